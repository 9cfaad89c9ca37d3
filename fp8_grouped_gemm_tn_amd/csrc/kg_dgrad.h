// kg_dgrad.h -- M-grouped data-gradient GEMM (dgrad) on gfx950, C ABI kg_dgrad.
//
// The other backward GEMM of an MoE expert (GitHub issue "Is DeepGEMM directly
// applicable to backward in training?": the backward pass of a GEMM is two GEMMs,
// YouJiacheng 2025-02-26; the library first shipped this one, LyricZhao
// 2025-02-26; 128x128 block scales belong to weights only, activations carry 1x128
// scales, soundOfDestiny 2025-02-28). With y = x w^T in the forward pass, the data
// gradient is dx = dy w. Expert g owns the contiguous token rows [off[g], off[g+1])
// of dy; for such a row t and output column n:
//
//   D[t][n] = sum over 128-channel blocks kb of the contraction axis of
//             sa[kb][t] * sw[g][kb][n/128] * sum_{k in kb} dy[t][k] * w[g][k][n]
//
// with dy [M_total, K] e4m3 (K contiguous), sa [K/128, M_total] fp32, w [G, K, N]
// e4m3 (the forward pass's weight, N contiguous), sw [G, K/128, N/128] fp32, D
// [M_total, N] fp32 or bf16.
//
// Design (gfx950): one persistent launch; every workgroup scans the expert sizes
// (token offsets and tiles of 256 tokens per expert, kg_sched.h) and walks items
// (expert m-tile, n-tile of 128 columns: one weight-scale column), in panels of four
// m-tiles so that an XCD's workgroups share token rows and weight columns in its L2
// (measured +3-7% over a walk with n-tiles fastest). A stage is one
// 128-channel scale block: 256 token rows of 128 channel bytes (read by the MFMA
// lanes directly, the channels being contiguous) and 128 weight rows of 128 column
// bytes (read with transposing LDS reads, as the K-grouped kernel reads its
// operands), plus the 256 token scales; two stages in a ring. Token rows past the
// expert's end lie outside the buffer range and read as zero. Each block's partial
// sum (bf16 MFMA on exactly widened fp8, or the fp8 MFMA with KG_FLAG_FP8_MFMA) is
// multiplied by sa[kb][t] * sw[g][kb][n/128] and added to the fp32 accumulators.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kg_device.h"
#include "kg_sched.h"
#include "kgwgrad.h"

namespace kg {

struct DParams {
  const unsigned char* A;  // dy [M_total, K] e4m3fn
  const float* sa;         // [K/128, M_total]
  const unsigned char* W;  // [G, K, N] e4m3fn
  const float* sw;         // [G, K/128, N/128]
  float* D;                // [M_total, N] fp32, or bf16 in the bf16-output kernels
  const int32_t* ms;       // [G] tokens per expert
  int G, N, K;
  int64_t M_total;
  int tiles_n;
};

// 256 token rows x BN columns per workgroup (BN = 128 or 256); 8 waves (4 x 2) of
// 64 x BN/2; stages of 128 channels. The epilogue reuses the K-grouped kernel's
// (the same tile and wave layout as its 256 x BN configuration, whose stage area is
// no larger than ours). A wave's BN/2 columns lie inside one 128-column weight-scale
// block.
template <int BN_>
struct DCfgT {
  static constexpr int BM = 256, BN = BN_, TK = 128, NS = 2, THREADS = 512, WAVES = 8;
  static constexpr int WAVES_M = 4, WM = 64, WN = BN / 2, NI = 4, NJ = WN / 16;
  static constexpr int ROWA = TK + 16;  // one token: 128 channel bytes + 16 pad
  static constexpr int ROWB = BN + 16;  // one channel: BN column bytes + 16 pad
  static constexpr int CHA = ROWA / 16, CHB = ROWB / 16;  // 16-byte chunks per row (8 data)
  static constexpr int OPA = BM * ROWA, OPB = TK * ROWB;
  static constexpr int SA_OFF = OPA + OPB;
  static constexpr int STAGE = SA_OFF + BM * 4;
  static constexpr int LOADS_A = BM * CHA / 64, LOADS_B = TK * CHB / 64;
  static constexpr int LOADS = LOADS_A + LOADS_B + 1;  // + the token scales
  // the two 4-wave halves take turns issuing a whole stage (as the K-grouped fp8 kernels)
  static constexpr int SLOTS4 = (LOADS + 3) / 4;
  using Epi = std::conditional_t<BN == 128, CfgF8h, CfgF8>;
  static_assert(BM * CHA % 64 == 0 && TK * CHB % 64 == 0, "stage must be whole wave loads");
  static_assert(Epi::BM == BM && Epi::BN == BN && Epi::WAVES_M == WAVES_M &&
                    Epi::THREADS == THREADS && Epi::NI == NI && Epi::NJ == NJ,
                "epilogue geometry");
  static_assert(Epi::EPI_BYTES <= NS * STAGE, "epilogue fits the stages");
  static_assert(SLOTS4 <= 31, "loads per wave");
  static_assert(WN <= 128, "a wave's columns in one weight-scale block");
};
using DCfg = DCfgT<128>;
// the wide tile, for the fp8-MFMA mode: a third fewer operand bytes per flop
using DCfg256 = DCfgT<256>;
// largest G of the wide tile (its stages and the schedule must fit the LDS)
constexpr int kDgradWideMaxGroups = 512;

// This lane's byte offset for load k of a stage, relative to the stage's first token
// row / weight row / scale; pad chunks load zeros from an offset past any range.
template <class DC>
__device__ inline uint32_t dgrad_off(const DParams& p, int k, int lane) {
  if (k < DC::LOADS_A) {
    const int idx = 64 * k + lane, row = idx / DC::CHA, ch = idx - row * DC::CHA;
    return ch < DC::TK / 16 ? (uint32_t)(row * p.K + 16 * ch) : kOobOffset;
  } else if (k < DC::LOADS_A + DC::LOADS_B) {
    const int idx = 64 * (k - DC::LOADS_A) + lane, row = idx / DC::CHB,
              ch = idx - row * DC::CHB;
    return ch < DC::BN / 16 ? (uint32_t)(row * p.N + 16 * ch) : kOobOffset;
  }
  return 16 * lane;  // 256 token scales
}

// Stage kb of a tile: token rows [row0, row0 + rows) of dy, channels [128 kb, 128 kb +
// 128); weight rows 128 kb .. 128 kb + 127 of expert g, columns [n0, n0 + 128); the
// tokens' scales of block kb. Rows past `rows` read as zero.
template <class DC>
__device__ inline void dgrad_load_stage(const DParams& p, unsigned char* st,
                                        int64_t row0, int rows, int g, int kb, int n0) {
  const int w = uniform(threadIdx.x >> 6);
  const v4i ra = make_rsrc(p.A + row0 * p.K + (int64_t)kb * DC::TK,
                           (uint32_t)((rows - 1) * p.K + DC::TK));
  const v4i rb = make_rsrc(p.W + ((int64_t)g * p.K + (int64_t)kb * DC::TK) * p.N + n0,
                           (uint32_t)((DC::TK - 1) * p.N + DC::BN));
  const v4i rs = make_rsrc(p.sa + (int64_t)kb * p.M_total + row0, (uint32_t)(rows * 4));
  const uint32_t sA = lds_addr(st), sB = sA + DC::OPA, sS = sA + DC::SA_OFF;
  // the waves of half kb & 1 (one wave per SIMD) issue the whole stage
  if ((w >> 2) != (kb & 1)) return;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int s = 0; s < DC::SLOTS4; ++s) {
    const int k = (w & 3) + 4 * s;
    if (k < DC::LOADS_A + DC::LOADS_B) {
      const bool is_a = k < DC::LOADS_A;
      load16_lds(is_a ? ra : rb, is_a ? sA + 1024 * k : sB + 1024 * (k - DC::LOADS_A),
                 dgrad_off<DC>(p, k, lane));
    } else if (k == DC::LOADS_A + DC::LOADS_B) {
      load16_lds(rs, sS, dgrad_off<DC>(p, k, lane));
    }
  }
}

// One stage: acc[i][jn] += (sa[row] * swv) * (this block's partial of sub-tile (i, jn)).
// Sub-tile (i, jn) of wave (wm, wn): token rows wm*64 + 16 i .., columns wn*64 + 16 jn
// ..; this lane holds rows 4q .. 4q+3, column j of it. The rescale of a sub-tile is
// issued after the next sub-tile's MFMAs, so the two overlap.
template <bool FAST, class DC>
__device__ inline void dgrad_compute(const unsigned char* st, float swv,
                                     v4f (&acc)[DC::NI][DC::NJ]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int q = lane >> 4, j = lane & 15;
  const int wm = w % DC::WAVES_M, wn = w / DC::WAVES_M;
  const float* sS = (const float*)(st + DC::SA_OFF);
  const unsigned char* aRow = st + (wm * DC::WM + j) * DC::ROWA;
  auto rescale = [&](int pi, int pj, const v4f& x) {
    const v4f sa = *(const v4f*)(sS + wm * DC::WM + 16 * pi + 4 * q);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[pi][pj][r] = fmaf(sa[r] * swv, x[r], acc[pi][pj][r]);
  };
  constexpr int S = DC::NI * DC::NJ;
  if constexpr (FAST) {
    // fp8 MFMA 16x16x128: lane (q, i) holds channels 16q..16q+15 and 64+16q..64+16q+15
    // of its row (A: read directly) or column (B: four transposing reads of 8 rows)
    v8i af[DC::NI];
#pragma unroll
    for (int i = 0; i < DC::NI; ++i) {
      const unsigned char* r = aRow + 16 * i * DC::ROWA;
      const v4i lo4 = *(const v4i*)(r + 16 * q), hi4 = *(const v4i*)(r + 64 + 16 * q);
      af[i] = v8i{lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
    }
    const unsigned char* bBase =
        st + DC::OPA + (16 * q + (j >> 1)) * DC::ROWB + 8 * (j & 1) + wn * DC::WN;
    auto bfrag = [&](int jn) {
      const unsigned char* b = bBase + 16 * jn;
      const v2i x0 = tr8(b), x1 = tr8(b + 8 * DC::ROWB);
      const v2i x2 = tr8(b + 64 * DC::ROWB), x3 = tr8(b + 72 * DC::ROWB);
      return v8i{x0.x, x0.y, x1.x, x1.y, x2.x, x2.y, x3.x, x3.y};
    };
    v8i bcur = bfrag(0), bnext = bcur;
    v4f prev = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int jn = s / DC::NI, i = s % DC::NI;
      if (i == 0 && jn + 1 < DC::NJ) bnext = bfrag(jn + 1);
      const v4f part = mfma_fp8(af[i], bcur, v4f{0.f, 0.f, 0.f, 0.f});
      if (s > 0) rescale((s - 1) % DC::NI, (s - 1) / DC::NI, prev);
      prev = part;
      if (i == DC::NI - 1) bcur = bnext;
    }
    rescale(DC::NI - 1, DC::NJ - 1, prev);
  } else {
    // bf16 MFMA 16x16x32 on exactly widened fp8: step kk takes channels 32kk + 8q ..
    // 32kk + 8q + 7 of this lane's row (A) or column (B)
    constexpr int KK = DC::TK / 32;
    v8bf af[DC::NI][KK];
#pragma unroll
    for (int i = 0; i < DC::NI; ++i)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        af[i][kk] = widen8(*(const v2i*)(aRow + 16 * i * DC::ROWA + 32 * kk + 8 * q), 1.0f);
    const unsigned char* bBase =
        st + DC::OPA + (8 * q + (j >> 1)) * DC::ROWB + 8 * (j & 1) + wn * DC::WN;
    v2i rnext[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) rnext[kk] = tr8(bBase + 32 * kk * DC::ROWB);
    // one column of sub-tiles at a time, its NI MFMA chains advanced together; the
    // previous column is rescaled between this column's first MFMAs
    v8bf bf[KK];
    v4f xprev[DC::NI];
#pragma unroll
    for (int jn = 0; jn < DC::NJ; ++jn) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) bf[kk] = widen8(rnext[kk], 1.0f);
      if (jn + 1 < DC::NJ) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          rnext[kk] = tr8(bBase + 32 * kk * DC::ROWB + 16 * (jn + 1));
      }
      v4f x[DC::NI];
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
        for (int i = 0; i < DC::NI; ++i)
          x[i] = mfma_bf16(af[i][kk], bf[kk], kk == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : x[i]);
        if (kk == 0 && jn > 0) {
#pragma unroll
          for (int i = 0; i < DC::NI; ++i) rescale(i, jn - 1, xprev[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < DC::NI; ++i) xprev[i] = x[i];
    }
#pragma unroll
    for (int i = 0; i < DC::NI; ++i) rescale(i, DC::NJ - 1, xprev[i]);
  }
}

template <bool FAST, bool OUTB, class DC = DCfg>
__global__ __launch_bounds__(DC::THREADS, 1) void kg_dgrad_kernel(DParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int64_t wsum_k[kMaxWaves];
  __shared__ int32_t wsum_b[kMaxWaves];
  // token offsets (s.off) and tiles of BM tokens per expert (s.boff)
  Sched s = sched_carve(smem + DC::NS * DC::STAGE, p.G);
  if (sched_build<DC::THREADS>(p.ms, p.G, DC::BM, p.M_total, s, wsum_k, wsum_b) != KG_OK) {
    if (blockIdx.x == 0 && threadIdx.x == 0) kgwgrad_status_word = KG_ERR_KSUM;
    return;
  }
  const int total = s.boff[p.G] * p.tiles_n;
  const int grid = gridDim.x, b = blockIdx.x;
  // as in the K-grouped kernel: XCD-contiguous runs when the items take several rounds
  const int slot = (grid % 8 == 0 && total > grid) ? (b % 8) * (grid / 8) + b / 8 : b;
  const int nk = p.K / DC::TK, nsc = p.N / 128;  // weight-scale blocks along K and N
  for (int base = 0; base < total; base += grid) {
    const int idx = base + slot;
    if (idx >= total) break;
    // panels of kPanelM m-tiles, m-tiles fastest within a panel: an XCD's run of
    // items covers a few m-tiles (token rows) by several n-tiles (weight columns) that
    // its L2 shares, instead of one m-tile by many n-tiles
    const int mt_total = s.boff[p.G];
    const int per_panel = kPanelM * p.tiles_n;
    const int panel = idx / per_panel, wi = idx - panel * per_panel;
    const int pm = min(kPanelM, mt_total - panel * kPanelM);
    const int mtg = panel * kPanelM + wi % pm, nt = wi / pm;
    // expert of m-tile mtg: the last g with boff[g] <= mtg (boff[G] > mtg)
    int lo_g = 0, hi_g = p.G;
    while (hi_g - lo_g > 1) {
      const int mid = (lo_g + hi_g) >> 1;
      if (s.boff[mid] <= mtg) lo_g = mid; else hi_g = mid;
    }
    const int g = uniform(lo_g);
    const int64_t row0 = s.off[g] + (int64_t)(mtg - s.boff[g]) * DC::BM;
    const int rows = uniform((int)min((int64_t)DC::BM, s.off[g + 1] - row0));
    const int n0 = nt * DC::BN;
    const float* swg = p.sw + (int64_t)g * nk * nsc + nt * (DC::BN / 128);
    __syncthreads();  // the previous item is done with the stage buffers
    v4f acc[DC::NI][DC::NJ];
#pragma unroll
    for (int i = 0; i < DC::NI; ++i)
#pragma unroll
      for (int jn = 0; jn < DC::NJ; ++jn) acc[i][jn] = v4f{0.f, 0.f, 0.f, 0.f};
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the previous item's stores
    if (nk > 0) dgrad_load_stage<DC>(p, smem, row0, rows, g, 0, n0);
    for (int kb = 0; kb < nk; ++kb) {
      // stage kb is in buffer kb % 2; stage kb + 1 loads into the other one while
      // stage kb computes
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __syncthreads();
      if (kb + 1 < nk)
        dgrad_load_stage<DC>(p, smem + ((kb + 1) & 1) * DC::STAGE, row0, rows, g, kb + 1, n0);
      // this wave's weight-scale column (its BN/2 columns lie in one 128-column block)
      const float swv = swg[(int64_t)kb * nsc + (threadIdx.x >> 6) / DC::WAVES_M * DC::WN / 128];
      dgrad_compute<FAST, DC>(smem + (kb & 1) * DC::STAGE, swv, acc);
    }
    store_tile_gen<typename DC::Epi, false, OUTB>(smem, acc,
                                           OUTB ? (float*)((unsigned short*)p.D + row0 * p.N + n0)
                                                : p.D + row0 * p.N + n0,
                                           p.N, rows, DC::BN, nullptr, 0, nullptr, nullptr, 0,
                                           0);
  }
}

}  // namespace kg

extern "C" int kg_dgrad(const void* A, const float* sa, const void* W, const float* sw, void* D,
                        const int32_t* ms, int G, int N, int K, int64_t M_total, int flags,
                        void* stream) {
  using namespace kg;
  if (flags & ~(KG_FLAG_FP8_MFMA | KG_FLAG_D_BF16)) return KG_ERR_DTYPE;
  const bool fast = (flags & KG_FLAG_FP8_MFMA) != 0, outb = (flags & KG_FLAG_D_BF16) != 0;
  if (G < 0 || N < 0 || K < 0 || M_total < 0) return KG_ERR_SHAPE;
  if (G > kMaxGroups || N > (1 << 24) || K > (1 << 24) || M_total > INT32_MAX)
    return KG_ERR_UNSUPPORTED;
  if (K % 128 != 0 || N % 128 != 0) return KG_ERR_ALIGN;
  if (G == 0 || N == 0 || M_total == 0) return KG_OK;
  if (D == nullptr || ms == nullptr) return KG_ERR_NULL;
  if (K > 0 && (A == nullptr || sa == nullptr || W == nullptr || sw == nullptr))
    return KG_ERR_NULL;
  if (((uintptr_t)A & 15) || ((uintptr_t)sa & 15) || ((uintptr_t)W & 15) || ((uintptr_t)sw & 3) ||
      ((uintptr_t)D & 15) || ((uintptr_t)ms & 3))
    return KG_ERR_ALIGN;
  if ((int64_t)DCfg::BM * K > INT32_MAX || (int64_t)DCfg::TK * N > INT32_MAX ||
      (int64_t)DCfg::BM * N * 4 > INT32_MAX)
    return KG_ERR_UNSUPPORTED;  // 32-bit offsets within a tile
  const size_t dbytes = (size_t)M_total * N * (outb ? 2 : 4);
  auto overlap = [](const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || !na || !nb) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
  };
  if (overlap(A, (size_t)M_total * K, D, dbytes) ||
      overlap(W, (size_t)G * K * N, D, dbytes) ||
      overlap(sa, (size_t)(K / 128) * M_total * 4, D, dbytes) ||
      overlap(sw, (size_t)G * (K / 128) * (N / 128) * 4, D, dbytes) ||
      overlap(ms, (size_t)G * 4, D, dbytes))
    return KG_ERR_ALIAS;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return KG_ERR_HIP;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return KG_ERR_HIP;
  // the wide tile for the fp8-MFMA mode when N allows it and the schedule fits beside
  // its stages
  const bool wide = fast && N % DCfg256::BN == 0 && G <= kDgradWideMaxGroups;
  const void* fns[2][2] = {{(const void*)kg_dgrad_kernel<false, false>,
                            (const void*)kg_dgrad_kernel<false, true>},
                           {(const void*)kg_dgrad_kernel<true, false>,
                            (const void*)kg_dgrad_kernel<true, true>}};
  const void* fns_wide[2] = {(const void*)kg_dgrad_kernel<true, false, DCfg256>,
                             (const void*)kg_dgrad_kernel<true, true, DCfg256>};
  const void* fn = wide ? fns_wide[outb ? 1 : 0] : fns[fast ? 1 : 0][outb ? 1 : 0];
  const int stage_bytes = wide ? DCfg256::NS * DCfg256::STAGE : DCfg::NS * DCfg::STAGE;
  const int bn = wide ? DCfg256::BN : DCfg::BN;
  const int lds = stage_bytes + sched_bytes(G);
  {
    static std::mutex mu;
    static bool set[64][2][2][2];
    std::lock_guard<std::mutex> lk(mu);
    if (dev < 0 || dev >= 64) return KG_ERR_HIP;
    if (!set[dev][wide][fast][outb]) {
      e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                              stage_bytes + sched_bytes(wide ? kDgradWideMaxGroups : kMaxGroups));
      if (e != hipSuccess) return KG_ERR_HIP;
      set[dev][wide][fast][outb] = true;
    }
  }
  DParams p;
  p.A = (const unsigned char*)A;
  p.sa = sa;
  p.W = (const unsigned char*)W;
  p.sw = sw;
  p.D = (float*)D;
  p.ms = ms;
  p.G = G;
  p.N = N;
  p.K = K;
  p.M_total = M_total;
  p.tiles_n = N / bn;
  // at most ceil(M_total / BM) + G m-tiles (the experts' sizes are only known on the
  // device)
  const int64_t max_items = (M_total / DCfg::BM + G) * (int64_t)p.tiles_n;  // BM alike
  if (max_items > INT32_MAX) return KG_ERR_UNSUPPORTED;
  const int grid = (int)(max_items < cus ? max_items : cus);
  void* args[] = {&p};
  e = hipLaunchKernel(fn, dim3(grid), dim3(DCfg::THREADS), args, lds, (hipStream_t)stream);
  if (e != hipSuccess) return KG_ERR_HIP;
  return KG_OK;
}
