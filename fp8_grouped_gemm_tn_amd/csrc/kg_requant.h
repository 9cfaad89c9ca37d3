// kg_requant.h -- requantiser on MI355X (gfx950), C ABI: the step that produces the
// K-grouped GEMM's fp8 operands. Included at the end of kgwgrad.hip, so that it
// shares the library's single translation unit (and its device status word).
//
// The issue page "Is DeepGEMM directly applicable to backward in training?" explains
// that the weight-gradient GEMM needs its operands scaled per channel per 128 tokens
// of an expert, while the forward pass stores activations as fp8 with one scale per
// token per 128 channels, so a requantisation is needed in between (comments of
// soundOfDestiny, 2025-03-12). For expert g's token block kb (gran_k tokens from the
// expert's first token, the last one partial) and channel h, with x the binary32
// source value (bf16 widened, or e4m3 decoded times the token's 1x128 scale as one
// binary32 product) and amax the block's largest |x|:
//   fp32 scales: s = amax / 448 (1 if amax is 0) and q = e4m3(x / s), both binary32
//                quotients rounded to nearest;
//   UE8M0:       e = 127 + the smallest k with 2^k >= amax / 448, clamped to
//                [0, 254] (127 if amax is 0), and q = e4m3(x * 2^(127 - e));
// where e4m3() rounds to the nearest e4m3fn value, ties to the even code, with
// saturation at +-448 and the sign kept. Scale rows are packed per expert exactly
// as kg_wgrad reads them.
//
// Design: HBM-bound, one pass. A work item is (scale row, channel tile); each wave
// owns a 128-channel slab of the tile (16 lanes of 8 channels per row, 4 rows at a
// time) and, with the other waves of its slab, the block's rows. The raw source
// words stay in registers between a pass that takes the column maxima (lane shuffles,
// then one LDS exchange when a slab spans several waves) and a pass that writes
// 8-byte runs of fp8 codes. Loads and stores go through buffer resources over the
// block's rows, whose range check turns rows past the block into zero reads and
// dropped writes. A persistent grid walks the items; each workgroup scans ks once
// (the same scan as the GEMM) and finds an item's expert by binary search over the
// scale-row offsets.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kg_device.h"
#include "kg_sched.h"
#include "kgwgrad.h"

namespace kg {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

constexpr int kQCols = 128;      // channels per slab
constexpr int kQColGroups = 16;  // lanes per row: 8 channels each

// Slabs per item and waves per slab. gran_k 32: four one-wave slabs (8 rows per
// lane). gran_k 128: bf16 sources two slabs of two waves (16 rows per lane); e4m3
// sources four one-wave slabs (32 rows per lane, whose raw words take half the
// registers of bf16 ones). Measured on MI355X among 1-8 slabs of 1-4 waves.
constexpr int q_slabs(int src, int gran) { return gran == 32 ? 4 : src == KG_SRC_BF16 ? 2 : 4; }
constexpr int q_wps(int src, int gran) { return gran == 32 ? 1 : src == KG_SRC_BF16 ? 2 : 1; }

struct QParams {
  const unsigned char* X;  // bf16 or e4m3 [K_total, H]
  const float* xs;         // [K_total, H/128] for the e4m3 source
  unsigned char* Q;        // e4m3 [K_total, H]
  void* S;                 // fp32 or uint8 [nblk, H]
  const int32_t* ks;
  int G, H;
  int64_t K_total;
  int64_t s_rows;  // rows of S
  int gran;
};

// e4m3fn codes of four binary32 values, one per byte (a in the low byte): the
// nearest e4m3fn value, ties to the even code, sign kept (also for zero). gfx950's
// fp32 -> fp8 conversion instruction rounds this way; the values handed to it lie
// within +-448 (1 + 2^-18), where no saturation is needed (448 rounds to itself up to
// the midpoint 464), or are NaN, which it encodes as 0xFF and which is mapped to 0x7F
// (a byte whose low seven bits are all ones carries into bit 7 when 1 is added).
__device__ inline uint32_t e4m3x4(float a, float b, float c, float d) {
  uint32_t q = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  q = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)q, true);
  const uint32_t nan = ((q & 0x7F7F7F7Fu) + 0x01010101u) & q & 0x80808080u;
  return q ^ nan;
}

// Magnitudes above 448 (here only infinities) saturate to +-448; NaN stays NaN.
__device__ inline float e4m3_sat(float y) {
  return __builtin_fabsf(y) > 448.0f ? __builtin_copysignf(448.0f, y) : y;
}

// Codes of four values of one row: e4m3(x_k / s_k) for fp32 scales, e4m3(x_k * m_k)
// for UE8M0 (m_k = 2^(127 - e_k), an exact product).
//
// fp32 scales, common case (every s_k a normal number, so inv_k = fl(1 / s_k) = m_k
// is one too): y_k = x_k * inv_k lies within 2^-22 (relative) of the binary32 quotient
// fl(x_k / s_k). When y_k (1 - 2^-19) and y_k (1 + 2^-19) round to the same codes,
// rounding being monotone, fl(x_k / s_k) between them rounds to those codes too;
// otherwise (a value within about 2^-16 of a step of a rounding midpoint) the
// quotients are divided out. (A y_k that is subnormal or zero rounds to a signed zero
// code, as the quotient does.)
//
// EXACT (a column of the thread has a scale outside the normal range, or an infinite
// maximum): the quotients or products themselves, infinities saturated.
template <int SK, bool EXACT>
__device__ __forceinline__ uint32_t e4m3x4_scaled(const float (&x)[4], const float (&s)[4],
                                                  const float (&m)[4]) {
  if constexpr (EXACT) {
    float y[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      y[k] = e4m3_sat(SK == KG_E4M3_F32SCALE ? x[k] / s[k] : x[k] * m[k]);
    return e4m3x4(y[0], y[1], y[2], y[3]);
  } else if constexpr (SK == KG_E4M3_F32SCALE) {
    constexpr float lo = 1.0f - 0x1p-19f, hi = 1.0f + 0x1p-19f;
    float y[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) y[k] = x[k] * m[k];
    const uint32_t ql = e4m3x4(y[0] * lo, y[1] * lo, y[2] * lo, y[3] * lo);
    const uint32_t qh = e4m3x4(y[0] * hi, y[1] * hi, y[2] * hi, y[3] * hi);
    if (ql == qh) return ql;
    return e4m3x4(x[0] / s[0], x[1] / s[1], x[2] / s[2], x[3] / s[3]);
  } else {
    return e4m3x4(x[0] * m[0], x[1] * m[1], x[2] * m[2], x[3] * m[3]);
  }
}

// One thread's rows of codes: 8 channels (two 4-byte words) per row.
template <int SK, bool EXACT, int ROWS, int RG, class W>
__device__ __forceinline__ void store_codes(__amdgpu_buffer_rsrc_t qr, int H, uint32_t qoff,
                                            W widen, const float (&sdiv)[8],
                                            const float (&mul)[8]) {
#pragma unroll
  for (int i = 0; i < ROWS; ++i) {
    {
      float v[8];
      widen(i, v);
      uint32_t w4[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float xv[4] = {v[4 * h], v[4 * h + 1], v[4 * h + 2], v[4 * h + 3]};
        const float sv[4] = {sdiv[4 * h], sdiv[4 * h + 1], sdiv[4 * h + 2], sdiv[4 * h + 3]};
        const float mv[4] = {mul[4 * h], mul[4 * h + 1], mul[4 * h + 2], mul[4 * h + 3]};
        w4[h] = e4m3x4_scaled<SK, EXACT>(xv, sv, mv);
      }
      __builtin_amdgcn_raw_buffer_store_b64(v2u{w4[0], w4[1]}, qr, (int)qoff, i * RG * H, 2 /* nt */);
    }
  }
}

// E8M0 byte of the smallest power of two >= r (r = amax / 448 > 0), clamped to
// [0, 254].
__device__ inline int e8m0_ceil(float r) {
  const uint32_t b = __builtin_bit_cast(uint32_t, r);
  const int ex = (int)((b >> 23) & 0xFFu);
  const uint32_t mant = b & 0x7FFFFFu;
  int e;
  if (ex > 0)
    e = ex + (mant != 0 ? 1 : 0);   // (ex - 127 + carry) + 127
  else
    e = mant > (1u << 22) ? 1 : 0;  // subnormal r: 2^-126 > r > 2^-127 -> 1
  return e < 0 ? 0 : e > 254 ? 254 : e;
}

// Layout of an item (scale row, SLABS x 128 channels): wave w works on slab
// w / WPS; its lanes hold channel group cg = lane % 16 (8 channels) of rows
// rg + RG i, rg = 4 (w % WPS) + lane / 16, RG = 4 WPS.
template <int SRC, int SK, int GRAN>
__global__ __launch_bounds__(q_slabs(SRC, GRAN) * q_wps(SRC, GRAN) * 64) void kg_requant_kernel(
    QParams p) {
  constexpr int SLABS = q_slabs(SRC, GRAN), WPS = q_wps(SRC, GRAN);
  constexpr int NT = SLABS * WPS * 64;  // threads
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int64_t wsum_k[kMaxWaves];
  __shared__ int32_t wsum_b[kMaxWaves];
  __shared__ float red[NT / 64][kQCols];
  Sched s = sched_carve(smem, p.G);
  const int sched_rc =
      sched_build<NT>(p.ks, p.G, p.gran, p.K_total, s, wsum_k, wsum_b, false, p.s_rows);
  if (sched_rc != KG_OK) {
    if (blockIdx.x == 0 && threadIdx.x == 0) kgwgrad_status_word = sched_rc;
    return;
  }
  constexpr int RG = 4 * WPS;          // row groups per slab
  constexpr int kMaxRows = GRAN / RG;  // rows per thread
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int cg = tid % kQColGroups;
  const int slab = w / WPS;
  const int rg = (w % WPS) * 4 + lane / kQColGroups;
  const int ctiles = (p.H + kQCols * SLABS - 1) / (kQCols * SLABS);
  const int64_t nblk = s.boff[p.G];
  const int64_t total = nblk * ctiles;
  for (int64_t item = blockIdx.x; item < total; item += gridDim.x) {
    const int b = (int)(item / ctiles), ct = (int)(item - (int64_t)b * ctiles);
    // expert of scale row b: the last g with boff[g] <= b (binary search; empty
    // experts own no rows and are skipped by the strict comparison)
    int lo = 0, hi = p.G;  // boff[lo] <= b < boff[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s.boff[mid] <= b)
        lo = mid;
      else
        hi = mid;
    }
    const int g = lo;
    const int kb = b - s.boff[g];
    const int64_t t0 = s.off[g] + (int64_t)kb * p.gran;
    const int hs = (ct * SLABS + slab) * kQCols;  // the wave's first channel
    const int h0 = hs + cg * 8;
    // rows of the block this wave's slab covers (none past the last channel)
    const int rows = hs < p.H ? (int)min((int64_t)GRAN, s.off[g + 1] - t0) : 0;
    // buffers over those rows from the slab's first channel: rows past them read as
    // zeros and their codes are dropped by the range check (offsets below 2^32: H is
    // at most 2^23)
    constexpr int XB = SRC == KG_SRC_BF16 ? 2 : 1;  // source bytes per value
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.X + (t0 * p.H + hs) * XB), 0, (int)((uint32_t)rows * p.H * XB), kRsrcWord3);
    const uint32_t xoff = (uint32_t)(rg * p.H + cg * 8) * XB;
    constexpr int RAW = SRC == KG_SRC_BF16 ? 4 : 2;  // 32-bit words per row
    uint32_t raw[kMaxRows][RAW];
    float xsc[kMaxRows];
    const int HB = p.H / 128;
    const float* xs_rows = SRC == KG_SRC_BF16 ? nullptr : p.xs + t0 * HB + hs / 128;
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)xs_rows, 0, SRC == KG_SRC_BF16 ? 0 : rows * HB * 4, kRsrcWord3);
    // this thread's rows (rg, rg + RG, ...) of its 8 channels: every load is issued
    // before any is used
#pragma unroll
    for (int i = 0; i < kMaxRows; ++i) {
      const int soff = i * RG * p.H * XB;
      if constexpr (SRC == KG_SRC_BF16) {
        const v4u x = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)xoff, soff, 2 /* nt */);
        raw[i][0] = x.x;
        raw[i][1] = x.y;
        raw[i][2] = x.z;
        raw[i][3] = x.w;
        xsc[i] = 0.0f;
      } else {
        const v2u x = __builtin_amdgcn_raw_buffer_load_b64(xr, (int)xoff, soff, 2 /* nt */);
        raw[i][0] = x.x;
        raw[i][1] = x.y;
        xsc[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                               sr, rg * HB * 4, i * RG * HB * 4, 0));
      }
    }
    // binary32 values of row i (recomputed from the raw words in each pass, so that
    // only the raw words stay live between the passes)
    auto widen = [&](int i, float (&o)[8]) {
      if constexpr (SRC == KG_SRC_BF16) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          o[2 * k] = __builtin_bit_cast(float, raw[i][k] << 16);
          o[2 * k + 1] = __builtin_bit_cast(float, raw[i][k] & 0xFFFF0000u);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const v2bf d0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[i][k], 1.0f, false);
          const v2bf d1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[i][k], 1.0f, true);
          o[4 * k + 0] = (float)d0[0] * xsc[i];
          o[4 * k + 1] = (float)d0[1] * xsc[i];
          o[4 * k + 2] = (float)d1[0] * xsc[i];
          o[4 * k + 3] = (float)d1[1] * xsc[i];
        }
      }
    };
    float amax[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) amax[c] = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxRows; ++i) {
      float o[8];
      widen(i, o);
      // rows past the block are zeros here: they leave the maxima unchanged
#pragma unroll
      for (int c = 0; c < 8; ++c) amax[c] = __builtin_fmaxf(amax[c], __builtin_fabsf(o[c]));
    }
    // the passes must not share their values (an empty asm that the compiler takes
    // as rewriting the raw words: the values of the first pass die here)
#pragma unroll
    for (int i = 0; i < kMaxRows; ++i) {
#pragma unroll
      for (int k = 0; k < RAW; ++k) asm volatile("" : "+v"(raw[i][k]));
    }
    // column maxima: the 4 row groups of a wave share a channel group at lanes
    // l, l + 16, l + 32, l + 48; then across the slab's waves through LDS
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      amax[c] = __builtin_fmaxf(amax[c], __shfl_xor(amax[c], 16, 64));
      amax[c] = __builtin_fmaxf(amax[c], __shfl_xor(amax[c], 32, 64));
    }
    if constexpr (WPS > 1) {
      if (lane < kQColGroups) {
#pragma unroll
        for (int c = 0; c < 8; ++c) red[w][cg * 8 + c] = amax[c];
      }
      __syncthreads();
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float m = red[slab * WPS][cg * 8 + c];
#pragma unroll
        for (int ww = 1; ww < WPS; ++ww) m = __builtin_fmaxf(m, red[slab * WPS + ww][cg * 8 + c]);
        amax[c] = m;
      }
      __syncthreads();  // red is rewritten by the next item
    }
    // scales and codes
    float mul[8];   // UE8M0: 2^(127 - e); fp32 scales: 1 / s
    float sdiv[8];  // fp32 scales: s
    uint32_t eb[8];
    bool exact = false;  // a scale outside the normal range or an infinite maximum
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if constexpr (SK == KG_E4M3_F32SCALE) {
        sdiv[c] = amax[c] == 0.0f ? 1.0f : amax[c] / 448.0f;
        mul[c] = 1.0f / sdiv[c];
        exact |= !(sdiv[c] >= 0x1p-126f && sdiv[c] <= 0x1p126f);
      } else {
        const int e = amax[c] == 0.0f ? 127 : e8m0_ceil(amax[c] / 448.0f);
        eb[c] = (uint32_t)e;
        mul[c] = __builtin_ldexpf(1.0f, 127 - e);
        sdiv[c] = 1.0f;  // unused
        exact |= amax[c] > 3.40282347e38f;
      }
    }
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.Q + t0 * p.H + hs), 0, rows * p.H, kRsrcWord3);
    const uint32_t qoff = (uint32_t)(rg * p.H + cg * 8);
    if (exact)
      store_codes<SK, true, kMaxRows, RG>(qr, p.H, qoff, widen, sdiv, mul);
    else
      store_codes<SK, false, kMaxRows, RG>(qr, p.H, qoff, widen, sdiv, mul);
    if (rg == 0 && h0 < p.H) {
      if constexpr (SK == KG_E4M3_F32SCALE) {
        float4* dst = (float4*)((float*)p.S + (int64_t)b * p.H + h0);
        dst[0] = float4{sdiv[0], sdiv[1], sdiv[2], sdiv[3]};
        dst[1] = float4{sdiv[4], sdiv[5], sdiv[6], sdiv[7]};
      } else {
        uint32_t lo4 = 0, hi4 = 0;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          if (c < 4)
            lo4 |= eb[c] << (8 * c);
          else
            hi4 |= eb[c] << (8 * (c - 4));
        }
        *(uint2*)((unsigned char*)p.S + (int64_t)b * p.H + h0) = uint2{lo4, hi4};
      }
    }
  }
}

}  // namespace kg

using namespace kg;

extern "C" int kg_requant(const void* X, const float* xs, const int32_t* ks, int G, int H,
                          int64_t K_total, int gran_k, int src, int scale_kind, void* Q, void* S,
                          int64_t s_rows, void* stream) {
  if (src != KG_SRC_BF16 && src != KG_SRC_E4M3_1X128) return KG_ERR_DTYPE;
  if (scale_kind != KG_E4M3_F32SCALE && scale_kind != KG_E4M3_UE8M0) return KG_ERR_DTYPE;
  if (G < 0 || H < 0 || K_total < 0) return KG_ERR_SHAPE;
  if (gran_k != 32 && gran_k != 128) return KG_ERR_GRAN;
  if (G > kMaxGroups || H > (1 << 23)) return KG_ERR_UNSUPPORTED;
  if (K_total > INT32_MAX || (int64_t)H * K_total > ((int64_t)1 << 46)) return KG_ERR_UNSUPPORTED;
  if (G == 0 || H == 0) return KG_OK;
  if (ks == nullptr) return KG_ERR_NULL;
  if (K_total > 0 && (X == nullptr || Q == nullptr || S == nullptr)) return KG_ERR_NULL;
  if (src == KG_SRC_E4M3_1X128 && K_total > 0 && xs == nullptr) return KG_ERR_NULL;
  if (src == KG_SRC_BF16 && xs != nullptr) return KG_ERR_NULL;
  // S needs a row per block: at least ceil(K_total / gran_k) (the exact count,
  // sum ceil(ks[g] / gran_k), is checked on the device)
  if (K_total > 0 && (s_rows < 0 || s_rows < K_total / gran_k + (K_total % gran_k != 0)))
    return KG_ERR_SCALE_ROWS;
  if (H % 128 != 0) return KG_ERR_ALIGN;
  if (((uintptr_t)X & 15) || ((uintptr_t)Q & 15) || ((uintptr_t)S & 15) || ((uintptr_t)xs & 3) ||
      ((uintptr_t)ks & 3))
    return KG_ERR_ALIGN;
  const size_t qbytes = (size_t)K_total * H;
  const size_t xbytes = qbytes * (src == KG_SRC_BF16 ? 2 : 1);
  auto overlap = [](const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || !na || !nb) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
  };
  const int64_t srows = s_rows < K_total ? s_rows : K_total;
  const size_t sbytes = (size_t)srows * H * (scale_kind == KG_E4M3_F32SCALE ? 4 : 1);
  if (overlap(X, xbytes, Q, qbytes) || overlap(S, sbytes, Q, qbytes) ||
      overlap(X, xbytes, S, sbytes) || overlap(xs, (size_t)K_total * (H / 128) * 4, S, sbytes) ||
      overlap(ks, (size_t)G * 4, S, sbytes) || overlap(ks, (size_t)G * 4, Q, qbytes))
    return KG_ERR_ALIAS;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return KG_ERR_HIP;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return KG_ERR_HIP;
  QParams p;
  p.X = (const unsigned char*)X;
  p.xs = xs;
  p.Q = (unsigned char*)Q;
  p.S = S;
  p.ks = ks;
  p.G = G;
  p.H = H;
  p.K_total = K_total;
  p.s_rows = s_rows;
  p.gran = gran_k;
  // items are not known on the host (they depend on ks): enough persistent
  // workgroups for the largest case: 8192 threads per CU (more than stay resident;
  // the rest start as resident ones finish)
  const int slabs = q_slabs(src, gran_k), nt = slabs * q_wps(src, gran_k) * 64;
  const int tile = kQCols * slabs;  // channels per item
  const int64_t max_items = ((K_total + (int64_t)G * (gran_k - 1)) / gran_k) * ((H + tile - 1) / tile);
  const int64_t wgs = (int64_t)cus * 32 * 256 / nt;
  const int grid = (int)(max_items < wgs ? (max_items > 0 ? max_items : 1) : wgs);
  const void* fns[2][2][2] = {
      {{(const void*)kg_requant_kernel<KG_SRC_BF16, KG_E4M3_F32SCALE, 32>,
        (const void*)kg_requant_kernel<KG_SRC_BF16, KG_E4M3_F32SCALE, 128>},
       {(const void*)kg_requant_kernel<KG_SRC_BF16, KG_E4M3_UE8M0, 32>,
        (const void*)kg_requant_kernel<KG_SRC_BF16, KG_E4M3_UE8M0, 128>}},
      {{(const void*)kg_requant_kernel<KG_SRC_E4M3_1X128, KG_E4M3_F32SCALE, 32>,
        (const void*)kg_requant_kernel<KG_SRC_E4M3_1X128, KG_E4M3_F32SCALE, 128>},
       {(const void*)kg_requant_kernel<KG_SRC_E4M3_1X128, KG_E4M3_UE8M0, 32>,
        (const void*)kg_requant_kernel<KG_SRC_E4M3_1X128, KG_E4M3_UE8M0, 128>}}};
  const void* fn = fns[src == KG_SRC_BF16 ? 0 : 1][scale_kind == KG_E4M3_F32SCALE ? 0 : 1]
                      [gran_k == 32 ? 0 : 1];
  void* args[] = {&p};
  e = hipLaunchKernel(fn, dim3(grid), dim3(nt), args, sched_bytes(G), (hipStream_t)stream);
  if (e != hipSuccess) return KG_ERR_HIP;
  return KG_OK;
}
