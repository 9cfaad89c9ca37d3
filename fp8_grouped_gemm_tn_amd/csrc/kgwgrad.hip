// kgwgrad.hip -- K-grouped weight-gradient GEMM on MI355X (gfx950), C ABI.
//
// For every expert g, D[g] = C[g] (or 0) + sum over the expert's token blocks of
// (sa_kb outer sb_kb) * (A_kb^T . B_kb), where expert g owns token rows
// [off[g], off[g+1]) of A [K_total, M] and B [K_total, N] (page "How to Use
// DeepGEMM Weight Gradient Kernels for Training Backward Passes", sections
// "Understanding K-Grouped Weight Gradient Kernels" and "FP8 Implementation
// Example"). Scales are shared by each gran_k-token run of one expert and are
// applied to the run's partial sum after it is accumulated (GitHub issue "Is
// DeepGEMM directly applicable to backward in training?", qijiaxing 2025-03-26).
//
// Design (MI355X-first, not the pages' TMA design):
//  * One persistent launch. Every workgroup rebuilds the schedule in LDS
//    (kg_sched.h) and walks work items (expert, m-tile, n-tile), longest experts
//    first. The hardware places workgroup b on XCD b % 8. When the items take
//    several rounds of the grid, each XCD's workgroups take a contiguous run of
//    neighbouring tiles of one expert and share their operand rows in that XCD's
//    L2; in a single round each XCD takes an eighth of the GEMM items and an eighth
//    of the fill items, so that every L2 serves GEMM tiles.
//  * Empty experts become copy/fill items (D = C, or 0), placed between the live
//    experts' items in multi-round launches so their stores overlap GEMM tiles.
//  * Operands move global -> LDS with buffer loads that write LDS directly; token
//    rows past the expert's end are outside the buffer's range and read as zero,
//    which masks ragged tails in both operands.
//  * The contraction runs over tokens, the leading (strided) dimension of both
//    operands: LDS holds token-major rows, and transposing LDS reads
//    (ds_read_b64_tr_b8 / _tr_b16) hand every lane token-contiguous fragments.
//  * Math policies:
//      bf16              16x16x32 bf16 MFMA, fp32 accumulation.
//      fp8, precise      fragments are widened to bf16 in registers (exact for
//                        e4m3; an E8M0 scale is folded into the widening, also
//                        exact) and contracted with the bf16 MFMA, whose fp32
//                        accumulation is exact to rounding. fp32 scales: the
//                        block's four chained MFMAs give its partial sum, which is
//                        rescaled by sa (x) sb on the VALU and accumulated.
//      fp8, fast         the 16x16x128 fp8 MFMA (the scaled form applies E8M0
//                        scales per 32 tokens). gfx950 sums each group of 8 fp8
//                        products aligned to the largest with about 13 bits, so
//                        this policy trades accuracy (~1e-4 of sum|ab|) for twice
//                        the MFMA rate. Selected by KG_FLAG_FP8_MFMA.
//  * 8 waves per workgroup (2 per SIMD); two LDS stages (block kb+1 loads while
//    block kb computes); an LDS-staged epilogue with float4 C loads and
//    non-temporal float4 D stores.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "kg_device.h"
#include "kg_sched.h"
#include "kgwgrad.h"

// Per-device status word (KG_OK or KG_ERR_KSUM); read and cleared by kg_status.
__device__ int kgwgrad_status_word;

namespace kg {

// F32S32: fp32 scales per 32 tokens (a scale row per 32-token block).
enum Kind { F32S = 0, E8M0 = 1, BF16 = 2, F32S32 = 3 };

struct Params {
  const unsigned char* A;
  const unsigned char* sa;
  const unsigned char* B;
  const unsigned char* sb;
  const float* C;  // bf16 [G, M, N] in the bf16-output kernels
  float* D;        // bf16 [G, M, N] in the bf16-output kernels
  const int32_t* ks;
  int G, M, N;

  int64_t K_total;
  int64_t scale_rows;     // rows of sa and sb (INT64_MAX for bf16: no scales)
  uint32_t lda_b, ldb_b;  // K-major kernels: row strides of A and B in bytes
  int gran;  // tokens per scale row
  int tiles_m, tiles_n;
  // stream-K mode when ws != nullptr: two partial-tile slots per workgroup and an
  // arrival counter per workgroup (for the cut tile whose first stage it holds)
  float* ws;
  int* wscnt;
};

// Tile configuration: BM x BN per workgroup, THREADS / 64 waves as WAVES_M x WAVES_N,
// TK tokens per LDS stage, NS stages in the ring, ELT bytes per operand element,
// SCALE_BYTES of scale tile per operand. PIPE: one 32-token MFMA step per stage, and
// each wave reads stage kb+1's fragments into registers before it issues stage kb's
// MFMAs (bf16 only).
// SWZ (token-major fp8 only): LDS rows without padding; each row's 16-byte chunks are
// XOR-permuted by a key of the row index (logical chunk c of row r sits at
// c ^ swz_key(r)), so that the rows the transposing reads of a half-wave touch still
// fall in distinct banks. The LDS the padding took then holds a third stage.
template <int BM_, int BN_, int WAVES_M_, int TK_, int NS_, int ELT_, int SCALE_BYTES_,
          int THREADS_ = 512, bool PIPE_ = false, bool NT_ = false, bool SWZ_ = false>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, TK = TK_, NS = NS_, ELT = ELT_;
  static constexpr int THREADS = THREADS_, WAVES = THREADS_ / 64;
  static constexpr bool PIPE = PIPE_;
  // NT: K-major operands (token index contiguous in memory)
  static constexpr bool NT = NT_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES / WAVES_M_;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int NI = WM / 16, NJ = WN / 16;
  // Token-major operands: LDS rows of one token each, BM (BN) elements + PAD bytes.
  // With the lane-to-row maps of the compute policies, the rows one half-wave reads
  // then start in distinct bank windows (fp8: 16-byte reads, row stride = 17 x 16 B;
  // bf16: 32-byte reads, row stride = 34 x 16 B).
  // K-major operands: LDS rows of one channel each, the stage's TK tokens (128
  // bytes); every pair of rows is followed by 16 bytes of padding, so that the 16
  // rows of a sub-tile, read at one byte offset, start in 16 distinct 4-bank groups.
  // The load layout's "row" is then a pair of channels (ROW = 272 bytes).
  static constexpr bool SWZ = SWZ_;
  static constexpr int PAD = SWZ ? 0 : NT ? 16 : ELT == 2 ? 32 : 16;
  static constexpr int ROWA = NT ? 2 * TK * ELT + PAD : BM * ELT + PAD;
  static constexpr int ROWB = NT ? 2 * TK * ELT + PAD : BN * ELT + PAD;
  static constexpr int CHA = ROWA / 16, CHB = ROWB / 16;  // 16-byte chunks per row
  static constexpr int DCA = (ROWA - PAD) / 16;           // of which data
  static constexpr int DCB = (ROWB - PAD) / 16;
  static constexpr int RA = NT ? BM / 2 : TK, RB = NT ? BN / 2 : TK;  // LDS rows per operand
  // K-major: byte offset of channel row r within its operand, and of 16 channels
  static __host__ __device__ constexpr int nt_row(int r) { return (r >> 1) * ROWA + (r & 1) * TK * ELT; }
  // Swizzled rows (SWZ): LDS chunk ch of row r holds the row's 16-byte chunk
  // ch ^ swz_key(r). The 16 rows that a half-wave's transposing reads name then fall
  // in distinct bank groups: a row of 256 bytes spans all 64 banks (key r mod 16),
  // rows of 128 bytes alternate between the two bank halves (key r / 2 mod 8).
  // Measured with an LDS probe: the key r mod 8 left these reads 2-way conflicted.
  static __host__ __device__ constexpr int swz_key(int r, int row_bytes) {
    return row_bytes >= 256 ? (r & 15) : ((r >> 1) & 7);
  }
  static constexpr int NT_SUB = 8 * ROWA;
  // A stage is LOADS wave loads of 1 KB: LOADS_A of A rows, LOADS_B of B rows and,
  // with scales, one scale tile per operand. Load k of a stage is issued by wave
  // k % WAVES, so the first HEAVY waves issue PER + 1 loads and the others PER.
  static constexpr int LOADS_A = RA * CHA / 64, LOADS_B = RB * CHB / 64;
  // scale tiles of more than 1 KB take SCALE_LOADS wave loads per operand
  static constexpr int SCALE_LOADS = SCALE_BYTES_ > 1024 ? SCALE_BYTES_ / 1024 : 1;
  static constexpr int LOADS = LOADS_A + LOADS_B + (SCALE_BYTES_ > 0 ? 2 * SCALE_LOADS : 0);
  static constexpr int SLOTS = (LOADS + WAVES - 1) / WAVES;  // per wave
  // ALT (fp8, two plain stages, 8 waves): the waves of one half (one wave per SIMD)
  // issue all of a stage's loads, the halves taking turns by stage, so that on every
  // SIMD one wave can run MFMAs while the other waits to issue loads (measured +2-6%
  // on the fp8 workloads; the load-bound bf16 half tiles lose 10% with half the
  // waves issuing loads)
  // (with three stages too: a wave then owns every other stage's loads)
  static constexpr bool ALT = (NS == 2 || NS == 3) && WAVES == 8 && !PIPE && ELT == 1;
  static constexpr int SLOTS4 = (LOADS + 3) / 4;
  // loads of a stage that wave w of the issuing half issues (ALT)
  static __host__ __device__ constexpr int alt_loads(int w) { return (LOADS - (w & 3) + 3) / 4; }
  static constexpr int PER = LOADS / WAVES, HEAVY = LOADS % WAVES;
  static constexpr int OPA = RA * ROWA, OPB = RB * ROWB;
  static constexpr int SCALE_BYTES = SCALE_BYTES_;
  static constexpr int SA_OFF = OPA + OPB, SB_OFF = SA_OFF + SCALE_BYTES;
  static constexpr int STAGE = SB_OFF + SCALE_BYTES;
  // epilogue passes: column pair pc (sub-tile columns 2pc, 2pc+1 of every wave) x
  // row block ph of EPI_ROWS rows; LDS holds the pass's accumulators (padded rows)
  // and its C tile (dense rows of EPI_COLS floats)
  static constexpr int EPI_COLS = WAVES_N * 32;
  static constexpr int EPI_STRIDE = EPI_COLS + 4;
  static constexpr int EPI_ROWS =
      BM * (EPI_STRIDE + EPI_COLS) * 4 <= NS * STAGE ? BM
      : (BM / 2) * (EPI_STRIDE + EPI_COLS) * 4 <= NS * STAGE ? BM / 2 : BM / 4;
  static constexpr int EPI_C_OFF = EPI_ROWS * EPI_STRIDE * 4;
  static constexpr int EPI_BYTES = EPI_C_OFF + EPI_ROWS * EPI_COLS * 4;
  static constexpr int EPI_CPR = EPI_COLS / 4;                    // float4 per row
  static constexpr int EPI_PER = EPI_ROWS * EPI_CPR / THREADS;    // float4 per thread
  static constexpr int EPI_LOADS = EPI_ROWS * EPI_CPR / 64;       // wave loads of C
  static_assert(WM % 16 == 0 && WN % 32 == 0, "wave tile must be whole sub-tile pairs");
  static_assert(RA * CHA % 64 == 0 && RB * CHB % 64 == 0, "stage must be whole wave loads");
  static_assert(!NT || (TK * ELT == 128 && !PIPE), "K-major rows: 128 bytes, plain stages");
  static_assert(!SWZ || (!NT && !PIPE && ELT == 1 && (BM * ELT == 128 || BM * ELT == 256) &&
                          (BN * ELT == 128 || BN * ELT == 256)),
                "swizzled rows: token-major fp8, rows of 128 or 256 bytes");
  static_assert(EPI_BYTES <= NS * STAGE, "epilogue must fit the stages");
  static_assert(NS >= 2, "at least two stages");
  static_assert(EPI_ROWS * EPI_CPR % THREADS == 0, "epilogue work must split evenly");
  static_assert(!PIPE || (TK == 32 && NS >= 3 && ELT == 2), "pipelined stages: bf16, 32 tokens");
  static_assert(EPI_ROWS % WM == 0, "epilogue row blocks hold whole wave rows");
  static_assert(SCALE_BYTES <= 1024 || SCALE_BYTES % 1024 == 0, "whole wave loads per scale tile");
  static_assert((PER + 1) * (NS - 1) <= 63, "stage loads in flight fit the wait counter");
};

// fp8 with the fp8 MFMA: 256 x 256 per workgroup, 64 x 128 per wave, two stages of
// 128 tokens (one MFMA consumes 128 tokens)
using CfgF8 = Cfg<256, 256, 4, 128, 2, 1, 1024>;
// fp8 widened to bf16 with fp32 scales: 256 x 128 per workgroup, 64 x 64 per wave (the
// widened fragments and the block partials need the registers a wider wave tile would
// take; UE8M0 scales, folded into the widening, need no partials and use CfgF8: 17%
// faster on 256 experts); two stages of 128. Long experts take CfgF8 instead, each
// column of sub-tiles rescaled right after its MFMAs (fewer conversions per MFMA).
using CfgF8h = Cfg<256, 128, 4, 128, 2, 1, 1024>;
// CfgF8h with three stages in the LDS the row padding took (swizzled rows): two stages in
// flight instead of one, for problems whose schedule leaves the LDS room (the kernel's
// loads are bound by the bytes in flight per CU, not by bandwidth)
using CfgF8h3 = Cfg<256, 128, 4, 128, 3, 1, 1024, 512, false, false, true>;
// fp8 with fp32 scales per 32 tokens: the 256 x 128 tile of CfgF8h, four scale rows
// per 128-token stage (4 KB of scale tile per operand)
using CfgF8h32 = Cfg<256, 128, 4, 128, 2, 1, 4096>;
// bf16: 256 x 256 per workgroup, 8 waves of 64 x 128 (two per SIMD), a ring of four
// 32-token stages; each wave reads stage kb+1's fragments while it runs stage kb's
// MFMAs
using CfgB16 = Cfg<256, 256, 4, 32, 4, 2, 0, 512, true>;
// bf16, 128 x 256 per workgroup (64 x 64 per wave) for problems with few tiles
using CfgB16s = Cfg<128, 256, 2, 64, 2, 2, 0>;

// K-major operands: the same tiles with 128-byte channel rows per stage (fp8: 128
// tokens; bf16: 64 tokens in two plain stages instead of the pipelined ring)
using CfgF8N = Cfg<256, 256, 4, 128, 2, 1, 1024, 512, false, true>;
using CfgF8hN = Cfg<256, 128, 4, 128, 2, 1, 1024, 512, false, true>;
using CfgF8h32N = Cfg<256, 128, 4, 128, 2, 1, 4096, 512, false, true>;
using CfgB16N = Cfg<256, 256, 4, 64, 2, 2, 0, 512, false, true>;
using CfgB16sN = Cfg<128, 256, 2, 64, 2, 2, 0, 512, false, true>;

// the configurations of one operand layout
template <bool NT>
struct Cfgs {
  using F8 = CfgF8;
  using F8h = CfgF8h;
  using F8hD = CfgF8h3;  // CfgF8h with three stages (when the LDS holds them)
  using F8h32 = CfgF8h32;
  using B16 = CfgB16;
  using B16s = CfgB16s;
};
template <>
struct Cfgs<true> {
  using F8 = CfgF8N;
  using F8h = CfgF8hN;
  using F8hD = CfgF8hN;
  using F8h32 = CfgF8h32N;
  using B16 = CfgB16N;
  using B16s = CfgB16sN;
};

// This lane's global byte offsets for its loads of a stage (slot s: load
// k = w + WAVES * s), relative to the stage's first byte (row 0, column m0 or n0) of
// the operand the load belongs to; the same for every stage and item of a launch.
// Padding chunks get an offset past any buffer range, so they load zeros. Scale
// loads are addressed per stage.
template <class CF>
struct LoadOffsets {
  uint32_t off[CF::SLOTS];
};

// Global byte offset of this lane's chunk in operand load k (k < LOADS_A + LOADS_B),
// relative to the stage's first byte of the operand; padding chunks are out of range.
template <class CF>
__device__ inline uint32_t load_off(const Params& p, int k, int lane) {
  const bool is_a = k < CF::LOADS_A;
  const int idx = 64 * (is_a ? k : k - CF::LOADS_A) + lane;
  if constexpr (CF::NT) {
    // chunk ch of channel pair `pair`: chunk ch & 7 of channel 2 pair + ch / 8
    const int pair = idx / CF::CHA, ch = idx - pair * CF::CHA;
    return ch < CF::DCA ? (2 * pair + (ch >> 3)) * (is_a ? p.lda_b : p.ldb_b) + 16 * (ch & 7)
                        : kOobOffset;
  } else if (is_a) {
    const int row = idx / CF::CHA, ch = idx - row * CF::CHA;
    // swizzled rows: LDS chunk ch of row `row` holds the row's chunk ch ^ swz_key(row)
    const int gch = CF::SWZ ? ch ^ CF::swz_key(row, CF::ROWA) : ch;
    return ch < CF::DCA ? row * (uint32_t)(p.M * CF::ELT) + 16 * gch : kOobOffset;
  } else {
    const int row = idx / CF::CHB, ch = idx - row * CF::CHB;
    const int gch = CF::SWZ ? ch ^ CF::swz_key(row, CF::ROWB) : ch;
    return ch < CF::DCB ? row * (uint32_t)(p.N * CF::ELT) + 16 * gch : kOobOffset;
  }
}

template <class CF>
__device__ inline LoadOffsets<CF> load_offsets(const Params& p) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t eM = p.M * CF::ELT, eN = p.N * CF::ELT;
  LoadOffsets<CF> o;
#pragma unroll
  for (int s = 0; s < CF::SLOTS; ++s) {
    const int k = w + CF::WAVES * s;
    o.off[s] = kOobOffset;
    if constexpr (CF::NT) {
      // chunk ch of channel pair `pair`: chunk ch & 7 of channel 2 pair + ch / 8
      if (k < CF::LOADS_A + CF::LOADS_B) {
        const bool is_a = k < CF::LOADS_A;
        const int idx = 64 * (is_a ? k : k - CF::LOADS_A) + lane;
        const int pair = idx / CF::CHA, ch = idx - pair * CF::CHA;
        if (ch < CF::DCA)
          o.off[s] = (2 * pair + (ch >> 3)) * (is_a ? p.lda_b : p.ldb_b) + 16 * (ch & 7);
      }
    } else if (k < CF::LOADS_A) {
      const int idx = 64 * k + lane;
      const int row = idx / CF::CHA, ch = idx - row * CF::CHA;
      const int gch = CF::SWZ ? ch ^ CF::swz_key(row, CF::ROWA) : ch;
      if (ch < CF::DCA) o.off[s] = row * eM + 16 * gch;
    } else if (k < CF::LOADS_A + CF::LOADS_B) {
      const int idx = 64 * (k - CF::LOADS_A) + lane;
      const int row = idx / CF::CHB, ch = idx - row * CF::CHB;
      const int gch = CF::SWZ ? ch ^ CF::swz_key(row, CF::ROWB) : ch;
      if (ch < CF::DCB) o.off[s] = row * eN + 16 * gch;
    }
  }
  return o;
}

// Wait until this wave's loads of all but the last n stages it issued are done
// (0 <= n <= NS - 2): loads complete in issue order, and every stage is PER or
// PER + 1 loads of this wave.
template <int PERW, int NS>
__device__ inline void wait_stages_n(int n) {
  if (NS > 3 && n >= 2) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * PERW));
  } else if (n == 1) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(PERW));
  } else {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }
}

template <class CF>
__device__ inline void wait_stages(int n) {
  static_assert(CF::NS <= 4, "waits cover at most two stages in flight");
  const int w = threadIdx.x >> 6;
  if (CF::HEAVY > 0 && w < CF::HEAVY)
    wait_stages_n<CF::PER + 1, CF::NS>(n);
  else
    wait_stages_n<CF::PER, CF::NS>(n);
}

// ---------------------------------------------------------------- bf16 output

typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// four bf16 codes (two per dword, lower half first) -> fp32, exact
__device__ inline v4f bf16x4_to_f32(v2u x) {
  return v4f{__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xFFFF0000u),
             __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xFFFF0000u)};
}

// fp32 -> four bf16 codes, rounded to nearest, ties to even
__device__ inline v2u f32x4_to_bf16(v4f v) {
  return __builtin_bit_cast(v2u, __builtin_convertvector(v, v4bf));
}

// ---------------------------------------------------------------- fill

// D tile = C tile (or 0) for an empty expert.
template <class CF>
__device__ void fill_tile_bf16(const Params& p, int g, int m0, int n0) {
  const int t = threadIdx.x;
  constexpr int kCols8 = CF::BN / 8;  // 16-byte runs of 8 bf16 per tile row
  constexpr int kPer = CF::BM * kCols8 / CF::THREADS;
  constexpr int kBatch = kPer < 16 ? kPer : 16;
  static_assert(kPer % kBatch == 0, "fill batches");
  const size_t base = (size_t)g * p.M * p.N;
  const unsigned short* C = (const unsigned short*)p.C;
  unsigned short* D = (unsigned short*)p.D;
#pragma unroll
  for (int b0 = 0; b0 < kPer; b0 += kBatch) {
    v4u v[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int e = t + CF::THREADS * (b0 + k);
      const int r = e / kCols8, c8 = e - r * kCols8;
      const int m = m0 + r, n = n0 + 8 * c8;
      v[k] = v4u{0u, 0u, 0u, 0u};
      if (C && m < p.M && n < p.N)
        v[k] = __builtin_nontemporal_load((const v4u*)(C + base + (size_t)m * p.N + n));
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int e = t + CF::THREADS * (b0 + k);
      const int r = e / kCols8, c8 = e - r * kCols8;
      const int m = m0 + r, n = n0 + 8 * c8;
      if (m < p.M && n < p.N)
        __builtin_nontemporal_store(v[k], (v4u*)(D + base + (size_t)m * p.N + n));
    }
  }
}

template <class CF, bool OUTB = false>
__device__ void fill_tile(const Params& p, int g, int m0, int n0) {
  if (p.C == p.D) return;  // in place: D already holds C
  if constexpr (OUTB) {
    fill_tile_bf16<CF>(p, g, m0, n0);
    return;
  }
  const int t = threadIdx.x;
  constexpr int kCols4 = CF::BN / 4;
  constexpr int kPer = CF::BM * kCols4 / CF::THREADS;
  constexpr int kBatch = kPer < 16 ? kPer : 16;
  static_assert(kPer % kBatch == 0, "fill batches");
  const size_t base = (size_t)g * p.M * p.N;
#pragma unroll
  for (int b0 = 0; b0 < kPer; b0 += kBatch) {
    v4f v[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int e = t + CF::THREADS * (b0 + k);
      const int r = e / kCols4, c4 = e - r * kCols4;
      const int m = m0 + r, n = n0 + 4 * c4;
      v[k] = v4f{0.f, 0.f, 0.f, 0.f};
      if (p.C && m < p.M && n < p.N)
        v[k] = __builtin_nontemporal_load((const v4f*)(p.C + base + (size_t)m * p.N + n));
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int e = t + CF::THREADS * (b0 + k);
      const int r = e / kCols4, c4 = e - r * kCols4;
      const int m = m0 + r, n = n0 + 4 * c4;
      if (m < p.M && n < p.N)
        __builtin_nontemporal_store(v[k], (v4f*)(p.D + base + (size_t)m * p.N + n));
    }
  }
}

// ---------------------------------------------------------------- epilogue

// Thread element idx of a pass -> LDS row / float column and global (m, n).
template <class CF>
__device__ inline void epi_coords(int idx, int ph, int pc, int m0, int n0, int& row, int& lcol,
                                  int& m, int& n) {
  row = idx / CF::EPI_CPR;
  const int c4 = idx - row * CF::EPI_CPR;
  const int strip = c4 >> 3;  // wave column
  lcol = 4 * c4;
  m = m0 + ph * CF::EPI_ROWS + row;
  n = n0 + strip * CF::WN + 32 * pc + 4 * (c4 & 7);
}

// Stream-K epilogue of one tile: acc (this lane's 4 rows x 1 column of each 16x16 sub-tile),
// plus an optional addend tile `add` (C), plus `nparts` partial tiles (stream-K),
// added in that order, stored to `dst`. Tiles are row-major from the tile origin:
// dst and add with row stride `ld` floats (rows and columns past rows x cols are
// not stored; addend bytes past add_bytes read as zero), partial 0 at parts0 and
// partial q > 0 at parts + (q - 1) * part_stride floats, each with row stride BN. Per pass (EPI_ROWS rows x two 16-column sub-tiles of
// every wave column): the waves owning the pass's rows write their accumulators to
// LDS while the addend goes global -> LDS by buffer loads; every thread adds the
// addend to its float4 runs, then each partial in turn through the same LDS
// buffer, and stores whole float4 runs along N, non-temporally.
// With OUTB, dst holds bf16 (the sums are rounded to nearest even; no addend or
// partials are allowed then).
template <class CF, bool SYS_STORE = false, bool OUTB = false>
__device__ inline void store_tile_gen(unsigned char* lds, const v4f (&acc)[CF::NI][CF::NJ],
                                      float* dst, int ld, int rows, int cols, const float* add,
                                      uint32_t add_bytes, const float* parts0, const float* parts,
                                      size_t part_stride, int nparts) {
  static_assert(!(OUTB && SYS_STORE), "bf16 output is stored with ordinary stores");
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int q = lane >> 4, j = lane & 15;
  const int wm = w % CF::WAVES_M, wn = w / CF::WAVES_M;
  float* e = (float*)lds;
  const float* cl = (const float*)(lds + CF::EPI_C_OFF);
  const uint32_t cl_lds = lds_addr(lds + CF::EPI_C_OFF);
  const v4i rc = make_rsrc(add, add_bytes);
  constexpr int kPH = CF::BM / CF::EPI_ROWS;
#pragma unroll
  for (int ph = 0; ph < kPH; ++ph) {
#pragma unroll
    for (int pc = 0; pc < CF::NJ / 2; ++pc) {
      __syncthreads();  // stage buffers / previous pass no longer read
      if (add) {
        for (int k = w; k < CF::EPI_LOADS; k += CF::WAVES) {
          int row, lcol, m, n;
          epi_coords<CF>(64 * k + lane, ph, pc, 0, 0, row, lcol, m, n);
          load16_lds(rc, cl_lds + 1024 * k, (uint32_t)((m * ld + n) * 4));
        }
      }
      const int wrow0 = wm * CF::WM - ph * CF::EPI_ROWS;  // this wave's first row in the pass
      if (wrow0 >= 0 && wrow0 < CF::EPI_ROWS) {
#pragma unroll
        for (int i = 0; i < CF::NI; ++i)
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int row = wrow0 + 16 * i + 4 * q + r;
              const int col = wn * 32 + 16 * jj + j;
              e[row * CF::EPI_STRIDE + col] = acc[i][2 * pc + jj][r];
            }
      }
      wait_all_and_barrier();  // accumulators and addend of this pass are in LDS
      // partial tiles: every thread adds each one, in order, to its own float4 runs
      // of the staged sums (LDS read-modify-write; no cross-thread hazards)
      for (int pq = 0; pq < nparts; ++pq) {
        if (add || pq > 0) {
#pragma unroll
          for (int k = 0; k < CF::EPI_PER; ++k) {
            int row, lcol, m, n;
            epi_coords<CF>(threadIdx.x + CF::THREADS * k, ph, pc, 0, 0, row, lcol, m, n);
            *(v4f*)(e + row * CF::EPI_STRIDE + lcol) += *(const v4f*)(cl + row * CF::EPI_COLS + lcol);
          }
        }
        const v4i rp = make_rsrc(pq == 0 ? parts0 : parts + (size_t)(pq - 1) * part_stride,
                                 CF::BM * CF::BN * 4);
        __syncthreads();  // the previous addend in LDS is no longer read
        for (int k = w; k < CF::EPI_LOADS; k += CF::WAVES) {
          int row, lcol, m, n;
          epi_coords<CF>(64 * k + lane, ph, pc, 0, 0, row, lcol, m, n);
          load16_lds_sys(rp, cl_lds + 1024 * k, (uint32_t)((m * CF::BN + n) * 4));
        }
        wait_all_and_barrier();
      }
      // the LDS addend buffer holds C (no partials) or the last partial
      const bool addl = add != nullptr || nparts > 0;
#pragma unroll
      for (int k = 0; k < CF::EPI_PER; ++k) {
        int row, lcol, m, n;
        epi_coords<CF>(threadIdx.x + CF::THREADS * k, ph, pc, 0, 0, row, lcol, m, n);
        if (m < rows && n < cols) {
          v4f v = *(const v4f*)(e + row * CF::EPI_STRIDE + lcol);
          if (addl) v += *(const v4f*)(cl + row * CF::EPI_COLS + lcol);
          if constexpr (SYS_STORE)
            store16_sys(dst, (uint32_t)((size_t)rows * ld * 4), (uint32_t)((m * ld + n) * 4), v);
          else if constexpr (OUTB)
            __builtin_nontemporal_store(
                f32x4_to_bf16(v), (v2u*)((unsigned short*)dst + (size_t)m * ld + n));
          else
            __builtin_nontemporal_store(v, (v4f*)(dst + (size_t)m * ld + n));
        }
      }
    }
  }
}

// acc + C + partial tiles -> D for expert g's tile at (m0, n0) (stream-K mode; the
// partial tiles as for store_tile_gen).
template <class CF>
__device__ inline void store_tile_parts(const Params& p, unsigned char* lds, int g, int m0, int n0,
                                        const v4f (&acc)[CF::NI][CF::NJ], const float* parts0,
                                        const float* parts, size_t part_stride, int nparts) {
  const size_t org = (size_t)g * p.M * p.N + (size_t)m0 * p.N + n0;
  // C from the tile origin to the end of the expert's matrix
  const uint32_t cbytes = (uint32_t)((((size_t)(p.M - m0) - 1) * p.N + (p.N - n0)) * 4);
  store_tile_gen<CF>(lds, acc, p.D + org, p.N, p.M - m0, p.N - n0, p.C ? p.C + org : nullptr,
                     cbytes, parts0, parts, part_stride, nparts);
}

// acc (this lane's 4 rows x 1 column of each 16x16 sub-tile) + C -> D. Per pass:
// the C tile goes global -> LDS by buffer loads (rows past M read as zero) while
// the waves owning the pass's rows write their accumulators to LDS; then every
// thread adds and stores whole float4 runs along N, non-temporally.
template <class CF, bool OUTB>
__device__ inline void store_tile(const Params& p, unsigned char* lds, int g, int m0, int n0,
                                  const v4f (&acc)[CF::NI][CF::NJ]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int q = lane >> 4, j = lane & 15;
  const int wm = w % CF::WAVES_M, wn = w / CF::WAVES_M;
  float* e = (float*)lds;
  const float* cl = (const float*)(lds + CF::EPI_C_OFF);
  const size_t gbase = (size_t)g * p.M * p.N;
  // C of this expert, from (m0, 0) to the expert's end (4- or 2-byte elements)
  constexpr int osz = OUTB ? 2 : 4;
  const v4i rc = make_rsrc((const unsigned char*)p.C + (gbase + (size_t)m0 * p.N) * osz,
                           (uint32_t)((size_t)(p.M - m0) * p.N * osz));
  constexpr int kPH = CF::BM / CF::EPI_ROWS;
#pragma unroll
  for (int ph = 0; ph < kPH; ++ph) {
#pragma unroll
    for (int pc = 0; pc < CF::NJ / 2; ++pc) {
      __syncthreads();  // stage buffers / previous pass no longer read
      if (p.C && !OUTB) {
        for (int k = w; k < CF::EPI_LOADS; k += CF::WAVES) {
          int row, lcol, m, n;
          epi_coords<CF>(64 * k + lane, ph, pc, m0, n0, row, lcol, m, n);
          load16_lds(rc, lds_addr(lds + CF::EPI_C_OFF) + 1024 * k,
                     (uint32_t)(((m - m0) * p.N + n) * 4));
        }
      } else if (p.C) {
        // bf16 C: lane j of load k brings the 8 columns of float4 runs 2j and 2j+1
        // (same row and wave strip); in LDS, bf16 element (row, lcol) sits at
        // row * EPI_COLS + lcol
        for (int k = w; k < CF::EPI_LOADS / 2; k += CF::WAVES) {
          int row, lcol, m, n;
          epi_coords<CF>(2 * (64 * k + lane), ph, pc, m0, n0, row, lcol, m, n);
          load16_lds(rc, lds_addr(lds + CF::EPI_C_OFF) + 1024 * k,
                     (uint32_t)(((m - m0) * p.N + n) * 2));
        }
      }
      const int wrow0 = wm * CF::WM - ph * CF::EPI_ROWS;  // this wave's first row in the pass
      if (wrow0 >= 0 && wrow0 < CF::EPI_ROWS) {
#pragma unroll
        for (int i = 0; i < CF::NI; ++i)
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int row = wrow0 + 16 * i + 4 * q + r;
              const int col = wn * 32 + 16 * jj + j;
              e[row * CF::EPI_STRIDE + col] = acc[i][2 * pc + jj][r];
            }
      }
      wait_all_and_barrier();  // accumulators and C of this pass are in LDS
#pragma unroll
      for (int k = 0; k < CF::EPI_PER; ++k) {
        int row, lcol, m, n;
        epi_coords<CF>(threadIdx.x + CF::THREADS * k, ph, pc, m0, n0, row, lcol, m, n);
        if (m < p.M && n < p.N) {
          v4f v = *(const v4f*)(e + row * CF::EPI_STRIDE + lcol);
          if constexpr (!OUTB) {
            if (p.C) v += *(const v4f*)(cl + row * CF::EPI_COLS + lcol);
            __builtin_nontemporal_store(v, (v4f*)(p.D + gbase + (size_t)m * p.N + n));
          } else {
            if (p.C)
              v += bf16x4_to_f32(*(const v2u*)((const unsigned short*)cl + row * CF::EPI_COLS + lcol));
            __builtin_nontemporal_store(
                f32x4_to_bf16(v), (v2u*)((unsigned short*)p.D + gbase + (size_t)m * p.N + n));
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- stage loads

// Stage kb of an item: token rows [TK*kb, TK*kb + TK) of the expert's A and B
// slices (rows past the expert's end read as zero), plus the scale rows that
// cover them.
template <int KIND, class CF>
__device__ inline void load_stage(const Params& p, const LoadOffsets<CF>& lo, unsigned char* st,
                                  int64_t t_begin, int Kg, int boff_g, int kb, int m0, int n0) {
  // the wave index is uniform: the slot tests below become scalar selects
  const int lane = threadIdx.x & 63, w = uniform(threadIdx.x >> 6);
  const int rows = uniform(min(CF::TK, Kg - CF::TK * kb));
  const int64_t t0 = t_begin + (int64_t)CF::TK * kb;
  const int eM = p.M * CF::ELT, eN = p.N * CF::ELT;
  v4i ra, rb;
  // K-major: chunks of the stage's last 16-byte unit that hold no token of the
  // expert load as zero (one partial chunk per row remains, see nt_tail_zero)
  const bool nt_tail = CF::NT && rows < CF::TK;
  if constexpr (CF::NT) {
    // the resource starts at (channel m0, token t0) and ends with the operand: rows
    // past the last channel read as zero. The host keeps the offsets of 256 rows
    // below 0xFFFFFF80; a longer range is cut at kOobOffset, so that the masked
    // chunks (offset kOobOffset) stay out of range.
    const int64_t ta = t0 * CF::ELT;
    const int64_t na = (int64_t)(p.M - m0) * p.lda_b - ta, nb = (int64_t)(p.N - n0) * p.ldb_b - ta;
    ra = make_rsrc(p.A + (int64_t)m0 * p.lda_b + ta, (uint32_t)min(na, (int64_t)kOobOffset));
    rb = make_rsrc(p.B + (int64_t)n0 * p.ldb_b + ta, (uint32_t)min(nb, (int64_t)kOobOffset));
  } else {
    // the resource starts at (row 0, column m0) and ends with the expert's last row
    // of this stage: rows past it, and columns past the row end of the last row,
    // read as zero (rows * eM reaches 2^31 for M = 2^24: unsigned arithmetic)
    ra = make_rsrc(p.A + t0 * eM + m0 * CF::ELT, (uint32_t)rows * (uint32_t)eM - (uint32_t)(m0 * CF::ELT));
    rb = make_rsrc(p.B + t0 * eN + n0 * CF::ELT, (uint32_t)rows * (uint32_t)eN - (uint32_t)(n0 * CF::ELT));
  }
  const uint32_t sA = lds_addr(st), sB = sA + CF::OPA;
  auto issue = [&](int k, uint32_t off0) {
    if (k < CF::LOADS_A + CF::LOADS_B) {
      // one load instruction per slot; the operand (resource and LDS base) is a
      // scalar select, not a branch
      const bool is_a = k < CF::LOADS_A;
      uint32_t off = off0;
      if (nt_tail) {
        // chunks past the expert's tokens load zeros. The partial chunk of the
        // operand's last channel could run past the end of the buffer: it loads
        // the 16 bytes that end there instead (nt_tail_zero moves its bytes into
        // place).
        const int idx = 64 * (is_a ? k : k - CF::LOADS_A) + lane;
        const int pair = idx / CF::CHA, ch = idx - pair * CF::CHA;
        const int c = ch & 7, nbytes = rows * CF::ELT;
        if (ch < CF::DCA) {
          if (16 * c >= nbytes) {
            off = kOobOffset;
          } else if (16 * c + 16 > nbytes && 2 * pair + (ch >> 3) == (is_a ? p.M - m0 : p.N - n0) - 1) {
            const int64_t d = t0 * CF::ELT + 16 * c + 16 - (is_a ? p.lda_b : p.ldb_b);
            if (d > 0) off -= (uint32_t)d;
          }
        }
      }
      load16_lds(is_a ? ra : rb, is_a ? sA + 1024 * k : sB + 1024 * (k - CF::LOADS_A), off);
    } else if (KIND != BF16 && k < CF::LOADS) {
      // scale tiles: TK/gran rows of BM (BN) scales (fp32 or E8M0), or the one row of
      // the block when gran >= TK; rows are stored one after the other in LDS. Load q
      // of an operand's SCALE_LOADS brings its q-th kilobyte.
      constexpr int esz = KIND == F32S || KIND == F32S32 ? 4 : 1;
      // rows per stage: compile-time for the fp32 kinds (gran 128 and 32)
      const int per = KIND == F32S ? 1 : KIND == F32S32 ? CF::TK / 32
                      : p.gran >= CF::TK ? 1 : CF::TK / p.gran;
      const int gran = KIND == F32S ? 128 : KIND == F32S32 ? 32 : p.gran;
      const int nb_g = (Kg + gran - 1) / gran;
      const int r0 = (CF::TK * kb) / gran;
      const int nrows = uniform(min(per, nb_g - r0));
      const int64_t r = (int64_t)boff_g + r0;
      const int qs = k - (CF::LOADS_A + CF::LOADS_B);
      const bool is_a = CF::SCALE_LOADS == 1 ? qs == 0 : qs < CF::SCALE_LOADS;
      const int part = CF::SCALE_LOADS == 1 ? 0 : (is_a ? qs : qs - CF::SCALE_LOADS);
      const int ext = is_a ? p.M : p.N, c0 = is_a ? m0 : n0;
      const int width = is_a ? CF::BM : CF::BN;
      const int cpr = width * esz / 16;  // 16-byte chunks per scale row
      const int idx = 64 * part + lane;
      const int sr = idx / cpr, c = idx - sr * cpr;
      const v4i rs = make_rsrc((is_a ? p.sa : p.sb) + r * ext * esz, (uint32_t)(nrows * ext * esz));
      load16_lds(rs, sA + (is_a ? CF::SA_OFF : CF::SB_OFF) + 1024 * part,
                 sr < per ? (uint32_t)(sr * ext * esz + c0 * esz + 16 * c) : kOobOffset);
    }
  };
  if constexpr (CF::ALT) {
    if ((w >> 2) != (kb & 1)) return;  // the other half issues this stage
#pragma unroll
    for (int s = 0; s < CF::SLOTS4; ++s) {
      const int k = (w & 3) + 4 * s;
      if (k < CF::LOADS) issue(k, k < CF::LOADS_A + CF::LOADS_B ? load_off<CF>(p, k, lane) : 0u);
    }
  } else {
#pragma unroll
    for (int s = 0; s < CF::SLOTS; ++s) issue(w + CF::WAVES * s, lo.off[s]);
  }
}

// K-major stage whose last 16-byte unit is partial (the expert's token count times
// the element size is not a multiple of 16): that chunk of every row of both
// operands also holds the next bytes of the row (another expert's tokens, or
// padding). Zero its bytes past the expert's last token. In the operand's last
// channel, whose chunk was loaded d bytes early when it would have run past the end
// of the buffer (load_stage), first move the valid bytes down by d. The stage's
// loads must be complete and visible; the caller barriers afterwards.
template <class CF>
__device__ inline void nt_tail_zero(const Params& p, unsigned char* st, int rows, int64_t t0,
                                    int m0, int n0) {
  const int nbytes = rows * CF::ELT;
  const int c = nbytes >> 4, rem = nbytes & 15;
  for (int r = threadIdx.x; r < CF::BM + CF::BN; r += CF::THREADS) {
    const bool is_a = r < CF::BM;
    const int rr = is_a ? r : r - CF::BM;
    unsigned char* chp = st + (is_a ? 0 : CF::OPA) + CF::nt_row(rr) + 16 * c;
    if (rr == (is_a ? p.M - m0 : p.N - n0) - 1) {
      const int d = (int)(t0 * CF::ELT + 16 * c + 16 - (is_a ? p.lda_b : p.ldb_b));
      if (d > 0)
        for (int x = 0; x < rem; ++x) chp[x] = chp[x + d];  // rem + d <= 16
    }
    v4i v = *(v4i*)chp;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int keep = rem - 4 * w;  // bytes of dword w to keep
      const unsigned m = keep >= 4 ? 0xFFFFFFFFu : keep <= 0 ? 0u : (1u << (8 * keep)) - 1u;
      v[w] &= (int)m;
    }
    *(v4i*)chp = v;
  }
}

// ---------------------------------------------------------------- fragments

// fast fp8: the 32 contraction bytes of lane group q for the 16x16x128 MFMA. Byte
// run p (8 bytes, p = 0..3) of group q falls in the instruction's 32-element scale
// block b = 2*(p>>1) + (q>>1); it carries tokens 32b + 16*(p&1) + 8*(q&1) + 0..7 of
// the stage, so every scale block of 32 tokens lands in one hardware block, and a
// half-wave's reads touch 16 consecutive token rows. `p` is the lane's base: row
// 8*(q&1) + 32*(q>>1) + j/2, byte 8*(j&1).
__device__ inline int fast_row(int q, int j) { return 8 * (q & 1) + 32 * (q >> 1) + (j >> 1); }

template <int ROW>
__device__ inline v8i frag_f8(const unsigned char* p) {
  const v2i x0 = tr8(p + 0 * ROW);
  const v2i x1 = tr8(p + 16 * ROW);
  const v2i x2 = tr8(p + 64 * ROW);
  const v2i x3 = tr8(p + 80 * ROW);
  return v8i{x0.x, x0.y, x1.x, x1.y, x2.x, x2.y, x3.x, x3.y};
}

// precise fp8: 8 tokens widened to bf16 (times a power-of-two scale, exact).
__device__ inline v8bf widen8(v2i x, float scale) {
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)x.x, scale, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)x.x, scale, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)x.y, scale, false);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)x.y, scale, true);
  return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Fragment readers. `base` is this lane's base in the operand: token-major, its row
// of the transposing read; K-major, its channel row of the wave's first sub-tile
// plus its first token byte (the K-major offsets below are then immediates). Both
// layouts give a lane the same tokens, so the MFMAs see the same operands, except in
// the K-major paths that read whole 16-byte runs instead (the split runs of the
// token-major order conflicted in the LDS banks, also when the compiler merged two
// steps' reads into one ds_read2_b64): bf16 (compute_bf16) and fp32 scales per 128
// tokens in both modes (rdf8n; compute_precise_f32s); the MFMA sums those orders with
// different roundings.
// fp8, tokens 32kk + 8q .. +7 of sub-tile row (column) i (K-major base: + 8q):
template <class CF, int ROW>
__device__ inline v2i rd8(const unsigned char* base, int i, int kk) {
  if constexpr (CF::NT)
    return *(const v2i*)(base + i * CF::NT_SUB + 32 * kk);
  else
    return tr8(base + 32 * kk * ROW + 16 * i);
}

// fast fp8, the 32 bytes of frag_f8: token runs 32(q>>1) + 8(q&1) + {0, 16, 64, 80}
// (K-major base: + 32(q>>1) + 8(q&1))
template <class CF, int ROW>
__device__ inline v8i rdf8(const unsigned char* base, int i) {
  if constexpr (CF::NT) {
    const unsigned char* r = base + i * CF::NT_SUB;
    const v2i x0 = *(const v2i*)(r);
    const v2i x1 = *(const v2i*)(r + 16);
    const v2i x2 = *(const v2i*)(r + 64);
    const v2i x3 = *(const v2i*)(r + 80);
    return v8i{x0.x, x0.y, x1.x, x1.y, x2.x, x2.y, x3.x, x3.y};
  } else {
    return frag_f8<ROW>(base + 16 * i);
  }
}

// bf16 token-major, tokens 32kk + 16h + 4q .. +3 of sub-tile row (column) i (the
// K-major bf16 path reads 8 consecutive tokens per lane instead, see compute_bf16)
template <class CF, int ROW>
__device__ inline v4bf rd16(const unsigned char* base, int i, int kk, int h) {
  return tr16(base + (32 * kk + 16 * h) * ROW + 32 * i);
}

// ---------------------------------------------------------------- compute policies

// All policies: wave (wm, wn) owns rows [wm*WM, +WM) and cols [wn*WN, +WN) of the
// tile; acc[i][jn] is the 16x16 sub-tile (i, jn), this lane holding rows 4q..4q+3,
// column j.

// fast fp8 + fp32 scales: one fp8 MFMA per sub-tile gives the block partial; the
// rescale of sub-tile s-1 is issued after the MFMA of sub-tile s so they overlap.
// K-major fp8-MFMA mode with fp32 scales: lane group q takes tokens 32q .. 32q+31 of
// the 128-token step, two aligned 16-byte reads (the split runs of the token-major
// order conflict in the LDS banks; the block partial is rescaled after the MFMA, so
// any order shared by A and B gives it, with its own roundings)
template <class CF>
__device__ inline v8i rdf8n(const unsigned char* base, int i) {
  if constexpr (CF::NT) {
    const unsigned char* r = base + i * CF::NT_SUB;
    const v4i x0 = *(const v4i*)(r);
    const v4i x1 = *(const v4i*)(r + 16);
    return v8i{x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  } else {
    return rdf8<CF, CF::ROWA>(base, i);
  }
}

template <class CF>
__device__ __forceinline__ void compute_fast_f32s(const unsigned char* st, v4f (&acc)[CF::NI][CF::NJ]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int q = lane >> 4, j = lane & 15;
  const int wm = w % CF::WAVES_M, wn = w / CF::WAVES_M;
  const int lrow = fast_row(q, j);
  const int lbyte = CF::NT ? 32 * q : 32 * (q >> 1) + 8 * (q & 1);  // K-major: first token byte
  const unsigned char* aBase = CF::NT ? st + CF::nt_row(wm * CF::WM + j) + lbyte
                                      : st + lrow * CF::ROWA + 8 * (j & 1) + wm * CF::WM;
  const unsigned char* bBase = CF::NT ? st + CF::OPA + CF::nt_row(wn * CF::WN + j) + lbyte
                                      : st + CF::OPA + lrow * CF::ROWB + 8 * (j & 1) + wn * CF::WN;
  const float* sSa = (const float*)(st + CF::SA_OFF);
  const float* sSb = (const float*)(st + CF::SB_OFF);
  v8i af[CF::NI];
#pragma unroll
  for (int i = 0; i < CF::NI; ++i) af[i] = CF::NT ? rdf8n<CF>(aBase, i) : rdf8<CF, CF::ROWA>(aBase, i);
  constexpr int S = CF::NI * CF::NJ;
  v8i bcur = CF::NT ? rdf8n<CF>(bBase, 0) : rdf8<CF, CF::ROWB>(bBase, 0), bnext = bcur;
  v4f prev = v4f{0.f, 0.f, 0.f, 0.f};
  // rescale of sub-tile (pi, pj): acc += (sa[rows] * sb[col]) * partial
  auto rescale = [&](int pi, int pj, const v4f& part) {
    const v4f sa = *(const v4f*)(sSa + wm * CF::WM + 16 * pi + 4 * q);
    const float sb = sSb[wn * CF::WN + 16 * pj + j];
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[pi][pj][r] = fmaf(sa[r] * sb, part[r], acc[pi][pj][r]);
  };
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int jn = s / CF::NI, i = s % CF::NI;
    if (i == 0 && jn + 1 < CF::NJ) bnext = CF::NT ? rdf8n<CF>(bBase, jn + 1) : rdf8<CF, CF::ROWB>(bBase, jn + 1);
    const v4f part = mfma_fp8(af[i], bcur, v4f{0.f, 0.f, 0.f, 0.f});
    if (s > 0) rescale((s - 1) % CF::NI, (s - 1) / CF::NI, prev);
    prev = part;
    if (i == CF::NI - 1) bcur = bnext;
  }
  rescale(CF::NI - 1, CF::NJ - 1, prev);
}

// fast fp8 + E8M0: the scaled MFMA takes lane 16b+i's exponent for (row i, 32-token
// block b) and accumulates directly.
template <class CF>
__device__ __forceinline__ void compute_fast_e8m0(const unsigned char* st, int gran,
                                         v4f (&acc)[CF::NI][CF::NJ]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int q = lane >> 4, j = lane & 15;
  const int wm = w % CF::WAVES_M, wn = w / CF::WAVES_M;
  const int lrow = fast_row(q, j);
  const int lbyte = 32 * (q >> 1) + 8 * (q & 1);  // K-major: first token byte
  const unsigned char* aBase = CF::NT ? st + CF::nt_row(wm * CF::WM + j) + lbyte
                                      : st + lrow * CF::ROWA + 8 * (j & 1) + wm * CF::WM;
  const unsigned char* bBase = CF::NT ? st + CF::OPA + CF::nt_row(wn * CF::WN + j) + lbyte
                                      : st + CF::OPA + lrow * CF::ROWB + 8 * (j & 1) + wn * CF::WN;
  const unsigned char* sSa = st + CF::SA_OFF;
  const unsigned char* sSb = st + CF::SB_OFF;
  const int srow = gran == 32 ? q : 0;
  v8i af[CF::NI];
  int ea[CF::NI];
#pragma unroll
  for (int i = 0; i < CF::NI; ++i) {
    af[i] = rdf8<CF, CF::ROWA>(aBase, i);
    ea[i] = sSa[srow * CF::BM + wm * CF::WM + 16 * i + j];
  }
  v8i bcur = rdf8<CF, CF::ROWB>(bBase, 0);
#pragma unroll
  for (int jn = 0; jn < CF::NJ; ++jn) {
    const v8i bnext = jn + 1 < CF::NJ ? rdf8<CF, CF::ROWB>(bBase, jn + 1) : bcur;
    const int eb = sSb[srow * CF::BN + wn * CF::WN + 16 * jn + j];
#pragma unroll
    for (int i = 0; i < CF::NI; ++i) acc[i][jn] = mfma_fp8_e8m0(af[i], bcur, acc[i][jn], ea[i], eb);
    bcur = bnext;
  }
}

// precise fp8: lane base row 8q + j/2; MFMA kk (tokens 32kk..32kk+31) takes this
// lane's 8 tokens 32kk+8q..32kk+8q+7 for its row (A) or column (B).

// precise fp8 + fp32 scales: a 128-token block spans 128/TK stages. Each stage
// chains its TK/32 bf16 MFMAs (K = 32 each) onto part[i][jn]; on the block's last
// stage (PROMOTE) the finished partial sum of sub-tile (i, jn) is rescaled by
// sa (x) sb on the VALU, one sub-tile behind the MFMAs, and part is cleared.
template <class CF, bool PROMOTE>
__device__ __forceinline__ void compute_precise_f32s(const unsigned char* st, v4f (&acc)[CF::NI][CF::NJ],
                                            v4f (&part)[CF::NI][CF::NJ]) {
  constexpr int KK = CF::TK / 32;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int q = lane >> 4, j = lane & 15;
  const int wm = w % CF::WAVES_M, wn = w / CF::WAVES_M;
  const int lrow = 8 * q + (j >> 1);
  const int lbyte = 16 * q;  // K-major: first token byte of the lane's 16-byte runs
  const unsigned char* aBase = CF::NT ? st + CF::nt_row(wm * CF::WM + j) + lbyte
                                      : st + lrow * CF::ROWA + 8 * (j & 1) + wm * CF::WM;
  const unsigned char* bBase = CF::NT ? st + CF::OPA + CF::nt_row(wn * CF::WN + j) + lbyte
                                      : st + CF::OPA + lrow * CF::ROWB + 8 * (j & 1) + wn * CF::WN;
  const float* sSa = (const float*)(st + CF::SA_OFF);
  const float* sSb = (const float*)(st + CF::SB_OFF);
  // K-major: step kk takes the lane's tokens 64(kk/2) + 16q + 8(kk%2) .. +7, so that
  // steps 2m and 2m+1 read one 16-byte run per lane
  auto rdn = [&](const unsigned char* base, int i, int kk) __attribute__((always_inline)) {
    const v4i r = *(const v4i*)(base + i * CF::NT_SUB + 64 * (kk >> 1));
    return (kk & 1) ? v2i{r.z, r.w} : v2i{r.x, r.y};
  };
  // swizzled rows: the lane's rows lrow + 32 kk all have the key of lrow, so each
  // sub-tile's chunk moves by a fixed XOR; one base per sub-tile row (column), the
  // token offsets stay immediates
  const int swa = CF::swz_key(lrow, CF::ROWA), swb = CF::swz_key(lrow, CF::ROWB);
  auto swz_a = [&](int i) __attribute__((always_inline)) {
    return st + lrow * CF::ROWA + 16 * (((wm * CF::WM) / 16 + i) ^ swa) + 8 * (j & 1);
  };
  auto swz_b = [&](int jn) __attribute__((always_inline)) {
    return st + CF::OPA + lrow * CF::ROWB + 16 * (((wn * CF::WN) / 16 + jn) ^ swb) + 8 * (j & 1);
  };
  auto rda = [&](int i, int kk) __attribute__((always_inline)) {
    if constexpr (CF::SWZ)
      return tr8(swz_a(i) + 32 * kk * CF::ROWA);
    else if constexpr (CF::NT)
      return rdn(aBase, i, kk);
    else
      return rd8<CF, CF::ROWA>(aBase, i, kk);
  };
  auto rdb = [&](int jn, int kk) __attribute__((always_inline)) {
    if constexpr (CF::SWZ)
      return tr8(swz_b(jn) + 32 * kk * CF::ROWB);
    else if constexpr (CF::NT)
      return rdn(bBase, jn, kk);
    else
      return rd8<CF, CF::ROWB>(bBase, jn, kk);
  };
  v8bf af[CF::NI][KK];
#pragma unroll
  for (int i = 0; i < CF::NI; ++i)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      af[i][kk] = widen8(rda(i, kk), 1.0f);
  auto rescale = [&](int pi, int pj, const v4f& x) {
    const v4f sa = *(const v4f*)(sSa + wm * CF::WM + 16 * pi + 4 * q);
    const float sb = sSb[wn * CF::WN + 16 * pj + j];
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[pi][pj][r] = fmaf(sa[r] * sb, x[r], acc[pi][pj][r]);
  };
  // One column jn of sub-tiles at a time: its NI partial sums are NI independent MFMA
  // chains advanced together (step kk of every chain before step kk + 1 of any), so
  // no MFMA waits for the result of the one before it. With at most four columns per
  // wave the previous column's rescale runs between this column's first MFMAs; with
  // more, each column is rescaled right after its MFMAs, which frees the registers
  // of the deferred partial sums (the 64 x 128 wave tile would spill otherwise).
  constexpr bool DEFER = CF::NJ <= 4;
  v2i rnext[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) rnext[kk] = rdb(0, kk);
  v8bf bf[KK];
  v4f xprev[CF::NI];
#pragma unroll
  for (int jn = 0; jn < CF::NJ; ++jn) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) bf[kk] = widen8(rnext[kk], 1.0f);
    if (jn + 1 < CF::NJ) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) rnext[kk] = rdb(jn + 1, kk);
    }
    v4f x[CF::NI];
    // K-major 64 x 128 wave tiles: the wave issues a column's MFMAs at raised priority,
    // so that the SIMD's other wave fills the MFMAs' cycles with its VALU work
    // (measured 6-7% on long K-major experts; the token-major kernels gained 1-3% or
    // lost as much depending on the variant, and keep the default priority)
    constexpr bool kPrio = !DEFER && CF::NT;
    if constexpr (kPrio) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int i = 0; i < CF::NI; ++i)
        x[i] = mfma_bf16(af[i][kk], bf[kk], kk == 0 ? part[i][jn] : x[i]);
      if (DEFER && PROMOTE && kk == 0 && jn > 0) {
#pragma unroll
        for (int i = 0; i < CF::NI; ++i) rescale(i, jn - 1, xprev[i]);
      }
    }
    if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int i = 0; i < CF::NI; ++i) {
      if constexpr (PROMOTE) {
        if constexpr (DEFER)
          xprev[i] = x[i];
        else
          rescale(i, jn, x[i]);
        part[i][jn] = v4f{0.f, 0.f, 0.f, 0.f};
      } else {
        part[i][jn] = x[i];
      }
    }
  }
  if constexpr (PROMOTE && DEFER) {
#pragma unroll
    for (int i = 0; i < CF::NI; ++i) rescale(i, CF::NJ - 1, xprev[i]);
  }
}

// fp32 scales per 32 tokens: every 32-token step kk of a stage is its own block
// (scale row kk). Each step's MFMA gives the block partial of sub-tile (i, jn), which
// is rescaled by sa (x) sb on the VALU one MFMA behind. Precise: bf16 MFMA on widened
// fp8; fast: the 16x16x32 fp8 MFMA, whose operand is this lane's 8 tokens as they
// come from the transposing read.
template <class CF, bool FAST>
__device__ __forceinline__ void compute_f32s32(const unsigned char* st, v4f (&acc)[CF::NI][CF::NJ]) {
  constexpr int KK = CF::TK / 32;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int q = lane >> 4, j = lane & 15;
  const int wm = w % CF::WAVES_M, wn = w / CF::WAVES_M;
  const int lrow = 8 * q + (j >> 1);
  const int lbyte = 8 * q;  // K-major: first token byte
  const unsigned char* aBase = CF::NT ? st + CF::nt_row(wm * CF::WM + j) + lbyte
                                      : st + lrow * CF::ROWA + 8 * (j & 1) + wm * CF::WM;
  const unsigned char* bBase = CF::NT ? st + CF::OPA + CF::nt_row(wn * CF::WN + j) + lbyte
                                      : st + CF::OPA + lrow * CF::ROWB + 8 * (j & 1) + wn * CF::WN;
  const float* sSa = (const float*)(st + CF::SA_OFF);
  const float* sSb = (const float*)(st + CF::SB_OFF);
  v2i ar[CF::NI][KK];
#pragma unroll
  for (int i = 0; i < CF::NI; ++i)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) ar[i][kk] = rd8<CF, CF::ROWA>(aBase, i, kk);
  auto rescale = [&](int pi, int pj, int pk, const v4f& x) {
    const v4f sa = *(const v4f*)(sSa + pk * CF::BM + wm * CF::WM + 16 * pi + 4 * q);
    const float sb = sSb[pk * CF::BN + wn * CF::WN + 16 * pj + j];
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[pi][pj][r] = fmaf(sa[r] * sb, x[r], acc[pi][pj][r]);
  };
  v2i rnext[KK], bcur[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) rnext[kk] = rd8<CF, CF::ROWB>(bBase, 0, kk);
  v4f prev = v4f{0.f, 0.f, 0.f, 0.f};
  constexpr int S = CF::NI * CF::NJ;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int jn = s / CF::NI, i = s % CF::NI;
    if (i == 0) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) bcur[kk] = rnext[kk];
      if (jn + 1 < CF::NJ) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) rnext[kk] = rd8<CF, CF::ROWB>(bBase, jn + 1, kk);
      }
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      v4f x;
      if constexpr (FAST)
        x = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(__builtin_bit_cast(long, ar[i][kk]),
                                                       __builtin_bit_cast(long, bcur[kk]),
                                                       v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      else
        x = mfma_bf16(widen8(ar[i][kk], 1.0f), widen8(bcur[kk], 1.0f), v4f{0.f, 0.f, 0.f, 0.f});
      const int t = s * KK + kk;  // step index; rescale step t - 1
      if (t > 0) {
        const int tp = t - 1, sp = tp / KK;
        rescale(sp % CF::NI, sp / CF::NI, tp % KK, prev);
      }
      prev = x;
    }
  }
  rescale(CF::NI - 1, CF::NJ - 1, KK - 1, prev);
}

// UE8M0 exponents whose scale 2^(e-127) can be folded into the bf16 widening exactly:
// every scaled e4m3 magnitude (2^-9 .. 448) then stays a normal bf16 (2^-126 .. 2^128).
constexpr int kE8FoldLo = 10, kE8FoldHi = 246;

// True if a byte of x lies outside [kE8FoldLo, kE8FoldHi]: a byte below 10, or one
// whose complement is below 9. Each test is the per-byte borrow test "(x - n) & ~x"
// on the bytes' top bits, exact as a whole-word answer for n <= 128.
__device__ inline bool e8_outside_fold(uint32_t x) {
  const uint32_t y = ~x;
  return (((x - 0x0A0A0A0Au) & y) | ((y - 0x09090909u) & x)) & 0x80808080u;
}

// 2^(e-127-c) as fp32, for 1 <= e - c <= 254: the exponent field e - c. cb = -c << 23
// (one shift-and-add).
__device__ inline float e8_pow2(uint32_t e, uint32_t cb) { return __uint_as_float((e << 23) + cb); }

// Lane-wise minimum / maximum over the wave.
__device__ inline int wave_min(int v) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) v = min(v, __shfl_xor(v, d, 64));
  return v;
}
__device__ inline int wave_max(int v) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) v = max(v, __shfl_xor(v, d, 64));
  return v;
}

// The widening and bf16 MFMAs of one E8M0 stage with A's scales folded as
// 2^(ea - c - 127) and B's as 2^(eb + c - 127), c the shift of the step's scale row
// (ca[row] = -c << 23, cb[row] = c << 23).
template <class CF>
__device__ __forceinline__ void e8m0_fold_stage(const unsigned char* aBase, const unsigned char* bBase,
                                                const unsigned char* sSa, const unsigned char* sSb,
                                                int g32, const uint32_t (&ca)[CF::TK / 32],
                                                const uint32_t (&cb)[CF::TK / 32],
                                                v4f (&acc)[CF::NI][CF::NJ]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j = lane & 15;
  const int wm = w % CF::WAVES_M, wn = w / CF::WAVES_M;
  constexpr int KK = CF::TK / 32;
  v8bf af[CF::NI][KK];
#pragma unroll
  for (int i = 0; i < CF::NI; ++i)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const float sc = e8_pow2(sSa[g32 * kk * CF::BM + wm * CF::WM + 16 * i + j], ca[kk]);
      af[i][kk] = widen8(rd8<CF, CF::ROWA>(aBase, i, kk), sc);
    }
  v2i rnext[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) rnext[kk] = rd8<CF, CF::ROWB>(bBase, 0, kk);
#pragma unroll
  for (int jn = 0; jn < CF::NJ; ++jn) {
    v8bf bf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const float sc = e8_pow2(sSb[g32 * kk * CF::BN + wn * CF::WN + 16 * jn + j], cb[kk]);
      bf[kk] = widen8(rnext[kk], sc);
    }
    if (jn + 1 < CF::NJ) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) rnext[kk] = rd8<CF, CF::ROWB>(bBase, jn + 1, kk);
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int i = 0; i < CF::NI; ++i) acc[i][jn] = mfma_bf16(af[i][kk], bf[kk], acc[i][jn]);
  }
}

// precise fp8 + E8M0: each fragment is widened with its power-of-two scale (exact) and
// the bf16 MFMAs accumulate straight into acc. The scaled values must be normal bf16s:
// the wave first checks the exponents it uses in the stage (4 per dword read; channels
// past M or N, mlim / nlim from the tile origin, and scale rows past srows, which hold
// no token of the expert, are not looked at). If some lie outside [kE8FoldLo,
// kE8FoldHi], then for each scale row (block) A's scales are folded as 2^(ea-c-127) and
// B's as 2^(eb+c-127) with one shift c that brings the row's exponents inside (the
// products keep 2^(ea+eb-254)). No such c exists only when the wave's exponents of one
// operand in one block span more than 236, or the block's scale products leave fp32's
// range (2^(ea+eb-254) above 2^238 or below 2^-234), or a scale is NaN (255): that
// block then takes the nearest shift and KG_ERR_SCALE_RANGE is reported.
template <class CF>
__device__ __forceinline__ void compute_precise_e8m0(const unsigned char* st, int gran, int srows,
                                                     int mlim, int nlim,
                                                     v4f (&acc)[CF::NI][CF::NJ]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int q = lane >> 4, j = lane & 15;
  const int wm = w % CF::WAVES_M, wn = w / CF::WAVES_M;
  const int lrow = 8 * q + (j >> 1);
  const int lbyte = 8 * q;  // K-major: first token byte
  const unsigned char* aBase = CF::NT ? st + CF::nt_row(wm * CF::WM + j) + lbyte
                                      : st + lrow * CF::ROWA + 8 * (j & 1) + wm * CF::WM;
  const unsigned char* bBase = CF::NT ? st + CF::OPA + CF::nt_row(wn * CF::WN + j) + lbyte
                                      : st + CF::OPA + lrow * CF::ROWB + 8 * (j & 1) + wn * CF::WN;
  const unsigned char* sSa = st + CF::SA_OFF;
  const unsigned char* sSb = st + CF::SB_OFF;
  // 32-token run kk of the stage uses scale row kk (gran 32) or row 0 (gran 128)
  const int g32 = gran == 32 ? 1 : 0;
  constexpr int KK = CF::TK / 32;
  // the wave's WM exponents of A and WN of B in a scale row: a dword per lane (M and N
  // are multiples of 16, so a dword never straddles the tile's edge)
  constexpr int DA = CF::WM / 4, DB = CF::WN / 4;
  static_assert(DA + DB <= 64, "one dword per lane covers a scale row");
  const int nrow = g32 ? srows : 1;
  auto row_dword = [&](int row, uint32_t& x) __attribute__((always_inline)) {
    const bool is_a = lane < DA;
    const int ch = is_a ? wm * CF::WM + 4 * lane : wn * CF::WN + 4 * (lane - DA);
    x = is_a ? *(const uint32_t*)(sSa + row * CF::BM + ch) : *(const uint32_t*)(sSb + row * CF::BN + ch);
    return lane < DA + DB && ch < (is_a ? mlim : nlim);
  };
  bool outside = false;
#pragma unroll
  for (int row = 0; row < KK; ++row) {
    uint32_t x;
    if (row < nrow && row_dword(row, x)) outside |= e8_outside_fold(x);
  }
  uint32_t ca[KK], cb[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) ca[kk] = cb[kk] = 0;
  if (__builtin_amdgcn_ballot_w64(outside) != 0) {
#pragma unroll
    for (int row = 0; row < KK; ++row) {
      if (row >= nrow) break;
      // the row's exponent ranges and shift
      int amin = 255, amax = 0, bmin = 255, bmax = 0;
      uint32_t x;
      if (row_dword(row, x)) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = (x >> (8 * r)) & 0xFF;
          if (lane < DA) {
            amin = min(amin, e);
            amax = max(amax, e);
          } else {
            bmin = min(bmin, e);
            bmax = max(bmax, e);
          }
        }
      }
      amin = wave_min(amin), amax = wave_max(amax), bmin = wave_min(bmin), bmax = wave_max(bmax);
      const int c_lo = max(amax - kE8FoldHi, kE8FoldLo - bmin);
      const int c_hi = min(amin - kE8FoldLo, kE8FoldHi - bmax);
      int c = c_lo;
      if (c_lo > c_hi || amax == 255 || bmax == 255) {
        // no exact shift (or a NaN scale): avoid overflow first
        c = max(min(c_lo, kE8FoldHi - bmax), amax - kE8FoldHi);
        if (lane == 0) kgwgrad_status_word = KG_ERR_SCALE_RANGE;
      }
      c = uniform(c);
      ca[row] = (uint32_t)(-c) << 23;
      cb[row] = (uint32_t)c << 23;
    }
    if (!g32) {
#pragma unroll
      for (int kk = 1; kk < KK; ++kk) ca[kk] = ca[0], cb[kk] = cb[0];
    }
  }
  e8m0_fold_stage<CF>(aBase, bBase, sSa, sSb, g32, ca, cb, acc);
}

// bf16: lane 4r+c of a 16-lane group names token row r, halfwords 4c..4c+3; lane
// base row 4q + j/4. For MFMA kk lane group q takes tokens 32kk + 4q + 0..3 and
// 32kk + 16 + 4q + 0..3 (a half-wave reads 8 consecutive rows per transposing read).
// K-major: lane (q, j) reads tokens 32kk + 8q .. +7 of channel row j in one 16-byte
// read (A and B alike, so the MFMA pairs the same tokens).
template <class CF>
__device__ __forceinline__ void compute_bf16(const unsigned char* st, v4f (&acc)[CF::NI][CF::NJ]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int q = lane >> 4, j = lane & 15;
  const int wm = w % CF::WAVES_M, wn = w / CF::WAVES_M;
  const int lrow = 4 * q + (j >> 2);
  const unsigned char* aBase = CF::NT ? st + CF::nt_row(wm * CF::WM + j) + 16 * q
                                      : st + lrow * CF::ROWA + 8 * (j & 3) + 2 * (wm * CF::WM);
  const unsigned char* bBase = CF::NT ? st + CF::OPA + CF::nt_row(wn * CF::WN + j) + 16 * q
                                      : st + CF::OPA + lrow * CF::ROWB + 8 * (j & 3) +
                                            2 * (wn * CF::WN);
#pragma unroll
  for (int kk = 0; kk < CF::TK / 32; ++kk) {
    v8bf af[CF::NI];
#pragma unroll
    for (int i = 0; i < CF::NI; ++i) {
      if constexpr (CF::NT) {
        af[i] = *(const v8bf*)(aBase + i * CF::NT_SUB + 64 * kk);
      } else {
        const v4bf x0 = rd16<CF, CF::ROWA>(aBase, i, kk, 0);
        const v4bf x1 = rd16<CF, CF::ROWA>(aBase, i, kk, 1);
        af[i] = v8bf{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      }
    }
    v8bf bf[CF::NJ];
#pragma unroll
    for (int jn = 0; jn < CF::NJ; ++jn) {
      if constexpr (CF::NT) {
        bf[jn] = *(const v8bf*)(bBase + jn * CF::NT_SUB + 64 * kk);
      } else {
        const v4bf y0 = rd16<CF, CF::ROWB>(bBase, jn, kk, 0);
        const v4bf y1 = rd16<CF, CF::ROWB>(bBase, jn, kk, 1);
        bf[jn] = v8bf{y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
      }
    }
    // K-major: keep the step's B reads ahead of its MFMAs (with the earlier 8-byte
    // runs the scheduler read one fragment, waited and ran its four MFMAs, fragment
    // after fragment; with the 16-byte reads it keeps them together by itself and
    // this barrier changes nothing measurable)
    if constexpr (CF::NT) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int jn = 0; jn < CF::NJ; ++jn)
#pragma unroll
      for (int i = 0; i < CF::NI; ++i) acc[i][jn] = mfma_bf16(af[i], bf[jn], acc[i][jn]);
  }
}

// bf16, pipelined stages of 32 tokens (same lane-to-token map as compute_bf16):
// this lane's byte offsets of its A and B fragments within a stage, and the
// fragment readers.
template <class CF>
struct PipeBase {
  uint32_t a, b;
};

template <class CF>
__device__ inline PipeBase<CF> pipe_base() {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int q = lane >> 4, j = lane & 15;
  const int wm = w % CF::WAVES_M, wn = w / CF::WAVES_M;
  const int lrow = 4 * q + (j >> 2);
  PipeBase<CF> pb;
  pb.a = lrow * CF::ROWA + 8 * (j & 3) + 2 * (wm * CF::WM);
  pb.b = CF::OPA + lrow * CF::ROWB + 8 * (j & 3) + 2 * (wn * CF::WN);
  return pb;
}

template <int ROW>
__device__ inline v8bf frag_b16(const unsigned char* p) {
  const v4bf x0 = tr16(p);
  const v4bf x1 = tr16(p + 16 * ROW);
  return v8bf{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
}

// E8M0: srows, the scale rows of the stage that belong to the expert's tokens; mlim and
// nlim, the tile's channels inside M and N
template <int KIND, bool FAST, class CF>
__device__ __forceinline__ void compute_stage(const unsigned char* st, int gran, bool promote,
                                              int srows, int mlim, int nlim,
                                              v4f (&acc)[CF::NI][CF::NJ],
                                              v4f (&part)[CF::NI][CF::NJ]) {
  static_assert(!CF::SWZ || (KIND == F32S && !FAST),
                "swizzled stages: only the precise fp32-scale compute reads them");
  if constexpr (KIND == BF16) {
    compute_bf16<CF>(st, acc);
  } else if constexpr (KIND == F32S32) {
    compute_f32s32<CF, FAST>(st, acc);
  } else if constexpr (KIND == F32S && FAST) {
    compute_fast_f32s<CF>(st, acc);
  } else if constexpr (KIND == F32S) {
    if (promote)
      compute_precise_f32s<CF, true>(st, acc, part);
    else
      compute_precise_f32s<CF, false>(st, acc, part);
  } else if constexpr (FAST) {
    compute_fast_e8m0<CF>(st, gran, acc);
  } else {
    compute_precise_e8m0<CF>(st, gran, srows, mlim, nlim, acc);
  }
}

// ---------------------------------------------------------------- the kernel

// Stages [kb0, kb1) of one item (expert g's tile at (m0, n0)), accumulated into acc.
// nk is the expert's stage count; stage kb is token rows [TK*kb, TK*kb + TK) of the
// expert. The stage buffers must be free on entry (callers barrier first); on
// return every load of the unit has completed (LDS may still be read by other waves).
template <int KIND, bool FAST, class CF>
__device__ __forceinline__ void item_gemm(const Params& p, const LoadOffsets<CF>& lo, unsigned char* smem,
                                 int64_t t_begin, int Kg, int boff_g, int m0, int n0, int nk,
                                 int kb0, int kb1, v4f (&acc)[CF::NI][CF::NJ]) {
  const int n = kb1 - kb0;  // stages of this unit
  // partial sums of the open 128-token block (used by fp32 scales with TK < 128;
  // dead and removed by the compiler for the other policies)
  v4f part[CF::NI][CF::NJ];
#pragma unroll
  for (int i = 0; i < CF::NI; ++i)
#pragma unroll
    for (int jn = 0; jn < CF::NJ; ++jn) part[i][jn] = v4f{0.f, 0.f, 0.f, 0.f};

  // Ring of NS stage buffers: step j (stage kb0 + j) lives in buffer j % NS. Each
  // wave waits only for its own loads of a stage (the later stages' loads may stay in
  // flight), then the barrier makes every wave's loads visible.
#pragma unroll
  for (int j = 0; j < CF::NS - 1; ++j)
    if (j < n) load_stage<KIND, CF>(p, lo, smem + j * CF::STAGE, t_begin, Kg, boff_g, kb0 + j, m0, n0);
  if constexpr (CF::PIPE) {
    // Step j's fragments are read into registers during step j-1, so at the top of
    // step j (after the barrier) buffer j % NS is free and receives step j + NS.
    const PipeBase<CF> pb = pipe_base<CF>();
    wait_stages<CF>(min(CF::NS - 2, n - 1));
    __syncthreads();
    if (CF::NS - 1 < n)
      load_stage<KIND, CF>(p, lo, smem + (CF::NS - 1) * CF::STAGE, t_begin, Kg, boff_g,
                           kb0 + CF::NS - 1, m0, n0);
    // fragment halves: [2i] tokens 4q..4q+3, [2i+1] tokens 16+4q..16+4q+3
    v4bf xa[2 * CF::NI], xb[2 * CF::NJ], ya[2 * CF::NI], yb[2 * CF::NJ];
#pragma unroll
    for (int i = 0; i < CF::NI; ++i) {
      xa[2 * i] = tr16(smem + pb.a + 32 * i);
      xa[2 * i + 1] = tr16(smem + pb.a + 32 * i + 16 * CF::ROWA);
    }
#pragma unroll
    for (int jn = 0; jn < CF::NJ; ++jn) {
      xb[2 * jn] = tr16(smem + pb.b + 32 * jn);
      xb[2 * jn + 1] = tr16(smem + pb.b + 32 * jn + 16 * CF::ROWB);
    }
    // Step j: wait for step j+1's stage and barrier, refill the freed buffer, then
    // the stage's MFMAs from (ca, cb) with the reads of step j+1 into (na, nb) spread
    // between them. On the last step the reads fetch a stale but valid buffer and
    // are never used.
    auto step = [&](int j, v4bf (&ca)[2 * CF::NI], v4bf (&cb)[2 * CF::NJ],
                    v4bf (&na)[2 * CF::NI], v4bf (&nb)[2 * CF::NJ]) {
      if (j + 1 < n) {
        wait_stages<CF>(min(CF::NS - 2, n - 2 - j));
        __syncthreads();
        if (j + CF::NS < n)
          load_stage<KIND, CF>(p, lo, smem + (j % CF::NS) * CF::STAGE, t_begin, Kg, boff_g,
                               kb0 + j + CF::NS, m0, n0);
      }
      const unsigned char* nxt = smem + ((j + 1) % CF::NS) * CF::STAGE;
      constexpr int R = 2 * (CF::NI + CF::NJ);  // reads of the next stage
      constexpr int S = CF::NI * CF::NJ;        // MFMAs of this stage
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int jn = s / CF::NI, i = s % CF::NI;
        const v8bf a = __builtin_shufflevector(ca[2 * i], ca[2 * i + 1], 0, 1, 2, 3, 4, 5, 6, 7);
        const v8bf b = __builtin_shufflevector(cb[2 * jn], cb[2 * jn + 1], 0, 1, 2, 3, 4, 5, 6, 7);
        acc[i][jn] = mfma_bf16(a, b, acc[i][jn]);
#pragma unroll
        for (int r = (s * R + S - 1) / S; r < ((s + 1) * R + S - 1) / S; ++r) {
          if (r < 2 * CF::NI)
            na[r] = tr16(nxt + pb.a + 32 * (r / 2) + 16 * CF::ROWA * (r % 2));
          else
            nb[r - 2 * CF::NI] = tr16(nxt + pb.b + 32 * ((r - 2 * CF::NI) / 2) +
                                      16 * CF::ROWB * (r % 2));
        }
      }
    };
    // two steps per trip so that the register sets swap roles without copies
    int j = 0;
    for (; j + 1 < n; j += 2) {
      step(j, xa, xb, ya, yb);
      step(j + 1, ya, yb, xa, xb);
    }
    if (j < n) step(j, xa, xb, ya, yb);
    return;
  }
  int buf = 0;  // j % NS
  for (int j = 0; j < n; ++j) {
    if constexpr (CF::ALT && CF::NS == 3) {
      // a wave issued only every other stage: if the stage in flight after this one
      // is its own, it may stay in flight (loads complete in issue order); else this
      // wave's outstanding loads all belong to this stage
      const int w = threadIdx.x >> 6;
      if (j + 1 < n && (w >> 2) == ((kb0 + j + 1) & 1))
        wait_vmcnt(CF::alt_loads(w));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    } else {
      const int ahead = min(CF::NS - 2, n - 1 - j);
      wait_stages<CF>(ahead);
    }
    __syncthreads();
    if constexpr (CF::NT) {
      if (kb0 + j == nk - 1 && (Kg * CF::ELT) % 16 != 0) {
        nt_tail_zero<CF>(p, smem + buf * CF::STAGE, Kg - CF::TK * (nk - 1),
                         t_begin + (int64_t)CF::TK * (nk - 1), m0, n0);
        __syncthreads();
      }
    }
    if (j + CF::NS - 1 < n) {
      const int nb = buf == 0 ? CF::NS - 1 : buf - 1;  // (j + NS - 1) % NS
      load_stage<KIND, CF>(p, lo, smem + nb * CF::STAGE, t_begin, Kg, boff_g, kb0 + j + CF::NS - 1,
                           m0, n0);
    }
    const int kb = kb0 + j;
    const bool promote = ((kb + 1) % (128 / CF::TK) == 0) || kb + 1 == nk;
    // E8M0, gran 32: scale rows of the stage's tokens (the last stage may hold fewer)
    const int srows = KIND == E8M0 ? (min(CF::TK, Kg - CF::TK * kb) + 31) / 32 : 0;
    compute_stage<KIND, FAST, CF>(smem + buf * CF::STAGE, p.gran, promote, srows, p.M - m0,
                                  p.N - n0, acc, part);
    buf = buf + 1 == CF::NS ? 0 : buf + 1;
  }
}

template <class CF>
__device__ inline void zero_acc(v4f (&acc)[CF::NI][CF::NJ]) {
#pragma unroll
  for (int i = 0; i < CF::NI; ++i)
#pragma unroll
    for (int jn = 0; jn < CF::NJ; ++jn) acc[i][jn] = v4f{0.f, 0.f, 0.f, 0.f};
}

// Split-tile partial sums (stream-K mode): workgroup c owns slots 2c (the cut tile its
// range starts with) and 2c + 1 (the cut tile its range ends with, when that is
// another one), row-major BM x BN tiles.
template <class CF>
__device__ inline float* partial_slot(const Params& p, int s) {
  return p.ws + (size_t)s * CF::BM * CF::BN;
}

template <int KIND, bool FAST, class CF>
__device__ void split_tiles(const Params& p, const Sched& s, unsigned char* smem,
                            const LoadOffsets<CF>& lo, int slot);

template <int KIND, bool FAST, class CF, bool SPLIT = false, bool OUTB = false>
__global__ __launch_bounds__(CF::THREADS, 1) void kg_wgrad_kernel(Params p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int64_t wsum_k[kMaxWaves];
  __shared__ int32_t wsum_b[kMaxWaves];
  Sched s = sched_carve(smem + CF::NS * CF::STAGE, p.G);
  const int gran = KIND == BF16 ? CF::TK : p.gran;
  const int T = p.tiles_m * p.tiles_n;
  const int grid = gridDim.x;
  const bool one_round = (int64_t)p.G * T <= grid;
  // Multi-round whole-tile launches spread the empty experts' fill tiles between the
  // GEMM tiles; stream-K, and a launch whose items all run at once, take the live
  // experts first and the fill tiles last.
  const int sched_rc = sched_build<CF::THREADS>(p.ks, p.G, gran, p.K_total, s, wsum_k, wsum_b,
                                                !SPLIT && !one_round, p.scale_rows);
  if (sched_rc != KG_OK) {
    if (blockIdx.x == 0 && threadIdx.x == 0) kgwgrad_status_word = sched_rc;
    return;
  }
  // Workgroup b runs on XCD b % 8. With several rounds of items, each XCD takes a
  // contiguous run of every round (neighbouring tiles that share operand rows in
  // its L2), mostly the runs of odd rounds in reverse XCD order (see below). When all
  // items fit in one round, XCD x takes the x-th eighth of the GEMM tiles (a
  // contiguous run: mostly one expert, sharing operand rows in its L2) and the x-th
  // eighth of the fill tiles, so that every L2 serves GEMM tiles; if an XCD's share
  // would not fit its workgroups, items are dealt round-robin.
  const int b = blockIdx.x;
  int slot = b;
  if (grid % 8 == 0 && !one_round) {
    slot = (b % 8) * (grid / 8) + b / 8;
  } else if (grid % 8 == 0 && !SPLIT && p.G <= 256) {  // live experts first (see above)
    int live = 0;
    for (int g = 0; g < p.G; ++g) live += s.ks[g] > 0;
    const int gm = live * T, nf = p.G * T - gm, per = grid / 8;
    if ((gm + 7) / 8 + (nf + 7) / 8 <= per) {
      const int x = b % 8, r = b / 8;
      const int g_lo = x * gm / 8, g_n = (x + 1) * gm / 8 - g_lo;
      const int f_lo = x * nf / 8, f_n = (x + 1) * nf / 8 - f_lo;
      slot = r < g_n ? g_lo + r : r - g_n < f_n ? gm + f_lo + (r - g_n) : p.G * T;
    }
  }
  const LoadOffsets<CF> lo = load_offsets<CF>(p);

  if constexpr (SPLIT) {
    split_tiles<KIND, FAST, CF>(p, s, smem, lo, slot);
  } else {
    // One item (expert, m-tile, n-tile) at a time, longest experts first.
    const int total = p.G * T;
    for (int base = 0; base < total; base += grid) {
      // odd rounds dealt in reverse (XCD x takes run 7 - x): the items come longest
      // first, and this evens out the work of the XCDs' and workgroups' shares. Not in
      // the fp8-MFMA mode with fp32 scales, whose load-bound long experts gain more
      // from each XCD keeping its panel position from round to round (measured).
      constexpr bool kReverse = !(FAST && KIND == F32S);
      const int idx = base + ((kReverse && ((base / grid) & 1)) ? grid - 1 - slot : slot);
      if (idx >= total) break;
      const Item it = decode_item(idx, T, p.tiles_m, p.tiles_n, s.order);
      const int g = it.g;
      const int m0 = it.tm * CF::BM, n0 = it.tn * CF::BN;
      const int64_t t_begin = s.off[g];
      const int Kg = uniform((int)(s.off[g + 1] - t_begin));
      __syncthreads();  // the previous item is done with the stage buffers
      if (Kg == 0) {
        fill_tile<CF, OUTB>(p, g, m0, n0);
        continue;
      }
      const int boff_g = uniform(s.boff[g]);
      const int nk = (Kg + CF::TK - 1) / CF::TK;
      v4f acc[CF::NI][CF::NJ];
      zero_acc<CF>(acc);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the previous item's stores
      item_gemm<KIND, FAST, CF>(p, lo, smem, t_begin, Kg, boff_g, m0, n0, nk, 0, nk, acc);
      store_tile<CF, OUTB>(p, smem, g, m0, n0, acc);
    }
  }
}

// Stream-K mode (few tiles): the stages of all non-empty tiles, in item order, form
// one line of length W; workgroup `slot` takes [W*slot/grid, W*(slot+1)/grid). A tile
// that lies inside one range is finished by that workgroup. A tile cut by range ends
// has parts in workgroups c0 .. c1: every part writes its partial to its own slot
// (write-through stores), waits for them, and adds one to the tile's arrival counter
// (counter c0). The part that arrives last (the counter reached c1 - c0 + 1) resets the
// counter and adds C and all the partials in workgroup order, so the result does not
// depend on timing, and no workgroup ever waits for another: the mode needs neither
// co-resident workgroups nor an idle GPU. Empty experts' fill tiles follow.
//
// Visibility of the partials: a part's stores bypass the caches (sc0 sc1) and the wave
// waits for their completion (vmcnt) before the workgroup barrier that precedes its
// counter increment; the last part reads the partials with loads that bypass the
// caches too, after its own increment has returned. Every increment thus follows the
// completion of its part's stores, and the reads follow every increment, without a
// cache-wide write-back or invalidation.
template <int KIND, bool FAST, class CF>
__device__ void split_tiles(const Params& p, const Sched& s, unsigned char* smem,
                            const LoadOffsets<CF>& lo, int slot) {
  __shared__ int64_t sk_cum[kMaxSplitGroups + 1];
  __shared__ int sk_last;
  const int T = p.tiles_m * p.tiles_n;
  const int grid = gridDim.x;
  if (threadIdx.x == 0) {
    int64_t c = 0;
    for (int r = 0; r < p.G; ++r) {
      sk_cum[r] = c;
      c += (int64_t)T * ((s.ks[s.order[r]] + CF::TK - 1) / CF::TK);
    }
    sk_cum[p.G] = c;
  }
  __syncthreads();
  const int64_t W = sk_cum[p.G];
  // with fewer stages than workgroups, workgroup c < W takes stage c and the rest none
  auto range_lo = [&](int c) { return W >= grid ? W * c / grid : (int64_t)min(c, (int)W); };
  const int64_t lo_pos = range_lo(slot), hi_pos = range_lo(slot + 1);
  constexpr size_t kTile = (size_t)CF::BM * CF::BN;
  for (int64_t pos = lo_pos; pos < hi_pos;) {
    int r = 0;
    while (sk_cum[r + 1] <= pos) ++r;
    const int g = uniform((int)s.order[r]);
    const int64_t t_begin = s.off[g];
    const int Kg = uniform((int)(s.off[g + 1] - t_begin));
    const int nk = (Kg + CF::TK - 1) / CF::TK;
    const int64_t rel = pos - sk_cum[r];
    const int t = (int)(rel / nk);
    const int kb0 = (int)(rel - (int64_t)t * nk);
    const int kb1 = (int)min((int64_t)nk, kb0 + (hi_pos - pos));
    const Item it = decode_item(r * T + t, T, p.tiles_m, p.tiles_n, s.order);
    const int m0 = it.tm * CF::BM, n0 = it.tn * CF::BN;
    const int boff_g = uniform(s.boff[g]);
    __syncthreads();  // the previous unit is done with the stage buffers
    v4f acc[CF::NI][CF::NJ];
    zero_acc<CF>(acc);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the previous unit's stores
    item_gemm<KIND, FAST, CF>(p, lo, smem, t_begin, Kg, boff_g, m0, n0, nk, kb0, kb1, acc);
    const int64_t tile_lo = sk_cum[r] + (int64_t)t * nk, tile_hi = tile_lo + nk;
    if (tile_lo >= lo_pos && tile_hi <= hi_pos) {
      store_tile_parts<CF>(p, smem, g, m0, n0, acc, nullptr, nullptr, 0, 0);
    } else {
      // the workgroups holding the tile: c0 (its first stage) .. c1 (its last)
      int c0 = slot, c1 = slot;
      while (c0 > 0 && range_lo(c0) > tile_lo) --c0;
      while (c1 + 1 < grid && range_lo(c1 + 1) < tile_hi) ++c1;
      const int nparts = c1 - c0 + 1;
      // publish this part: slot 2c for the unit a range starts with, else 2c + 1
      store_tile_gen<CF, true>(smem, acc, partial_slot<CF>(p, 2 * slot + (pos == lo_pos ? 0 : 1)),
                               CF::BN, CF::BM, CF::BN, nullptr, 0, nullptr, nullptr, 0, 0);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // this wave's partial stores are done
      __syncthreads();
      if (threadIdx.x == 0) {
        const int before =
            __hip_atomic_fetch_add(p.wscnt + c0, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sk_last = before == nparts - 1;
        if (sk_last) __hip_atomic_store(p.wscnt + c0, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
      if (sk_last) {
        // C + the partials of c0 .. c1 in that order (read around the caches)
        zero_acc<CF>(acc);
        const int s0 = 2 * c0 + (range_lo(c0) == tile_lo ? 0 : 1);
        store_tile_parts<CF>(p, smem, g, m0, n0, acc, partial_slot<CF>(p, s0),
                             partial_slot<CF>(p, 2 * (c0 + 1)), 2 * kTile, nparts);
      }
    }
    pos += kb1 - kb0;
  }
  // fill tiles of the empty experts (at the end of the longest-first order)
  int first_empty = 0;
  while (first_empty < p.G && sk_cum[first_empty + 1] > sk_cum[first_empty]) ++first_empty;
  const int nfill = (p.G - first_empty) * T;
  for (int f = slot; f < nfill; f += grid) {
    const Item it = decode_item(first_empty * T + f, T, p.tiles_m, p.tiles_n, s.order);
    __syncthreads();
    fill_tile<CF>(p, it.g, it.tm * CF::BM, it.tn * CF::BN);
  }
}

// Same scan as the main kernel, written out for tests.
constexpr int kOffThreads = 512;
__global__ __launch_bounds__(kOffThreads, 1) void kg_offsets_kernel(const int32_t* ks, int G,
                                                                    int gran, int64_t* off,
                                                                    int32_t* boff) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int64_t wsum_k[kMaxWaves];
  __shared__ int32_t wsum_b[kMaxWaves];
  Sched s = sched_carve(smem, G);
  // K_total is not known here: the sum check fails, the scans are still written
  sched_build<kOffThreads>(ks, G, gran, -1, s, wsum_k, wsum_b);
  for (int g = threadIdx.x; g <= G; g += kOffThreads) {
    off[g] = s.off[g];
    boff[g] = s.boff[g];
  }
}

// ---------------------------------------------------------------- host side

// KG_VERBOSE=1 in the environment prints HIP errors to stderr.
static int hip_fail(hipError_t e, const char* what) {
  static const bool verbose = getenv("KG_VERBOSE") != nullptr;
  if (verbose) fprintf(stderr, "kgwgrad: %s: %s\n", what, hipGetErrorString(e));
  return KG_ERR_HIP;
}

struct Launch {
  const void* fn;
  int stage_bytes;  // all stages
  int bm, bn, threads;
  int tk, ns;       // tokens per stage, stages in the ring
};

template <int KIND, bool FAST, class CF, bool SPLIT = false, bool OUTB = false>
static Launch launch_of() {
  return Launch{(const void*)kg_wgrad_kernel<KIND, FAST, CF, SPLIT, OUTB>, CF::NS * CF::STAGE,
                CF::BM, CF::BN, CF::THREADS, CF::TK, CF::NS};
}

// bf16 output (whole tiles only: stream-K is not taken with a bf16 D)
template <bool NT>
static Launch pick_outb(int kind, bool fast, bool small, bool deep, bool wide) {
  using S = Cfgs<NT>;
  if (wide && kind == F32S && !fast) return launch_of<F32S, false, typename S::F8, false, true>();
  if (kind == F32S32)
    return fast ? launch_of<F32S32, true, typename S::F8h32, false, true>()
                : launch_of<F32S32, false, typename S::F8h32, false, true>();
  if (kind == BF16)
    return small ? launch_of<BF16, false, typename S::B16s, false, true>()
                 : launch_of<BF16, false, typename S::B16, false, true>();
  if (kind == F32S)
    return fast   ? launch_of<F32S, true, typename S::F8, false, true>()
           : deep ? launch_of<F32S, false, typename S::F8hD, false, true>()
                  : launch_of<F32S, false, typename S::F8h, false, true>();
  return fast ? launch_of<E8M0, true, typename S::F8, false, true>()
              : launch_of<E8M0, false, typename S::F8, false, true>();
}

template <bool NT>
static Launch pick_t(int kind, bool fast, bool small, bool split, bool outb, bool deep,
                     bool wide) {
  using S = Cfgs<NT>;
  if (outb) return pick_outb<NT>(kind, fast, small, deep, wide);
  if (wide && kind == F32S && !fast && !split) return launch_of<F32S, false, typename S::F8>();
  if (kind == F32S32)
    return fast ? (split ? launch_of<F32S32, true, typename S::F8h32, true>()
                         : launch_of<F32S32, true, typename S::F8h32>())
                : (split ? launch_of<F32S32, false, typename S::F8h32, true>()
                         : launch_of<F32S32, false, typename S::F8h32>());
  if (split) {
    if (kind == BF16) return launch_of<BF16, false, typename S::B16, true>();
    if (kind == F32S)
      return fast   ? launch_of<F32S, true, typename S::F8, true>()
             : deep ? launch_of<F32S, false, typename S::F8hD, true>()
                    : launch_of<F32S, false, typename S::F8h, true>();
    return fast ? launch_of<E8M0, true, typename S::F8, true>()
                : launch_of<E8M0, false, typename S::F8, true>();
  }
  if (kind == BF16)
    return small ? launch_of<BF16, false, typename S::B16s>()
                 : launch_of<BF16, false, typename S::B16>();
  if (kind == F32S)
    return fast   ? launch_of<F32S, true, typename S::F8>()
           : deep ? launch_of<F32S, false, typename S::F8hD>()
                  : launch_of<F32S, false, typename S::F8h>();
  return fast ? launch_of<E8M0, true, typename S::F8>() : launch_of<E8M0, false, typename S::F8>();
}

// small: half tiles (bf16) for problems with few full tiles; split: stream-K over the
// full-size tiles; outb: bf16 D; nt: K-major operands; deep: the three-stage precise
// fp32-scale tile (token-major) when its stages and the schedule fit the LDS
static Launch pick(int kind, bool fast, bool small = false, bool split = false,
                   bool outb = false, bool nt = false, bool deep = false, bool wide = false) {
  return nt ? pick_t<true>(kind, fast, small, split, outb, deep, wide)
            : pick_t<false>(kind, fast, small, split, outb, deep, wide);
}

// Dynamic LDS a workgroup may take on gfx950: 160 KB less 1 KB for the kernels' static
// __shared__ arrays (at most about 0.6 KB: the scan's wave sums, stream-K's offsets).
constexpr int kMaxLds = 159 * 1024;

// The three-stage precise tile fits beside the schedule of G experts.
static bool deep_fits(int G) { return CfgF8h3::NS * CfgF8h3::STAGE + sched_bytes(G) <= kMaxLds; }

// Stream-K workspace: one int arrival counter per workgroup (the counter area is padded
// to a multiple of 256 bytes), then two partial tiles per workgroup of the largest
// (256 x 256) tile configuration.
static constexpr size_t split_flag_bytes(int cus) {
  return ((size_t)cus * sizeof(int) + 255) & ~(size_t)255;
}

static constexpr size_t split_ws_bytes(int cus) {
  return split_flag_bytes(cus) + 2 * (size_t)cus * CfgB16::BM * CfgB16::BN * sizeof(float);
}

// The scratch of kg_wgrad_noalloc: the stream-K workspace for up to kScratchCUs compute
// units (128 MiB + 1 KiB), one copy per device, held until the process ends. In host
// code `scratch` names a host-side stand-in: its device address is taken once per
// device with hipGetSymbolAddress (DeviceInfo::scratch) and only that is used.
constexpr int kScratchCUs = 256;
static __device__ __align__(256) unsigned char scratch[split_ws_bytes(kScratchCUs)];

struct DeviceInfo {
  int cus = 0;
  void* scratch = nullptr;  // device address of this device's `scratch`
  bool ready = false;
};
static std::mutex g_mu;
static DeviceInfo g_dev[64];

static int device_setup(int dev) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (dev < 0 || dev >= 64) return KG_ERR_HIP;
  DeviceInfo& d = g_dev[dev];
  if (!d.ready) {
    int cus = 0;
    hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    // every kernel the launches can pick: layouts x kinds x modes
    const int kinds[4] = {F32S, E8M0, BF16, F32S32};
    for (int v = 0; v < 2 * 4 * 2 * 2 * 2 * 2 * 2 * 2; ++v) {
      const bool nt = v & 1, fast = (v >> 3) & 1, small = (v >> 4) & 1;
      const bool split = (v >> 5) & 1, outb = (v >> 6) & 1, deep = (v >> 7) & 1;
      const bool wide = (v >> 8) & 1;
      const int kind = kinds[(v >> 1) & 3];
      if ((fast && kind == BF16) || (split && outb)) continue;
      const Launch l = pick(kind, fast, small, split, outb, nt, deep, wide);
      const int lds = l.stage_bytes + sched_bytes(kMaxGroups);
      e = hipFuncSetAttribute(l.fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                              lds < kMaxLds ? lds : kMaxLds);
      if (e != hipSuccess) return hip_fail(e, "hipFuncSetAttribute");
    }
    void* sp = nullptr;
    e = hipGetSymbolAddress(&sp, HIP_SYMBOL(scratch));
    if (e != hipSuccess || sp == nullptr) return hip_fail(e, "hipGetSymbolAddress");
    d.cus = cus;
    d.scratch = sp;
    d.ready = true;
  }
  return KG_OK;
}

// Zeroes n ints (the stream-K arrival counters of kg_wgrad_noalloc's scratch) with
// ordinary stores, so that a call captured in a HIP graph holds no memset node.
__global__ void kg_clear_kernel(int* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

static bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

static bool misaligned(const void* ptr) { return ((uintptr_t)ptr & 15) != 0; }

}  // namespace kg

using namespace kg;

extern "C" int kg_max_groups(void) { return kMaxGroups; }

static int current_cus(int* cus) {
  int dev = 0;
  const hipError_t eg = hipGetDevice(&dev);
  if (eg != hipSuccess) return hip_fail(eg, "hipGetDevice");
  const int rc = device_setup(dev);
  if (rc != KG_OK) return rc;
  *cus = g_dev[dev].cus > 0 ? g_dev[dev].cus : 256;
  return KG_OK;
}

extern "C" int64_t kg_wgrad_workspace_bytes(void) {
  int cus = 0;
  if (current_cus(&cus) != KG_OK) return -1;
  return (int64_t)split_ws_bytes(cus);
}

extern "C" int64_t kg_wgrad_workspace_flag_bytes(void) {
  int cus = 0;
  if (current_cus(&cus) != KG_OK) return -1;
  return (int64_t)split_flag_bytes(cus);
}

// nt: K-major operands A [M, lda] and B [N, ldb] (elements), else token-major
// A [K_total, M] and B [K_total, N]
// clear_counters: zero the workspace's arrival counters before a stream-K launch (the
// library's own scratch, whose last user may have been any earlier call)
static int wgrad_run(bool nt, const void* A, int64_t lda, const void* sa, const void* B,
                     int64_t ldb, const void* sb, const void* C, void* D, const int32_t* ks, int G,
                     int M, int N, int64_t K_total, int64_t scale_rows, int gran_k,
                     int dtype_flags, void* workspace, int64_t workspace_bytes, void* stream,
                     bool clear_counters = false) {
  const int dtype = dtype_flags & 0xFF;
  const int flags = dtype_flags & ~0xFF;
  if (dtype != KG_E4M3_F32SCALE && dtype != KG_E4M3_UE8M0 && dtype != KG_BF16)
    return KG_ERR_DTYPE;
  if (flags & ~(KG_FLAG_FP8_MFMA | KG_FLAG_D_BF16)) return KG_ERR_DTYPE;
  const bool fast = (flags & KG_FLAG_FP8_MFMA) != 0;
  const bool out_bf16 = (flags & KG_FLAG_D_BF16) != 0;
  if (fast && dtype == KG_BF16) return KG_ERR_DTYPE;
  if (G < 0 || M < 0 || N < 0 || K_total < 0 || workspace_bytes < 0) return KG_ERR_SHAPE;
  if (nt && (lda < K_total || ldb < K_total)) return KG_ERR_SHAPE;
  if (dtype != KG_BF16 && gran_k != 32 && gran_k != 128) return KG_ERR_GRAN;
  if (G > kMaxGroups) return KG_ERR_UNSUPPORTED;
  if (M > (1 << 24) || N > (1 << 24) || K_total > INT32_MAX) return KG_ERR_UNSUPPORTED;
  if ((int64_t)M * N > (int64_t)1 << 29) return KG_ERR_UNSUPPORTED;  // 32-bit byte offsets in one expert's C
  if (G == 0 || M == 0 || N == 0) return KG_OK;
  if (D == nullptr || ks == nullptr) return KG_ERR_NULL;
  if (K_total > 0 && (A == nullptr || B == nullptr)) return KG_ERR_NULL;
  if (dtype == KG_BF16) {
    if (sa != nullptr || sb != nullptr) return KG_ERR_NULL;
  } else if (K_total > 0 && (sa == nullptr || sb == nullptr)) {
    return KG_ERR_NULL;
  }
  // every expert's blocks need their scale rows: at least ceil(K_total / gran_k) in
  // all (the exact count, sum ceil(ks[g] / gran_k), is checked on the device)
  if (dtype != KG_BF16 && K_total > 0 &&
      (scale_rows < 0 || scale_rows < K_total / gran_k + (K_total % gran_k != 0)))
    return KG_ERR_SCALE_ROWS;
  if (M % 16 != 0 || N % 16 != 0) return KG_ERR_ALIGN;
  if (misaligned(A) || misaligned(B) || misaligned(sa) || misaligned(sb) || misaligned(C) ||
      misaligned(D) || ((uintptr_t)ks & 3) != 0 || ((uintptr_t)workspace & 255) != 0)
    return KG_ERR_ALIGN;
  const int elt = dtype == KG_BF16 ? 2 : 1;
  if (nt) {
    // whole 16-byte units per K-major row; offsets within 256 rows of one load stay
    // below 2^32
    if ((lda * elt) % 16 != 0 || (ldb * elt) % 16 != 0) return KG_ERR_ALIGN;
    if (256 * lda * elt > (int64_t)0xFFFFFF00 || 256 * ldb * elt > (int64_t)0xFFFFFF00)
      return KG_ERR_UNSUPPORTED;
  }
  const size_t abytes = nt ? (size_t)M * lda * elt : (size_t)K_total * M * elt;
  const size_t bbytes = nt ? (size_t)N * ldb * elt : (size_t)K_total * N * elt;
  const size_t dbytes = (size_t)G * M * N * (out_bf16 ? 2 : 4);
  if (C != nullptr && C != D && overlap(C, dbytes, D, dbytes)) return KG_ERR_ALIAS;
  const size_t sesz = dtype == KG_E4M3_F32SCALE ? 4 : 1;
  // (the kernel reads at most K_total + G rows: sum ceil(ks[g] / gran_k) <= K_total)
  const int64_t srows = scale_rows < K_total ? scale_rows : K_total;
  const size_t sabytes = dtype == KG_BF16 ? 0 : (size_t)srows * M * sesz;
  const size_t sbbytes = dtype == KG_BF16 ? 0 : (size_t)srows * N * sesz;
  if (overlap(A, abytes, D, dbytes) || overlap(sa, sabytes, D, dbytes) ||
      overlap(sb, sbbytes, D, dbytes) ||
      overlap(B, bbytes, D, dbytes) || overlap(ks, (size_t)G * 4, D, dbytes) ||
      overlap(workspace, (size_t)workspace_bytes, D, dbytes) ||
      (C != nullptr && overlap(workspace, (size_t)workspace_bytes, C, dbytes)))
    return KG_ERR_ALIAS;

  const int kind = dtype == KG_E4M3_F32SCALE ? (gran_k == 32 ? F32S32 : F32S)
                   : dtype == KG_E4M3_UE8M0  ? E8M0
                                             : BF16;
  int cus = 0;
  const int rc = current_cus(&cus);
  if (rc != KG_OK) return rc;
  // bf16 problems with fewer than two full 256 x 256 tiles per CU use half tiles.
  // When even then at most half of the CUs would get a tile, and a workspace is
  // given (and G <= 64), the tiles' token ranges are cut across all CUs instead
  // (stream-K).
  auto tiles_of = [&](const Launch& l) {
    return (int64_t)G * ((M + l.bm - 1) / l.bm) * ((N + l.bn - 1) / l.bn);
  };
  const int64_t big_tiles = tiles_of(pick(BF16, false, false, false, false, nt));
  const bool small = kind == BF16 && big_tiles < 2 * (int64_t)cus;
  // Stream-K also when whole rounds of tiles would leave more than 30% of the
  // grid idle (e.g. 272 tiles on 256 CUs); the default bf16 problem's 192 half
  // tiles (75% of one round) stay whole: its partial-tile hand-off measured slower.
  const int64_t T = tiles_of(pick(kind, fast, small, false, false, nt));
  const int64_t rounds = (T + cus - 1) / cus;
  const bool split = workspace != nullptr && G <= kMaxSplitGroups && !out_bf16 &&
                     (size_t)workspace_bytes >= split_ws_bytes(cus) &&
                     (2 * T <= (int64_t)cus || 10 * T < 7 * rounds * (int64_t)cus);
  // precise fp32 scales, long experts (on average at least 4096 tokens): 256 x 256
  // tiles, which widen fewer fp8 values per MFMA (either layout); shorter experts (and
  // their C) keep the 256 x 128 tile, whose smaller work items balance better
  const bool wide = kind == F32S && !fast && !split &&
                    K_total >= (int64_t)4096 * G &&
                    CfgF8::NS * CfgF8::STAGE + sched_bytes(G) <= kMaxLds;
  const Launch L = pick(kind, fast, small && !split, split, out_bf16, nt, deep_fits(G), wide);
  const int tiles_m = (M + L.bm - 1) / L.bm, tiles_n = (N + L.bn - 1) / L.bn;
  const int64_t total = (int64_t)G * tiles_m * tiles_n;
  if (total > INT32_MAX) return KG_ERR_UNSUPPORTED;

  Params p;
  p.A = (const unsigned char*)A;
  p.sa = (const unsigned char*)sa;
  p.B = (const unsigned char*)B;
  p.sb = (const unsigned char*)sb;
  p.C = (const float*)C;
  p.D = (float*)D;
  p.ks = ks;
  p.G = G;
  p.M = M;
  p.N = N;
  p.K_total = K_total;
  p.scale_rows = dtype == KG_BF16 ? INT64_MAX : scale_rows;
  p.lda_b = nt ? (uint32_t)(lda * elt) : 0;
  p.ldb_b = nt ? (uint32_t)(ldb * elt) : 0;
  p.gran = dtype == KG_BF16 ? 0 : gran_k;
  p.tiles_m = tiles_m;
  p.tiles_n = tiles_n;
  p.ws = split ? (float*)((unsigned char*)workspace + split_flag_bytes(cus)) : nullptr;
  p.wscnt = split ? (int*)workspace : nullptr;
  const int grid = split ? cus : (int)(total < cus ? total : cus);
  if (split && clear_counters) {
    hipLaunchKernelGGL(kg_clear_kernel, dim3(1), dim3(256), 0, (hipStream_t)stream, p.wscnt,
                       (int)(split_flag_bytes(cus) / sizeof(int)));
    const hipError_t ec = hipGetLastError();
    if (ec != hipSuccess) return hip_fail(ec, "kernel launch");
  }
  // KG_PRINT_CONFIG=1 in the environment: the configuration of every launch on stderr
  static const bool print_config = getenv("KG_PRINT_CONFIG") != nullptr;
  if (print_config) {
    static const char* kind_names[4] = {"e4m3+f32", "e4m3+ue8m0", "bf16", "e4m3+f32"};
    fprintf(stderr,
            "kgwgrad: %s %s gran %d%s%s G %d M %d N %d K_total %lld | tile %dx%d, %d-token "
            "stages x %d, %d threads, %s, grid %d, %lld tiles (%d x %d per expert), LDS %d B\n",
            nt ? "K-major" : "token-major", kind_names[kind], dtype == KG_BF16 ? 0 : gran_k,
            fast ? " fp8-MFMA" : dtype == KG_BF16 ? "" : " precise", out_bf16 ? " bf16-out" : "",
            G, M, N, (long long)K_total, L.bm, L.bn, L.tk, L.ns, L.threads,
            split ? "stream-K" : "whole tiles", grid, (long long)total, tiles_m, tiles_n,
            L.stage_bytes + sched_bytes(G));
  }
  void* args[] = {&p};
  const hipError_t e = hipLaunchKernel(L.fn, dim3(grid), dim3(L.threads), args,
                                       L.stage_bytes + sched_bytes(G), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return KG_OK;
}

extern "C" int kg_wgrad_ws(const void* A, const void* sa, const void* B, const void* sb,
                           const void* C, void* D, const int32_t* ks, int G, int M, int N,
                           int64_t K_total, int64_t scale_rows, int gran_k, int dtype_flags,
                           void* workspace, int64_t workspace_bytes, void* stream) {
  return wgrad_run(false, A, 0, sa, B, 0, sb, C, D, ks, G, M, N, K_total, scale_rows, gran_k,
                   dtype_flags, workspace, workspace_bytes, stream);
}

extern "C" int kg_wgrad_nt_ws(const void* A, int64_t lda, const void* sa, const void* B,
                              int64_t ldb, const void* sb, const void* C, void* D,
                              const int32_t* ks, int G, int M, int N, int64_t K_total,
                              int64_t scale_rows, int gran_k, int dtype_flags, void* workspace,
                              int64_t workspace_bytes, void* stream) {
  return wgrad_run(true, A, lda, sa, B, ldb, sb, C, D, ks, G, M, N, K_total, scale_rows, gran_k,
                   dtype_flags, workspace, workspace_bytes, stream);
}

extern "C" int kg_wgrad_nt(const void* A, int64_t lda, const void* sa, const void* B, int64_t ldb,
                           const void* sb, const void* C, void* D, const int32_t* ks, int G, int M,
                           int N, int64_t K_total, int64_t scale_rows, int gran_k, int dtype_flags,
                           void* stream) {
  return wgrad_run(true, A, lda, sa, B, ldb, sb, C, D, ks, G, M, N, K_total, scale_rows, gran_k,
                   dtype_flags, nullptr, 0, stream);
}

extern "C" int kg_wgrad_noalloc(const void* A, const void* sa, const void* B, const void* sb,
                                const void* C, void* D, const int32_t* ks, int G, int M, int N,
                                int64_t K_total, int64_t scale_rows, int gran_k, int dtype_flags,
                                void* stream) {
  int dev = 0;
  const hipError_t eg = hipGetDevice(&dev);
  if (eg != hipSuccess) return hip_fail(eg, "hipGetDevice");
  const int rc = device_setup(dev);
  if (rc != KG_OK) return rc;
  // the scratch covers the stream-K workspace of kScratchCUs compute units
  if (split_ws_bytes(g_dev[dev].cus) > sizeof(scratch)) return KG_ERR_UNSUPPORTED;
  return wgrad_run(false, A, 0, sa, B, 0, sb, C, D, ks, G, M, N, K_total, scale_rows, gran_k,
                   dtype_flags, g_dev[dev].scratch, (int64_t)sizeof(scratch), stream, true);
}

extern "C" int kg_wgrad(const void* A, const void* sa, const void* B, const void* sb,
                        const void* C, void* D, const int32_t* ks, int G, int M, int N,
                        int64_t K_total, int64_t scale_rows, int gran_k, int dtype_flags,
                        void* stream) {
  return kg_wgrad_ws(A, sa, B, sb, C, D, ks, G, M, N, K_total, scale_rows, gran_k, dtype_flags,
                     nullptr, 0, stream);
}

extern "C" int kg_status(void* stream) {
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  int v = 0;
  e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(kgwgrad_status_word), sizeof v, 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyFromSymbol");
  if (v != 0) {
    const int zero = 0;
    e = hipMemcpyToSymbol(HIP_SYMBOL(kgwgrad_status_word), &zero, sizeof zero, 0,
                          hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyToSymbol");
  }
  return v;
}

extern "C" int kg_debug_offsets(const int32_t* ks, int G, int gran_k, int64_t* off, int32_t* boff,
                                void* stream) {
  if (G < 0 || G > kMaxGroups) return KG_ERR_SHAPE;
  if (gran_k <= 0) return KG_ERR_GRAN;
  if (off == nullptr || boff == nullptr || (G > 0 && ks == nullptr)) return KG_ERR_NULL;
  hipLaunchKernelGGL(kg_offsets_kernel, dim3(1), dim3(kOffThreads), sched_bytes(G),
                     (hipStream_t)stream, ks, G, gran_k, off, boff);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return KG_OK;
}

// The requantiser and the M-grouped dgrad GEMM share this translation unit (and the
// device status word).
#include "kg_requant.h"
#include "kg_dgrad.h"
