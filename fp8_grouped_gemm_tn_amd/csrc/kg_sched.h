// kg_sched.h -- per-workgroup schedule of the K-grouped wgrad kernels.
//
// Every workgroup of the persistent launch rebuilds the same schedule in LDS:
// the exclusive scans of the expert token counts (token offsets, int64) and of
// their scale-block counts (scale-row offsets), the check that the counts are
// non-negative and add up to K_total, and a longest-first order of the experts.
// Work items are (expert, m-tile, n-tile); every expert has the same number of
// tiles because M and N are shared by all experts.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kg_device.h"
#include "kgwgrad.h"

namespace kg {

constexpr int kMaxGroups = 1024;
constexpr int kMaxSplitGroups = 64;  // largest G that runs in stream-K mode
constexpr int kMaxWaves = 8;  // largest workgroup: 512 threads
constexpr int kPanelM = 4;    // m-tiles per panel of the tile walk

__host__ __device__ constexpr int align16(int x) { return (x + 15) & ~15; }

// LDS bytes of the schedule for G experts: off (int64), boff, ks (int32), order (uint16).
__host__ __device__ inline int sched_bytes(int G) {
  return align16((G + 1) * 8) + align16((G + 1) * 4) + align16(G * 4) + align16(G * 2) + 64;
}

struct Sched {
  int64_t* off;
  int32_t* boff;
  int32_t* ks;
  uint16_t* order;
  int* flag;
};

__device__ inline Sched sched_carve(unsigned char* base, int G) {
  Sched s;
  s.off = (int64_t*)base;
  base += align16((G + 1) * 8);
  s.boff = (int32_t*)base;
  base += align16((G + 1) * 4);
  s.ks = (int32_t*)base;
  base += align16(G * 4);
  s.order = (uint16_t*)base;
  base += align16(G * 2);
  s.flag = (int*)base;
  return s;
}

// Inclusive scan within a wave (64 lanes).
template <typename T>
__device__ inline T wave_incl_scan(T v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    T u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  return v;
}

// Block-wide: load ks, check counts, scan offsets, order experts. Returns KG_OK,
// KG_ERR_KSUM (a negative count, or counts that do not add up to K_total) or
// KG_ERR_SCALE_ROWS (more blocks than max_blocks, the rows the caller's scale
// tensors hold); every thread returns the same value. THREADS is the block size
// (256 or 512); each thread owns kMaxGroups / THREADS consecutive experts. spread:
// place the empty experts between the others (else last).
template <int THREADS>
__device__ int sched_build(const int32_t* ks, int G, int gran, int64_t K_total, Sched s,
                           int64_t* wsum_k, int32_t* wsum_b, bool spread = false,
                           int64_t max_blocks = INT64_MAX) {
  constexpr int E = kMaxGroups / THREADS, W = THREADS / 64;
  static_assert(E * THREADS == kMaxGroups && W <= kMaxWaves, "block size");
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int g0 = E * t;
  int kv[E], bv[E];
  int neg = 0;
  int64_t own_k = 0;
  int32_t own_b = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    kv[e] = g0 + e < G ? ks[g0 + e] : 0;
    neg |= kv[e] < 0;
    // ceil(kv / gran) without forming kv + gran - 1 (which overflows near 2^31)
    bv[e] = kv[e] > 0 ? kv[e] / gran + (kv[e] % gran != 0) : 0;
    if (g0 + e < G) s.ks[g0 + e] = kv[e];
    own_k += kv[e];
    own_b += bv[e];
  }
  const int64_t sk = wave_incl_scan<int64_t>(own_k);
  const int32_t sbk = wave_incl_scan<int32_t>(own_b);
  if (lane == 63) {
    wsum_k[w] = sk;
    wsum_b[w] = sbk;
  }
  const int any_neg = __syncthreads_or(neg);
  int64_t pk = 0;
  int32_t pb = 0;
  for (int i = 0; i < w; ++i) {
    pk += wsum_k[i];
    pb += wsum_b[i];
  }
  int64_t run_k = pk + sk - own_k;
  int32_t run_b = pb + sbk - own_b;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    run_k += kv[e];
    run_b += bv[e];
    if (g0 + e < G) {
      s.off[g0 + e + 1] = run_k;
      s.boff[g0 + e + 1] = run_b;
    }
  }
  if (t == 0) {
    s.off[0] = 0;
    s.boff[0] = 0;
  }
  int64_t total = 0, total_b = 0;
  for (int i = 0; i < W; ++i) {
    total += wsum_k[i];
    total_b += wsum_b[i];
  }
  __syncthreads();
  if (any_neg || total != K_total) return KG_ERR_KSUM;
  // (with consistent counts, total_b <= K_total / gran + G fits the int32 scan)
  if (total_b > max_blocks) return KG_ERR_SCALE_ROWS;
  // When G is small: experts with tokens longest first (ties by index), and the empty
  // ones (fill items: stores only) after them or, with spread, spread evenly between
  // them, so that their stores run beside other workgroups' GEMM tiles rather than
  // all at the end (measured 3% on 256 experts with 51 empty, precise mode). Live
  // expert of rank r sits at (r + 1/2) / L of the way, empty expert e (by index) at
  // (e + 1/2) / E, live first on ties. Identity order otherwise.
  if (G <= 256) {
    int L = 0;
    for (int h = 0; h < G; ++h) L += s.ks[h] > 0;
    const int Ez = G - L;
    // without spread every empty expert goes after every live one
    const int Ls = spread ? L : 0;
    for (int g = t; g < G; g += THREADS) {
      const int kt = s.ks[g];
      int pos = 0;
      if (kt > 0) {
        int r = 0;
        for (int h = 0; h < G; ++h) {
          const int kh = s.ks[h];
          r += (kh > kt) | ((kh == kt) & (h < g));
        }
        int before = 0;  // empty experts placed before live rank r
        for (int e = 0; e < Ez && spread; ++e) before += (2 * e + 1) * L < (2 * r + 1) * Ez;
        pos = r + before;
      } else {
        int e = 0;
        for (int h = 0; h < g; ++h) e += s.ks[h] == 0;
        int before = spread ? 0 : L;  // live experts placed before empty rank e
        for (int r = 0; r < Ls; ++r) before += (2 * r + 1) * Ez <= (2 * e + 1) * L;
        pos = e + before;
      }
      s.order[pos] = (uint16_t)g;
    }
  } else {
    for (int g = t; g < G; g += THREADS) s.order[g] = (uint16_t)g;
  }
  __syncthreads();
  return KG_OK;
}

struct Item {
  int g, tm, tn;
};

// Item index -> (expert, m-tile, n-tile). Within an expert, tiles are walked in
// panels of kPanelM m-tiles, n-tiles outer within the panel.
__device__ inline Item decode_item(int idx, int T, int tiles_m, int tiles_n, const uint16_t* order) {
  Item it;
  const int pos = idx / T;
  const int t = idx - pos * T;
  it.g = uniform((int)order[pos]);
  const int per_panel = kPanelM * tiles_n;
  const int panel = t / per_panel;
  const int w = t - panel * per_panel;
  const int rem = tiles_m - panel * kPanelM;
  const int pm = rem < kPanelM ? rem : kPanelM;
  it.tm = panel * kPanelM + w % pm;
  it.tn = w / pm;
  return it;
}

}  // namespace kg
