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
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kPanelM = 4;  // m-tiles per panel of the tile walk

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

// Block-wide: load ks, check counts, scan offsets, order experts. Returns KG_OK
// or KG_ERR_KSUM; every thread returns the same value.
__device__ int sched_build(const int32_t* ks, int G, int gran, int64_t K_total, Sched s,
                           int64_t* wsum_k, int32_t* wsum_b) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  // each thread owns experts 2t and 2t+1 (G <= 1024)
  const int g0 = 2 * t, g1 = 2 * t + 1;
  const int k0 = g0 < G ? ks[g0] : 0;
  const int k1 = g1 < G ? ks[g1] : 0;
  const int neg = (k0 < 0) | (k1 < 0);
  const int b0 = k0 > 0 ? (k0 + gran - 1) / gran : 0;
  const int b1 = k1 > 0 ? (k1 + gran - 1) / gran : 0;
  if (g0 < G) s.ks[g0] = k0;
  if (g1 < G) s.ks[g1] = k1;
  const int64_t sk = wave_incl_scan<int64_t>((int64_t)k0 + k1);
  const int32_t sbk = wave_incl_scan<int32_t>(b0 + b1);
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
  const int64_t ex_k = pk + sk - ((int64_t)k0 + k1);
  const int32_t ex_b = pb + sbk - (b0 + b1);
  if (g0 < G) {
    s.off[g0 + 1] = ex_k + k0;
    s.boff[g0 + 1] = ex_b + b0;
  }
  if (g1 < G) {
    s.off[g1 + 1] = ex_k + k0 + k1;
    s.boff[g1 + 1] = ex_b + b0 + b1;
  }
  if (t == 0) {
    s.off[0] = 0;
    s.boff[0] = 0;
  }
  int64_t total = 0;
  for (int i = 0; i < kWaves; ++i) total += wsum_k[i];
  __syncthreads();
  if (any_neg || total != K_total) return KG_ERR_KSUM;
  // Longest-first order of experts (ties by index) when G is small; identity otherwise.
  if (G <= 256) {
    if (t < G) {
      const int kt = s.ks[t];
      int rank = 0;
      for (int h = 0; h < G; ++h) {
        const int kh = s.ks[h];
        rank += (kh > kt) | ((kh == kt) & (h < t));
      }
      s.order[rank] = (uint16_t)t;
    }
  } else {
    for (int g = t; g < G; g += kThreads) s.order[g] = (uint16_t)g;
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
