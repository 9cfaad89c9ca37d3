// kg_device.h -- gfx950 device primitives used by the K-grouped wgrad kernels.
//
// Layout facts these helpers rely on (checked on gfx950 by lane-layout probes):
//  * v_mfma_f32_16x16x128_f8f6f4: lane l = 16*q + i holds row i of the 16-row
//    operand; its 32 bytes hold the contraction indices 16q..16q+15 (bytes 0-15)
//    and 64+16q..64+16q+15 (bytes 16-31). The fp32 result lane l, register r is
//    row 4*(l/16)+r, column l%16.
//  * The scaled form applies, to 32-index block b of row i, the E8M0 exponent
//    supplied by lane 16*b+i (bias 127); an exponent of 127 equals no scaling.
//  * v_mfma_f32_16x16x32_bf16: lane l = 16*q + i holds row i, contraction
//    indices 8q..8q+7; result layout as above.
//  * ds_read_b64_tr_b8: in each 16-lane group, lane 2r+h names 8 bytes of "row"
//    r (r < 8); lane c of the group receives byte c of the 16 named columns from
//    rows 0..7, i.e. one column, 8 rows deep.
//  * ds_read_b64_tr_b16: lane 4r+c names 4 halfwords of row r (r < 4); lane c
//    receives column c from rows 0..3.
//  * buffer_load_dwordx4 ... lds: lane l's 16 bytes land at the wave's LDS base
//    + 16*l; offsets at or past num_records write zeros.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kg {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

#define KG_LDS __attribute__((address_space(3)))

// Buffer resource word 3 for raw (unstructured) buffers on the gfx9 family.
constexpr int kRsrcWord3 = 0x00020000;
// An offset that is always out of range: the load writes zeros.
constexpr uint32_t kOobOffset = 0xFFFFFFF0u;

// Raw buffer resource over [base, base + bytes), wave-uniform (SGPRs).
__device__ __forceinline__ v4i make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  v4i r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = kRsrcWord3;
  return r;
}

// LDS byte address of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const KG_LDS void*)p;
}

// 16 bytes global -> LDS at `lds` + 16 * lane, no VGPR staging. `lds` must be
// wave-uniform. Issued as inline assembly on purpose: the compiler then does not
// track these writes, so it does not make reads of the other LDS stage wait for
// them. Callers wait with wait_all_and_barrier() before reading the stage.
__device__ __forceinline__ void load16_lds(v4i r, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane((int)lds))
               : "memory", "m0");
}

// load16_lds that reads around the L2 (sc0 sc1): sees data that other XCDs wrote
// with store16_sys without any cache-wide invalidation.
__device__ __forceinline__ void load16_lds_sys(v4i r, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen sc0 sc1 lds"
               :
               : "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane((int)lds))
               : "memory", "m0");
}

// 16-byte store at byte `voff` of [base, base + bytes), written through to memory
// (cache policy sc0 sc1): visible to every XCD once this wave's vmcnt reaches zero,
// without a cache-wide write-back.
__device__ __forceinline__ void store16_sys(void* base, uint32_t bytes, uint32_t voff, v4f v) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, kRsrcWord3);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), r, (int)voff, 0,
                                         /* sc0 | sc1 */ 1 | 16);
}

__device__ __forceinline__ v2i tr8(const unsigned char* lds) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((KG_LDS v2i*)lds);
}

__device__ __forceinline__ v4bf tr16(const unsigned char* lds) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((KG_LDS v4bf*)lds);
}

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c) {
  // scales 0 with op_sel 0 select the unscaled instruction
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v4f mfma_fp8_e8m0(const v8i& a, const v8i& b, const v4f& c, int sa,
                                             int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

__device__ __forceinline__ v4f mfma_bf16(const v8bf& a, const v8bf& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt
// and lgkmcnt left at their maxima, i.e. not waited for).
constexpr int vmcnt_imm(int n) { return (n & 0xF) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14); }

// Wait until at most n (0 <= n <= 31) of this wave's vector-memory operations are
// outstanding. Loads complete in issue order, so this waits for all but the n
// most recent ones.
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
#define KG_W(k) \
  case k:       \
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(k)); \
    break;
    KG_W(1) KG_W(2) KG_W(3) KG_W(4) KG_W(5) KG_W(6) KG_W(7) KG_W(8) KG_W(9) KG_W(10)
    KG_W(11) KG_W(12) KG_W(13) KG_W(14) KG_W(15) KG_W(16) KG_W(17) KG_W(18) KG_W(19)
    KG_W(20) KG_W(21) KG_W(22) KG_W(23) KG_W(24) KG_W(25) KG_W(26) KG_W(27) KG_W(28)
    KG_W(29) KG_W(30) KG_W(31)
#undef KG_W
    default:
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }
}

// Wait for every outstanding vector-memory operation of this wave (including
// loads into LDS), then barrier the workgroup.
__device__ __forceinline__ void wait_all_and_barrier() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

}  // namespace kg
