// Device-side building blocks for gfx950 (CDNA4): vector types, MFMA wrappers with their
// lane layouts, wave reductions and asynchronous global -> LDS copies.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace gsa {

constexpr int kWave = 64;

typedef __bf16 bf16_t;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------------------
// 16x16 MFMA lane layouts (wave64; g = lane / 16, c = lane % 16):
//   A (16 x K, row-major rows m):  lane holds row m = c, K-slots [kpl*g, kpl*g + kpl)
//   B (K x 16, columns n):         lane holds column n = c, the same K-slots
//   C/D (16 x 16 fp32):            lane holds column n = c, rows 4g + r, r = 0..3
// with kpl = 8 for v_mfma_f32_16x16x32_bf16 and kpl = 1 for v_mfma_f32_16x16x4_f32.
// Which K index a slot carries is irrelevant to the product as long as A and B agree,
// which lets the C tile of one product feed the next as a B operand: a lane's four C
// rows of two adjacent 16-row tiles become its eight K-slots, and the other operand is
// read with the same key order.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Reduce over the four lane groups that share a column (lanes c, c+16, c+32, c+48).
// A permlane swap of a value with itself leaves, in its two results, each lane's own
// value and that of the lane 16 (resp. 32) apart, so one ALU op per step reduces the
// pair without a trip through the LDS crossbar.
__device__ __forceinline__ float group_max4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// bf16 <-> fp32 (round to nearest even on the way down).
__device__ __forceinline__ bf16_t to_bf16(float x) { return (bf16_t)x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return (float)x; }

// ---------------------------------------------------------------------------------------
// Asynchronous global -> LDS copies through a buffer resource.  buffer_load_dword{,x4}
// with the lds flag writes each active lane's 4 or 16 bytes to LDS at (wave-uniform
// base) + lane * size; completion is tracked by the wave's vmcnt like any vector load.
// The resource (four scalar registers) holds the base and size of one tensor slice, the
// per-lane byte offset is a vector register that stays the same from copy to copy and
// the slice offset of the tile is a scalar, so a copy needs no vector address
// arithmetic; reads past the resource's size return zero.  The compiler does not track
// which LDS bytes a copy writes, so every read of copied data is preceded by an explicit
// vmcnt wait (and a barrier, for the other waves' copies).  Slice offsets are 32-bit:
// the largest slice of the built instances (131072 tokens x 128 bf16 features) is 32 MiB.
// ---------------------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void *lds_ptr_t;
typedef __amdgpu_buffer_rsrc_t rsrc_t;
// gfx9 buffer descriptor word 3: 32-bit data format (dword accesses), no swizzle.
constexpr int kRsrcWord3 = 0x00020000;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ void buf_copy16_to_lds(rsrc_t r, uint32_t voff, uint32_t soff, unsigned char *lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds_wave_base, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void buf_copy4_to_lds(rsrc_t r, uint32_t voff, uint32_t soff, unsigned char *lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds_wave_base, 4, voff, soff, 0, 0);
}

// s_waitcnt immediate for "vmcnt <= n" leaving the other counters alone (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14]).
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
constexpr int kLgkmZero = 15 | (7 << 4) | (0 << 8) | (3 << 14);   // "lgkmcnt <= 0" only

// Workgroup barrier for the copy pipelines.  __syncthreads() is a release fence, and the
// compiler counts asynchronous global -> LDS copies as pending LDS stores, so it drains
// every copy in flight (vmcnt(0)) at each one, which defeats prefetching.  Here the
// callers wait for the copies they need with explicit vmcnt counts; the barrier only
// finishes this wave's LDS accesses and stops the compiler from moving memory accesses
// across it (a compiler-only fence emits no instruction).
__device__ __forceinline__ void wg_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(kLgkmZero);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Read of a value that no thread of the kernel writes, at a wave-uniform address.  Through
// the constant address space it becomes a scalar load (counted by lgkmcnt, so waiting for
// it does not wait for the vector loads and copies in flight).
template <typename V>
__device__ __forceinline__ V load_uniform(const V *p) {
  return *(const __attribute__((address_space(4))) V *)p;
}

}  // namespace gsa
