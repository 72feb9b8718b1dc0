// Device-side building blocks for gfx950 (CDNA4): vector types, MFMA wrappers with their
// lane layouts, wave reductions and the XCD-aware workgroup order.
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

__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, kWave); }

// Reduce over the four lane groups that share a column (lanes c, c+16, c+32, c+48).
__device__ __forceinline__ float group_max4(float v) {
  v = fmaxf(v, shfl_xor(v, 16));
  return fmaxf(v, shfl_xor(v, 32));
}
__device__ __forceinline__ float group_sum4(float v) {
  v += shfl_xor(v, 16);
  return v + shfl_xor(v, 32);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// bf16 <-> fp32 (round to nearest even on the way down).
__device__ __forceinline__ bf16_t to_bf16(float x) { return (bf16_t)x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return (float)x; }

// ---------------------------------------------------------------------------------------
// Workgroup order.  The dispatcher hands consecutive workgroup ids to the 8 XCDs in turn,
// and each XCD has its own L2.  Workgroups that reuse the same K/V tiles sit next to each
// other in the work list, so runs of kChunk consecutive work-list positions are kept on
// one XCD while successive runs still rotate over all XCDs (which keeps the longest-first
// order balanced).  The grid is padded to a multiple of 8 * kChunk; ids mapping past the
// end return -1.
// ---------------------------------------------------------------------------------------
constexpr int kXcds = 8;
constexpr int kChunk = 4;

__host__ __device__ inline int64_t padded_grid(int64_t items) {
  const int64_t q = (int64_t)kXcds * kChunk;
  return (items + q - 1) / q * q;
}

__device__ __forceinline__ int64_t work_position(int64_t pid, int64_t items) {
  const int64_t xcd = pid % kXcds;
  const int64_t local = pid / kXcds;
  const int64_t pos = ((local / kChunk) * kXcds + xcd) * kChunk + (local % kChunk);
  return pos < items ? pos : -1;
}

}  // namespace gsa
