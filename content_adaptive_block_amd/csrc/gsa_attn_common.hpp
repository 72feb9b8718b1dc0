// Tile primitives shared by the attention kernels (forward, dK/dV, dQ).
//
// A "tile" is one mask block: BLK token rows of HD features, contiguous in memory
// ([B, H, T, d] layout, so a block of one head is a dense BLK x HD row-major matrix).
// Each wave owns 16 rows of the workgroup's own block; the other operand's block is
// staged in LDS, row-major ("rows") and/or transposed ("cols").
//
// Products used (16x16 MFMA tiles, see gsa_device.hpp for the lane layouts):
//   dot_rows:      C[m][n] = sum_d LDSrows[m][d] * F[n][d]   (A from LDS, B from the
//                  wave's register fragment F of its 16 rows)  -> C rows m = staged
//                  block's tokens (4 per lane), column n = one of the wave's rows
//   accumulate_pv: Acc[f][n] += sum_m LDScols[f][m] * C[m][n] (A from the transposed
//                  LDS block, B = a C tile from dot_rows fed back in place)
// The second product reads a lane's C rows 4g+r of 16-row tiles 2kk and 2kk+1 as its
// eight K-slots, and the transposed operand with the same token order.
#pragma once

#include <type_traits>

#include "gsa_device.hpp"
#include "gsa_internal.hpp"

namespace gsa {

__device__ __forceinline__ int head_class(int h, int n_loc, int n_lit) {
  return h < n_loc ? 0 : (h < n_loc + n_lit ? 1 : 2);
}

template <typename T, int BLK, int HD>
struct AttnShape {
  static constexpr bool kBf16 = std::is_same<T, bf16_t>::value;
  static_assert(kBf16 || std::is_same<T, float>::value, "bf16 or fp32 only");
  static_assert(BLK % (kBf16 ? 32 : 16) == 0 && HD % (kBf16 ? 32 : 16) == 0, "tile shape");
  static constexpr int kWaves = BLK / 16;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kKB = BLK / 16;                 // 16-row tiles of a staged block
  static constexpr int kDB = HD / 16;                  // 16-wide feature tiles
  static constexpr int kKS = kBf16 ? HD / 32 : HD / 4; // MFMA K-steps over the features
  static constexpr int kVec = 16 / sizeof(T);          // elements per 16-byte access
  static constexpr int kRowStride = HD + (kBf16 ? 8 : 4);   // padded LDS row (elements)
  static constexpr int kTStride = BLK + (kBf16 ? 8 : 4);    // padded LDS column block
  static constexpr int kRowChunks = BLK * HD / kVec;
  static_assert(kRowChunks % kThreads == 0, "row staging must divide evenly");

  using Frag = typename std::conditional<kBf16, bf16x8, float>::type;
  struct QFrag {
    Frag f[kKS];
  };

  // Register fragment of one token row (this lane's n = c), K-slots of lane group g.
  __device__ static __forceinline__ void load_row_frag(QFrag &qf, const T *row, int g) {
    if constexpr (kBf16) {
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) qf.f[ks] = *reinterpret_cast<const bf16x8 *>(row + ks * 32 + 8 * g);
    } else {
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) qf.f[ks] = row[4 * ks + g];
    }
  }

  // Copies a BLK x HD block to LDS row-major (row stride kRowStride).
  __device__ static __forceinline__ void stage_rows(T *lds, const T *src, int tid) {
#pragma unroll
    for (int it = 0; it < kRowChunks / kThreads; ++it) {
      const int u = tid + it * kThreads;
      const int row = u / (HD / kVec), col = (u % (HD / kVec)) * kVec;
      *reinterpret_cast<u32x4 *>(lds + row * kRowStride + col) =
          *reinterpret_cast<const u32x4 *>(src + row * HD + col);
    }
  }

  // Copies a BLK x HD block to LDS transposed: lds[f * kTStride + token].
  __device__ static __forceinline__ void stage_cols(T *lds, const T *src, int tid) {
    if constexpr (kBf16) {
      // Unit = 2 tokens x 8 features: two 16-byte loads, eight 4-byte LDS stores.
      constexpr int kUnits = BLK * HD / 16;
      static_assert(kUnits % kThreads == 0, "column staging must divide evenly");
#pragma unroll
      for (int it = 0; it < kUnits / kThreads; ++it) {
        const int u = tid + it * kThreads;
        const int m = u % (HD / 8), kp = u / (HD / 8);
        const u32x4 r0 = *reinterpret_cast<const u32x4 *>(src + (2 * kp) * HD + 8 * m);
        const u32x4 r1 = *reinterpret_cast<const u32x4 *>(src + (2 * kp + 1) * HD + 8 * m);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t a = r0[e], b = r1[e];
          // feature 8m + 2e: (low half of a, low half of b); 8m + 2e + 1: the high halves
          const uint32_t lo = (a & 0xFFFFu) | (b << 16);
          const uint32_t hi = (a >> 16) | (b & 0xFFFF0000u);
          *reinterpret_cast<uint32_t *>(lds + (8 * m + 2 * e) * kTStride + 2 * kp) = lo;
          *reinterpret_cast<uint32_t *>(lds + (8 * m + 2 * e + 1) * kTStride + 2 * kp) = hi;
        }
      }
    } else {
      constexpr int kUnits = BLK * HD / 4;
      static_assert(kUnits % kThreads == 0, "column staging must divide evenly");
#pragma unroll
      for (int it = 0; it < kUnits / kThreads; ++it) {
        const int u = tid + it * kThreads;
        const int m = u % (HD / 4), tok = u / (HD / 4);
        const f32x4 r = *reinterpret_cast<const f32x4 *>(src + tok * HD + 4 * m);
#pragma unroll
        for (int e = 0; e < 4; ++e) lds[(4 * m + e) * kTStride + tok] = r[e];
      }
    }
  }

  // C tile (16 staged rows starting at `row0 = 16 * tile`, lane's row row0 + c as A)
  // times the wave's fragment.
  __device__ static __forceinline__ f32x4 dot_rows(const T *lds, int row, int g, const QFrag &qf) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (kBf16) {
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(lds + row * kRowStride + ks * 32 + 8 * g);
        acc = mfma_bf16(a, qf.f[ks], acc);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) acc = mfma_f32(lds[row * kRowStride + 4 * ks + g], qf.f[ks], acc);
    }
    return acc;
  }

  // acc[db] += LDScols[db*16 + c][tokens] x C, C = kKB tiles of 16 staged tokens.
  __device__ static __forceinline__ void accumulate_pv(f32x4 *acc, const T *lds_t, const f32x4 *cm,
                                                        int c, int g) {
    if constexpr (kBf16) {
#pragma unroll
      for (int kk = 0; kk < kKB / 2; ++kk) {
        bf16x8 b;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          b[r] = to_bf16(cm[2 * kk][r]);
          b[4 + r] = to_bf16(cm[2 * kk + 1][r]);
        }
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          const T *rowp = lds_t + (db * 16 + c) * kTStride + 32 * kk + 4 * g;
          const bf16x4 a0 = *reinterpret_cast<const bf16x4 *>(rowp);
          const bf16x4 a1 = *reinterpret_cast<const bf16x4 *>(rowp + 16);
          const bf16x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          acc[db] = mfma_bf16(a, b, acc[db]);
        }
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int db = 0; db < kDB; ++db)
            acc[db] = mfma_f32(lds_t[(db * 16 + c) * kTStride + kb * 16 + 4 * g + r], cm[kb][r], acc[db]);
    }
  }

  // Stores four consecutive features.
  __device__ static __forceinline__ void store4(T *dst, const f32x4 &x) {
    if constexpr (kBf16) {
      const bf16x4 y = {to_bf16(x[0]), to_bf16(x[1]), to_bf16(x[2]), to_bf16(x[3])};
      *reinterpret_cast<bf16x4 *>(dst) = y;
    } else {
      *reinterpret_cast<f32x4 *>(dst) = x;
    }
  }
};

}  // namespace gsa
