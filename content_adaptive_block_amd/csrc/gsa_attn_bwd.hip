// Backward of gzip-guided block-sparse causal attention on gfx950.
//
// The pages give no backward; this is the gradient of sum(O * dO) for the masked
// softmax attention of "Gzip-guided Sparse Attention" (daiwk.github.io reproduction
// note, 核心公式 second display), taken over the kept set only.  With P the kept
// softmax of one head:  dV = P^T dO,  dP = dO V^T,  D_t = sum_f dO_tf O_tf,
// dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.  P is recomputed from the
// forward's log-sum-exp, so nothing of size T x T is stored.
//
// Three kernels, all deterministic (no atomics; every output element has one writer):
//   bwd_pre   D for every row (fp32), for callers that run dK/dV without dQ.
//   bwd_dkdv  one workgroup per (sample, head, kv-block j), walking the CSC column of j
//             (query blocks i that keep j); each wave keeps 16 or 32 keys of K_j, V_j in
//             registers and accumulates dK^T, dV^T tiles in fp32 while Q_i, dO_i, LSE_i
//             and D_i stream through two LDS stages by asynchronous global -> LDS copies
//             one piece ahead (32-row pieces at b = 64, whole blocks otherwise); Q_i^T
//             and dO_i^T come from transposing LDS reads.
//   bwd_dq    one workgroup per (sample, head, query block i), walking the CSR row of i;
//             each wave keeps 16 query rows of Q_i and dO_i in registers and accumulates
//             dQ^T while K_j and V_j stream through a ring of three LDS slots (V's slot
//             takes the next V as soon as dS is formed; K^T by transposing reads); at
//             b = 128, d = 128 the blocks stream as 64-row pieces.
//             It also forms D of its rows from O and dO and writes it for dK/dV, so the
//             full backward runs dQ, then dK/dV, with no separate pass for D.
#include <type_traits>

#include "gsa_attn_common.hpp"

namespace gsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <typename T, int HD>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T *__restrict__ o, const T *__restrict__ dout,
                                                      float *__restrict__ dvec, int64_t rows) {
  constexpr int kVec = 16 / sizeof(T);
  constexpr int kLanes = HD / kVec;           // lanes cooperating on one row
  static_assert(kLanes <= 64 && (64 % kLanes) == 0, "row split");
  const int64_t gtid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gtid / kLanes;
  const int part = (int)(gtid % kLanes);
  float acc = 0.f;
  if (row < rows) {
    const T *op = o + row * HD + part * kVec;
    const T *dp = dout + row * HD + part * kVec;
    if constexpr (kVec == 8) {
      const bf16x8 a = *reinterpret_cast<const bf16x8 *>(op);
      const bf16x8 b = *reinterpret_cast<const bf16x8 *>(dp);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf(to_f32(a[e]), to_f32(b[e]), acc);
    } else {
      const f32x4 a = *reinterpret_cast<const f32x4 *>(op);
      const f32x4 b = *reinterpret_cast<const f32x4 *>(dp);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = fmaf(a[e], b[e], acc);
    }
  }
#pragma unroll
  for (int off = 1; off < kLanes; off <<= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && part == 0) dvec[row] = acc;
}

// 16-key groups per wave in dK/dV: two where registers allow, so that each LDS operand
// read feeds two products.
#ifndef GSA_DKDV_GROUPS
#define GSA_DKDV_GROUPS 2
#endif
template <typename T, int BLK, int HD>
constexpr int dkdv_groups() {
  return std::is_same<T, bf16_t>::value && HD <= 64 && BLK % 32 == 0 ? GSA_DKDV_GROUPS : 1;
}

// Query rows per streamed piece of dK/dV (GSA_DKDV_PIECE at b = 64, d = 64, bf16).  With
// 32-row pieces a workgroup's two stages take 16.5 KiB instead of 33, and the kernel is
// asked for three waves per SIMD (<= 168 VGPRs), so six 2-wave workgroups share a CU
// instead of four: 3-5% faster at 8 x 8 KiB; the same pieces at two waves per SIMD were
// 3% slower than whole blocks.
#ifndef GSA_DKDV_PIECE
#define GSA_DKDV_PIECE 32
#endif
template <typename T, int BLK, int HD>
constexpr int dkdv_piece_rows() {
  return std::is_same<T, bf16_t>::value && BLK == 64 && HD == 64 ? GSA_DKDV_PIECE : BLK;
}

// dK, dV of one (sample, head, kv-block j): walk the query blocks i of column j.  Each
// wave owns R groups of 16 keys of block j.
template <typename T, int BLK, int HD, int R>
struct DkdvPolicy {
  static constexpr int KQ = dkdv_piece_rows<T, BLK, HD>();
  using S = AttnShape<T, BLK, HD, R, KQ>;
  using Item = WorkItem;
  static constexpr int kSub = BLK / KQ;   // pieces per query block
  // A stage holds KQ rows of Q_i and of dO_i, then KQ floats each of LSE_i and D_i.
  static constexpr int kStageBytes = 2 * S::kTileBytes + 2 * KQ * 4;
  static constexpr int kVecLanes = KQ / S::kWaves;   // floats of LSE_i (and D_i) per wave
  static_assert(kVecLanes <= 64, "vector slice per wave");

  const T *q, *k, *v, *dout;
  const float *lse, *dvec;
  T *dk, *dv;
  int64_t seq;
  float sl2, scale;
  unsigned char *lds;
  int tid, c, g, key0;   // key0: this lane's key of group 0 inside block j

  typename S::QFrag kf[R], vf[R];
  f32x4 dk_acc[R][S::kDB], dv_acc[R][S::kDB];

  __device__ void operands(const Item &it) {
#pragma unroll
    for (int kg = 0; kg < R; ++kg) {
      const int64_t key_row = it.sh * seq + (int64_t)it.blk * BLK + key0 + 16 * kg;
      S::load_row_frag(kf[kg], k + key_row * HD, g);
      S::load_row_frag(vf[kg], v + key_row * HD, g);
      // -V: dP is then formed as D - dP on the matrix core (accumulator starting at D),
      // so no per-block negation is needed; dK's final scale absorbs the sign.
#pragma unroll
      for (int ks = 0; ks < S::kKS; ++ks) {
        if constexpr (S::kBf16) {
          vf[kg].f[ks] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, vf[kg].f[ks]) ^ 0x80008000u);
        } else {
          vf[kg].f[ks] = -vf[kg].f[ks];
        }
      }
    }
  }
  __device__ void begin(const Item &) {
#pragma unroll
    for (int kg = 0; kg < R; ++kg)
#pragma unroll
      for (int db = 0; db < S::kDB; ++db) {
        dk_acc[kg][db] = f32x4{0.f, 0.f, 0.f, 0.f};
        dv_acc[kg][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
  }
  __device__ void copy(const Item &it, int i, int piece, int stage) {
    const int64_t row0 = it.sh * seq + (int64_t)i * BLK + piece * KQ;
    unsigned char *dst = lds + stage * kStageBytes;
    S::copy_tile(dst, q + row0 * HD, tid);
    S::copy_tile(dst + S::kTileBytes, dout + row0 * HD, tid);
    const int wave = tid >> 6, lane = tid & 63;
    if (lane < kVecLanes) {
      const int x = wave * kVecLanes + lane;
      copy4_to_lds(lse + row0 + x, dst + 2 * S::kTileBytes + wave * kVecLanes * 4);
      copy4_to_lds(dvec + row0 + x, dst + 2 * S::kTileBytes + KQ * 4 + wave * kVecLanes * 4);
    }
  }
  __device__ void compute(const Item &it, int e, int piece, int stage) {
    const unsigned char *lq = lds + stage * kStageBytes;
    const unsigned char *ldo = lq + S::kTileBytes;
    const float *ll = reinterpret_cast<const float *>(lq + 2 * S::kTileBytes);
    const float *ld = ll + KQ;
    const bool diag = e == it.beg;   // column j starts with its own block i = j
    // P[q][key] and dS[q][key], one part of 16*kPartTiles queries at a time;
    // lane: key c of each group, queries piece*KQ + qb*16 + 4g + r.
#pragma unroll
    for (int part = 0; part < S::kParts; ++part) {
      f32x4 p[R][S::kPartTiles], ds[R][S::kPartTiles];
#pragma unroll
      for (int t = 0; t < S::kPartTiles; ++t) {
        const int qb = part * S::kPartTiles + t;
        const f32x4 l2 = *reinterpret_cast<const f32x4 *>(ll + qb * 16 + 4 * g) * kLog2e;
        const f32x4 d4 = *reinterpret_cast<const f32x4 *>(ld + qb * 16 + 4 * g);
        f32x4 st[R], dpd[R];   // dpd = D - dP: -V against dO^T, starting from D
        S::template dot_rows_n<R>(lq, qb * 16 + c, g, kf, st);
        S::template dot_rows_n<R>(ldo, qb * 16 + c, g, vf, dpd, d4);
#pragma unroll
        for (int kg = 0; kg < R; ++kg)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float pr = fast_exp2(fmaf(st[kg][r], sl2, -l2[r]));
            p[kg][t][r] = pr;
            ds[kg][t][r] = pr * dpd[kg][r];   // -dS
          }
        if (diag) {   // token-causal mask, diagonal block only
#pragma unroll
          for (int kg = 0; kg < R; ++kg)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (key0 + 16 * kg > piece * KQ + qb * 16 + 4 * g + r) {
                p[kg][t][r] = 0.f;
                ds[kg][t][r] = 0.f;
              }
        }
      }
      S::template accumulate_part_n<R>(&dv_acc[0][0], ldo, &p[0][0], S::kPartTiles, part, c, g);
      S::template accumulate_part_n<R>(&dk_acc[0][0], lq, &ds[0][0], S::kPartTiles, part, c, g);
    }
  }
  __device__ void finish(const Item &it) {
    // Lane holds features db*16 + 4g + r of its key: four consecutive features.
#pragma unroll
    for (int kg = 0; kg < R; ++kg) {
      const int64_t key_row = it.sh * seq + (int64_t)it.blk * BLK + key0 + 16 * kg;
      T *dkr = dk + key_row * HD;
      T *dvr = dv + key_row * HD;
#pragma unroll
      for (int db = 0; db < S::kDB; ++db) {
        S::store4(dkr + db * 16 + 4 * g, dk_acc[kg][db] * -scale);   // the sum holds -dK / scale
        S::store4(dvr + db * 16 + 4 * g, dv_acc[kg][db]);
      }
    }
  }
};

template <typename T, int BLK, int HD>
__global__ __launch_bounds__((BLK / (16 * dkdv_groups<T, BLK, HD>()) * 64),
                             (dkdv_piece_rows<T, BLK, HD>() < BLK ? 3 : 1)) void bwd_dkdv_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, const T *__restrict__ dout,
    const float *__restrict__ lse, const float *__restrict__ dvec, T *__restrict__ dk, T *__restrict__ dv,
    WorkLists wl, float sl2, float scale) {
  constexpr int R = dkdv_groups<T, BLK, HD>();
  using P = DkdvPolicy<T, BLK, HD, R>;
  __shared__ __align__(16) unsigned char lds[2 * P::kStageBytes];
  const WorkItem it = wl.decode(dispatch_position(blockIdx.x, gridDim.x));

  P pol;
  pol.q = q;
  pol.k = k;
  pol.v = v;
  pol.dout = dout;
  pol.lse = lse;
  pol.dvec = dvec;
  pol.dk = dk;
  pol.dv = dv;
  pol.seq = (int64_t)wl.n * BLK;
  pol.sl2 = sl2;
  pol.scale = scale;
  pol.lds = lds;
  pol.tid = threadIdx.x;
  pol.c = threadIdx.x & 15;
  pol.g = (threadIdx.x & 63) >> 4;
  pol.key0 = (threadIdx.x >> 6) * 16 * R + pol.c;
  run_item(pol, it);
}

// dQ of one (sample, head, query block i): walk the kv-blocks j of row i.  The item's
// D = rowsum(dO * O) is formed from the rows it loads anyway and written out for dK/dV.
template <typename T, int BLK, int HD>
struct DqPolicy {
  static constexpr int KC = kv_piece_rows<T, BLK, HD>();
  using S = AttnShape<T, BLK, HD, 1, KC>;
  using Item = WorkItem;
  static constexpr int kSub = BLK / KC;                  // pieces per kv-block
  static constexpr int kLdsBytes = 3 * S::kTileBytes;   // the ring: K, V and a spare

  const T *q, *k, *v, *o, *dout;
  const float *lse;
  float *dvec;
  T *dq;
  int64_t seq;
  float sl2, scale;
  unsigned char *lds;
  int tid, c, g, q_in_blk;

  typename S::QFrag qf, dof;
  float lse2, dd;
  f32x4 acc[S::kDB];

  __device__ void operands(const Item &it) {
    const int64_t q_row = it.sh * seq + (int64_t)it.blk * BLK + q_in_blk;
    typename S::QFrag of;
    S::load_row_frag(qf, q + q_row * HD, g);
    S::load_row_frag(dof, dout + q_row * HD, g);
    S::load_row_frag(of, o + q_row * HD, g);
    lse2 = lse[q_row] * kLog2e;
    // D over this lane's feature slots, then across the four lane groups of the row.
    float part = 0.f;
#pragma unroll
    for (int ks = 0; ks < S::kKS; ++ks) {
      if constexpr (S::kBf16) {
#pragma unroll
        for (int x = 0; x < 8; ++x) part = fmaf(to_f32(dof.f[ks][x]), to_f32(of.f[ks][x]), part);
      } else {
        part = fmaf(dof.f[ks], of.f[ks], part);
      }
    }
    dd = group_sum4(part);
    if (g == 0) dvec[q_row] = dd;
  }
  __device__ void begin(const Item &) {
#pragma unroll
    for (int db = 0; db < S::kDB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  static constexpr bool kFreeK = false;   // V_j is done once dS is formed; K_j is read again
  __device__ void copy_k(const Item &it, int j, int piece, int slot) {
    S::copy_tile(lds + slot * S::kTileBytes, k + (it.sh * seq + (int64_t)j * BLK + piece * KC) * HD, tid);
  }
  __device__ void copy_v(const Item &it, int j, int piece, int slot) {
    S::copy_tile(lds + slot * S::kTileBytes, v + (it.sh * seq + (int64_t)j * BLK + piece * KC) * HD, tid);
  }
  // dS^T[key][q] of every key of the piece (lane holds keys piece*KC + kb*16 + 4g + r of its
  // query): S^T from K and dP^T - D from V.
  f32x4 dsr[S::kKB];
  __device__ void compute_a(const Item &it, int e, int piece, int k_slot, int v_slot) {
    const unsigned char *lk = lds + k_slot * S::kTileBytes;
    const unsigned char *lv = lds + v_slot * S::kTileBytes;
    const bool diag = e == it.end - 1;   // row i ends with its own block j = i
#pragma unroll
    for (int kb = 0; kb < S::kKB; ++kb) {
      const f32x4 st = S::dot_rows(lk, kb * 16 + c, g, qf);
      const f32x4 dpd = S::dot_rows(lv, kb * 16 + c, g, dof, f32x4{-dd, -dd, -dd, -dd});   // dP - D
#pragma unroll
      for (int r = 0; r < 4; ++r) dsr[kb][r] = fast_exp2(fmaf(st[r], sl2, -lse2)) * dpd[r];
      if (diag) {   // token-causal mask, diagonal block only
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (piece * KC + kb * 16 + 4 * g + r > q_in_blk) dsr[kb][r] = 0.f;
      }
    }
  }
  // dQ^T += K^T dS^T over the piece, one part of 16*kPartTiles keys at a time.
  __device__ void compute_b(const Item &, int, int, int k_slot, int) {
    const unsigned char *lk = lds + k_slot * S::kTileBytes;
#pragma unroll
    for (int part = 0; part < S::kParts; ++part)
      S::accumulate_part(acc, lk, &dsr[part * S::kPartTiles], part, c, g);
  }
  __device__ void finish(const Item &it) {
    const int64_t q_row = it.sh * seq + (int64_t)it.blk * BLK + q_in_blk;
    T *dqr = dq + q_row * HD;
#pragma unroll
    for (int db = 0; db < S::kDB; ++db) S::store4(dqr + db * 16 + 4 * g, acc[db] * scale);
  }
};

template <typename T, int BLK, int HD>
__global__ __launch_bounds__(BLK / 16 * 64, HD <= 64 ? 1 : 2) void bwd_dq_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, const T *__restrict__ o,
    const T *__restrict__ dout, const float *__restrict__ lse, float *__restrict__ dvec, T *__restrict__ dq,
    WorkLists wl, float sl2, float scale) {
  using P = DqPolicy<T, BLK, HD>;
  __shared__ __align__(16) unsigned char lds[P::kLdsBytes];
  const WorkItem it = wl.decode(dispatch_position(blockIdx.x, gridDim.x));

  P pol;
  pol.q = q;
  pol.k = k;
  pol.v = v;
  pol.o = o;
  pol.dout = dout;
  pol.lse = lse;
  pol.dvec = dvec;
  pol.dq = dq;
  pol.seq = (int64_t)wl.n * BLK;
  pol.sl2 = sl2;
  pol.scale = scale;
  pol.lds = lds;
  pol.tid = threadIdx.x;
  pol.c = threadIdx.x & 15;
  pol.g = (threadIdx.x & 63) >> 4;
  pol.q_in_blk = (threadIdx.x >> 6) * 16 + pol.c;
  run_item_ring(pol, it);
}

template <typename T, int BLK, int HD>
gsa_status launch_dq_instance(const gsa_bwd_args &a, const gsa_mask &m, hipStream_t stream) {
  using S = AttnShape<T, BLK, HD>;
  const gsa_fwd_args &f = a.f;
  const int64_t items = f.batch * f.heads * (int64_t)m.n_blocks;
  const float scale = f.scale > 0.f ? f.scale : 1.0f / sqrtf((float)HD);
  const WorkLists wl{m.work_row, m.col_idx, f.heads, m.n_blocks, m.n_heads[0], m.n_heads[1],
                     mask_cap(m.n_blocks)};
  hipLaunchKernelGGL((bwd_dq_kernel<T, BLK, HD>), dim3((unsigned)items), dim3(S::kThreads), 0, stream,
                     static_cast<const T *>(f.q), static_cast<const T *>(f.k), static_cast<const T *>(f.v),
                     static_cast<const T *>(f.o), static_cast<const T *>(a.dout), f.lse, a.workspace,
                     static_cast<T *>(a.dq), wl, scale * kLog2e, scale);
  return check_launch("bwd_dq_kernel");
}

#ifndef GSA_WIDE_TU
template <typename T, int BLK, int HD>
gsa_status launch_bwd_instance(const gsa_bwd_args &a, const gsa_mask &m, hipStream_t stream, int stages) {
  using SK = AttnShape<T, BLK, HD, dkdv_groups<T, BLK, HD>()>;
  const gsa_fwd_args &f = a.f;
  const int64_t items = f.batch * f.heads * (int64_t)m.n_blocks;
  const int64_t rows = f.batch * f.heads * f.seq_len;
  const float scale = f.scale > 0.f ? f.scale : 1.0f / sqrtf((float)HD);
  const float sl2 = scale * kLog2e;
  const T *q = static_cast<const T *>(f.q);
  const T *k = static_cast<const T *>(f.k);
  const T *v = static_cast<const T *>(f.v);
  const T *o = static_cast<const T *>(f.o);
  const T *dout = static_cast<const T *>(a.dout);

  constexpr int kLanes = HD / (16 / sizeof(T));
  if (stages & kBwdPrep) {
    const int64_t pre_threads = rows * kLanes;
    hipLaunchKernelGGL((bwd_pre_kernel<T, HD>), dim3((unsigned)((pre_threads + 255) / 256)), dim3(256), 0,
                       stream, o, dout, a.workspace, rows);
    gsa_status st = check_launch("bwd_pre_kernel");
    if (st != GSA_OK) return st;
  }
  if (stages & kBwdDq) {
    gsa_status st;
    if constexpr (std::is_same<T, bf16_t>::value && BLK == 128 && HD == 128) {
      st = launch_dq_wide(a, m, stream);
    } else {
      st = launch_dq_instance<T, BLK, HD>(a, m, stream);
    }
    if (st != GSA_OK) return st;
  }
  if (stages & kBwdDkdv) {
    const WorkLists wl{m.work_col, m.row_idx, f.heads, m.n_blocks, m.n_heads[0], m.n_heads[1],
                       mask_cap(m.n_blocks)};
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, BLK, HD>), dim3((unsigned)items), dim3(SK::kThreads), 0, stream, q, k,
                       v, dout, f.lse, a.workspace, static_cast<T *>(a.dk), static_cast<T *>(a.dv), wl, sl2,
                       scale);
    gsa_status st = check_launch("bwd_dkdv_kernel");
    if (st != GSA_OK) return st;
  }
  return GSA_OK;
}
#endif

}  // namespace

#ifdef GSA_WIDE_TU
gsa_status launch_dq_wide(const gsa_bwd_args &a, const gsa_mask &m, hipStream_t stream) {
  return launch_dq_instance<bf16_t, 128, 128>(a, m, stream);
}
#else
gsa_status launch_attn_bwd(const gsa_bwd_args &a, const gsa_mask &m, hipStream_t stream, int stages) {
  const gsa_fwd_args &f = a.f;
  if (f.dtype == GSA_F32 && f.block == 16 && f.head_dim == 32)
    return launch_bwd_instance<float, 16, 32>(a, m, stream, stages);
  if (f.dtype == GSA_BF16 && f.block == 64 && f.head_dim == 64)
    return launch_bwd_instance<bf16_t, 64, 64>(a, m, stream, stages);
  if (f.dtype == GSA_BF16 && f.block == 128 && f.head_dim == 128)
    return launch_bwd_instance<bf16_t, 128, 128>(a, m, stream, stages);
  return fail(GSA_ERR_UNSUPPORTED, "no backward kernel for dtype %d, block %d, head_dim %d", f.dtype, f.block,
              f.head_dim);
}
#endif

}  // namespace gsa
