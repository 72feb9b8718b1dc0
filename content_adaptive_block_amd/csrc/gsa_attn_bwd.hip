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
//   bwd_pre   D for every row (fp32).
//   bwd_dkdv  one workgroup per (sample, head, kv-block j), walking the CSC column of j
//             (query blocks i that keep j); each wave keeps 16 keys of K_j, V_j in
//             registers and accumulates dK^T, dV^T tiles in fp32 while Q_i and dO_i are
//             staged in LDS (row-major and transposed).
//   bwd_dq    one workgroup per (sample, head, query block i), walking the CSR row of i;
//             each wave keeps 16 query rows of Q_i and dO_i in registers and accumulates
//             dQ^T while K_j (both layouts) and V_j are staged in LDS.
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

template <typename T, int BLK, int HD>
__global__ __launch_bounds__(BLK / 16 * 64) void bwd_dkdv_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, const T *__restrict__ dout,
    const float *__restrict__ lse, const float *__restrict__ dvec, T *__restrict__ dk, T *__restrict__ dv,
    const int32_t *__restrict__ col_ptr, const int32_t *__restrict__ row_idx, const int32_t *__restrict__ work,
    int heads, int n, int64_t cap, int n_loc, int n_lit, int64_t items, float sl2, float scale) {
  using S = AttnShape<T, BLK, HD>;
  __shared__ __align__(16) T s_q[BLK * S::kRowStride];
  __shared__ __align__(16) T s_qt[HD * S::kTStride];
  __shared__ __align__(16) T s_do[BLK * S::kRowStride];
  __shared__ __align__(16) T s_dot[HD * S::kTStride];
  __shared__ float s_lse[BLK];
  __shared__ float s_d[BLK];

  const int64_t pos = work_position(blockIdx.x, items);
  if (pos < 0) return;
  const int64_t item = work[pos];
  const int j = (int)(item % n);
  const int64_t sh = item / n;
  const int h = (int)(sh % heads);
  const int64_t s = sh / heads;
  const int cls = head_class(h, n_loc, n_lit);
  const int32_t *cp = col_ptr + (s * 3 + cls) * (int64_t)(n + 1);
  const int32_t *ridx = row_idx + (s * 3 + cls) * cap;
  const int beg = cp[j], end = cp[j + 1];

  const int64_t seq = (int64_t)n * BLK;
  const int64_t head_off = sh * seq * HD;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int key_in_blk = wave * 16 + c;
  const int64_t key_row = (int64_t)j * BLK + key_in_blk;

  typename S::QFrag kf, vf;
  S::load_row_frag(kf, k + head_off + key_row * HD, g);
  S::load_row_frag(vf, v + head_off + key_row * HD, g);

  f32x4 dk_acc[S::kDB], dv_acc[S::kDB];
#pragma unroll
  for (int db = 0; db < S::kDB; ++db) {
    dk_acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    dv_acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int e = beg; e < end; ++e) {
    const int i = ridx[e];
    const int64_t blk_off = head_off + (int64_t)i * BLK * HD;
    __syncthreads();
    S::stage_rows(s_q, q + blk_off, tid);
    S::stage_cols(s_qt, q + blk_off, tid);
    S::stage_rows(s_do, dout + blk_off, tid);
    S::stage_cols(s_dot, dout + blk_off, tid);
    for (int t = tid; t < BLK; t += S::kThreads) {
      s_lse[t] = lse[sh * seq + (int64_t)i * BLK + t] * kLog2e;
      s_d[t] = dvec[sh * seq + (int64_t)i * BLK + t];
    }
    __syncthreads();

    // P[q][key] and dS[q][key] for the 16-query tiles of block i; lane: key c, queries 4g+r.
    f32x4 p[S::kKB], ds[S::kKB];
#pragma unroll
    for (int qb = 0; qb < S::kKB; ++qb) {
      const f32x4 st = S::dot_rows(s_q, qb * 16 + c, g, kf);
      const f32x4 dp = S::dot_rows(s_do, qb * 16 + c, g, vf);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qi = qb * 16 + 4 * g + r;
        float pr = fast_exp2(fmaf(st[r], sl2, -s_lse[qi]));
        if (i == j && key_in_blk > qi) pr = 0.f;
        p[qb][r] = pr;
        ds[qb][r] = pr * (dp[r] - s_d[qi]);
      }
    }
    S::accumulate_pv(dv_acc, s_dot, p, c, g);
    S::accumulate_pv(dk_acc, s_qt, ds, c, g);
  }

  // Lane holds features db*16 + 4g + r of key key_row: four consecutive features.
  T *dkr = dk + head_off + key_row * HD;
  T *dvr = dv + head_off + key_row * HD;
#pragma unroll
  for (int db = 0; db < S::kDB; ++db) {
    S::store4(dkr + db * 16 + 4 * g, dk_acc[db] * scale);
    S::store4(dvr + db * 16 + 4 * g, dv_acc[db]);
  }
}

template <typename T, int BLK, int HD>
__global__ __launch_bounds__(BLK / 16 * 64) void bwd_dq_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, const T *__restrict__ dout,
    const float *__restrict__ lse, const float *__restrict__ dvec, T *__restrict__ dq,
    const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ col_idx, const int32_t *__restrict__ work,
    int heads, int n, int64_t cap, int n_loc, int n_lit, int64_t items, float sl2, float scale) {
  using S = AttnShape<T, BLK, HD>;
  __shared__ __align__(16) T s_k[BLK * S::kRowStride];
  __shared__ __align__(16) T s_kt[HD * S::kTStride];
  __shared__ __align__(16) T s_v[BLK * S::kRowStride];

  const int64_t pos = work_position(blockIdx.x, items);
  if (pos < 0) return;
  const int64_t item = work[pos];
  const int i = (int)(item % n);
  const int64_t sh = item / n;
  const int h = (int)(sh % heads);
  const int64_t s = sh / heads;
  const int cls = head_class(h, n_loc, n_lit);
  const int32_t *rp = row_ptr + (s * 3 + cls) * (int64_t)(n + 1);
  const int32_t *cidx = col_idx + (s * 3 + cls) * cap;
  const int beg = rp[i], end = rp[i + 1];

  const int64_t seq = (int64_t)n * BLK;
  const int64_t head_off = sh * seq * HD;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int q_in_blk = wave * 16 + c;
  const int64_t q_row = (int64_t)i * BLK + q_in_blk;

  typename S::QFrag qf, dof;
  S::load_row_frag(qf, q + head_off + q_row * HD, g);
  S::load_row_frag(dof, dout + head_off + q_row * HD, g);
  const float lse2 = lse[sh * seq + q_row] * kLog2e;
  const float dd = dvec[sh * seq + q_row];

  f32x4 acc[S::kDB];
#pragma unroll
  for (int db = 0; db < S::kDB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int e = beg; e < end; ++e) {
    const int j = cidx[e];
    const int64_t blk_off = head_off + (int64_t)j * BLK * HD;
    __syncthreads();
    S::stage_rows(s_k, k + blk_off, tid);
    S::stage_cols(s_kt, k + blk_off, tid);
    S::stage_rows(s_v, v + blk_off, tid);
    __syncthreads();

    // dS^T[key][q]: lane holds keys kb*16 + 4g + r of its query.
    f32x4 ds[S::kKB];
#pragma unroll
    for (int kb = 0; kb < S::kKB; ++kb) {
      const f32x4 st = S::dot_rows(s_k, kb * 16 + c, g, qf);
      const f32x4 dp = S::dot_rows(s_v, kb * 16 + c, g, dof);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float pr = fast_exp2(fmaf(st[r], sl2, -lse2));
        if (j == i && kb * 16 + 4 * g + r > q_in_blk) pr = 0.f;
        ds[kb][r] = pr * (dp[r] - dd);
      }
    }
    S::accumulate_pv(acc, s_kt, ds, c, g);
  }

  T *dqr = dq + head_off + q_row * HD;
#pragma unroll
  for (int db = 0; db < S::kDB; ++db) S::store4(dqr + db * 16 + 4 * g, acc[db] * scale);
}

template <typename T, int BLK, int HD>
gsa_status launch_bwd_instance(const gsa_bwd_args &a, const gsa_mask &m, hipStream_t stream, int stages) {
  using S = AttnShape<T, BLK, HD>;
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
  const unsigned grid = (unsigned)padded_grid(items);
  if (stages & kBwdDkdv) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, BLK, HD>), dim3(grid), dim3(S::kThreads), 0, stream, q, k, v, dout,
                       f.lse, a.workspace, static_cast<T *>(a.dk), static_cast<T *>(a.dv), m.col_ptr, m.row_idx,
                       m.work_col, f.heads, m.n_blocks, mask_cap(m.n_blocks), m.n_heads[0], m.n_heads[1], items,
                       sl2, scale);
    gsa_status st = check_launch("bwd_dkdv_kernel");
    if (st != GSA_OK) return st;
  }
  if (stages & kBwdDq) {
    hipLaunchKernelGGL((bwd_dq_kernel<T, BLK, HD>), dim3(grid), dim3(S::kThreads), 0, stream, q, k, v, dout,
                       f.lse, a.workspace, static_cast<T *>(a.dq), m.row_ptr, m.col_idx, m.work_row, f.heads,
                       m.n_blocks, mask_cap(m.n_blocks), m.n_heads[0], m.n_heads[1], items, sl2, scale);
    gsa_status st = check_launch("bwd_dq_kernel");
    if (st != GSA_OK) return st;
  }
  return GSA_OK;
}

}  // namespace

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

}  // namespace gsa
