// Forward of gzip-guided block-sparse causal attention on gfx950.
//
// What is computed ("Gzip-guided Sparse Attention", daiwk.github.io reproduction note,
// 核心公式 second display, and 复现边界, where the reproduction takes the dense scores and
// masks them): for head h of class k(h) and query block i, softmax(scale Q_i K^T) V over
// the keys of the kv-blocks j in row i of that class's mask, token-causal inside the
// diagonal block.  Keys outside the kept blocks carry exactly zero weight in the dense
// masked form, so visiting only the kept blocks gives the same result.
//
// Design (one workgroup per (sample, head, query block); BLK/16 waves, 16 query rows
// each):
//   * The query rows of a wave stay in registers as the B operand of S^T = K Q^T, so
//     each lane owns one query column of every score tile and its online-softmax state
//     (running max m and a lane-partial sum l) without cross-lane traffic except two
//     shuffles for the row max.
//   * K_j is staged row-major and V_j transposed in LDS, once per kv-block, shared by all
//     waves.  O^T = V^T P^T accumulates in fp32 registers; P re-enters the MFMA straight
//     from the S^T accumulator (rounded to bf16 in the bf16 instance).
//   * Scores are scaled by scale * log2(e) so every exponential is one exp2.
//   * Only the diagonal block applies the token-causal mask.  Rows are never empty: the
//     diagonal block is always kept and a query always sees itself.
//   * Workgroups run in the mask kernel's longest-row-first order, with runs of adjacent
//     items kept on one XCD (see work_position).
#include <type_traits>

#include "gsa_attn_common.hpp"

namespace gsa {
namespace {

template <typename T, int BLK, int HD>
__global__ __launch_bounds__(BLK / 16 * 64) void attn_fwd_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, T *__restrict__ o,
    float *__restrict__ lse, const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ col_idx,
    const int32_t *__restrict__ work, int heads, int n, int64_t cap, int n_loc, int n_lit,
    int64_t items, float sl2) {
  using S = AttnShape<T, BLK, HD>;
  __shared__ __align__(16) T s_k[BLK * S::kRowStride];   // K_j, row-major
  __shared__ __align__(16) T s_vt[HD * S::kTStride];     // V_j transposed: [d][key]

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
  const T *qh = q + head_off;
  const T *kh = k + head_off;
  const T *vh = v + head_off;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int q_in_blk = wave * 16 + c;            // this lane's query row inside block i
  const int64_t q_row = (int64_t)i * BLK + q_in_blk;

  typename S::QFrag qf;
  S::load_row_frag(qf, qh + q_row * HD, g);

  f32x4 acc[S::kDB];
#pragma unroll
  for (int db = 0; db < S::kDB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.f;

  for (int e = beg; e < end; ++e) {
    const int j = cidx[e];
    __syncthreads();
    S::stage_rows(s_k, kh + (int64_t)j * BLK * HD, tid);
    S::stage_cols(s_vt, vh + (int64_t)j * BLK * HD, tid);
    __syncthreads();

    // S^T tile: lane holds keys kb*16 + 4g + r of query q_in_blk.
    f32x4 st[S::kKB];
#pragma unroll
    for (int kb = 0; kb < S::kKB; ++kb) st[kb] = S::dot_rows(s_k, kb * 16 + c, g, qf);

    if (j == i) {
#pragma unroll
      for (int kb = 0; kb < S::kKB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (kb * 16 + 4 * g + r > q_in_blk) st[kb][r] = -INFINITY;
    }

    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < S::kKB; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, st[kb][r]);
    mx = group_max4(mx);
    const float m_new = fmaxf(m_run, mx * sl2);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    l_part *= alpha;
#pragma unroll
    for (int db = 0; db < S::kDB; ++db) acc[db] *= alpha;

#pragma unroll
    for (int kb = 0; kb < S::kKB; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(fmaf(st[kb][r], sl2, -m_new));
        st[kb][r] = p;
        l_part += p;
      }
    S::accumulate_pv(acc, s_vt, st, c, g);
  }

  const float l = group_sum4(l_part);
  const float inv = 1.0f / l;
  T *oh = o + head_off + q_row * HD;
#pragma unroll
  for (int db = 0; db < S::kDB; ++db) S::store4(oh + db * 16 + 4 * g, acc[db] * inv);
  if (lse != nullptr && g == 0) lse[sh * seq + q_row] = (m_run + __log2f(l)) * 0.69314718055994531f;
}

template <typename T, int BLK, int HD>
gsa_status launch_fwd_instance(const gsa_fwd_args &a, const gsa_mask &m, hipStream_t stream) {
  using S = AttnShape<T, BLK, HD>;
  const int64_t items = a.batch * a.heads * (int64_t)m.n_blocks;
  const float scale = a.scale > 0.f ? a.scale : 1.0f / sqrtf((float)HD);
  const float sl2 = scale * 1.4426950408889634f;
  hipLaunchKernelGGL((attn_fwd_kernel<T, BLK, HD>), dim3((unsigned)padded_grid(items)),
                     dim3(S::kThreads), 0, stream, static_cast<const T *>(a.q),
                     static_cast<const T *>(a.k), static_cast<const T *>(a.v), static_cast<T *>(a.o),
                     a.lse, m.row_ptr, m.col_idx, m.work_row, a.heads, m.n_blocks, mask_cap(m.n_blocks),
                     m.n_heads[0], m.n_heads[1], items, sl2);
  return check_launch("attn_fwd_kernel");
}

}  // namespace

bool attn_instance_built(int32_t dtype, int32_t block, int32_t head_dim) {
  if (dtype == GSA_F32) return block == 16 && head_dim == 32;
  if (dtype == GSA_BF16) return (block == 64 && head_dim == 64) || (block == 128 && head_dim == 128);
  return false;
}

gsa_status launch_attn_fwd(const gsa_fwd_args &a, const gsa_mask &m, hipStream_t stream) {
  if (a.dtype == GSA_F32 && a.block == 16 && a.head_dim == 32)
    return launch_fwd_instance<float, 16, 32>(a, m, stream);
  if (a.dtype == GSA_BF16 && a.block == 64 && a.head_dim == 64)
    return launch_fwd_instance<bf16_t, 64, 64>(a, m, stream);
  if (a.dtype == GSA_BF16 && a.block == 128 && a.head_dim == 128)
    return launch_fwd_instance<bf16_t, 128, 128>(a, m, stream);
  return fail(GSA_ERR_UNSUPPORTED, "no forward kernel for dtype %d, block %d, head_dim %d", a.dtype,
              a.block, a.head_dim);
}

}  // namespace gsa
