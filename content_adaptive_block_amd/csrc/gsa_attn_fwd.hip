// Forward of gzip-guided block-sparse causal attention on gfx950.
//
// What is computed ("Gzip-guided Sparse Attention", daiwk.github.io reproduction note,
// 核心公式 second display, and 复现边界, where the reproduction takes the dense scores and
// masks them): for head h of class k(h) and query block i, softmax(scale Q_i K^T) V over
// the keys of the kv-blocks j in row i of that class's mask, token-causal inside the
// diagonal block.  Keys outside the kept blocks carry exactly zero weight in the dense
// masked form, so visiting only the kept blocks gives the same result.
//
// Design (one workgroup of BLK/16 waves per (sample, head, query block); each wave owns
// 16 of its query rows):
//   * The query rows of a wave stay in registers as the B operand of S^T = K Q^T, so
//     each lane owns one query column of every score tile and its online-softmax state
//     (running max m and a lane-partial sum l); the row max needs two permlane swaps.
//   * K_j and V_j stream row-major (swizzled) into two LDS stages by asynchronous
//     global -> LDS copies, one kept block ahead of the one being computed.  O^T =
//     V^T P^T reads V^T with transposing LDS loads and takes P straight from the S^T
//     accumulator (rounded to bf16 in the bf16 instance).
//   * Scores are scaled by scale * log2(e) so every exponential is one exp2.  The
//     reference max is raised only when a row's max exceeds it by more than 2^8; O and l
//     share that reference, so the result is unchanged and most rescales are skipped.
//   * Only the diagonal block applies the token-causal mask.  Rows are never empty: the
//     diagonal block is always kept and a query always sees itself.
//   * Workgroups run in the mask kernel's work order (longest rows first, by octave of
//     length), runs of 16 consecutive items per XCD.
#include <type_traits>

#include "gsa_attn_common.hpp"

namespace gsa {
namespace {

constexpr float kRescaleSlack = 8.0f;   // log2 units

template <typename T, int BLK, int HD>
struct FwdPolicy {
  using S = AttnShape<T, BLK, HD>;
  using Item = WorkItem;
  static constexpr int kStageBytes = 2 * S::kTileBytes;

  WorkLists wl;
  const T *q, *k, *v;
  T *o;
  float *lse;
  int64_t seq;
  float sl2;
  unsigned char *lds;
  int tid, c, g, q_in_blk;

  typename S::QFrag qf;
  f32x4 acc[S::kDB];
  float m_run, l_part;

  __device__ void operands(const Item &it) {
    S::load_row_frag(qf, q + (it.sh * seq + (int64_t)it.blk * BLK + q_in_blk) * HD, g);
  }
  __device__ void begin(const Item &) {
#pragma unroll
    for (int db = 0; db < S::kDB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;
    l_part = 0.f;
  }
  __device__ void copy(const Item &it, int j, int stage) {
    const int64_t off = (it.sh * seq + (int64_t)j * BLK) * HD;
    unsigned char *dst = lds + stage * kStageBytes;
    S::copy_tile(dst, k + off, tid);
    S::copy_tile(dst + S::kTileBytes, v + off, tid);
  }
  __device__ void compute(const Item &it, int e, int stage) {
    const unsigned char *lk = lds + stage * kStageBytes;
    const unsigned char *lv = lk + S::kTileBytes;
    // S^T tile: lane holds keys kb*16 + 4g + r of query q_in_blk.
    f32x4 st[S::kKB];
#pragma unroll
    for (int kb = 0; kb < S::kKB; ++kb) st[kb] = S::dot_rows(lk, kb * 16 + c, g, qf);
    if (e == it.end - 1) {   // the diagonal block is the last (largest) entry of row i
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
    mx = group_max4(mx) * sl2;
    if (mx > m_run + kRescaleSlack) {
      const float alpha = fast_exp2(m_run - mx);
      m_run = mx;
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < S::kDB; ++db) acc[db] *= alpha;
    }
#pragma unroll
    for (int kb = 0; kb < S::kKB; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(fmaf(st[kb][r], sl2, -m_run));
        st[kb][r] = p;
        l_part += p;
      }
    S::accumulate_pv(acc, lv, st, c, g);
  }
  __device__ void finish(const Item &it) {
    const float l = group_sum4(l_part);
    const float inv = 1.0f / l;
    const int64_t q_row = it.sh * seq + (int64_t)it.blk * BLK + q_in_blk;
    T *orow = o + q_row * HD;
#pragma unroll
    for (int db = 0; db < S::kDB; ++db) S::store4(orow + db * 16 + 4 * g, acc[db] * inv);
    if (lse != nullptr && g == 0) lse[q_row] = (m_run + __log2f(l)) * 0.69314718055994531f;
  }
};

template <typename T, int BLK, int HD>
__global__ __launch_bounds__(BLK / 16 * 64) void attn_fwd_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, T *__restrict__ o,
    float *__restrict__ lse, WorkLists wl, float sl2) {
  using P = FwdPolicy<T, BLK, HD>;
  __shared__ __align__(16) unsigned char lds[2 * P::kStageBytes];
  const WorkItem it = wl.decode(dispatch_position(blockIdx.x, gridDim.x));

  P pol;
  pol.wl = wl;
  pol.q = q;
  pol.k = k;
  pol.v = v;
  pol.o = o;
  pol.lse = lse;
  pol.seq = (int64_t)wl.n * BLK;
  pol.sl2 = sl2;
  pol.lds = lds;
  pol.tid = threadIdx.x;
  pol.c = threadIdx.x & 15;
  pol.g = (threadIdx.x & 63) >> 4;
  pol.q_in_blk = (threadIdx.x >> 6) * 16 + pol.c;
  run_item(pol, it);
}

template <typename T, int BLK, int HD>
gsa_status launch_fwd_instance(const gsa_fwd_args &a, const gsa_mask &m, hipStream_t stream) {
  using S = AttnShape<T, BLK, HD>;
  const int64_t items = a.batch * a.heads * (int64_t)m.n_blocks;
  const float scale = a.scale > 0.f ? a.scale : 1.0f / sqrtf((float)HD);
  const float sl2 = scale * 1.4426950408889634f;
  const WorkLists wl{m.work_row, m.col_idx, a.heads, m.n_blocks, m.n_heads[0], m.n_heads[1],
                     mask_cap(m.n_blocks)};
  hipLaunchKernelGGL((attn_fwd_kernel<T, BLK, HD>), dim3((unsigned)items), dim3(S::kThreads), 0, stream,
                     static_cast<const T *>(a.q), static_cast<const T *>(a.k), static_cast<const T *>(a.v),
                     static_cast<T *>(a.o), a.lse, wl, sl2);
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
