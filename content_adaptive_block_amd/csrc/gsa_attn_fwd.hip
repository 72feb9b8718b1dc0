// Forward of gzip-guided block-sparse causal attention on gfx950.
//
// What is computed ("Gzip-guided Sparse Attention", daiwk.github.io reproduction note,
// 核心公式 second display, and 复现边界, where the reproduction takes the dense scores and
// masks them): for head h of class k(h) and query block i, softmax(scale Q_i K^T) V over
// the keys of the kv-blocks j in row i of that class's mask, token-causal inside the
// diagonal block.  Keys outside the kept blocks carry exactly zero weight in the dense
// masked form, so visiting only the kept blocks gives the same result.
//
// Design (one workgroup per (sample, head, query block); each wave owns 16 of its query
// rows, 32 at b = d = 128):
//   * The query rows of a wave stay in registers as the B operand of S^T = K Q^T, so
//     each lane owns one query column of every score tile and its online-softmax state
//     (running max m and a lane-partial sum l); the row max needs two permlane swaps.
//     With two 16-row groups per wave every K and V read from LDS feeds two products.
//   * K_j and V_j stream row-major (swizzled) into a ring of three LDS tiles by
//     asynchronous global -> LDS copies: K_{j+1} lands in the spare tile while block j
//     is computed, V_{j+1} in K_j's tile once the scores of block j are done.  At
//     b = 128, d = 128 they stream in 64-row pieces through four slots (this piece's K
//     and V, and the next piece's, copied as the step starts), so that two workgroups
//     fit a CU and a step needs one barrier.  O^T = V^T P^T reads V^T with transposing
//     LDS loads and takes P straight from the S^T accumulator (rounded to bf16 in the
//     bf16 instance); O leaves through LDS in whole rows.
//   * Scores are scaled by scale * log2(e) so every exponential is one exp2.  The
//     reference max is raised only when a row's max exceeds it by more than 2^8; O and l
//     share that reference, so the result is unchanged and most rescales are skipped.
//   * Only the diagonal block applies the token-causal mask.  Rows are never empty: the
//     diagonal block is always kept and a query always sees itself.
//   * Workgroups run in the mask kernel's work order (longest rows first, by octave of
//     length), runs of 8 consecutive items per XCD.
#include <type_traits>

#include "gsa_attn_common.hpp"

namespace gsa {
namespace {

constexpr float kRescaleSlack = 8.0f;   // log2 units
// Score of a masked key and the initial running max: finite (the build assumes finite
// math), and exp2 of it minus any real score is exactly 0.
constexpr float kMaskedScore = -1.0e30f;

#ifndef GSA_FWD_GROUPS
#define GSA_FWD_GROUPS 1
#endif
// 16-row query groups per wave.  Two groups halve the LDS reads per tile (every K and V
// read feeds two products) but need more registers.  At b = d = 64 (GSA_FWD_GROUPS) they
// need 146 VGPRs, which halves the resident waves at the same six items per CU: 98.2-98.5
// vs 97.6-98.4 us at 8 x 8 KiB, equal, so one group, with the fewer registers.  At b = d = 128 (GSA_FWD_GROUPS_WIDE) eight one-group waves read 512 KiB of LDS
// per kept tile, about 90 bytes per clock per CU, so LDS bandwidth binds; two groups (4
// waves, 215 VGPRs, two waves per SIMD) read half of it: 2.36-2.46 vs 2.56-2.61 ms at
// 2 x 64 KiB.
#ifndef GSA_FWD_GROUPS_WIDE
#define GSA_FWD_GROUPS_WIDE 2
#endif
// Four LDS slots (K and V of this piece and of the next, one barrier per step) at b = 128,
// where registers, not LDS, limit the kernel to two workgroups per CU: 2.05-2.06 vs
// 2.19-2.20 ms at 2 x 64 KiB (fewer registers too, 201 vs 222).  At b = 64
// (GSA_FWD_RING4) the three-slot ring keeps six workgroups per CU instead of five:
// 97.6-98.4 vs 102.5-102.9 us at 8 x 8 KiB.
#ifndef GSA_FWD_RING4_WIDE
#define GSA_FWD_RING4_WIDE 1
#endif
#ifndef GSA_FWD_RING4
#define GSA_FWD_RING4 0
#endif
template <typename T, int BLK, int HD>
constexpr int fwd_groups() {
  if (std::is_same<T, bf16_t>::value && HD <= 64 && BLK % 32 == 0) return GSA_FWD_GROUPS;
  if (std::is_same<T, bf16_t>::value && HD == 128 && BLK == 128) return GSA_FWD_GROUPS_WIDE;
  return 1;
}

template <typename T, int BLK, int HD, int R>
struct FwdPolicy {
  static constexpr int KC = kv_piece_rows<T, BLK, HD>();
  using S = AttnShape<T, BLK, HD, R, KC>;
  using Item = WorkItem;
  static constexpr int kSub = BLK / KC;   // pieces per kv-block
  static constexpr bool kRing4 = BLK == 128 ? GSA_FWD_RING4_WIDE : GSA_FWD_RING4;
  static constexpr int kLdsBytes = (kRing4 ? 4 : 3) * S::kTileBytes;
  static_assert(S::kWaves * S::kAreaBytes <= (kRing4 ? 2 : 1) * S::kTileBytes, "output staging fits the free slots");

  const T *q, *k, *v;
  T *o;
  float *lse;
  int64_t seq;
  float sl2;
  unsigned char *lds;
  int tid, c, g, q0;   // q0: this lane's query of group 0 in the block; group r: q0 + 16 r
  int wave, lane;      // wave: wave-uniform
  rsrc_t rk, rv;       // K and V of the item's (sample, head)

  typename S::QFrag qf[R];
  f32x4 acc[R][S::kDB];
  float m_run[R], l_part[R];

  __device__ void resources(const Item &it) {
    const int64_t slice = seq * HD;
    rk = make_rsrc(k + it.sh * slice, (uint32_t)(slice * sizeof(T)));
    rv = make_rsrc(v + it.sh * slice, (uint32_t)(slice * sizeof(T)));
  }
  __device__ void operands(const Item &it) {
    const int64_t row0 = it.sh * seq + (int64_t)it.blk * BLK + q0;
#pragma unroll
    for (int r = 0; r < R; ++r) S::load_row_frag(qf[r], q + (row0 + 16 * r) * HD, g);
  }
  __device__ void begin(const Item &) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int db = 0; db < S::kDB; ++db) acc[r][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      m_run[r] = kMaskedScore;
      l_part[r] = 0.f;
    }
  }
  static constexpr bool kFreeK = true;   // K_j is done once the scores are
  __device__ void copy_k(const Item &it, int j, int piece, int slot) {
    S::copy_tile_buf(lds + slot * S::kTileBytes, rk, (uint32_t)((j * BLK + piece * KC) * S::kRowBytes), wave, lane);
  }
  __device__ void copy_v(const Item &it, int j, int piece, int slot) {
    S::copy_tile_buf(lds + slot * S::kTileBytes, rv, (uint32_t)((j * BLK + piece * KC) * S::kRowBytes), wave, lane);
  }
  // S^T tiles: lane holds keys piece*KC + kb*16 + 4g + rr of query q0 + 16 r.
  f32x4 st[R][S::kKB];
  __device__ void compute_a(const Item &it, int e, int piece, int k_slot, int) {
    compute_a_at(lds + k_slot * S::kTileBytes, nullptr, it, e, piece);
  }
  __device__ __forceinline__ void compute_a_at(const unsigned char *lk, const unsigned char *, const Item &it, int e,
                                               int piece) {
#pragma unroll
    for (int kb = 0; kb < S::kKB; ++kb) {
      f32x4 t[R];
      S::template dot_rows_n<R>(lk, kb * 16 + c, g, qf, t);
#pragma unroll
      for (int r = 0; r < R; ++r) st[r][kb] = t[r];
    }
    if (e == it.end - 1) {   // the diagonal block is the last (largest) entry of row i
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int kb = 0; kb < S::kKB; ++kb)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            if (piece * KC + kb * 16 + 4 * g + rr > q0 + 16 * r) st[r][kb][rr] = kMaskedScore;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float mx = kMaskedScore;
#pragma unroll
      for (int kb = 0; kb < S::kKB; ++kb)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) mx = fmaxf(mx, st[r][kb][rr]);
      mx = group_max4(mx) * sl2;
      if (mx > m_run[r] + kRescaleSlack) {
        const float alpha = fast_exp2(m_run[r] - mx);
        m_run[r] = mx;
        l_part[r] *= alpha;
#pragma unroll
        for (int db = 0; db < S::kDB; ++db) acc[r][db] *= alpha;
      }
#pragma unroll
      for (int kb = 0; kb < S::kKB; ++kb)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float p = fast_exp2(fmaf(st[r][kb][rr], sl2, -m_run[r]));
          st[r][kb][rr] = p;
          l_part[r] += p;
        }
    }
  }
  // The second half of a step: the next piece's V into `wr` (when `more`), then P V from
  // this piece's V at `rd`.  The slots never overlap; saying so (restrict) keeps the
  // transposing reads from waiting for the copy just issued.
  __device__ __forceinline__ void step_b(unsigned char *__restrict__ wr, const unsigned char *__restrict__ rd,
                                         const Item &it, int e, int piece, bool more, int j_next, int h_next) {
    if (more) S::copy_tile_buf(wr, rv, (uint32_t)((j_next * BLK + h_next * KC) * S::kRowBytes), wave, lane);
    compute_b_at(rd, it, e, piece);
  }
  // One step of the four-slot ring: the next piece's K and V into `wk`, `wv` (when `more`),
  // then this piece from `lk`, `lv`; no two of the four tiles overlap.
  __device__ __forceinline__ void step4(unsigned char *__restrict__ wk, unsigned char *__restrict__ wv,
                                        const unsigned char *__restrict__ lk, const unsigned char *__restrict__ lv,
                                        const Item &it, int e, int piece, bool more, int j_next, int h_next) {
    if (more) {
      const uint32_t off = (uint32_t)((j_next * BLK + h_next * KC) * S::kRowBytes);
      S::copy_tile_buf(wk, rk, off, wave, lane);
      S::copy_tile_buf(wv, rv, off, wave, lane);
    }
    compute_a_at(lk, lv, it, e, piece);
    compute_b_at(lv, it, e, piece);
  }
  __device__ __forceinline__ void compute_b_at(const unsigned char *lv, const Item &, int, int) {
#pragma unroll
    for (int part = 0; part < S::kParts; ++part)
      S::template accumulate_part_n<R>(&acc[0][0], lv, &st[0][part * S::kPartTiles], S::kKB, part, c, g);
  }
  __device__ void finish(const Item &it, unsigned char *area) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float l = group_sum4(l_part[r]);
      const float inv = 1.0f / l;
      const int64_t q_row = it.sh * seq + (int64_t)it.blk * BLK + q0 + 16 * r;   // this lane's row
      S::store_rows(o + q_row * HD, acc[r], inv, area + wave * S::kAreaBytes, c, g, lane);
      if (lse != nullptr && g == 0) lse[q_row] = (m_run[r] + __log2f(l)) * 0.69314718055994531f;
    }
  }
};

template <typename T, int BLK, int HD>
// At head_dim <= 64 the kernel is asked to fit five waves per SIMD (<= 96 VGPRs; three
// with two row groups per wave): the three-tile ring lets five or six workgroups share a
// CU's LDS, and registers must not be the tighter limit.
__global__ __launch_bounds__((BLK / (16 * fwd_groups<T, BLK, HD>()) * 64),
                             (HD <= 64 ? (fwd_groups<T, BLK, HD>() == 1 ? 5 : 3) : 2)) void attn_fwd_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, T *__restrict__ o,
    float *__restrict__ lse, WorkLists wl, float sl2) {
  constexpr int R = fwd_groups<T, BLK, HD>();
  using P = FwdPolicy<T, BLK, HD, R>;
  __shared__ __align__(16) unsigned char lds[P::kLdsBytes];
  const WorkItem it = wl.decode(dispatch_position(blockIdx.x, gridDim.x));

  P pol;
  pol.q = q;
  pol.k = k;
  pol.v = v;
  pol.o = o;
  pol.lse = lse;
  pol.seq = (int64_t)wl.n * BLK;
  pol.sl2 = sl2;
  pol.lds = lds;
  pol.tid = threadIdx.x;
  pol.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  pol.lane = threadIdx.x & 63;
  pol.c = threadIdx.x & 15;
  pol.g = (threadIdx.x & 63) >> 4;
  pol.q0 = (threadIdx.x >> 6) * 16 * R + pol.c;
  if constexpr (P::kRing4) {
    run_item_ring4(pol, it);
  } else {
    run_item_ring(pol, it);
  }
}

template <typename T, int BLK, int HD>
gsa_status launch_fwd_instance(const gsa_fwd_args &a, const gsa_mask &m, hipStream_t stream) {
  using S = AttnShape<T, BLK, HD, fwd_groups<T, BLK, HD>()>;
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

#ifdef GSA_WIDE_TU
gsa_status launch_attn_fwd_wide(const gsa_fwd_args &a, const gsa_mask &m, hipStream_t stream) {
  return launch_fwd_instance<bf16_t, 128, 128>(a, m, stream);
}
#else
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
  if (a.dtype == GSA_BF16 && a.block == 128 && a.head_dim == 128) return launch_attn_fwd_wide(a, m, stream);
  return fail(GSA_ERR_UNSUPPORTED, "no forward kernel for dtype %d, block %d, head_dim %d", a.dtype,
              a.block, a.head_dim);
}
#endif

}  // namespace gsa
