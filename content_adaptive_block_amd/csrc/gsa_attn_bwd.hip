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
//             registers and accumulates dK^T, dV^T tiles in fp32 while Q_i, dO_i, LSE_i
//             and D_i stream through two LDS stages by asynchronous global -> LDS copies
//             one block ahead; Q_i^T and dO_i^T come from transposing LDS reads.
//   bwd_dq    one workgroup per (sample, head, query block i), walking the CSR row of i;
//             each wave keeps 16 query rows of Q_i and dO_i in registers and accumulates
//             dQ^T while K_j and V_j stream the same way (K_j^T by transposing reads).
// Short lists run in packets of neighbouring blocks (see packet_of).
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

// Packet size: neighbouring blocks share one workgroup when tiles are small.
template <typename T, int BLK, int HD>
constexpr int bwd_group() {
  return AttnShape<T, BLK, HD>::kTileBytes <= 8 * 1024 ? kGroup : 1;
}

// dK, dV of one (sample, head, kv-block j): walk the query blocks i of column j.
template <typename T, int BLK, int HD>
struct DkdvPolicy {
  using S = AttnShape<T, BLK, HD>;
  using Item = WorkItem;
  // A stage holds Q_i, dO_i, then LSE_i and D_i (BLK floats each).
  static constexpr int kStageBytes = 2 * S::kTileBytes + 2 * BLK * 4;
  static constexpr int kStores = 2 * S::kDB;
  // Each wave copies 16 of the BLK floats of LSE_i and of D_i (4-byte copies, 16 lanes).
  static_assert(BLK == 16 * S::kWaves, "vector slice per wave");
  // At d = 128 a wave's 256 registers cannot also hold the next item's K/V rows; those
  // instances run one item per workgroup and load them directly.
  static constexpr bool kAhead = HD <= 64;
  struct NoFrag {};
  using NextFrag = typename std::conditional<kAhead, typename S::QFrag, NoFrag>::type;

  WorkLists wl;
  const T *q, *k, *v, *dout;
  const float *lse, *dvec;
  T *dk, *dv;
  int64_t seq;
  float sl2, scale;
  unsigned char *lds;
  int tid, c, g, key_in_blk;

  typename S::QFrag kf, vf;
  NextFrag kn, vn;
  f32x4 dk_acc[S::kDB], dv_acc[S::kDB];

  __device__ Item decode(int64_t pos) const { return wl.decode(pos); }
  __device__ void operands(const Item &it) {
    const int64_t key_row = it.sh * seq + (int64_t)it.blk * BLK + key_in_blk;
    if constexpr (kAhead) {
      S::load_row_frag(kn, k + key_row * HD, g);
      S::load_row_frag(vn, v + key_row * HD, g);
    } else {
      S::load_row_frag(kf, k + key_row * HD, g);
      S::load_row_frag(vf, v + key_row * HD, g);
    }
  }
  __device__ void begin(const Item &) {
    if constexpr (kAhead) {
      kf = kn;
      vf = vn;
    }
#pragma unroll
    for (int db = 0; db < S::kDB; ++db) {
      dk_acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
      dv_acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  __device__ void copy(const Item &it, int i, int stage) {
    const int64_t row0 = it.sh * seq + (int64_t)i * BLK;
    unsigned char *dst = lds + stage * kStageBytes;
    S::copy_tile(dst, q + row0 * HD, tid);
    S::copy_tile(dst + S::kTileBytes, dout + row0 * HD, tid);
    const int wave = tid >> 6, lane = tid & 63;
    if (lane < 16) {
      const int x = wave * 16 + lane;
      copy4_to_lds(lse + row0 + x, dst + 2 * S::kTileBytes + wave * 64);
      copy4_to_lds(dvec + row0 + x, dst + 2 * S::kTileBytes + BLK * 4 + wave * 64);
    }
  }
  __device__ void compute(const Item &it, int e, int stage) {
    const unsigned char *lq = lds + stage * kStageBytes;
    const unsigned char *ldo = lq + S::kTileBytes;
    const float *ll = reinterpret_cast<const float *>(lq + 2 * S::kTileBytes);
    const float *ld = ll + BLK;
    const bool diag = e == it.beg;   // column j starts with its own block i = j
    // P[q][key] and dS[q][key], one part of 16*kPartTiles queries at a time;
    // lane: key c, queries qb*16 + 4g + r.
#pragma unroll
    for (int part = 0; part < S::kParts; ++part) {
      f32x4 p[S::kPartTiles], ds[S::kPartTiles];
#pragma unroll
      for (int t = 0; t < S::kPartTiles; ++t) {
        const int qb = part * S::kPartTiles + t;
        const f32x4 st = S::dot_rows(lq, qb * 16 + c, g, kf);
        const f32x4 dp = S::dot_rows(ldo, qb * 16 + c, g, vf);
        const f32x4 l4 = *reinterpret_cast<const f32x4 *>(ll + qb * 16 + 4 * g);
        const f32x4 d4 = *reinterpret_cast<const f32x4 *>(ld + qb * 16 + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float pr = fast_exp2(fmaf(st[r], sl2, -l4[r] * kLog2e));
          if (diag && key_in_blk > qb * 16 + 4 * g + r) pr = 0.f;
          p[t][r] = pr;
          ds[t][r] = pr * (dp[r] - d4[r]);
        }
      }
      S::accumulate_part(dv_acc, ldo, p, part, c, g);
      S::accumulate_part(dk_acc, lq, ds, part, c, g);
    }
  }
  __device__ void finish(const Item &it) {
    // Lane holds features db*16 + 4g + r of its key: four consecutive features.
    const int64_t key_row = it.sh * seq + (int64_t)it.blk * BLK + key_in_blk;
    T *dkr = dk + key_row * HD;
    T *dvr = dv + key_row * HD;
#pragma unroll
    for (int db = 0; db < S::kDB; ++db) {
      S::store4(dkr + db * 16 + 4 * g, dk_acc[db] * scale);
      S::store4(dvr + db * 16 + 4 * g, dv_acc[db]);
    }
  }
};

template <typename T, int BLK, int HD>
__global__ __launch_bounds__(BLK / 16 * 64) void bwd_dkdv_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, const T *__restrict__ dout,
    const float *__restrict__ lse, const float *__restrict__ dvec, T *__restrict__ dk, T *__restrict__ dv,
    WorkLists wl, const int32_t *__restrict__ n_long_ptr, int64_t items, float sl2, float scale) {
  using P = DkdvPolicy<T, BLK, HD>;
  constexpr int G = bwd_group<T, BLK, HD>();
  __shared__ __align__(16) unsigned char lds[2 * P::kStageBytes];
  int64_t first;
  int count;
  packet_of(blockIdx.x, items, G > 1 ? *n_long_ptr : items, G, &first, &count);
  if (count == 0) return;

  P pol;
  pol.wl = wl;
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
  pol.key_in_blk = (threadIdx.x >> 6) * 16 + pol.c;
  run_packet<G>(pol, first, count);
}

// dQ of one (sample, head, query block i): walk the kv-blocks j of row i.
template <typename T, int BLK, int HD>
struct DqPolicy {
  using S = AttnShape<T, BLK, HD>;
  using Item = WorkItem;
  static constexpr int kStageBytes = 2 * S::kTileBytes;
  static constexpr int kStores = S::kDB;

  WorkLists wl;
  const T *q, *k, *v, *dout;
  const float *lse, *dvec;
  T *dq;
  int64_t seq;
  float sl2, scale;
  unsigned char *lds;
  int tid, c, g, q_in_blk;

  typename S::QFrag qf, dof, qn, don;
  float lse2, dd, lsen, ddn;
  f32x4 acc[S::kDB];

  __device__ Item decode(int64_t pos) const { return wl.decode(pos); }
  __device__ void operands(const Item &it) {
    const int64_t q_row = it.sh * seq + (int64_t)it.blk * BLK + q_in_blk;
    S::load_row_frag(qn, q + q_row * HD, g);
    S::load_row_frag(don, dout + q_row * HD, g);
    lsen = lse[q_row];
    ddn = dvec[q_row];
  }
  __device__ void begin(const Item &) {
    qf = qn;
    dof = don;
    lse2 = lsen * kLog2e;
    dd = ddn;
#pragma unroll
    for (int db = 0; db < S::kDB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
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
    const bool diag = e == it.end - 1;   // row i ends with its own block j = i
    // dS^T[key][q], one part of 16*kPartTiles keys at a time: lane holds keys
    // kb*16 + 4g + r of its query.
#pragma unroll
    for (int part = 0; part < S::kParts; ++part) {
      f32x4 ds[S::kPartTiles];
#pragma unroll
      for (int t = 0; t < S::kPartTiles; ++t) {
        const int kb = part * S::kPartTiles + t;
        const f32x4 st = S::dot_rows(lk, kb * 16 + c, g, qf);
        const f32x4 dp = S::dot_rows(lv, kb * 16 + c, g, dof);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float pr = fast_exp2(fmaf(st[r], sl2, -lse2));
          if (diag && kb * 16 + 4 * g + r > q_in_blk) pr = 0.f;
          ds[t][r] = pr * (dp[r] - dd);
        }
      }
      S::accumulate_part(acc, lk, ds, part, c, g);
    }
  }
  __device__ void finish(const Item &it) {
    const int64_t q_row = it.sh * seq + (int64_t)it.blk * BLK + q_in_blk;
    T *dqr = dq + q_row * HD;
#pragma unroll
    for (int db = 0; db < S::kDB; ++db) S::store4(dqr + db * 16 + 4 * g, acc[db] * scale);
  }
};

template <typename T, int BLK, int HD>
__global__ __launch_bounds__(BLK / 16 * 64) void bwd_dq_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, const T *__restrict__ dout,
    const float *__restrict__ lse, const float *__restrict__ dvec, T *__restrict__ dq, WorkLists wl,
    const int32_t *__restrict__ n_long_ptr, int64_t items, float sl2, float scale) {
  using P = DqPolicy<T, BLK, HD>;
  constexpr int G = bwd_group<T, BLK, HD>();
  __shared__ __align__(16) unsigned char lds[2 * P::kStageBytes];
  int64_t first;
  int count;
  packet_of(blockIdx.x, items, G > 1 ? *n_long_ptr : items, G, &first, &count);
  if (count == 0) return;

  P pol;
  pol.wl = wl;
  pol.q = q;
  pol.k = k;
  pol.v = v;
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
  run_packet<G>(pol, first, count);
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
  const int32_t *n_long = m.sched + sched_words(m.batch, m.n_blocks);   // [0] rows, [1] columns

  constexpr int kLanes = HD / (16 / sizeof(T));
  if (stages & kBwdPrep) {
    const int64_t pre_threads = rows * kLanes;
    hipLaunchKernelGGL((bwd_pre_kernel<T, HD>), dim3((unsigned)((pre_threads + 255) / 256)), dim3(256), 0,
                       stream, o, dout, a.workspace, rows);
    gsa_status st = check_launch("bwd_pre_kernel");
    if (st != GSA_OK) return st;
  }
  if (stages & kBwdDkdv) {
    const WorkLists wl{m.work_col, m.col_ptr, m.row_idx, f.heads, m.n_blocks, m.n_heads[0], m.n_heads[1],
                       mask_cap(m.n_blocks)};
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, BLK, HD>), dim3((unsigned)items), dim3(S::kThreads), 0, stream, q, k,
                       v, dout, f.lse, a.workspace, static_cast<T *>(a.dk), static_cast<T *>(a.dv), wl, n_long + 1,
                       items, sl2, scale);
    gsa_status st = check_launch("bwd_dkdv_kernel");
    if (st != GSA_OK) return st;
  }
  if (stages & kBwdDq) {
    const WorkLists wl{m.work_row, m.row_ptr, m.col_idx, f.heads, m.n_blocks, m.n_heads[0], m.n_heads[1],
                       mask_cap(m.n_blocks)};
    hipLaunchKernelGGL((bwd_dq_kernel<T, BLK, HD>), dim3((unsigned)items), dim3(S::kThreads), 0, stream, q, k, v,
                       dout, f.lse, a.workspace, static_cast<T *>(a.dq), wl, n_long, items, sl2, scale);
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
