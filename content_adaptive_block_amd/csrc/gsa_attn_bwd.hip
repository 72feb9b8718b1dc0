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
//             and D_i stream through LDS by asynchronous global -> LDS copies: at b = 64
//             as 32-row pieces on three stages, each copied two pieces ahead; otherwise
//             as whole blocks on two stages, one ahead.  Q_i^T and dO_i^T come from
//             transposing LDS reads.
//   bwd_dq    one workgroup per (sample, head, query block i), walking the CSR row of i;
//             each wave keeps 16 query rows (32 at b = d = 128) of Q_i and dO_i in
//             registers and accumulates dQ^T while K_j and V_j stream through a ring of
//             three LDS slots (V's slot takes the next V as soon as dS is formed; K^T by
//             transposing reads); at b = d = 128 the blocks stream as 64-row pieces
//             through four slots (this piece's K and V, and the next piece's).
//             It also forms D of its rows from O and dO and writes it for dK/dV, so the
//             full backward runs dQ, then dK/dV, with no separate pass for D.
// dK, dV and dQ leave through LDS in whole rows (AttnShape::store_rows).
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
// At b = d = 128 (the _WIDE options): one 16-key group per wave, whole query blocks, one
// 8-wave workgroup per CU.  Two groups need 128 VGPRs of accumulators alone and spill
// (176-352 bytes per lane) at the two waves per SIMD that 64-row query pieces would allow.
#ifndef GSA_DKDV_GROUPS_WIDE
#define GSA_DKDV_GROUPS_WIDE 1
#endif
#ifndef GSA_DKDV_PIECE_WIDE
#define GSA_DKDV_PIECE_WIDE 128
#endif
// One-group dK/dV (the 128 x 128 instance) applies the diagonal block's mask once per part
// of two query tiles instead of once per tile: a branch ends the compiler's scheduling
// region, and with two tiles per region their four MFMA chains interleave (dK/dV 0.6-1.3%
// faster at 2 x 64 KiB over six interleaved runs).  The two-group instance would spill.
#ifndef GSA_DKDV_MASK_PER_PART
#define GSA_DKDV_MASK_PER_PART 1
#endif
#ifndef GSA_DKDV_WAVES_WIDE
#define GSA_DKDV_WAVES_WIDE 1
#endif
template <typename T, int BLK, int HD>
constexpr int dkdv_groups() {
  if (std::is_same<T, bf16_t>::value && HD <= 64 && BLK % 32 == 0) return GSA_DKDV_GROUPS;
  if (std::is_same<T, bf16_t>::value && HD == 128 && BLK == 128) return GSA_DKDV_GROUPS_WIDE;
  return 1;
}

// Query rows per streamed piece of dK/dV (GSA_DKDV_PIECE at b = 64, d = 64, bf16).  With
// 32-row pieces a workgroup's two stages take 16.5 KiB instead of 33, and the kernel is
// asked for three waves per SIMD (<= 168 VGPRs), so six 2-wave workgroups share a CU
// instead of four: 3-5% faster at 8 x 8 KiB; the same pieces at two waves per SIMD were
// 3% slower than whole blocks.
#ifndef GSA_DKDV_PIECE
#define GSA_DKDV_PIECE 32
#endif
// LDS stages of dK/dV at b = 64 (32-row query pieces): three let every copy run two
// pieces ahead of its use at the same six workgroups per CU (24.75 KiB each); dK/dV
// 167.2-170.3 vs 169.1-171.7 us at 8 x 8 KiB over three interleaved runs.
#ifndef GSA_DKDV_STAGES
#define GSA_DKDV_STAGES 3
#endif
template <typename T, int BLK, int HD>
constexpr int dkdv_piece_rows() {
  if (std::is_same<T, bf16_t>::value && BLK == 64 && HD == 64) return GSA_DKDV_PIECE;
  if (std::is_same<T, bf16_t>::value && BLK == 128 && HD == 128) return GSA_DKDV_PIECE_WIDE;
  return BLK;
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
  // LDS stages: three (copies two pieces ahead) where pieces are small, else two.
  static constexpr int kStages = kSub == 2 ? GSA_DKDV_STAGES : 2;
  // Vector memory instructions per piece and wave: the Q and dO tiles, LSE and D (every
  // wave has lanes below kVecLanes, so every wave issues both vector copies).
  static constexpr int kCopyOps = 2 * S::kTileCopies + 2;
  static_assert(kVecLanes >= 1, "every wave copies part of LSE and D");

  const T *q, *k, *v, *dout;
  const float *lse, *dvec;
  T *dk, *dv;
  int64_t seq;
  float sl2, scale;
  unsigned char *lds;
  int tid, c, g, key0;   // key0: this lane's key of group 0 inside block j
  int wave, lane;        // wave: wave-uniform
  rsrc_t rq, rdo, rl, rd;   // Q, dO, LSE, D of the item's (sample, head)

  typename S::QFrag kf[R], vf[R];
  f32x4 dk_acc[R][S::kDB], dv_acc[R][S::kDB];

  __device__ void operands(const Item &it) {
    rq = make_rsrc(q + it.sh * seq * HD, (uint32_t)(seq * S::kRowBytes));
    rdo = make_rsrc(dout + it.sh * seq * HD, (uint32_t)(seq * S::kRowBytes));
    rl = make_rsrc(lse + it.sh * seq, (uint32_t)(seq * 4));
    rd = make_rsrc(dvec + it.sh * seq, (uint32_t)(seq * 4));
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
    copy_to(lds + stage * kStageBytes, it, i, piece);
  }
  __device__ __forceinline__ void copy_to(unsigned char *dst, const Item &, int i, int piece) {
    const int r0 = i * BLK + piece * KQ;   // first row of the piece in the (sample, head) slice
    S::copy_tile_buf(dst, rq, (uint32_t)(r0 * S::kRowBytes), wave, lane);
    S::copy_tile_buf(dst + S::kTileBytes, rdo, (uint32_t)(r0 * S::kRowBytes), wave, lane);
    if (lane < kVecLanes) {
      const uint32_t x4 = (uint32_t)((wave * kVecLanes + lane) * 4);
      buf_copy4_to_lds(rl, x4, (uint32_t)(r0 * 4), dst + 2 * S::kTileBytes + wave * kVecLanes * 4);
      buf_copy4_to_lds(rd, x4, (uint32_t)(r0 * 4), dst + 2 * S::kTileBytes + KQ * 4 + wave * kVecLanes * 4);
    }
  }
  // One step of the three-stage pipeline: copy piece `piece` of query block j_next into the
  // stage at `wr` (when do_copy) and compute piece `piece` of entry e from the stage at
  // `rd`.  The two stages never overlap; saying so (restrict) lets the compiler keep the
  // step's LDS reads from waiting for the copies just issued.
  __device__ __forceinline__ void step(unsigned char *__restrict__ wr, const unsigned char *__restrict__ rd,
                                       const Item &it, int e, int piece, bool do_copy, int j_next) {
    if (do_copy) copy_to(wr, it, j_next, piece);
    compute_at(rd, it, e, piece);
  }
  // The same for the two-stage pipeline, whose copy is of another piece (`copy_piece` of
  // block `j_copy`).
  __device__ __forceinline__ void step_to(unsigned char *__restrict__ wr, const unsigned char *__restrict__ rd,
                                          const Item &it, int e, int piece, bool do_copy, int j_copy,
                                          int copy_piece) {
    if (do_copy) copy_to(wr, it, j_copy, copy_piece);
    compute_at(rd, it, e, piece);
  }
  __device__ __forceinline__ void compute_at(const unsigned char *lq, const Item &it, int e, int piece) {
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
        if (!(GSA_DKDV_MASK_PER_PART && R == 1) && diag) {   // token-causal mask, diagonal block only
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
      if (GSA_DKDV_MASK_PER_PART && R == 1 && diag) {   // the same, once per part
#pragma unroll
        for (int t = 0; t < S::kPartTiles; ++t)
#pragma unroll
          for (int kg = 0; kg < R; ++kg)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (key0 + 16 * kg > piece * KQ + (part * S::kPartTiles + t) * 16 + 4 * g + r) {
                p[kg][t][r] = 0.f;
                ds[kg][t][r] = 0.f;
              }
      }
      S::template accumulate_part_n<R>(&dv_acc[0][0], ldo, &p[0][0], S::kPartTiles, part, c, g);
      S::template accumulate_part_n<R>(&dk_acc[0][0], lq, &ds[0][0], S::kPartTiles, part, c, g);
    }
  }
  __device__ void finish(const Item &it, unsigned char *area) {
    static_assert(S::kWaves * S::kAreaBytes <= kStageBytes, "output staging fits a free stage");
    unsigned char *own = area + wave * S::kAreaBytes;
#pragma unroll
    for (int kg = 0; kg < R; ++kg) {
      const int64_t key_row = it.sh * seq + (int64_t)it.blk * BLK + key0 + 16 * kg;   // this lane's key
      S::store_rows(dk + key_row * HD, dk_acc[kg], -scale, own, c, g, lane);   // the sum holds -dK / scale
      S::store_rows(dv + key_row * HD, dv_acc[kg], 1.0f, own, c, g, lane);
    }
  }
};

template <typename T, int BLK, int HD>
__global__ __launch_bounds__((BLK / (16 * dkdv_groups<T, BLK, HD>()) * 64),
                             (HD == 128 ? GSA_DKDV_WAVES_WIDE : (dkdv_piece_rows<T, BLK, HD>() < BLK ? 3 : 1))) void bwd_dkdv_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, const T *__restrict__ dout,
    const float *__restrict__ lse, const float *__restrict__ dvec, T *__restrict__ dk, T *__restrict__ dv,
    WorkLists wl, float sl2, float scale) {
  constexpr int R = dkdv_groups<T, BLK, HD>();
  using P = DkdvPolicy<T, BLK, HD, R>;
  __shared__ __align__(16) unsigned char lds[P::kStages * P::kStageBytes];
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
  pol.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  pol.lane = threadIdx.x & 63;
  pol.c = threadIdx.x & 15;
  pol.g = (threadIdx.x & 63) >> 4;
  pol.key0 = (threadIdx.x >> 6) * 16 * R + pol.c;
  if constexpr (P::kStages == 3) {
    run_item3(pol, it);
  } else {
    run_item(pol, it);
  }
}

// 16-row query groups per wave in dQ.  At b = d = 128 eight one-group waves read 768 KiB
// of LDS per kept tile (K twice, V once), over 100 bytes per clock per CU; with two groups
// every K and V read feeds two products (4 waves, 235 VGPRs, two waves per SIMD):
// 3.19-3.20 vs 3.40-3.42 ms at 2 x 64 KiB.  At b = d = 64 two groups measured no faster.
#ifndef GSA_DQ_GROUPS_WIDE
#define GSA_DQ_GROUPS_WIDE 2
#endif
// Four LDS slots at b = 128 (as for the forward): 2.94-2.96 vs 3.02-3.04 ms at 2 x 64 KiB.
// At b = 64 (GSA_DQ_RING4) they leave room for five workgroups per CU instead of six:
// 141.5-141.8 vs 139.3-139.7 us at 8 x 8 KiB.
#ifndef GSA_DQ_RING4_WIDE
#define GSA_DQ_RING4_WIDE 1
#endif
#ifndef GSA_DQ_RING4
#define GSA_DQ_RING4 0
#endif
template <typename T, int BLK, int HD>
constexpr int dq_groups() {
  return std::is_same<T, bf16_t>::value && BLK == 128 && HD == 128 ? GSA_DQ_GROUPS_WIDE : 1;
}

// dQ of one (sample, head, query block i): walk the kv-blocks j of row i.  The item's
// D = rowsum(dO * O) is formed from the rows it loads anyway and written out for dK/dV.
// Each wave owns R groups of 16 query rows.
template <typename T, int BLK, int HD, int R>
struct DqPolicy {
  static constexpr int KC = kv_piece_rows<T, BLK, HD>();
  using S = AttnShape<T, BLK, HD, R, KC>;
  using Item = WorkItem;
  static constexpr int kSub = BLK / KC;                  // pieces per kv-block
  static constexpr bool kRing4 = BLK == 128 ? GSA_DQ_RING4_WIDE : GSA_DQ_RING4;
  // The ring: K, V and a spare (or K and V of this piece and of the next).
  static constexpr int kLdsBytes = (kRing4 ? 4 : 3) * S::kTileBytes;
  static_assert(S::kWaves * S::kAreaBytes <= (kRing4 ? 2 : 1) * S::kTileBytes, "output staging fits the free slots");

  const T *q, *k, *v, *o, *dout;
  const float *lse;
  float *dvec;
  T *dq;
  int64_t seq;
  float sl2, scale;
  unsigned char *lds;
  int tid, c, g, q_in_blk;   // q_in_blk: this lane's query of group 0; group r: + 16 r
  int wave, lane;            // wave: wave-uniform
  rsrc_t rk, rv;             // K and V of the item's (sample, head)

  typename S::QFrag qf[R], dof[R];
  float lse2[R], dd[R];
  f32x4 acc[R][S::kDB];

  __device__ void resources(const Item &it) {
    rk = make_rsrc(k + it.sh * seq * HD, (uint32_t)(seq * S::kRowBytes));
    rv = make_rsrc(v + it.sh * seq * HD, (uint32_t)(seq * S::kRowBytes));
  }
  __device__ void operands(const Item &it) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t q_row = it.sh * seq + (int64_t)it.blk * BLK + q_in_blk + 16 * r;
      typename S::QFrag of;
      S::load_row_frag(qf[r], q + q_row * HD, g);
      S::load_row_frag(dof[r], dout + q_row * HD, g);
      S::load_row_frag(of, o + q_row * HD, g);
      lse2[r] = lse[q_row] * kLog2e;
      // D over this lane's feature slots, then across the four lane groups of the row.
      float part = 0.f;
#pragma unroll
      for (int ks = 0; ks < S::kKS; ++ks) {
        if constexpr (S::kBf16) {
#pragma unroll
          for (int x = 0; x < 8; ++x) part = fmaf(to_f32(dof[r].f[ks][x]), to_f32(of.f[ks][x]), part);
        } else {
          part = fmaf(dof[r].f[ks], of.f[ks], part);
        }
      }
      dd[r] = group_sum4(part);
      if (g == 0) dvec[q_row] = dd[r];
    }
  }
  __device__ void begin(const Item &) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int db = 0; db < S::kDB; ++db) acc[r][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  static constexpr bool kFreeK = false;   // V_j is done once dS is formed; K_j is read again
  __device__ void copy_k(const Item &it, int j, int piece, int slot) {
    S::copy_tile_buf(lds + slot * S::kTileBytes, rk, (uint32_t)((j * BLK + piece * KC) * S::kRowBytes), wave, lane);
  }
  __device__ void copy_v(const Item &it, int j, int piece, int slot) {
    S::copy_tile_buf(lds + slot * S::kTileBytes, rv, (uint32_t)((j * BLK + piece * KC) * S::kRowBytes), wave, lane);
  }
  // dS^T[key][q] of every key of the piece (lane holds keys piece*KC + kb*16 + 4g + r of its
  // query of group rg): S^T from K and dP^T - D from V.
  f32x4 dsr[R][S::kKB];
  __device__ void compute_a(const Item &it, int e, int piece, int k_slot, int v_slot) {
    compute_a_at(lds + k_slot * S::kTileBytes, lds + v_slot * S::kTileBytes, it, e, piece);
  }
  __device__ __forceinline__ void compute_a_at(const unsigned char *lk, const unsigned char *lv, const Item &it, int e,
                                               int piece) {
    const bool diag = e == it.end - 1;   // row i ends with its own block j = i
    if constexpr (R == 1) {
#pragma unroll
      for (int kb = 0; kb < S::kKB; ++kb) {
        const f32x4 st = S::dot_rows(lk, kb * 16 + c, g, qf[0]);
        const f32x4 dpd = S::dot_rows(lv, kb * 16 + c, g, dof[0], f32x4{-dd[0], -dd[0], -dd[0], -dd[0]});   // dP - D
#pragma unroll
        for (int r = 0; r < 4; ++r) dsr[0][kb][r] = fast_exp2(fmaf(st[r], sl2, -lse2[0])) * dpd[r];
        if (diag) {   // token-causal mask, diagonal block only
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (piece * KC + kb * 16 + 4 * g + r > q_in_blk) dsr[0][kb][r] = 0.f;
        }
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < S::kKB; ++kb) {
        f32x4 st[R], dp[R];
        S::template dot_rows_n<R>(lk, kb * 16 + c, g, qf, st);
        S::template dot_rows_n<R>(lv, kb * 16 + c, g, dof, dp);
#pragma unroll
        for (int rg = 0; rg < R; ++rg) {
#pragma unroll
          for (int r = 0; r < 4; ++r) dsr[rg][kb][r] = fast_exp2(fmaf(st[rg][r], sl2, -lse2[rg])) * (dp[rg][r] - dd[rg]);
          if (diag) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (piece * KC + kb * 16 + 4 * g + r > q_in_blk + 16 * rg) dsr[rg][kb][r] = 0.f;
          }
        }
      }
    }
  }
  // dQ^T += K^T dS^T over the piece, one part of 16*kPartTiles keys at a time.
  // The second half of a step: the next piece's V into `wr` (when `more`), then dQ from
  // this piece's K at `rd`; the slots never overlap (restrict: the transposing reads of K
  // need not wait for the copy just issued).
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
    compute_b_at(lk, it, e, piece);
  }
  __device__ __forceinline__ void compute_b_at(const unsigned char *lk, const Item &, int, int) {
#pragma unroll
    for (int part = 0; part < S::kParts; ++part)
      S::template accumulate_part_n<R>(&acc[0][0], lk, &dsr[0][part * S::kPartTiles], S::kKB, part, c, g);
  }
  __device__ void finish(const Item &it, unsigned char *area) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t q_row = it.sh * seq + (int64_t)it.blk * BLK + q_in_blk + 16 * r;   // this lane's row
      S::store_rows(dq + q_row * HD, acc[r], scale, area + wave * S::kAreaBytes, c, g, lane);
    }
  }
};

template <typename T, int BLK, int HD>
__global__ __launch_bounds__(BLK / (16 * dq_groups<T, BLK, HD>()) * 64, HD <= 64 ? 1 : 2) void bwd_dq_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, const T *__restrict__ o,
    const T *__restrict__ dout, const float *__restrict__ lse, float *__restrict__ dvec, T *__restrict__ dq,
    WorkLists wl, float sl2, float scale) {
  constexpr int R = dq_groups<T, BLK, HD>();
  using P = DqPolicy<T, BLK, HD, R>;
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
  pol.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  pol.lane = threadIdx.x & 63;
  pol.c = threadIdx.x & 15;
  pol.g = (threadIdx.x & 63) >> 4;
  pol.q_in_blk = (threadIdx.x >> 6) * 16 * R + pol.c;
  if constexpr (P::kRing4) {
    run_item_ring4(pol, it);
  } else {
    run_item_ring(pol, it);
  }
}

template <typename T, int BLK, int HD>
gsa_status launch_dq_instance(const gsa_bwd_args &a, const gsa_mask &m, hipStream_t stream) {
  using S = AttnShape<T, BLK, HD, dq_groups<T, BLK, HD>()>;
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
