// Tile primitives shared by the attention kernels (forward, dK/dV, dQ).
//
// A "tile" is one mask block of one head: BLK token rows of HD features, contiguous in
// memory ([B, H, T, d] layout), i.e. a dense BLK x HD row-major matrix.  Each wave owns
// 16 rows (one group; 32 with two groups) of its workgroup's own block, kept in
// registers; the other side's tiles are staged row-major in LDS and read two ways:
//   dot_rows:        C[m][n] = sum_f LDS[m][f] * F[n][f]    (A = 16 staged rows, b128
//                    reads; B = the wave's register fragment F) -> a C tile whose rows m
//                    are staged tokens (4 per lane) and whose column n is one of the
//                    wave's rows
//   accumulate_part: Acc[f][n] += sum_m LDS[m][f] * C[m][n] (A = the staged tile
//                    transposed, read with ds_read_b64_tr_b16; B = C tiles from dot_rows
//                    fed back)
// The second product takes a lane's four C rows of two adjacent 16-row tiles as its eight
// K-slots; the transposed read delivers the other operand in the same token order.
//
// LDS tiles are unpadded; each 16-byte chunk of a row is stored at chunk ^ swz(row).
// Tiles arrive by asynchronous global -> LDS copies (no register staging).  The
// swizzle keeps both read forms free of bank conflicts (measured on gfx950: 128-byte rows
// use (row >> 1) & 7, 256-byte rows ((row & 7) << 1) | ((row >> 3) & 1)).
//
// The item pipelines below (run_item, run_item3, run_item_ring, run_item_ring4) drive a
// kernel's policy through its list, and store_rows writes a wave's outputs through LDS
// in whole rows.
//
// Lane layout of ds_read_b64_tr_b16 (measured on gfx950): within each group of 16 lanes,
// lane i receives element i % 4 of the 8 bytes addressed by lane 4e + i / 4, for
// e = 0..3.  Pointing lane j at row key0 + j / 4, columns f0 + 4 (j % 4) .. + 3 therefore
// gives lane i the four values T[key0 + e][f0 + i].
#pragma once

#include <type_traits>

#include "gsa_device.hpp"
#include "gsa_internal.hpp"

namespace gsa {

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int head_class(int h, int n_loc, int n_lit) {
  return h < n_loc ? 0 : (h < n_loc + n_lit ? 1 : 2);
}

// One work item: list `list[beg, end)` of block `blk` of head `sh` = s * H + h; `first`
// is list[beg].
struct WorkItem {
  int64_t sh;
  int blk, beg, end, first;
  const int32_t *list;
};

// Where work items live: the work descriptors (item index (s*H + h)*N + blk, beg, end,
// first entry) in schedule order, and the per-(sample, class) lists (CSR rows or CSC
// columns).  One 16-byte load describes an item, so the first tile copy waits on a single
// memory access.
struct WorkLists {
  const int32_t *work, *idx;
  int heads, n, n_loc, n_lit;
  int64_t cap;
  __device__ __forceinline__ WorkItem decode(int64_t pos) const {
    const u32x4 d = load_uniform(reinterpret_cast<const u32x4 *>(work) + pos);
    WorkItem it;
    const uint32_t item = d[0];
    it.blk = (int)(item % (uint32_t)n);
    const uint32_t sh = item / (uint32_t)n;
    it.sh = sh;
    const int h = (int)(sh % (uint32_t)heads);
    const int64_t s = sh / (uint32_t)heads;
    it.list = idx + (s * 3 + head_class(h, n_loc, n_lit)) * cap;
    it.beg = (int)d[1];
    it.end = (int)d[2];
    it.first = (int)d[3];
    return it;
  }
};

// Work position of workgroup b of a grid of `total`.  Workgroups are handed to the eight
// XCDs round-robin (b % 8) and each XCD has its own L2; with a chunk C > 0, every window
// of 8C consecutive work positions is split into eight runs of C, one per XCD, so that
// neighbouring items (which share kv-blocks) meet in one L2 while the window order keeps
// the longest-first schedule.  The tail past the last whole window keeps its order.
// Runs of 8 measured 1.4% (8 x 8 KiB) and 1.8% (2 x 64 KiB) faster per step than runs
// of 16, 4 no better than 8, and 32 or no remapping slower.
#ifndef GSA_XCD_CHUNK
#define GSA_XCD_CHUNK 8
#endif
__device__ __forceinline__ uint32_t dispatch_position(uint32_t b, uint32_t total) {
  constexpr uint32_t kX = 8, kC = GSA_XCD_CHUNK;
  if constexpr (kC == 0) {
    return b;
  } else {
    constexpr uint32_t kW = kX * kC;
    if (b >= total / kW * kW) return b;
    const uint32_t r = b % kW;
    return b - r + (r % kX) * kC + r / kX;
  }
}

// Rows of the K and V pieces that the forward and dQ kernels stream through their LDS
// ring.  A 128-row block of 128 bf16 features is a 32 KiB tile; streamed as two 64-row
// pieces, the three ring slots take 48 KiB, so two workgroups share a CU instead of one.
#ifndef GSA_PIECE_ROWS_128
#define GSA_PIECE_ROWS_128 64
#endif
template <typename T, int BLK, int HD>
constexpr int kv_piece_rows() {
  return std::is_same<T, bf16_t>::value && BLK == 128 && HD == 128 ? GSA_PIECE_ROWS_128 : BLK;
}

// Outputs (O, dQ, dK, dV) leave through LDS in whole rows (AttnShape::store_rows): at
// 8 x 8 KiB the step took 0.394-0.396 vs 0.425-0.428 ms (forward 98 vs 106 us, dQ 140 vs
// 146, dK/dV 148 vs 166); at 2 x 64 KiB neutral to 2% faster.
#ifndef GSA_STORE_VIA_LDS
#define GSA_STORE_VIA_LDS 1
#endif

// R = 16-row groups owned by each wave (1 or 2); the workgroup has BLK / (16 R) waves.
// KC = rows of a staged tile: the whole block (BLK), or a part of it when the other side
// streams each block in KC-row pieces.
template <typename T, int BLK, int HD, int R = 1, int KC = BLK>
struct AttnShape {
  static constexpr bool kBf16 = std::is_same<T, bf16_t>::value;
  static_assert(kBf16 || std::is_same<T, float>::value, "bf16 or fp32 only");
  static_assert(BLK % (kBf16 ? 32 : 16) == 0 && HD % (kBf16 ? 32 : 16) == 0, "tile shape");
  static_assert(KC % (kBf16 ? 32 : 16) == 0 && BLK % KC == 0, "staged rows");
  static_assert(R >= 1 && BLK % (16 * R) == 0, "row groups per wave");
  static constexpr int kWaves = BLK / (16 * R);
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kKB = KC / 16;                  // 16-row tiles of a staged tile
  static constexpr int kDB = HD / 16;                  // 16-wide feature tiles
  static constexpr int kKS = kBf16 ? HD / 32 : HD / 4; // MFMA K-steps over the features
  static constexpr int kVec = 16 / sizeof(T);          // elements per 16-byte chunk
  static constexpr int kRowBytes = HD * sizeof(T);
  static constexpr int kChunks = kRowBytes / 16;       // chunks per row
  static_assert(kChunks == 8 || kChunks == 16, "rows of 128 or 256 bytes");
  static constexpr int kTileBytes = KC * kRowBytes;
  static constexpr int kTileChunks = KC * kChunks;
  static_assert(kTileChunks % kThreads == 0, "staging must divide evenly");
  static constexpr int kChunksPerThread = kTileChunks / kThreads;

  using Frag = typename std::conditional<kBf16, bf16x8, float>::type;
  struct QFrag {
    Frag f[kKS];
  };

  __device__ static __forceinline__ int swz(int row) {
    return kChunks == 8 ? ((row >> 1) & 7) : (((row & 7) << 1) | ((row >> 3) & 1));
  }
  // Byte offset of 16-byte chunk `ch` of row `row` inside a staged tile.
  __device__ static __forceinline__ int chunk_off(int row, int ch) {
    return row * kRowBytes + ((ch ^ swz(row)) << 4);
  }

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

  // Asynchronous copy of a KC x HD tile into LDS in the swizzled layout, through a buffer
  // resource `r` over one tensor slice, the tile starting `soff` bytes into it: every copy
  // instruction fills 64 consecutive 16-byte LDS slots, so each lane fetches the chunk
  // whose swizzled home is its slot.  `wave` is wave-uniform (a scalar), so only the
  // loop-invariant lane offsets live in vector registers.  kTileCopies instructions per
  // thread.
  static constexpr int kTileCopies = kChunksPerThread;
  __device__ static __forceinline__ void copy_tile_buf(unsigned char *lds, rsrc_t r, uint32_t soff, int wave,
                                                       int lane) {
#pragma unroll
    for (int it = 0; it < kTileCopies; ++it) {
      const int first = it * kThreads + wave * 64;
      const int slot = it * kThreads + (lane & 63) + wave * 64;
      const int row = slot / kChunks, phys = slot % kChunks;
      buf_copy16_to_lds(r, (uint32_t)((row * kChunks + (phys ^ swz(row))) << 4), soff, lds + (first << 4));
    }
  }

  // C tile: staged rows 16*tile .. +15 (this lane's row = 16*tile + c) x the fragment,
  // added to `init` (the accumulator's starting value).
  __device__ static __forceinline__ f32x4 dot_rows(const unsigned char *lds, int row, int g, const QFrag &qf,
                                                   f32x4 init = f32x4{0.f, 0.f, 0.f, 0.f}) {
    f32x4 acc = init;
    if constexpr (kBf16) {
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(lds + chunk_off(row, 4 * ks + g));
        acc = mfma_bf16(a, qf.f[ks], acc);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        const float a = *reinterpret_cast<const float *>(lds + chunk_off(row, ks) + 4 * g);
        acc = mfma_f32(a, qf.f[ks], acc);
      }
    }
    return acc;
  }

  // N C tiles of the same 16 staged rows against N fragments f[0..N): one LDS read per
  // K-step feeds all N products.
  template <int N>
  __device__ static __forceinline__ void dot_rows_n(const unsigned char *lds, int row, int g, const QFrag *f,
                                                    f32x4 *c, f32x4 init = f32x4{0.f, 0.f, 0.f, 0.f}) {
    if constexpr (N == 1) {
      c[0] = dot_rows(lds, row, g, f[0], init);
    } else {
      static_assert(kBf16, "several fragments per read: bf16 only");
#pragma unroll
      for (int n = 0; n < N; ++n) c[n] = init;
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(lds + chunk_off(row, 4 * ks + g));
#pragma unroll
        for (int n = 0; n < N; ++n) c[n] = mfma_bf16(a, f[n].f[ks], c[n]);
      }
    }
  }

  // The second product runs in parts of kPartTiles 16-token tiles (32 tokens for bf16,
  // one MFMA K-step; 16 for fp32), so callers without a row-wide softmax can produce and
  // consume C one part at a time.
  static constexpr int kPartTiles = kBf16 ? 2 : 1;
  static constexpr int kParts = kKB / kPartTiles;

  // acc[db] += (staged tile)^T[db*16 + c][tokens of part] x C, cm = the part's C tiles.
  __device__ static __forceinline__ void accumulate_part(f32x4 *acc, const unsigned char *lds, const f32x4 *cm,
                                                          int part, int c, int g) {
    if constexpr (kBf16) {
      // Lane j = c of group g addresses rows 32*part + 16h + 4g + j/4, features db*16 + 4(j%4).
      const int row0 = 32 * part + 4 * g + (c >> 2), row1 = row0 + 16;
      const int fq = 4 * (c & 3);
      bf16x8 b;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        b[r] = to_bf16(cm[0][r]);
        b[4 + r] = to_bf16(cm[1][r]);
      }
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const int f = db * 16 + fq;
        const s16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)(lds + chunk_off(row0, f >> 3) + 2 * (f & 7)));
        const s16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)(lds + chunk_off(row1, f >> 3) + 2 * (f & 7)));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[db] = mfma_bf16(a, b, acc[db]);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = part * 16 + 4 * g + r;
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          const int f = db * 16 + c;
          const float a = *reinterpret_cast<const float *>(lds + chunk_off(row, f >> 2) + 4 * (f & 3));
          acc[db] = mfma_f32(a, cm[0][r], acc[db]);
        }
      }
    }
  }

  // accumulate_part for N operands sharing the transposed LDS reads: acc + n * kDB and
  // cm + n * cm_stride are operand n's accumulators and C tiles.
  template <int N>
  __device__ static __forceinline__ void accumulate_part_n(f32x4 *acc, const unsigned char *lds, const f32x4 *cm,
                                                           int cm_stride, int part, int c, int g) {
    if constexpr (N == 1) {
      accumulate_part(acc, lds, cm, part, c, g);
    } else {
      static_assert(kBf16, "several operands per read: bf16 only");
      const int row0 = 32 * part + 4 * g + (c >> 2), row1 = row0 + 16;
      const int fq = 4 * (c & 3);
      bf16x8 b[N];
#pragma unroll
      for (int n = 0; n < N; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          b[n][r] = to_bf16(cm[n * cm_stride][r]);
          b[n][4 + r] = to_bf16(cm[n * cm_stride + 1][r]);
        }
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const int f = db * 16 + fq;
        const s16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)(lds + chunk_off(row0, f >> 3) + 2 * (f & 7)));
        const s16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)(lds + chunk_off(row1, f >> 3) + 2 * (f & 7)));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int n = 0; n < N; ++n) acc[n * kDB + db] = mfma_bf16(a, b[n], acc[n * kDB + db]);
      }
    }
  }

  // Stores the 16 rows of one row group (row c of the group in lane c) whose HD features a
  // wave holds in the C layout (acc[db][r] = feature db*16 + 4g + r), times `mul`; `mine`
  // is this lane's row, and the group's rows are consecutive in memory.  With
  // kStoreViaLds (bf16) the rows pass through the wave's own 16-row area of LDS at `area`,
  // so that each store instruction writes 64 lanes x 16 contiguous bytes instead of
  // sixteen 32-byte pieces of rows.  Only this wave touches `area`, and a wave's LDS
  // accesses complete in order, so no barrier is needed.
  static constexpr bool kStoreViaLds = kBf16 && GSA_STORE_VIA_LDS;
  static constexpr int kAreaBytes = 16 * kRowBytes;   // LDS per wave for store_rows
  __device__ static __forceinline__ void store_rows(T *mine, const f32x4 *acc, float mul, unsigned char *area, int c,
                                                    int g, int lane) {
    if constexpr (!kStoreViaLds) {
#pragma unroll
      for (int db = 0; db < kDB; ++db) store4(mine + db * 16 + 4 * g, acc[db] * mul);
    } else {
      T *dst = mine - c * HD;   // the group's first row
      // Row c's 16-byte chunks sit at chunk ^ (c & 7), which spreads the sixteen rows that one
      // write instruction touches over the banks.
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const f32x4 x = acc[db] * mul;
        const bf16x4 y = {to_bf16(x[0]), to_bf16(x[1]), to_bf16(x[2]), to_bf16(x[3])};
        const int ch = 2 * db + (g >> 1);
        *reinterpret_cast<bf16x4 *>(area + c * kRowBytes + ((ch ^ (c & 7)) << 4) + (g & 1) * 8) = y;
      }
#pragma unroll
      for (int it = 0; it < 16 * kChunks / 64; ++it) {
        const int kx = it * 64 + lane, row = kx / kChunks, ch = kx % kChunks;
        const u32x4 val = *reinterpret_cast<const u32x4 *>(area + row * kRowBytes + ((ch ^ (row & 7)) << 4));
        *reinterpret_cast<u32x4 *>(dst + row * HD + ch * kVec) = val;
      }
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

// ---------------------------------------------------------------------------------------
// Per-item pipeline shared by the attention kernels.  A workgroup runs one work item,
// which walks one list (a CSR row or a CSC column); each list entry's block arrives as
// P::kSub pieces of BLK / kSub rows, each piece in one of two LDS stages by asynchronous
// copies issued one piece ahead.  The policy P supplies kSub, kStageBytes and:
//   operands(item)                   load the item's register operands (before the loop)
//   begin(item)                      clear the accumulators
//   copy(item, block, piece, stage)  issue the copies of one piece into `stage`
//   step_to(write, read, item, e, piece, do_copy, block, copy_piece)
//                                    copy piece `copy_piece` of `block` to the stage at
//                                    `write` (when do_copy), then compute piece `piece` of
//                                    list entry e from the stage at `read`
//   finish(item, area)               write the item's outputs (`area`: LDS free of reads
//                                    and copies, for store_rows)
// A step waits for its own copies, synchronises -- after which every wave has finished
// the previous step, so the other stage is free -- issues the next piece's copies and
// computes.  The two stage pointers are restrict, so that the compiler does not make the
// step's LDS reads wait for the copies just issued.
// ---------------------------------------------------------------------------------------
template <class P>
__device__ __forceinline__ void run_item(P &pol, const WorkItem &it) {
  // Entries after the first come from a lane-indexed register holding 64 of them (one
  // per lane), read with readlane: no step waits on memory for its next kv index.
  const int lane = threadIdx.x & (kWave - 1);
  int chunk = it.beg + 1 + lane < it.end ? it.list[it.beg + 1 + lane] : 0;
  constexpr int kSub = P::kSub;
  pol.operands(it);
  pol.copy(it, it.first, 0, 0);
  pol.begin(it);
  int stage = 0, j = it.first;
  for (int e = it.beg; e < it.end; ++e) {
    const int nx = e + 1 - (it.beg + 1);   // position of entry e + 1 after the first
#pragma unroll
    for (int h = 0; h < kSub; ++h) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      wg_barrier();
      bool do_copy = true;
      int h_copy = h + 1;
      if (h + 1 < kSub) {
      } else if (e + 1 < it.end) {
        if (nx > 0 && (nx & (kWave - 1)) == 0)
          chunk = e + 1 + lane < it.end ? it.list[e + 1 + lane] : 0;
        j = __builtin_amdgcn_readlane(chunk, nx & (kWave - 1));
        h_copy = 0;
      } else {
        do_copy = false;
      }
      pol.step_to(pol.lds + (stage ^ 1) * P::kStageBytes, pol.lds + stage * P::kStageBytes, it, e, h, do_copy, j,
                  h_copy);
      stage ^= 1;
    }
  }
  pol.finish(it, pol.lds + stage * P::kStageBytes);   // no copy went there in the last step
}


// ---------------------------------------------------------------------------------------
// run_item with three LDS stages for items whose entries arrive as two pieces: the copies
// of a piece are issued two pieces ahead (one entry), so each has two steps to land.  A
// step waits only for its own piece (the wave's kCopyOps newer copy instructions may stay
// in flight), synchronises -- after which every wave has finished the previous step, so
// that step's stage is free -- and calls pol.step(write stage, read stage, ...), which
// issues the copies of the same piece of the next entry into the free stage and computes.
// ---------------------------------------------------------------------------------------
template <class P>
__device__ __forceinline__ void run_item3(P &pol, const WorkItem &it) {
  static_assert(P::kSub == 2 && P::kStages == 3, "two pieces per entry, three stages");
  const int lane = threadIdx.x & (kWave - 1);
  int chunk = it.beg + 1 + lane < it.end ? it.list[it.beg + 1 + lane] : 0;
  pol.operands(it);
  pol.copy(it, it.first, 0, 0);
  pol.copy(it, it.first, 1, 1);
  pol.begin(it);
  int stage = 0;
  for (int e = it.beg; e < it.end; ++e) {
    const bool more = e + 1 < it.end;
    int j_next = 0;
    if (more) {
      const int nx = e - it.beg;   // position of entry e + 1 after the first
      if (nx > 0 && (nx & (kWave - 1)) == 0)
        chunk = e + 1 + lane < it.end ? it.list[e + 1 + lane] : 0;
      j_next = __builtin_amdgcn_readlane(chunk, nx & (kWave - 1));
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // In flight before this wait: piece (e, h), then (e, 1) or, at h = 1, (e + 1, 0).
      if (h == 0 || more) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(P::kCopyOps));
      } else {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      }
      wg_barrier();
      const int ws = stage == 0 ? 2 : stage - 1;   // the stage of the previous step
      pol.step(pol.lds + ws * P::kStageBytes, pol.lds + stage * P::kStageBytes, it, e, h, more, j_next);
      stage = stage == 2 ? 0 : stage + 1;
    }
  }
  pol.finish(it, pol.lds + stage * P::kStageBytes);   // neither read nor written in the last step
}

// ---------------------------------------------------------------------------------------
// Three-slot pipeline for items whose two streamed tiles (K_j and V_j) are used one after
// the other: 3 tiles of LDS instead of 4, which lets 6 rather than 4 workgroups share a
// CU (gfx950 fits six 24 KiB workgroups but only four 32 KiB ones).  Each list entry is
// streamed as P::kSub pieces of BLK / kSub rows (one piece unless the tiles are large);
// per piece:
//   wait for K and V, barrier (everyone left the previous piece, so the spare slot is
//   free); copy the next piece's K into the spare slot; compute_a (reads K, and V if it
//   wants); barrier (everyone is done with the slot the policy frees: K when kFreeK, else
//   V); step_b: copy the next piece's V into it and compute the second half.
// The policy supplies operands/begin/finish as for run_item, resources(item) (the buffer
// resources the copies need, set before operands), the constants kSub and kFreeK,
// copy_k(item, j, piece, slot), copy_v(item, j, piece, slot),
// compute_a(item, e, piece, k_slot, v_slot) and step_b(write, read, item, e, piece, more,
// j_next, piece_next), which copies the next piece's V (when `more`) to `write` and computes
// from the tile at `read` (V when kFreeK, else K).  The two pointers are restrict: the
// second half's transposing LDS reads then need not wait for the copy just issued (3-5%
// faster dQ at b = d = 128).
// ---------------------------------------------------------------------------------------
template <class P>
__device__ __forceinline__ void run_item_ring(P &pol, const WorkItem &it) {
  constexpr int kSub = P::kSub;
  const int lane = threadIdx.x & (kWave - 1);
  int chunk = it.beg + 1 + lane < it.end ? it.list[it.beg + 1 + lane] : 0;
  // The first tiles' copies go out before the register operands are loaded (dQ forms D
  // from its rows right away, and would otherwise hold the copies back until they land).
  pol.resources(it);
  int ks = 0, vs = 1, spare = 2;
  pol.copy_k(it, it.first, 0, ks);
  pol.copy_v(it, it.first, 0, vs);
  pol.operands(it);
  pol.begin(it);
  int j = it.first;
  for (int e = it.beg; e < it.end; ++e) {
    const int nx_pos = e - it.beg;   // entry e + 1 sits at this position of the chunk run
#pragma unroll
    for (int h = 0; h < kSub; ++h) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      wg_barrier();
      const bool last_piece = h + 1 == kSub;
      const bool more = !last_piece || e + 1 < it.end;
      int j_next = j;
      if (last_piece && e + 1 < it.end) {
        if (nx_pos > 0 && (nx_pos & (kWave - 1)) == 0)
          chunk = e + 1 + lane < it.end ? it.list[e + 1 + lane] : 0;
        j_next = __builtin_amdgcn_readlane(chunk, nx_pos & (kWave - 1));
      }
      const int h_next = last_piece ? 0 : h + 1;
      if (more) pol.copy_k(it, j_next, h_next, spare);
      pol.compute_a(it, e, h, ks, vs);
      wg_barrier();
      const int freed = P::kFreeK ? ks : vs;
      pol.step_b(pol.lds + freed * P::S::kTileBytes, pol.lds + (P::kFreeK ? vs : ks) * P::S::kTileBytes, it, e, h,
                 more, j_next, h_next);
      // The next piece's K sits in the spare slot and its V in the freed one; the other
      // is spare.
      const int next_spare = P::kFreeK ? vs : ks;
      ks = spare;
      vs = freed;
      spare = next_spare;
      j = j_next;
    }
  }
  pol.finish(it, pol.lds + ks * P::S::kTileBytes);   // the last step's spare slot: untouched
}

// ---------------------------------------------------------------------------------------
// Four-slot pipeline: K and V of the current piece in one pair of slots, the next piece's
// K and V copied into the other pair as the step starts.  One barrier per step (after it,
// every wave has left the previous step, so the other pair is free), and each copy has a
// whole step to land.  The policy supplies operands/begin/finish, kSub, copy_k, copy_v and
// step4(write K, write V, read K, read V, item, e, piece, more, j_next, piece_next).
// ---------------------------------------------------------------------------------------
template <class P>
__device__ __forceinline__ void run_item_ring4(P &pol, const WorkItem &it) {
  constexpr int kSub = P::kSub;
  constexpr int kTile = P::S::kTileBytes;
  const int lane = threadIdx.x & (kWave - 1);
  int chunk = it.beg + 1 + lane < it.end ? it.list[it.beg + 1 + lane] : 0;
  pol.resources(it);   // as in run_item_ring: the first copies go out first
  pol.copy_k(it, it.first, 0, 0);
  pol.copy_v(it, it.first, 0, 1);
  pol.operands(it);
  pol.begin(it);
  int cur = 0, j = it.first;
  for (int e = it.beg; e < it.end; ++e) {
    const int nx_pos = e - it.beg;   // entry e + 1 sits at this position of the chunk run
#pragma unroll
    for (int h = 0; h < kSub; ++h) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      wg_barrier();
      const bool last_piece = h + 1 == kSub;
      const bool more = !last_piece || e + 1 < it.end;
      int j_next = j;
      if (last_piece && e + 1 < it.end) {
        if (nx_pos > 0 && (nx_pos & (kWave - 1)) == 0)
          chunk = e + 1 + lane < it.end ? it.list[e + 1 + lane] : 0;
        j_next = __builtin_amdgcn_readlane(chunk, nx_pos & (kWave - 1));
      }
      const int h_next = last_piece ? 0 : h + 1;
      unsigned char *next = pol.lds + (2 - 2 * cur) * kTile;
      const unsigned char *now = pol.lds + 2 * cur * kTile;
      pol.step4(next, next + kTile, now, now + kTile, it, e, h, more, j_next, h_next);
      cur ^= 1;
      j = j_next;
    }
  }
  pol.finish(it, pol.lds + 2 * cur * kTile);   // the pair no copy went to in the last step
}

}  // namespace gsa
