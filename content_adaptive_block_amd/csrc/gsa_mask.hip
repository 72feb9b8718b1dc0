// Mask construction for gzip-guided sparse attention on gfx950.
//
// Method ("Gzip-guided Sparse Attention", daiwk.github.io reproduction note):
//   核心公式 first display: r_i = |gzip(x_i)| / b and l_i = 1[r_i > mean_j r_j] over the
//   sample's N blocks.  With integer sizes c_i this is exactly N * c_i > sum_j c_j.
//   核心公式 second display: M = M^lit U M^local U I, M^lit_ij = 1[l_i = l_j = 1],
//   M^local_ij = 1[|i - j| <= w], intersected with the causal mask (j <= i).
//   背景与主要改动: heads split into local (M^local U I), literal long-range (M^lit U I)
//   and their union (hybrid).
//
// Kernel 1 (a few 1024-thread workgroups per sample, one thread per block): each forms
// the sum of c, the flags, literal ranks by wave ballot + popcount prefix, row and column
// lengths in closed form and one combined exclusive scan into row_ptr/col_ptr (the first
// workgroup of the sample writes them), then the workgroups share the list entries, each
// written by its own thread (row found by binary search over the row starts).
// Row i of each class:
//   local   : j = max(0, i-w) .. i
//   literal : literal j <= i if l_i, else i alone
//   hybrid  : (literal j < i - w, if l_i) followed by j = max(0, i-w) .. i
// Column j: local i = j .. min(N-1, j+w); literal: literal i >= j if l_j, else j alone;
// hybrid: i = j .. min(N-1, j+w) followed by (literal i > j + w, if l_j).
//
// Work order: every (sample, head, block) item sorted by the octave of its list length,
// key = floor(log2 len) + 1, largest first, ties in ascending item index (s*H + h)*N + i,
// once over CSR row lengths and once over CSC column lengths.  Heads of one class share
// their lists, so the position of an item is a closed form of per-(sample, class) data:
//   pos(s, h, i) = base[s][k][key] + (h - first head of k) * hist[s][k][key] + rank[s][k][i]
// where hist[s][k][key] counts the blocks with that key in the (s, k) list, rank is the
// number of earlier blocks with the same key there (found by ballots over the key bits),
// and base[s][k][key] is the number of items with a larger key plus n_heads * hist summed
// over every earlier (s', k') for this key.  Kernel 1 writes hist and rank per sample;
// kernel 2 (one workgroup per list) scans hist over keys and segments into base; kernel 3
// places every item with one thread, as a descriptor (item, beg, end, first entry) that
// the attention kernels read with one load.
#include <mutex>

#include "gsa_device.hpp"
#include "gsa_internal.hpp"

namespace gsa {
namespace {

constexpr int kMaskThreads = 1024;
constexpr int kMaskWaves = kMaskThreads / kWave;
static_assert(kOrderKeys >= 32 - __builtin_clz(GSA_MAX_BLOCKS) + 1, "order keys of every length fit");

// Sort key of a list length: its octave, floor(log2 len) + 1 (0 for an empty list).
// Items of one head with similar lengths then sit next to each other in the work order,
// so the kv-blocks they share meet in one L2, while the order stays longest-first to
// within a factor of two.
__device__ __forceinline__ int order_key(int len) { return len <= 0 ? 0 : 32 - __clz(len); }

__device__ __forceinline__ uint64_t lanes_below(int lane) { return (1ull << lane) - 1ull; }

// Largest x in [0, n) with start[x] <= e, for strictly increasing start[0..n] with
// start[0] = 0 <= e: a fixed number of halving steps (n <= GSA_MAX_BLOCKS), so the
// searches of several lists have no data-dependent loop and can be interleaved.
__device__ __forceinline__ int find_segment(const int *start, int n, int e) {
  int x = 0;
#pragma unroll
  for (int step = GSA_MAX_BLOCKS / 2; step > 0; step >>= 1)
    if (x + step < n && start[x + step] <= e) x += step;
  return x;
}

// From the six list lengths of this thread's block t (rows of classes 0..2, then columns):
// one exclusive scan into row_ptr / col_ptr (also kept in s_start), the edge counts, and
// the work-order data (key histograms and packed ranks) in sched.  Every thread of the
// workgroup calls it (it synchronises); s_cnt must be zero and visible on entry.
__device__ void lengths_to_lists(const int (&len)[6], int n, int64_t s, int64_t batch, int32_t *__restrict__ row_ptr,
                                 int32_t *__restrict__ col_ptr, int64_t *__restrict__ n_edges,
                                 int32_t *__restrict__ sched, int (*s_start)[GSA_MAX_BLOCKS + 1],
                                 int (*s_wave)[kMaskWaves], int (*s_cnt)[kMaskWaves][kOrderKeys],
                                 bool writer = true) {
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const bool valid = t < n;
  const int active = (n + kWave - 1) / kWave;
  const bool busy = wave < active;
  // One exclusive scan of the six lengths, and the ranks among equal keys: lanes with the
  // same key agree on every key bit, so AND-ing the ballots of the bits (or of their
  // complements) gives the wave's lanes with this lane's key.
  const uint64_t live = __ballot(valid);
  int incl[6] = {}, key[6] = {}, in_rank[6] = {};
  if (busy) {
#pragma unroll
  for (int q = 0; q < 6; ++q) {
    incl[q] = len[q];
    key[q] = valid ? order_key(len[q]) : 0;
    uint64_t same = live;
#pragma unroll
    for (int bit = 0; bit < 4; ++bit) {
      const bool on = (key[q] >> bit) & 1;
      const uint64_t b = __ballot(on);
      same &= on ? b : ~b;
    }
    in_rank[q] = __popcll(same & lanes_below(lane));
    if (valid && in_rank[q] == 0) s_cnt[q][wave][key[q]] = __popcll(same);
  }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
#pragma unroll
    for (int q = 0; q < 6; ++q) {
      const int y = __shfl_up(incl[q], off, kWave);
      if (lane >= off) incl[q] += y;
    }
  }
  if (lane == kWave - 1) {
#pragma unroll
    for (int q = 0; q < 6; ++q) s_wave[q][wave] = incl[q];
  }
  }
  __syncthreads();

  // Per (list-class q, key): exclusive scan of the wave counts over waves; the total is the
  // (s, class) histogram entry.
  int32_t *hist = sched;
  int32_t *packed = sched + 4 * batch * 3 * kOrderKeys;
  if (t < 6 * kOrderKeys) {
    const int q = t / kOrderKeys, kk = t % kOrderKeys;
    int run = 0;
    for (int w2 = 0; w2 < active; ++w2) {
      const int v = s_cnt[q][w2][kk];
      s_cnt[q][w2][kk] = run;
      run += v;
    }
    if (writer) hist[(((q / 3) * batch + s) * 3 + q % 3) * kOrderKeys + kk] = run;
  }
#pragma unroll
  for (int q = 0; q < 6 && busy; ++q) {
    int base = 0, tot = 0;
    for (int w2 = 0; w2 < active; ++w2) {
      const int v = s_wave[q][w2];
      if (w2 < wave) base += v;
      tot += v;
    }
    const int start = base + incl[q] - len[q];
    int32_t *ptr = (q < 3 ? row_ptr : col_ptr) + (s * 3 + q % 3) * (int64_t)(n + 1);
    if (valid) {
      if (writer) ptr[t] = start;
      s_start[q][t] = start;
    }
    if (t == 0) {
      if (writer) ptr[n] = tot;
      s_start[q][n] = tot;
      if (writer && q < 3) n_edges[s * 3 + q] = tot;
    }
  }
  __syncthreads();
  if (valid && writer) {
#pragma unroll
    for (int q = 0; q < 6; ++q)
      packed[(((q / 3) * batch + s) * 3 + q % 3) * (int64_t)n + t] =
          ((s_cnt[q][wave][key[q]] + in_rank[q]) << 4) | key[q];
  }

}

__global__ __launch_bounds__(kMaskThreads) void mask_kernel(
    const int32_t *__restrict__ c, int n, int w, uint8_t *__restrict__ flags,
    int32_t *__restrict__ n_literal, int32_t *__restrict__ row_ptr, int32_t *__restrict__ col_idx,
    int32_t *__restrict__ col_ptr, int32_t *__restrict__ row_idx, int64_t *__restrict__ n_edges,
    int64_t cap, int32_t *__restrict__ sched, int64_t batch) {
  __shared__ int s_prefix[GSA_MAX_BLOCKS + 1];   // # literal blocks before position i
  __shared__ int s_list[GSA_MAX_BLOCKS];         // literal block ids, ascending
  __shared__ int s_start[6][GSA_MAX_BLOCKS + 1]; // row starts (k), then column starts (3 + k)
  __shared__ long long s_sum[kMaskWaves];
  __shared__ int s_wave[6][kMaskWaves];
  __shared__ int s_cnt[6][kMaskWaves][kOrderKeys];

  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const int64_t s = blockIdx.x;
  // gridDim.y workgroups share a sample: each derives its flags and list starts, the first
  // writes them, and all write a share of the list entries.
  const bool writer = blockIdx.y == 0;
  const bool valid = t < n;
  // Waves holding blocks; the others only help with the list entries.
  const int active = (n + kWave - 1) / kWave;
  const bool busy = wave < active;
  const int ci = valid ? c[s * n + t] : 0;
  for (int x = t; x < 6 * kMaskWaves * kOrderKeys; x += kMaskThreads) (&s_cnt[0][0][0])[x] = 0;

  // Sum of c over the sample, exactly, in 64 bits.
  if (busy) {
    long long part = ci;
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) part += __shfl_xor(part, off, kWave);
    if (lane == 0) s_sum[wave] = part;
  }
  __syncthreads();
  long long sum = 0;
  for (int w2 = 0; w2 < active; ++w2) sum += s_sum[w2];

  // l_i = [N c_i > sum c]  <=>  r_i > mean r.
  const bool lit = valid && (long long)n * ci > sum;
  const uint64_t bal = __ballot(lit);
  const int below = __popcll(bal & lanes_below(lane));
  if (lane == 0) s_wave[0][wave] = __popcll(bal);
  __syncthreads();
  int wave_base = 0, n_lit = 0;
  for (int w2 = 0; w2 < active; ++w2) {
    if (w2 < wave) wave_base += s_wave[0][w2];
    n_lit += s_wave[0][w2];
  }
  const int rank = wave_base + below;   // literal blocks j < t
  if (valid) {
    if (writer) flags[s * n + t] = lit ? 1 : 0;
    s_prefix[t] = rank;
    if (lit) s_list[rank] = t;
  }
  if (t == 0) {
    s_prefix[n] = n_lit;
    if (writer) n_literal[s] = n_lit;
  }
  __syncthreads();

  // List lengths in closed form (w >= n - 1 behaves like w = n): rows k, columns 3 + k.
  const int ww = w < n ? w : n;
  int len[6] = {0, 0, 0, 0, 0, 0};
  if (valid) {
    const int win = (t < ww ? t : ww) + 1;
    len[0] = win;
    len[1] = lit ? rank + 1 : 1;
    len[2] = win + (lit ? s_prefix[t - ww > 0 ? t - ww : 0] : 0);
    const int after = n - 1 - t;
    const int cwin = (after < ww ? after : ww) + 1;
    const int beyond = t + ww + 1 < n ? t + ww + 1 : n;
    len[3] = cwin;
    len[4] = lit ? n_lit - rank : 1;
    len[5] = cwin + (lit ? n_lit - s_prefix[beyond] : 0);
  }

  lengths_to_lists(len, n, s, batch, row_ptr, col_ptr, n_edges, sched, s_start, s_wave, s_cnt, writer);

  // List entries, one thread each; the six lists are walked together so that their row
  // searches interleave.  Entry e of row i (lists 0-2, col_idx) or of column j (lists
  // 3-5, row_idx) of class k:
  //   row i:    local lo + e; literal: s_list[e] if l_i, else i; hybrid: the literal
  //             j < lo first, then lo + ...   (lo = max(0, i - w))
  //   column j: local j + e; literal: s_list[prefix_j + e] if l_j, else j; hybrid:
  //             j .. j + w first, then the literal i > j + w
  int tot[6], most = 0;
#pragma unroll
  for (int q = 0; q < 6; ++q) {
    tot[q] = s_start[q][n];
    most = tot[q] > most ? tot[q] : most;
  }
  const int stride = kMaskThreads * (int)gridDim.y;
  for (int e0 = (int)blockIdx.y * kMaskThreads + t; e0 < most; e0 += stride) {
    int seg[6];
#pragma unroll
    for (int q = 0; q < 6; ++q) seg[q] = e0 < tot[q] ? find_segment(s_start[q], n, e0) : 0;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      if (e0 < tot[k]) {
        const int i = seg[k];
        const int e = e0 - s_start[k][i];
        const int lo = i - ww > 0 ? i - ww : 0;
        const bool li = s_prefix[i + 1] != s_prefix[i];
        int j;
        if (k == 0) {
          j = lo + e;
        } else if (k == 1) {
          j = li ? s_list[e] : i;
        } else {
          const int n_far = li ? s_prefix[lo] : 0;   // literal j < i - w
          j = e < n_far ? s_list[e] : lo + (e - n_far);
        }
        col_idx[(s * 3 + k) * cap + e0] = j;
      }
      if (e0 < tot[3 + k]) {
        const int j = seg[3 + k];
        const int e = e0 - s_start[3 + k][j];
        const bool lj = s_prefix[j + 1] != s_prefix[j];
        int i;
        if (k == 0) {
          i = j + e;
        } else if (k == 1) {
          i = lj ? s_list[s_prefix[j] + e] : j;
        } else {
          const int after = n - 1 - j;
          const int cwin = (after < ww ? after : ww) + 1;
          const int first_far = s_prefix[j + ww + 1 < n ? j + ww + 1 : n];
          i = e < cwin ? j + e : s_list[first_far + (e - cwin)];
        }
        row_idx[(s * 3 + k) * cap + e0] = i;
      }
    }
  }
}


// ---------------------------------------------------------------------------------------
// Lists of a caller-given block mask: u8 [B, 3, N, N], entry (s, k, i, j) nonzero when
// query block i of class k keeps kv-block j.  The lists follow the causal reading of the
// gzip mask: entries above the diagonal are ignored and the diagonal is always kept, so
// the attention kernels see the same list shape as for the gzip mask.  One workgroup per
// sample, thread t owns row t and column t of every class; flags and L are set to zero.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ bool block_kept(const uint8_t *m, int n, int i, int j) {
  return j == i || (j < i && m[(int64_t)i * n + j] != 0);
}

__global__ __launch_bounds__(kMaskThreads) void blocks_kernel(
    const uint8_t *__restrict__ blocks, int n, uint8_t *__restrict__ flags, int32_t *__restrict__ n_literal,
    int32_t *__restrict__ row_ptr, int32_t *__restrict__ col_idx, int32_t *__restrict__ col_ptr,
    int32_t *__restrict__ row_idx, int64_t *__restrict__ n_edges, int64_t cap, int32_t *__restrict__ sched,
    int64_t batch) {
  __shared__ int s_start[6][GSA_MAX_BLOCKS + 1];
  __shared__ int s_wave[6][kMaskWaves];
  __shared__ int s_cnt[6][kMaskWaves][kOrderKeys];
  const int t = threadIdx.x;
  const int64_t s = blockIdx.x;
  const bool valid = t < n;
  for (int x = t; x < 6 * kMaskWaves * kOrderKeys; x += kMaskThreads) (&s_cnt[0][0][0])[x] = 0;
  if (valid) flags[s * n + t] = 0;
  if (t == 0) n_literal[s] = 0;
  int len[6] = {0, 0, 0, 0, 0, 0};
  if (valid) {
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const uint8_t *m = blocks + (s * 3 + k) * (int64_t)n * n;
      for (int j = 0; j <= t; ++j) len[k] += block_kept(m, n, t, j) ? 1 : 0;
      for (int i = t; i < n; ++i) len[3 + k] += block_kept(m, n, i, t) ? 1 : 0;
    }
  }
  __syncthreads();
  lengths_to_lists(len, n, s, batch, row_ptr, col_ptr, n_edges, sched, s_start, s_wave, s_cnt);
  if (valid) {
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const uint8_t *m = blocks + (s * 3 + k) * (int64_t)n * n;
      int32_t *rows = col_idx + (s * 3 + k) * cap + s_start[k][t];
      int e = 0;
      for (int j = 0; j <= t; ++j)
        if (block_kept(m, n, t, j)) rows[e++] = j;
      int32_t *cols = row_idx + (s * 3 + k) * cap + s_start[3 + k][t];
      e = 0;
      for (int i = t; i < n; ++i)
        if (block_kept(m, n, i, t)) cols[e++] = i;
    }
  }
}

// BigBird-style fixed block mask, causal form, into class 0 of u8 [B, 3, N, N] (classes 1
// and 2 get the diagonal only): query block i keeps j <= i when j is within the window
// (i - j <= w), j is a global block (j < g), i is a global block (i < g, which then sees
// every earlier block), or j is one of the r random blocks drawn for row i.
__global__ __launch_bounds__(256) void bigbird_kernel(int64_t batch, int n, int w, int g, int r,
                                                      const int32_t *__restrict__ rnd,
                                                      uint8_t *__restrict__ blocks) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_sample = 3 * (int64_t)n * n;
  if (idx >= batch * per_sample) return;
  const int64_t s = idx / per_sample;
  const int64_t rem = idx % per_sample;
  const int k = (int)(rem / ((int64_t)n * n));
  const int i = (int)((rem / n) % n), j = (int)(rem % n);
  bool keep = j == i;
  if (k == 0 && j <= i) {
    keep = i - j <= w || j < g || i < g;
    const int32_t *ri = rnd + (s * n + i) * (int64_t)r;
    for (int q = 0; q < r && !keep; ++q) keep = ri[q] == j;
  }
  blocks[idx] = keep ? 1 : 0;
}

// base[list][s][k][key] from hist: one workgroup per list.  Segments (s, k) weigh their
// counts by the heads of class k; keys are taken largest first.
constexpr int kOrderThreads = 256;
constexpr int kOrderWaves = kOrderThreads / kWave;

// The 16 counts of segment `seg` (zeros past the end), weighted by its class's heads; four
// 16-byte loads issued together.
__device__ __forceinline__ void load_counts(const int32_t *hist, int64_t seg, int64_t nseg, const int *nh,
                                            int (&v)[kOrderKeys]) {
  static_assert(kOrderKeys == 16, "four int4 per segment");
  u32x4 x[4] = {};
  if (seg < nseg) {
    const u32x4 *src = reinterpret_cast<const u32x4 *>(hist + seg * kOrderKeys);
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = src[u];
  }
  const int wgt = seg < nseg ? nh[seg % 3] : 0;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) v[4 * u + e] = wgt * (int)x[u][e];
}

__global__ __launch_bounds__(kOrderThreads) void order_base_kernel(int64_t batch, int n_loc, int n_lit,
                                                                   int n_hyb, int32_t *__restrict__ sched) {
  __shared__ int s_tot[kOrderKeys][kOrderWaves], s_first[kOrderKeys], s_carry[kOrderKeys];
  __shared__ int s_part[kOrderKeys][kOrderWaves];
  const int list = blockIdx.x;
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const int nh[3] = {n_loc, n_lit, n_hyb};
  const int64_t nseg = 3 * batch;
  const int32_t *hist = sched + list * nseg * kOrderKeys;
  int32_t *base = sched + (2 + list) * nseg * kOrderKeys;
  int v[kOrderKeys];
  // Items per key over every segment (with a single chunk its counts stay in registers).
  int tot[kOrderKeys] = {};
  for (int64_t c0 = 0; c0 < nseg; c0 += kOrderThreads) {
    load_counts(hist, c0 + t, nseg, nh, v);
#pragma unroll
    for (int kk = 0; kk < kOrderKeys; ++kk) tot[kk] += v[kk];
  }
  const bool any = wave * kWave < nseg;   // this wave ever holds a segment
#pragma unroll
  for (int kk = 0; kk < kOrderKeys; ++kk) {
    int x = tot[kk];
    if (any) {
#pragma unroll
      for (int off = kWave / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
    }
    if (lane == 0) s_tot[kk][wave] = x;
  }
  if (t < kOrderKeys) s_carry[t] = 0;
  __syncthreads();
  if (t < kOrderKeys) {
    int first = 0;
    for (int k2 = t + 1; k2 < kOrderKeys; ++k2)
      for (int w2 = 0; w2 < kOrderWaves; ++w2) first += s_tot[k2][w2];
    s_first[t] = first;
  }
  // Exclusive scan over segments, per key, one chunk of segments at a time.
  for (int64_t c0 = 0; c0 < nseg; c0 += kOrderThreads) {
    const int64_t seg = c0 + t;
    if (nseg > kOrderThreads) load_counts(hist, seg, nseg, nh, v);
    int incl[kOrderKeys];
#pragma unroll
    for (int kk = 0; kk < kOrderKeys; ++kk) incl[kk] = v[kk];
    if (c0 + wave * kWave < nseg) {
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
#pragma unroll
      for (int kk = 0; kk < kOrderKeys; ++kk) {
        const int y = __shfl_up(incl[kk], off, kWave);
        if (lane >= off) incl[kk] += y;
      }
    }
    }
    if (lane == kWave - 1) {
#pragma unroll
      for (int kk = 0; kk < kOrderKeys; ++kk) s_part[kk][wave] = incl[kk];
    }
    __syncthreads();
    if (seg < nseg) {
      int out[kOrderKeys];
#pragma unroll
      for (int kk = 0; kk < kOrderKeys; ++kk) {
        int before = s_carry[kk];
        for (int w2 = 0; w2 < wave; ++w2) before += s_part[kk][w2];
        out[kk] = s_first[kk] + before + incl[kk] - v[kk];
      }
      u32x4 *dst = reinterpret_cast<u32x4 *>(base + seg * kOrderKeys);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        dst[u] = u32x4{(uint32_t)out[4 * u], (uint32_t)out[4 * u + 1], (uint32_t)out[4 * u + 2],
                       (uint32_t)out[4 * u + 3]};
    }
    __syncthreads();
    if (t < kOrderKeys) {
      int sum = 0;
      for (int w2 = 0; w2 < kOrderWaves; ++w2) sum += s_part[t][w2];
      s_carry[t] += sum;
    }
    __syncthreads();
  }
}

// Places every item of both work lists with its descriptor (item, beg, end, first entry):
// grid (items / 256, 2).
__global__ __launch_bounds__(256) void order_scatter_kernel(const int32_t *__restrict__ sched, int64_t batch, int n,
                                                            int n_loc, int n_lit, int n_hyb,
                                                            const int32_t *__restrict__ row_ptr,
                                                            const int32_t *__restrict__ col_idx,
                                                            const int32_t *__restrict__ col_ptr,
                                                            const int32_t *__restrict__ row_idx, int64_t cap,
                                                            int32_t *__restrict__ work_row,
                                                            int32_t *__restrict__ work_col) {
  const int heads = n_loc + n_lit + n_hyb;
  const int64_t items = batch * heads * (int64_t)n;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= items) return;
  const int list = blockIdx.y;
  const int i = (int)(idx % n);
  const int64_t sh = idx / n;
  const int h = (int)(sh % heads);
  const int64_t s = sh / heads;
  const int k = h < n_loc ? 0 : (h < n_loc + n_lit ? 1 : 2);
  const int h0 = k == 0 ? 0 : (k == 1 ? n_loc : n_loc + n_lit);
  const int64_t seg = (list * batch + s) * 3 + k;
  const int32_t pk = sched[4 * batch * 3 * kOrderKeys + seg * n + i];
  const int32_t *ptr = (list == 0 ? row_ptr : col_ptr) + (s * 3 + k) * (int64_t)(n + 1);
  const int beg = ptr[i], end = ptr[i + 1];
  const int first = (list == 0 ? col_idx : row_idx)[(s * 3 + k) * cap + beg];
  const int64_t slot = seg * kOrderKeys + (pk & 15);
  const int32_t *hist = sched;
  const int32_t *base = sched + 2 * batch * 3 * kOrderKeys;
  const int64_t pos = base[slot] + (h - h0) * hist[slot] + (pk >> 4);
  reinterpret_cast<u32x4 *>(list == 0 ? work_row : work_col)[pos] =
      u32x4{(uint32_t)idx, (uint32_t)beg, (uint32_t)end, (uint32_t)first};
}

// order_base_kernel and order_scatter_kernel in one launch, for batches whose per-list
// histograms fit in LDS: every workgroup loads the histogram of its list and forms the
// bases itself (a few hundred counts), which costs less than a kernel boundary.
constexpr int kFusedMaxBatch = 128;
constexpr int kFusedMaxSeg = 3 * kFusedMaxBatch;

__global__ __launch_bounds__(kOrderThreads) void order_fused_kernel(const int32_t *__restrict__ sched, int64_t batch,
                                                                    int n, int n_loc, int n_lit, int n_hyb,
                                                                    const int32_t *__restrict__ row_ptr,
                                                                    const int32_t *__restrict__ col_idx,
                                                                    const int32_t *__restrict__ col_ptr,
                                                                    const int32_t *__restrict__ row_idx, int64_t cap,
                                                                    int32_t *__restrict__ work_row,
                                                                    int32_t *__restrict__ work_col) {
  static_assert(kOrderThreads == kOrderKeys * 16, "16 chunks of segments per key");
  __shared__ int s_pre[kFusedMaxSeg][kOrderKeys];   // weighted counts, then exclusive prefixes
  __shared__ int s_chunk[16][kOrderKeys], s_tot[kOrderKeys], s_first[kOrderKeys];
  const int t = threadIdx.x;
  const int list = blockIdx.y;
  const int nseg = (int)(3 * batch);
  const int nh[3] = {n_loc, n_lit, n_hyb};
  const int32_t *hist = sched + (int64_t)list * nseg * kOrderKeys;
  for (int x = t; x < nseg * kOrderKeys; x += kOrderThreads)
    s_pre[x / kOrderKeys][x % kOrderKeys] = nh[(x / kOrderKeys) % 3] * hist[x];
  __syncthreads();
  // Thread (chunk, key): segments [lo, hi) of one key.
  const int key = t % kOrderKeys, chunk = t / kOrderKeys;
  const int per = (nseg + 15) / 16;
  const int lo = min(chunk * per, nseg), hi = min(lo + per, nseg);
  int sum = 0;
  for (int sg = lo; sg < hi; ++sg) sum += s_pre[sg][key];
  s_chunk[chunk][key] = sum;
  __syncthreads();
  int run = 0, total = 0;
  for (int c2 = 0; c2 < 16; ++c2) {
    const int v = s_chunk[c2][key];
    if (c2 < chunk) run += v;
    total += v;
  }
  for (int sg = lo; sg < hi; ++sg) {
    const int v = s_pre[sg][key];
    s_pre[sg][key] = run;
    run += v;
  }
  if (chunk == 0) s_tot[key] = total;
  __syncthreads();
  if (t < kOrderKeys) {
    int first = 0;
    for (int k2 = t + 1; k2 < kOrderKeys; ++k2) first += s_tot[k2];
    s_first[t] = first;
  }
  __syncthreads();

  const int heads = n_loc + n_lit + n_hyb;
  const int64_t items = batch * heads * (int64_t)n;
  const int64_t idx = (int64_t)blockIdx.x * kOrderThreads + t;
  if (idx >= items) return;
  const int i = (int)(idx % n);
  const int64_t sh = idx / n;
  const int h = (int)(sh % heads);
  const int64_t s = sh / heads;
  const int k = h < n_loc ? 0 : (h < n_loc + n_lit ? 1 : 2);
  const int h0 = k == 0 ? 0 : (k == 1 ? n_loc : n_loc + n_lit);
  const int seg = (int)(s * 3 + k);
  const int32_t pk = sched[4 * batch * 3 * kOrderKeys + ((int64_t)list * nseg + seg) * n + i];
  const int32_t *ptr = (list == 0 ? row_ptr : col_ptr) + seg * (int64_t)(n + 1);
  const int beg = ptr[i], end = ptr[i + 1];
  const int first = (list == 0 ? col_idx : row_idx)[seg * cap + beg];
  const int kk = pk & 15;
  const int64_t pos = s_first[kk] + s_pre[seg][kk] + (int64_t)(h - h0) * hist[seg * kOrderKeys + kk] + (pk >> 4);
  reinterpret_cast<u32x4 *>(list == 0 ? work_row : work_col)[pos] =
      u32x4{(uint32_t)idx, (uint32_t)beg, (uint32_t)end, (uint32_t)first};
}

}  // namespace

static gsa_status launch_order(const gsa_mask &m, hipStream_t stream) {
  const int n = m.n_blocks;
  const int64_t items = m.batch * (int64_t)(m.n_heads[0] + m.n_heads[1] + m.n_heads[2]) * n;
  if (items == 0) return GSA_OK;
  if (m.batch <= kFusedMaxBatch) {
    hipLaunchKernelGGL(order_fused_kernel, dim3((unsigned)((items + kOrderThreads - 1) / kOrderThreads), 2),
                       dim3(kOrderThreads), 0, stream, m.sched, m.batch, n, m.n_heads[0], m.n_heads[1],
                       m.n_heads[2], m.row_ptr, m.col_idx, m.col_ptr, m.row_idx, mask_cap(n), m.work_row,
                       m.work_col);
    return check_launch("order_fused_kernel");
  }
  hipLaunchKernelGGL(order_base_kernel, dim3(2), dim3(kOrderThreads), 0, stream, m.batch, m.n_heads[0],
                     m.n_heads[1], m.n_heads[2], m.sched);
  gsa_status st = check_launch("order_base_kernel");
  if (st != GSA_OK) return st;
  hipLaunchKernelGGL(order_scatter_kernel, dim3((unsigned)((items + 255) / 256), 2), dim3(256), 0, stream,
                     m.sched, m.batch, n, m.n_heads[0], m.n_heads[1], m.n_heads[2], m.row_ptr, m.col_idx,
                     m.col_ptr, m.row_idx, mask_cap(n), m.work_row, m.work_col);
  return check_launch("order_scatter_kernel");
}

// Workgroups per sample in mask_kernel: enough that each writes at most about 4K entries
// of the up to 6 N (N + 1) / 2 list entries of a sample (1 at N <= 64, 32 at N = 512).
static int mask_split(int n) {
  const int64_t cap = mask_cap(n);
  const int64_t split = cap / 4096;
  return (int)(split < 1 ? 1 : (split > 32 ? 32 : split));
}

gsa_status launch_build_mask(const int32_t *c, const gsa_mask &m, hipStream_t stream) {
  const int n = m.n_blocks;
  hipLaunchKernelGGL(mask_kernel, dim3((unsigned)m.batch, (unsigned)mask_split(n)), dim3(kMaskThreads), 0, stream, c, n,
                     m.window, m.flags, m.n_literal, m.row_ptr, m.col_idx, m.col_ptr, m.row_idx,
                     m.n_edges, mask_cap(n), m.sched, m.batch);
  gsa_status st = check_launch("mask_kernel");
  if (st != GSA_OK) return st;
  return launch_order(m, stream);
}

// Work-order scratch of gsa_build_mask_noalloc: a file-scope device array, one copy per
// GPU.  In host code `scratch` names a host-side stand-in, not the device memory, so the
// kernels get its device address, looked up once per device (with that device current)
// by hipGetSymbolAddress and kept in g_scratch.  Every entry of the scratch is written
// by the mask kernel or the order kernels before it is read, so nothing needs clearing
// between calls.
static __device__ __align__(256) int32_t scratch[GSA_NOALLOC_SCHED_BYTES / 4];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t *g_scratch[kMaxDevices] = {};

gsa_status scratch_on(int dev, int32_t **out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(GSA_ERR_UNSUPPORTED, "device %d outside 0..%d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return fail(GSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(GSA_ERR_HIP, "hipSetDevice(%d): %s", dev, hipGetErrorString(e));
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess && e2 != hipSuccess)
        return fail(GSA_ERR_HIP, "hipSetDevice(%d): %s", cur, hipGetErrorString(e2));
    }
    if (e != hipSuccess || !p)
      return fail(GSA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch[dev] = static_cast<int32_t *>(p);
  }
  *out = g_scratch[dev];
  return GSA_OK;
}
}  // namespace

gsa_status launch_build_mask_noalloc(const int32_t *c, const gsa_mask &m, hipStream_t stream) {
  int dev = 0;
  const hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return fail(GSA_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
  int32_t *ptr = nullptr;
  gsa_status st = scratch_on(dev, &ptr);
  if (st != GSA_OK) return st;
  gsa_mask mm = m;
  mm.sched = ptr;
  return launch_build_mask(c, mm, stream);
}

gsa_status launch_mask_from_blocks(const uint8_t *blocks, const gsa_mask &m, hipStream_t stream) {
  const int n = m.n_blocks;
  hipLaunchKernelGGL(blocks_kernel, dim3((unsigned)m.batch), dim3(kMaskThreads), 0, stream, blocks, n, m.flags,
                     m.n_literal, m.row_ptr, m.col_idx, m.col_ptr, m.row_idx, m.n_edges, mask_cap(n), m.sched,
                     m.batch);
  gsa_status st = check_launch("blocks_kernel");
  if (st != GSA_OK) return st;
  return launch_order(m, stream);
}

gsa_status launch_bigbird(int64_t batch, int32_t n, int32_t window, int32_t n_global, int32_t n_random,
                          const int32_t *rnd, uint8_t *blocks, hipStream_t stream) {
  const int64_t total = batch * 3 * (int64_t)n * n;
  hipLaunchKernelGGL(bigbird_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, batch, n, window,
                     n_global, n_random, rnd, blocks);
  return check_launch("bigbird_kernel");
}

}  // namespace gsa
