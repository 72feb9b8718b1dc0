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
// Kernel 1 (one workgroup of 1024 threads per sample, one thread per block): the sum of
// c, the flags, literal ranks by wave ballot + popcount prefix, row and column lengths
// in closed form, exclusive scans into row_ptr/col_ptr, then every wave writes whole
// rows (and columns) with its 64 lanes on consecutive entries.  Row i of each class:
//   local   : j = max(0, i-w) .. i
//   literal : literal j <= i if l_i, else i alone
//   hybrid  : (literal j < i - w, if l_i) followed by j = max(0, i-w) .. i
// Column j: local i = j .. min(N-1, j+w); literal: literal i >= j if l_j, else j alone;
// hybrid: i = j .. min(N-1, j+w) followed by (literal i > j + w, if l_j).
//
// Work order: every (sample, head, block) item sorted by list length, longest first, ties
// in ascending item index (s*H + h)*N + i, once over CSR row lengths and once over CSC
// column lengths.  Heads of one class share their lists, so the position of an item is
// a closed form of per-(sample, class) data:
//   pos(s, h, i) = start[len] + base[s][k][len] + (h - first head of k) * hist[s][k][len]
//                  + rank[s][k][i]
// where hist[s][k][len] counts the blocks of that length in the (s, k) lists, rank is the
// number of earlier blocks of the same length there, base sums n_heads * hist over every
// earlier (s', k') and start sums all items of every longer length.  Kernel 1 writes hist
// and rank per sample; kernel 2 (one workgroup per list) scans them over lengths and
// samples and scatters every item independently.
#include "gsa_device.hpp"
#include "gsa_internal.hpp"

namespace gsa {
namespace {

constexpr int kMaskThreads = 1024;
constexpr int kMaskWaves = kMaskThreads / kWave;

// Exclusive scan of one int per thread over the workgroup; returns the thread's prefix
// and writes the total to *total.  `scratch` holds kMaskWaves ints.
__device__ int block_exclusive_scan(int v, int *scratch, int *total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int y = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += y;
  }
  if (lane == kWave - 1) scratch[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w2 = 0; w2 < kMaskWaves; ++w2) {
    int s = scratch[w2];
    if (w2 < wave) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

__global__ __launch_bounds__(kMaskThreads) void mask_kernel(
    const int32_t *__restrict__ c, int n, int w, uint8_t *__restrict__ flags,
    int32_t *__restrict__ n_literal, int32_t *__restrict__ row_ptr, int32_t *__restrict__ col_idx,
    int32_t *__restrict__ col_ptr, int32_t *__restrict__ row_idx, int64_t *__restrict__ n_edges,
    int64_t cap, int32_t *__restrict__ sched, int64_t batch) {
  __shared__ int s_prefix[GSA_MAX_BLOCKS + 1];   // # literal blocks before position i
  __shared__ int s_list[GSA_MAX_BLOCKS];         // literal block ids, ascending
  __shared__ int s_rstart[3][GSA_MAX_BLOCKS + 1];
  __shared__ int s_cstart[3][GSA_MAX_BLOCKS + 1];
  __shared__ long long s_sum[kMaskWaves];
  __shared__ int s_scan[kMaskWaves];
  __shared__ int s_len[6][GSA_MAX_BLOCKS];       // row lengths (k), then column lengths (3 + k)
  __shared__ int s_hist[6][GSA_MAX_BLOCKS + 1];

  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const int64_t s = blockIdx.x;
  const int ci = t < n ? c[s * n + t] : 0;

  // Sum of c over the sample, exactly, in 64 bits.
  long long part = ci;
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) part += __shfl_xor(part, off, kWave);
  if (lane == 0) s_sum[wave] = part;
  __syncthreads();
  long long sum = 0;
  for (int w2 = 0; w2 < kMaskWaves; ++w2) sum += s_sum[w2];

  // l_i = [N c_i > sum c]  <=>  r_i > mean r.
  const bool lit = t < n && (long long)n * ci > sum;
  const uint64_t bal = __ballot(lit);
  const int below = __popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) s_scan[wave] = __popcll(bal);
  __syncthreads();
  int wave_base = 0, n_lit = 0;
  for (int w2 = 0; w2 < kMaskWaves; ++w2) {
    if (w2 < wave) wave_base += s_scan[w2];
    n_lit += s_scan[w2];
  }
  const int rank = wave_base + below;   // literal blocks j < t
  if (t < n) {
    flags[s * n + t] = lit ? 1 : 0;
    s_prefix[t] = rank;
    if (lit) s_list[rank] = t;
  }
  if (t == 0) {
    s_prefix[n] = n_lit;
    n_literal[s] = n_lit;
  }
  __syncthreads();

  // List lengths in closed form (w >= n - 1 behaves like w = n).
  const int ww = w < n ? w : n;
  int rlen[3] = {0, 0, 0}, clen[3] = {0, 0, 0};
  if (t < n) {
    const int win = (t < ww ? t : ww) + 1;
    rlen[0] = win;
    rlen[1] = lit ? rank + 1 : 1;
    rlen[2] = win + (lit ? s_prefix[t - ww > 0 ? t - ww : 0] : 0);
    const int after = n - 1 - t;
    const int cwin = (after < ww ? after : ww) + 1;
    const int beyond = t + ww + 1 < n ? t + ww + 1 : n;
    clen[0] = cwin;
    clen[1] = lit ? n_lit - rank : 1;
    clen[2] = cwin + (lit ? n_lit - s_prefix[beyond] : 0);
  }
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    int tot;
    const int rs = block_exclusive_scan(rlen[k], s_scan, &tot);
    int32_t *rp = row_ptr + (s * 3 + k) * (int64_t)(n + 1);
    if (t < n) {
      rp[t] = rs;
      s_rstart[k][t] = rs;
    }
    if (t == 0) {
      rp[n] = tot;
      s_rstart[k][n] = tot;
      n_edges[s * 3 + k] = tot;
    }
    const int cs = block_exclusive_scan(clen[k], s_scan, &tot);
    int32_t *cp = col_ptr + (s * 3 + k) * (int64_t)(n + 1);
    if (t < n) {
      cp[t] = cs;
      s_cstart[k][t] = cs;
    }
    if (t == 0) {
      cp[n] = tot;
      s_cstart[k][n] = tot;
    }
  }
  // Per-(list, class) length histograms and stable ranks among equal lengths.
  for (int x = t; x < 6 * (GSA_MAX_BLOCKS + 1); x += kMaskThreads) (&s_hist[0][0])[x] = 0;
  if (t < n) {
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      s_len[k][t] = rlen[k];
      s_len[3 + k][t] = clen[k];
    }
  }
  __syncthreads();
  if (t < n) {
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      atomicAdd(&s_hist[k][rlen[k]], 1);
      atomicAdd(&s_hist[3 + k][clen[k]], 1);
    }
  }
  int rank6[6] = {0, 0, 0, 0, 0, 0};
  if (t < n) {
    int mine[6];
#pragma unroll
    for (int q = 0; q < 6; ++q) mine[q] = s_len[q][t];
    for (int j2 = 0; j2 < t; ++j2) {
#pragma unroll
      for (int q = 0; q < 6; ++q) rank6[q] += s_len[q][j2] == mine[q] ? 1 : 0;
    }
  }
  __syncthreads();
  {
    const int seg = 3 * n + 2;
#pragma unroll
    for (int q = 0; q < 6; ++q) {
      const int list = q / 3, k = q % 3;
      int32_t *sg = sched + ((list * batch + s) * 3 + k) * (int64_t)seg;
      for (int l = t; l <= n; l += kMaskThreads) sg[l] = s_hist[q][l];
      if (t < n) sg[2 * n + 2 + t] = rank6[q];
    }
  }

  // Rows: wave-per-row, lanes on consecutive entries.
  for (int k = 0; k < 3; ++k) {
    int32_t *ci_out = col_idx + (s * 3 + k) * cap;
    int32_t *ri_out = row_idx + (s * 3 + k) * cap;
    for (int i = wave; i < n; i += kMaskWaves) {
      const int lo = i - ww > 0 ? i - ww : 0;
      const bool li = s_prefix[i + 1] != s_prefix[i];
      const int beg = s_rstart[k][i], len = s_rstart[k][i + 1] - beg;
      const int n_far = (k == 2 && li) ? s_prefix[lo] : 0;   // literal j < i - w
      for (int e = lane; e < len; e += kWave) {
        int j;
        if (k == 0) j = lo + e;
        else if (k == 1) j = li ? s_list[e] : i;
        else j = e < n_far ? s_list[e] : lo + (e - n_far);
        ci_out[beg + e] = j;
      }
      // Column i (the same i, used as a kv-block index).
      const int cbeg = s_cstart[k][i], clen2 = s_cstart[k][i + 1] - cbeg;
      const int after = n - 1 - i;
      const int cwin = (after < ww ? after : ww) + 1;
      const int first_far = s_prefix[i + ww + 1 < n ? i + ww + 1 : n];
      const int rank_i = s_prefix[i];
      for (int e = lane; e < clen2; e += kWave) {
        int r;
        if (k == 0) r = i + e;
        else if (k == 1) r = li ? s_list[rank_i + e] : i;
        else r = e < cwin ? i + e : s_list[first_far + (e - cwin)];
        ri_out[cbeg + e] = r;
      }
    }
  }
}

constexpr int kSortThreads = 1024;

// blockIdx.x == 0 orders by CSR row length into work_row, 1 by CSC column length into
// work_col.  See the work-order note at the top of this file.
__global__ __launch_bounds__(kSortThreads) void worklist_kernel(
    const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ col_ptr, int64_t batch, int n,
    int n_loc, int n_lit, int n_hyb, int32_t *__restrict__ sched, int32_t *__restrict__ work_row,
    int32_t *__restrict__ work_col) {
  __shared__ int s_scan[kSortThreads / kWave];

  const int list = blockIdx.x;
  const int32_t *ptr = list == 0 ? row_ptr : col_ptr;
  int32_t *out = list == 0 ? work_row : work_col;
  const int nh[3] = {n_loc, n_lit, n_hyb};
  const int heads = n_loc + n_lit + n_hyb;
  const int seg = 3 * n + 2;
  int32_t *base_list = sched + list * batch * 3 * (int64_t)seg;
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const int64_t nseg = batch * 3;

  // Totals per length, over every sample and class, weighted by heads per class.  The
  // (sample, class) loop is unrolled in groups so its loads are in flight together.
  int tot = 0;
  const int len = n - t;                 // thread t owns length n - t (bin t: longest first)
  if (t < n) {
    for (int64_t q0 = 0; q0 < nseg; q0 += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = q0 + u < nseg ? base_list[(q0 + u) * seg + len] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) tot += v[u] * (q0 + u < nseg ? nh[(q0 + u) % 3] : 0);
    }
  }
  // Exclusive scan over bins (longest first) gives each length's start position.
  int incl = tot;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int y = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += y;
  }
  if (lane == kWave - 1) s_scan[wave] = incl;
  __syncthreads();
  int wbase = 0;
  for (int w2 = 0; w2 < wave; ++w2) wbase += s_scan[w2];
  int running = wbase + incl - tot;
  // base[s][k][len]: start of the first head of class k of sample s among this length.
  if (t < n) {
    for (int64_t q0 = 0; q0 < nseg; q0 += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = q0 + u < nseg ? base_list[(q0 + u) * seg + len] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (q0 + u < nseg) {
          base_list[(q0 + u) * seg + n + 1 + len] = running;
          running += v[u] * nh[(q0 + u) % 3];
        }
      }
    }
  }
  __syncthreads();

  // Scatter: every item computes its own position.
  const int64_t items = batch * heads * (int64_t)n;
  for (int64_t idx = t; idx < items; idx += kSortThreads) {
    const int i = (int)(idx % n);
    const int64_t sh = idx / n;
    const int h = (int)(sh % heads);
    const int64_t s = sh / heads;
    const int k = h < n_loc ? 0 : (h < n_loc + n_lit ? 1 : 2);
    const int h0 = k == 0 ? 0 : (k == 1 ? n_loc : n_loc + n_lit);
    const int32_t *p = ptr + (s * 3 + k) * (int64_t)(n + 1);
    const int l = p[i + 1] - p[i];
    const int32_t *sg = base_list + (s * 3 + k) * (int64_t)seg;
    out[sg[n + 1 + l] + (h - h0) * sg[l] + sg[2 * n + 2 + i]] = (int32_t)idx;
  }
}

}  // namespace

gsa_status launch_build_mask(const int32_t *c, const gsa_mask &m, hipStream_t stream) {
  const int n = m.n_blocks;
  hipLaunchKernelGGL(mask_kernel, dim3((unsigned)m.batch), dim3(kMaskThreads), 0, stream, c, n,
                     m.window, m.flags, m.n_literal, m.row_ptr, m.col_idx, m.col_ptr, m.row_idx,
                     m.n_edges, mask_cap(n), m.sched, m.batch);
  gsa_status st = check_launch("mask_kernel");
  if (st != GSA_OK) return st;
  if (m.n_heads[0] + m.n_heads[1] + m.n_heads[2] == 0) return GSA_OK;
  hipLaunchKernelGGL(worklist_kernel, dim3(2), dim3(kSortThreads), 0, stream, m.row_ptr, m.col_ptr,
                     m.batch, n, m.n_heads[0], m.n_heads[1], m.n_heads[2], m.sched, m.work_row,
                     m.work_col);
  return check_launch("worklist_kernel");
}

}  // namespace gsa
