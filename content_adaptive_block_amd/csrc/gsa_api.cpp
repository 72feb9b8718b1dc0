// C ABI entry points: argument validation and kernel launches.  Every check here runs
// before any HIP call, so a rejected call has no side effects.  Status strings and the
// thread-local error detail live in gsa_error.cpp.
#include <cstdio>
#include <cstring>
#include <string>

#include "gsa_internal.hpp"

namespace gsa {

gsa_status check_launch(const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return GSA_OK;
}

static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// building: the call fills the mask (flags, counts and, unless own_sched, sched needed).
static gsa_status check_mask(const gsa_mask *m, bool building, bool own_sched = false) {
  if (!m) return fail(GSA_ERR_ARG, "mask is NULL");
  if (m->batch < 0) return fail(GSA_ERR_ARG, "mask batch %lld < 0", (long long)m->batch);
  if (m->window < 0) return fail(GSA_ERR_ARG, "window %d < 0", m->window);
  for (int k = 0; k < 3; ++k)
    if (m->n_heads[k] < 0) return fail(GSA_ERR_ARG, "n_heads[%d] = %d < 0", k, m->n_heads[k]);
  if (m->batch == 0) return GSA_OK;
  if (m->n_blocks < 1 || m->n_blocks > GSA_MAX_BLOCKS)
    return fail(GSA_ERR_UNSUPPORTED, "n_blocks %d outside 1..%d", m->n_blocks, GSA_MAX_BLOCKS);
  if (!m->row_ptr || !m->col_idx || !m->col_ptr || !m->row_idx || !m->work_row || !m->work_col)
    return fail(GSA_ERR_ARG, "mask list buffer is NULL");
  if (!aligned16(m->work_row) || !aligned16(m->work_col))
    return fail(GSA_ERR_ARG, "mask work buffers are not 16-byte aligned");
  if (building && (!m->flags || !m->n_literal || !m->n_edges))
    return fail(GSA_ERR_ARG, "mask flag/count buffer is NULL");
  if (building && !own_sched && !m->sched) return fail(GSA_ERR_ARG, "mask sched buffer is NULL");
  if (building && !own_sched && !aligned16(m->sched))
    return fail(GSA_ERR_ARG, "mask sched buffer is not 16-byte aligned");
  int64_t items = m->batch * (int64_t)(m->n_heads[0] + m->n_heads[1] + m->n_heads[2]) * m->n_blocks;
  if (items > INT32_MAX) return fail(GSA_ERR_UNSUPPORTED, "B*H*N = %lld exceeds int32", (long long)items);
  return GSA_OK;
}

static gsa_status check_fwd(const gsa_fwd_args *a, const gsa_mask *m) {
  if (!a) return fail(GSA_ERR_ARG, "args is NULL");
  if (a->batch < 0 || a->seq_len < 0 || a->heads < 0)
    return fail(GSA_ERR_ARG, "negative batch/seq_len/heads");
  if (a->block <= 0 || a->head_dim <= 0) return fail(GSA_ERR_ARG, "block and head_dim must be > 0");
  if (a->dtype != GSA_F32 && a->dtype != GSA_BF16) return fail(GSA_ERR_ARG, "unknown dtype %d", a->dtype);
  if (a->seq_len % a->block)
    return fail(GSA_ERR_SHAPE, "seq_len %lld is not a multiple of block %d", (long long)a->seq_len, a->block);
  if (!(a->scale >= 0.0f)) return fail(GSA_ERR_ARG, "scale must be >= 0 (0 selects 1/sqrt(d))");
  gsa_status st = check_mask(m, false);
  if (st != GSA_OK) return st;
  if (a->heads != m->n_heads[0] + m->n_heads[1] + m->n_heads[2])
    return fail(GSA_ERR_ARG, "heads %d != mask head counts %d+%d+%d", a->heads, m->n_heads[0],
                m->n_heads[1], m->n_heads[2]);
  if (a->batch == 0 || a->seq_len == 0 || a->heads == 0) return GSA_OK;
  if (m->batch != a->batch || (int64_t)m->n_blocks * a->block != a->seq_len)
    return fail(GSA_ERR_SHAPE, "mask (batch %lld, N %d) does not match tensors (batch %lld, T/b %lld)",
                (long long)m->batch, m->n_blocks, (long long)a->batch, (long long)(a->seq_len / a->block));
  if (!attn_instance_built(a->dtype, a->block, a->head_dim))
    return fail(GSA_ERR_UNSUPPORTED, "no kernel for dtype %d, block %d, head_dim %d", a->dtype, a->block,
                a->head_dim);
  if (!a->q || !a->k || !a->v || !a->o) return fail(GSA_ERR_ARG, "q/k/v/o is NULL");
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o))
    return fail(GSA_ERR_ARG, "q/k/v/o must be 16-byte aligned");
  if (a->lse && !aligned16(a->lse)) return fail(GSA_ERR_ARG, "lse must be 16-byte aligned");
  return GSA_OK;
}

}  // namespace gsa

using namespace gsa;

extern "C" {

int32_t gsa_abi_version(void) { return GSA_ABI_VERSION; }

gsa_status gsa_mask_bytes(int64_t batch, int32_t n_blocks, const int32_t n_heads[3],
                          size_t sizes_out[GSA_MASK_NBUF]) {
  clear_error();
  if (!n_heads || !sizes_out) return fail(GSA_ERR_ARG, "NULL argument");
  if (batch < 0 || n_blocks < 0) return fail(GSA_ERR_ARG, "negative batch or n_blocks");
  for (int k = 0; k < 3; ++k)
    if (n_heads[k] < 0) return fail(GSA_ERR_ARG, "n_heads[%d] < 0", k);
  const size_t B = (size_t)batch, N = (size_t)n_blocks;
  const size_t H = (size_t)n_heads[0] + n_heads[1] + n_heads[2];
  const size_t cap = N * (N + 1) / 2;
  sizes_out[0] = B * N;                      // flags
  sizes_out[1] = B * 4;                      // n_literal
  sizes_out[2] = B * 3 * (N + 1) * 4;        // row_ptr
  sizes_out[3] = B * 3 * cap * 4;            // col_idx
  sizes_out[4] = B * 3 * (N + 1) * 4;        // col_ptr
  sizes_out[5] = B * 3 * cap * 4;            // row_idx
  sizes_out[6] = B * 3 * 8;                  // n_edges
  sizes_out[7] = B * H * N * 16;             // work_row: 4 int32 per item
  sizes_out[8] = B * H * N * 16;             // work_col
  sizes_out[9] = (size_t)sched_words(batch, n_blocks) * 4;  // sched: work-order scratch
  return GSA_OK;
}

gsa_status gsa_mask_sizes(int64_t batch, int32_t n_blocks, const int32_t n_heads[3],
                          size_t sizes_out[GSA_MASK_NBUF]) {
  return gsa_mask_bytes(batch, n_blocks, n_heads, sizes_out);
}

gsa_status gsa_default_head_counts(int32_t heads, int32_t n_heads_out[3]) {
  clear_error();
  if (!n_heads_out) return fail(GSA_ERR_ARG, "n_heads_out is NULL");
  if (heads < 0) return fail(GSA_ERR_ARG, "heads %d < 0", heads);
  n_heads_out[0] = heads / 2;
  n_heads_out[1] = heads / 4;
  n_heads_out[2] = heads - heads / 2 - heads / 4;
  return GSA_OK;
}

gsa_status gsa_build_mask(const int32_t *c_dev, const gsa_mask *m, hipStream_t stream) {
  clear_error();
  gsa_status st = check_mask(m, true);
  if (st != GSA_OK) return st;
  if (m->batch == 0) return GSA_OK;
  if (!c_dev) return fail(GSA_ERR_ARG, "c_dev is NULL");
  return launch_build_mask(c_dev, *m, stream);
}

gsa_status gsa_build_mask_noalloc(const int32_t *c_dev, const gsa_mask *m, hipStream_t stream) {
  clear_error();
  gsa_status st = check_mask(m, true, true);
  if (st != GSA_OK) return st;
  if (m->batch == 0) return GSA_OK;
  if (!c_dev) return fail(GSA_ERR_ARG, "c_dev is NULL");
  const int64_t need = sched_words(m->batch, m->n_blocks) * 4;
  if (need > (int64_t)GSA_NOALLOC_SCHED_BYTES)
    return fail(GSA_ERR_UNSUPPORTED,
                "batch %lld x %d blocks needs %lld bytes of work-order scratch; gsa_build_mask_noalloc "
                "holds %u (use gsa_build_mask with a caller-allocated sched buffer)",
                (long long)m->batch, m->n_blocks, (long long)need, (unsigned)GSA_NOALLOC_SCHED_BYTES);
  return launch_build_mask_noalloc(c_dev, *m, stream);
}

gsa_status gsa_build_mask_from_blocks(const uint8_t *blocks_dev, const gsa_mask *m, hipStream_t stream) {
  clear_error();
  gsa_status st = check_mask(m, true);
  if (st != GSA_OK) return st;
  if (m->batch == 0) return GSA_OK;
  if (!blocks_dev) return fail(GSA_ERR_ARG, "blocks_dev is NULL");
  return launch_mask_from_blocks(blocks_dev, *m, stream);
}

gsa_status gsa_bigbird_blocks(int64_t batch, int32_t n_blocks, int32_t window, int32_t n_global,
                              int32_t n_random, const int32_t *random_dev, uint8_t *blocks_dev,
                              hipStream_t stream) {
  clear_error();
  if (batch < 0) return fail(GSA_ERR_ARG, "batch %lld < 0", (long long)batch);
  if (window < 0 || n_global < 0 || n_random < 0)
    return fail(GSA_ERR_ARG, "window, n_global and n_random must be >= 0");
  if (batch == 0) return GSA_OK;
  if (n_blocks < 1 || n_blocks > GSA_MAX_BLOCKS)
    return fail(GSA_ERR_UNSUPPORTED, "n_blocks %d outside 1..%d", n_blocks, GSA_MAX_BLOCKS);
  if (!blocks_dev || (n_random > 0 && !random_dev)) return fail(GSA_ERR_ARG, "blocks_dev or random_dev is NULL");
  return launch_bigbird(batch, n_blocks, window, n_global, n_random, random_dev, blocks_dev, stream);
}

gsa_status gsa_attn_fwd(const gsa_fwd_args *a, const gsa_mask *m, hipStream_t stream) {
  clear_error();
  gsa_status st = check_fwd(a, m);
  if (st != GSA_OK) return st;
  if (a->batch == 0 || a->seq_len == 0 || a->heads == 0) return GSA_OK;
  return launch_attn_fwd(*a, *m, stream);
}

static gsa_status attn_bwd_stages(const gsa_bwd_args *a, const gsa_mask *m, hipStream_t stream, int stages) {
  clear_error();
  if (!a) return fail(GSA_ERR_ARG, "args is NULL");
  gsa_status st = check_fwd(&a->f, m);
  if (st != GSA_OK) return st;
  if (a->f.batch == 0 || a->f.seq_len == 0 || a->f.heads == 0) return GSA_OK;
  if (!a->f.lse || !a->dout || !a->dq || !a->dk || !a->dv || !a->workspace)
    return fail(GSA_ERR_ARG, "lse/dout/dq/dk/dv/workspace is NULL");
  if (!aligned16(a->dout) || !aligned16(a->dq) || !aligned16(a->dk) || !aligned16(a->dv) ||
      !aligned16(a->workspace))
    return fail(GSA_ERR_ARG, "dout/dq/dk/dv/workspace must be 16-byte aligned");
  return launch_attn_bwd(*a, *m, stream, stages);
}

gsa_status gsa_attn_bwd(const gsa_bwd_args *a, const gsa_mask *m, hipStream_t stream) {
  return attn_bwd_stages(a, m, stream, kBwdAll);
}

gsa_status gsa_attn_bwd_prep(const gsa_bwd_args *a, const gsa_mask *m, hipStream_t stream) {
  return attn_bwd_stages(a, m, stream, kBwdPrep);
}

gsa_status gsa_attn_bwd_dkdv(const gsa_bwd_args *a, const gsa_mask *m, hipStream_t stream) {
  return attn_bwd_stages(a, m, stream, kBwdDkdv);
}

gsa_status gsa_attn_bwd_dq(const gsa_bwd_args *a, const gsa_mask *m, hipStream_t stream) {
  return attn_bwd_stages(a, m, stream, kBwdDq);
}

}  // extern "C"
