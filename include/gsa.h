/*
 * gsa.h - C ABI of the gzip-guided block-sparse causal attention library (libgsa.so),
 * built for AMD Instinct MI355X (gfx950).
 *
 * Method sources (web pages, cited by title and section):
 *   [note]  "Gzip-guided Sparse Attention：用压缩率选择长程内容" (daiwk.github.io reproduction
 *           of arXiv 2607.21752): flowchart under 背景与主要改动; 核心公式 first display
 *           (ratio r_i = |gzip(block i)| / b and literal flag l_i = 1[r_i > mean r]); second
 *           display (M = M^lit U M^local U I intersected with the causal mask); third display
 *           (O(L^2 + N w) edges); 背景与主要改动 (head split 50% local / 25% literal / 25% both,
 *           no fixed global tokens).
 *
 * Notation: B batch, T bytes (= tokens) per sample, b block size in bytes, N = T / b blocks,
 * w window in blocks, H heads, d head dimension, L number of literal blocks of a sample.
 * Head classes: 0 = local (M^local U I), 1 = literal (M^lit U I), 2 = hybrid (all three);
 * heads are ordered by class: [0, n_heads[0]) local, then literal, then hybrid.
 *
 * Conventions shared by every entry point:
 *   - The caller owns every buffer.  The library never allocates device memory and keeps
 *     no state between calls.
 *   - Device work is enqueued on the caller's stream and is asynchronous; nothing
 *     synchronises implicitly.  gsa_prepare is host-only and synchronous.
 *   - Arguments are validated before any HIP call; a rejected call returns its status
 *     and has touched no buffer.  gsa_last_error() then describes the problem.
 *   - A launch failure returns GSA_ERR_HIP; faults inside a kernel surface at the
 *     caller's next synchronisation.  No C++ exception crosses this boundary.
 *   - Empty work (batch == 0 or seq_len == 0) returns GSA_OK and enqueues nothing.
 */
#ifndef GSA_H
#define GSA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GSA_ABI_VERSION 1

typedef enum {
  GSA_OK = 0,
  GSA_ERR_ARG = 1,          /* NULL pointer, negative size, misaligned buffer, head counts */
  GSA_ERR_SHAPE = 2,        /* seq_len % block != 0, or mask shape differs from tensors   */
  GSA_ERR_ZLIB = 3,         /* zlib failed in gsa_prepare                                  */
  GSA_ERR_HIP = 4,          /* a HIP runtime call or kernel launch failed                  */
  GSA_ERR_UNSUPPORTED = 5   /* (dtype, block, head_dim) or N outside the built instances   */
} gsa_status;

typedef enum { GSA_F32 = 0, GSA_BF16 = 1 } gsa_dtype;

enum { GSA_CLASS_LOCAL = 0, GSA_CLASS_LITERAL = 1, GSA_CLASS_HYBRID = 2, GSA_N_CLASSES = 3 };

/* Largest block count per sample gsa_build_mask accepts (a sample's flags, ranks and
 * list starts are formed inside one 1024-thread workgroup). */
#define GSA_MAX_BLOCKS 1024

/* Short name of a status code; never NULL. */
const char *gsa_status_str(int32_t status);

/* Detail of the last failure on the calling thread ("" if none); valid until the next
 * library call on this thread. */
const char *gsa_last_error(void);

/* zlibVersion() of the libz this library is linked against. */
const char *gsa_zlib_version(void);

/* GSA_ABI_VERSION this library was built with. */
int32_t gsa_abi_version(void);

/* ------------------------------------------------------------------------------------
 * (1) Host stage: per-block gzip level-1 compressed lengths.
 *     [note] flowchart (fixed-size blocks, gzip level 1 per block) and 核心公式 first
 *     display (|gzip(x_{ib:(i+1)b})|).
 *
 *   bytes     host, uint8 [batch, seq_len] row-major; sample s, block i is
 *             bytes[s*seq_len + i*block, ... + block) (0-based, half-open).
 *   c_out     host, int32 [batch, seq_len/block] row-major: c_out[s*N + i] = size in bytes
 *             of the whole gzip member (10-byte header, deflate body, 8-byte trailer)
 *             produced by zlib deflate at level 1, windowBits 15 (+16: gzip wrapper),
 *             memLevel 8, default strategy.
 *   n_threads host worker threads; <= 0 uses every online core.
 * Errors: NULL pointers or batch/seq_len < 0 or block <= 0 -> GSA_ERR_ARG;
 *         seq_len % block != 0 -> GSA_ERR_SHAPE; any zlib failure -> GSA_ERR_ZLIB.
 * Synchronous; touches no device.
 * ------------------------------------------------------------------------------------ */
gsa_status gsa_prepare(const uint8_t *bytes, int64_t batch, int64_t seq_len, int32_t block,
                       int32_t n_threads, int32_t *c_out);

/* ------------------------------------------------------------------------------------
 * (1b) Host-stage pipeline: the same sizes as gsa_prepare from a persistent pool of
 *      deflate workers, computed asynchronously so that the next batch's sizes can be
 *      prepared while the device runs the current batch ([note] flowchart: the gzip
 *      stage comes before everything else on the path).
 *
 *   gsa_prep_pool_create   starts n_threads workers (<= 0: every online core); *pool
 *                          receives the handle (NULL on failure).
 *   gsa_prep_pool_submit   waits until the previous batch is done, then starts this one
 *                          and returns at once.  Arguments as for gsa_prepare; `bytes` and
 *                          `c_out` must stay valid until the batch is done.  If the
 *                          previous batch failed, returns its error and starts nothing.
 *   gsa_prep_pool_wait     blocks until the current batch is done; returns its status
 *                          (GSA_OK if nothing was submitted).
 *   gsa_prep_pool_destroy  waits for the current batch, stops the workers and frees the
 *                          pool (NULL is a no-op).
 * c_out equals gsa_prepare's output byte for byte.  One pool serves one caller thread at
 * a time.  Errors: as gsa_prepare (synchronous ones from submit, zlib failures from the
 * next wait or submit); NULL pool -> GSA_ERR_ARG.
 * ------------------------------------------------------------------------------------ */
typedef struct gsa_prep_pool gsa_prep_pool;
gsa_status gsa_prep_pool_create(int32_t n_threads, gsa_prep_pool **pool);
gsa_status gsa_prep_pool_submit(gsa_prep_pool *pool, const uint8_t *bytes, int64_t batch, int64_t seq_len,
                                int32_t block, int32_t *c_out);
gsa_status gsa_prep_pool_wait(gsa_prep_pool *pool);
gsa_status gsa_prep_pool_destroy(gsa_prep_pool *pool);

/* ------------------------------------------------------------------------------------
 * (2) Mask: literal flags and per-class block lists.
 *     [note] 核心公式 first display (l_i = 1[r_i > mean r], evaluated exactly as the
 *     integer test N * c_i > sum_j c_j of the sample), second display (the mask
 *     sets and the causal intersection) and 背景与主要改动 (head classes).
 *
 * Device buffers, all caller-allocated; cap = N (N + 1) / 2 entries per (sample, class):
 *   flags     uint8 [B, N]            1 for literal blocks
 *   n_literal int32 [B]               L per sample
 *   row_ptr   int32 [B, 3, N + 1]     CSR offsets into col_idx's (s, class) segment
 *   col_idx   int32 [B, 3, cap]       kept kv-blocks j of each query block i, ascending
 *   col_ptr   int32 [B, 3, N + 1]     CSC offsets into row_idx's (s, class) segment
 *   row_idx   int32 [B, 3, cap]       query blocks i keeping kv-block j, ascending
 *   n_edges   int64 [B, 3]            kept block pairs per (sample, class)
 *   work_row  int32 [B * H * N, 4]    one descriptor per (s, h, i), in schedule order:
 *                                     (item (s*H + h)*N + i, beg, end, first), where
 *                                     [beg, end) is row i's range in col_idx's (s, class)
 *                                     segment and first = its first entry; sorted by the
 *                                     octave floor(log2 len) + 1 of the row length
 *                                     len = end - beg, largest first, ties in ascending
 *                                     item (forward and dQ order); 16-byte aligned
 *   work_col  int32 [B * H * N, 4]    the same over CSC columns and row_idx (dK/dV order)
 *   sched     int32 [2*3*B*(N+32)]    scratch of the work-order construction, 16-byte
 *                                     aligned (contents unspecified after the call)
 * Entries of col_idx/row_idx past a segment's total are left untouched.
 * ------------------------------------------------------------------------------------ */
typedef struct {
  int64_t batch;
  int32_t n_blocks;            /* N, 1 .. GSA_MAX_BLOCKS                                   */
  int32_t window;              /* w >= 0, in blocks                                        */
  int32_t n_heads[3];          /* heads per class (local, literal, hybrid), each >= 0       */
  uint8_t *flags;
  int32_t *n_literal;
  int32_t *row_ptr;
  int32_t *col_idx;
  int32_t *col_ptr;
  int32_t *row_idx;
  int64_t *n_edges;
  int32_t *work_row;
  int32_t *work_col;
  int32_t *sched;
} gsa_mask;

#define GSA_MASK_NBUF 10

/* Byte sizes of the GSA_MASK_NBUF mask buffers, in the struct's field order (flags ..
 * sched), for a caller that allocates them.  The work list is two descriptor arrays
 * (rows for the forward and dQ, columns for dK/dV) plus the sched scratch that builds
 * them, hence ten buffers.
 * Errors: NULL n_heads/sizes_out, negative batch, n_blocks or head count -> GSA_ERR_ARG. */
gsa_status gsa_mask_bytes(int64_t batch, int32_t n_blocks, const int32_t n_heads[3],
                          size_t sizes_out[GSA_MASK_NBUF]);
/* The same as gsa_mask_bytes (earlier name, kept for existing callers). */
gsa_status gsa_mask_sizes(int64_t batch, int32_t n_blocks, const int32_t n_heads[3],
                          size_t sizes_out[GSA_MASK_NBUF]);

/* Default head split of [note] 背景与主要改动: half of the heads local, a quarter
 * literal, the rest hybrid, i.e. (floor(H/2), floor(H/4), H - floor(H/2) - floor(H/4));
 * for H = 4, 12, 16 this is (2,1,1), (6,3,3), (8,4,4).  Callers may pass any other
 * split to the mask and attention calls.
 * Errors: heads < 0 or NULL n_heads_out -> GSA_ERR_ARG. */
gsa_status gsa_default_head_counts(int32_t heads, int32_t n_heads_out[3]);

/* Fills every buffer of *m from c_dev (device, int32 [B, N], lengths from gsa_prepare).
 * Errors: NULL pointers, window < 0, negative head counts -> GSA_ERR_ARG;
 *         N outside 1 .. GSA_MAX_BLOCKS -> GSA_ERR_UNSUPPORTED. */
gsa_status gsa_build_mask(const int32_t *c_dev, const gsa_mask *m, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * (2') gsa_build_mask for callers that cannot allocate device memory (code under HIP graph
 *      capture, tight serving loops, harnesses that forbid allocation).
 *
 *   Same arguments, outputs and errors as gsa_build_mask, except that m->sched is not
 *   used (it may be NULL): the work-order scratch lives in a library-owned device array
 *   of GSA_NOALLOC_SCHED_BYTES, one per GPU, placed when the library is loaded and held
 *   until the process ends.  The call allocates nothing (no hipMalloc, no allocating
 *   library routine); the first call on a device looks the array's address up once.
 *   Every call on one GPU shares that array and leaves its last contents there; calls
 *   that overlap on one GPU (concurrent streams or host threads) race on it.
 * Extra error: a batch whose scratch (2 * 3 * batch * (N + 32) int32 words) exceeds
 * GSA_NOALLOC_SCHED_BYTES -> GSA_ERR_UNSUPPORTED, before anything is enqueued.
 * ------------------------------------------------------------------------------------ */
#define GSA_NOALLOC_SCHED_BYTES (2u << 20)
gsa_status gsa_build_mask_noalloc(const int32_t *c_dev, const gsa_mask *m, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * (2b) Lists of a caller-given block mask, for comparisons with other block-sparse
 *      patterns through the same attention kernels (the pages compare the method with
 *      BigBird: [note] 论文离线与线上效果).
 *
 *   blocks_dev  device, uint8 [B, 3, N, N]: nonzero (s, k, i, j) = query block i of class
 *               k keeps kv-block j.  Entries with j > i are ignored and (i, i) is always
 *               kept (causal blocks, as for the gzip mask).
 *   m           as for gsa_build_mask (same buffers and sizes); flags and n_literal are
 *               set to zero, the lists, counts and work descriptors follow the mask.
 * Errors as gsa_build_mask; NULL blocks_dev -> GSA_ERR_ARG.  Asynchronous on `stream`.
 * ------------------------------------------------------------------------------------ */
gsa_status gsa_build_mask_from_blocks(const uint8_t *blocks_dev, const gsa_mask *m, hipStream_t stream);

/* BigBird-style fixed block mask (causal form) into class 0 of blocks_dev u8 [B, 3, N, N];
 * classes 1 and 2 get the diagonal only.  Query block i keeps j <= i when i - j <= window,
 * j < n_global, i < n_global, or j is one of the n_random entries random_dev[s, i, :]
 * (device int32 [B, N, n_random], each in 0..i; drawn by the caller).  The pages do not
 * give BigBird's parameters; callers choose them.
 * Errors: negative batch/window/n_global/n_random -> GSA_ERR_ARG; N outside
 * 1..GSA_MAX_BLOCKS -> GSA_ERR_UNSUPPORTED; NULL buffers -> GSA_ERR_ARG. */
gsa_status gsa_bigbird_blocks(int64_t batch, int32_t n_blocks, int32_t window, int32_t n_global,
                              int32_t n_random, const int32_t *random_dev, uint8_t *blocks_dev,
                              hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * (3) Forward: O = softmax(scale Q K^T restricted to the kept set) V per head.
 *     [note] 核心公式 second display: head h of class k(h), query block i attends the
 *     kv-blocks j of its CSR row; inside the diagonal block only keys u <= t are kept;
 *     off-diagonal kept blocks are fully visible.
 *
 *   q, k, v, o  device [B, H, T, d] contiguous, dtype GSA_BF16 or GSA_F32, 16-byte aligned
 *   lse         device fp32 [B, H, T], 16-byte aligned: natural-log sum of exp of the kept
 *               scaled scores; may be NULL when no backward follows
 *   scale       softmax scale; 0 selects 1/sqrt(d)
 * Built instances (dtype, block, head_dim): (F32, 16, 32), (BF16, 64, 64), (BF16, 128, 128).
 * Errors: NULL/misaligned pointers, heads != sum of mask head counts -> GSA_ERR_ARG;
 *         T % block != 0, mask batch or N differing from (B, T / block) -> GSA_ERR_SHAPE;
 *         other instances -> GSA_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------------------ */
typedef struct {
  const void *q;
  const void *k;
  const void *v;
  void *o;
  float *lse;
  int32_t dtype;               /* gsa_dtype */
  int64_t batch;
  int32_t heads;
  int64_t seq_len;
  int32_t head_dim;
  int32_t block;
  float scale;
} gsa_fwd_args;

gsa_status gsa_attn_fwd(const gsa_fwd_args *a, const gsa_mask *m, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * (4) Backward: dQ, dK, dV of sum(O * dO) through the same block lists.
 *     The pages give no backward; this is the softmax-attention gradient restricted to
 *     the kept set of [note] 核心公式 second display: with P the kept softmax,
 *     dV = P^T dO, dP = dO V^T, D = rowsum(dO * O), dS = P * (dP - D),
 *     dQ = scale dS K, dK = scale dS^T Q.
 *
 *   f           forward arguments; f.o and f.lse (required) are read as inputs
 *   dout        device [B, H, T, d], same dtype as q
 *   dq, dk, dv  device [B, H, T, d] outputs, same dtype, 16-byte aligned
 *   workspace   device fp32 [B, H, T] scratch for D, owned by the caller
 * Errors: as gsa_attn_fwd, plus NULL lse/dout/dq/dk/dv/workspace -> GSA_ERR_ARG.
 * ------------------------------------------------------------------------------------ */
typedef struct {
  gsa_fwd_args f;
  const void *dout;
  void *dq;
  void *dk;
  void *dv;
  float *workspace;
} gsa_bwd_args;

gsa_status gsa_attn_bwd(const gsa_bwd_args *a, const gsa_mask *m, hipStream_t stream);

/* Stages of the backward, for callers that time or schedule them separately (same
 * arguments, validation and errors as gsa_attn_bwd):
 *   gsa_attn_bwd_dq    dQ over the CSR row lists; also writes D_t = sum_f dO_tf O_tf of
 *                      every row into a->workspace;
 *   gsa_attn_bwd_dkdv  dK, dV over the CSC column lists; reads D from a->workspace;
 *   gsa_attn_bwd_prep  D alone, for running dK/dV without dQ.
 * gsa_attn_bwd enqueues gsa_attn_bwd_dq, then gsa_attn_bwd_dkdv. */
gsa_status gsa_attn_bwd_prep(const gsa_bwd_args *a, const gsa_mask *m, hipStream_t stream);
gsa_status gsa_attn_bwd_dkdv(const gsa_bwd_args *a, const gsa_mask *m, hipStream_t stream);
gsa_status gsa_attn_bwd_dq(const gsa_bwd_args *a, const gsa_mask *m, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GSA_H */
