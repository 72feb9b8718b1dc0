// Internal declarations shared by the C ABI layer and the kernel translation units.
#pragma once

#include <cstdarg>
#include <cstdint>

#include <hip/hip_runtime_api.h>

#include "gsa.h"

namespace gsa {

// Records a thread-local failure detail and returns `st`.
gsa_status fail(gsa_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the thread-local failure detail.
void clear_error();
// Maps a HIP error after a launch to GSA_ERR_HIP with a detail; GSA_OK otherwise.
gsa_status check_launch(const char *what);

// Kernel launchers (arguments already validated).
gsa_status launch_build_mask(const int32_t *c, const gsa_mask &m, hipStream_t stream);
// gsa_build_mask with the work-order scratch in the library's static device array.
gsa_status launch_build_mask_noalloc(const int32_t *c, const gsa_mask &m, hipStream_t stream);
gsa_status launch_mask_from_blocks(const uint8_t *blocks, const gsa_mask &m, hipStream_t stream);
gsa_status launch_bigbird(int64_t batch, int32_t n, int32_t window, int32_t n_global, int32_t n_random,
                          const int32_t *rnd, uint8_t *blocks, hipStream_t stream);
gsa_status launch_attn_fwd(const gsa_fwd_args &a, const gsa_mask &m, hipStream_t stream);
// Backward stages: bit 0 = D alone, bit 1 = dK/dV (reads D), bit 2 = dQ (writes D);
// enqueued in the order D alone, dQ, dK/dV.
enum : int { kBwdPrep = 1, kBwdDkdv = 2, kBwdDq = 4, kBwdAll = kBwdDq | kBwdDkdv };
gsa_status launch_attn_bwd(const gsa_bwd_args &a, const gsa_mask &m, hipStream_t stream, int stages);
// The 128 x 128 bf16 forward and dQ, built in a translation unit of their own with the
// occupancy-first instruction scheduler (it keeps them within 128 VGPRs, so two
// workgroups share a CU).
gsa_status launch_attn_fwd_wide(const gsa_fwd_args &a, const gsa_mask &m, hipStream_t stream);
gsa_status launch_dq_wide(const gsa_bwd_args &a, const gsa_mask &m, hipStream_t stream);

// Whether a (dtype, block, head_dim) instance is compiled in.
bool attn_instance_built(int32_t dtype, int32_t block, int32_t head_dim);

inline int64_t mask_cap(int32_t n) { return (int64_t)n * (n + 1) / 2; }

// Work-order scratch in the mask's sched buffer (int32 words): per (list, sample, class)
// a histogram and a base over kOrderKeys length keys, then one packed rank/key per block.
constexpr int kOrderKeys = 16;
#if defined(__HIPCC__)
#define GSA_HOST_DEVICE __host__ __device__
#else
#define GSA_HOST_DEVICE
#endif
GSA_HOST_DEVICE inline int64_t sched_words(int64_t batch, int32_t n) {
  return 2 * 3 * batch * ((int64_t)n + 2 * kOrderKeys);
}

}  // namespace gsa
