// Host stage of gzip-guided sparse attention: the compressed size of every fixed
// block, as the flowchart of "Gzip-guided Sparse Attention" (daiwk.github.io
// reproduction note, 背景与主要改动) and the ratio formula of its 核心公式 section
// define it: gzip at level 1 applied to each block x_{ib:(i+1)b} on its own.
//
// Each worker thread owns one deflate stream, initialised once and reset per block
// (a reset costs far less than a fresh init), and compresses a contiguous range of
// (sample, block) pairs into a private output buffer.
//
// gsa_prep_pool_* keeps such workers alive between batches: a submitted batch is split
// into chunks of blocks that the workers claim from an atomic counter, and the caller
// returns at once, so the next batch's sizes can be computed while the device runs the
// current one.
#include <zlib.h>

#include <algorithm>
#include <atomic>
#include <condition_variable>
#include <memory>
#include <mutex>
#include <thread>
#include <vector>

#include "gsa_internal.hpp"

#ifdef GSA_TEST_HOOKS
// Test builds only (the library is never built with GSA_TEST_HOOKS): deflate's
// allocations succeed while a countdown lasts and then fail, so that the zlib error path
// of the host stage can be reached.  gsa_test_fail_zalloc_after(n) lets n more
// allocations succeed; n < 0 switches the failures off.
#include <cstdlib>
static std::atomic<long> g_zalloc_left{-1};
extern "C" void gsa_test_fail_zalloc_after(long n) { g_zalloc_left.store(n); }
static voidpf test_zalloc(voidpf, uInt items, uInt size) {
  long left = g_zalloc_left.load();
  while (left >= 0) {
    if (left == 0) return Z_NULL;
    if (g_zalloc_left.compare_exchange_weak(left, left - 1)) break;
  }
  return calloc(items, size);
}
static void test_zfree(voidpf, voidpf p) { free(p); }
#endif

namespace {

struct BlockDeflater {
  z_stream zs{};
  int init_err = Z_OK;
  std::vector<unsigned char> out;

  explicit BlockDeflater(uLong max_in) {
#ifdef GSA_TEST_HOOKS
    zs.zalloc = test_zalloc;
    zs.zfree = test_zfree;
#endif
    // level 1, deflate, windowBits 15 + 16 (gzip wrapper), memLevel 8, default strategy.
    init_err = deflateInit2(&zs, 1, Z_DEFLATED, 15 + 16, 8, Z_DEFAULT_STRATEGY);
    if (init_err == Z_OK) out.resize(deflateBound(&zs, max_in) + 64);
  }
  ~BlockDeflater() {
    if (init_err == Z_OK) deflateEnd(&zs);
  }
  BlockDeflater(const BlockDeflater &) = delete;
  BlockDeflater &operator=(const BlockDeflater &) = delete;

  // Size of the gzip member of p[0, n), or a negative zlib status on failure.
  int64_t member_size(const unsigned char *p, uInt n) {
    int e = deflateReset(&zs);
    if (e != Z_OK) return e < 0 ? e : Z_STREAM_ERROR;
    zs.next_in = const_cast<Bytef *>(p);
    zs.avail_in = n;
    zs.next_out = out.data();
    zs.avail_out = (uInt)out.size();
    e = deflate(&zs, Z_FINISH);
    if (e != Z_STREAM_END) return e < 0 ? e : Z_BUF_ERROR;
    return (int64_t)zs.total_out;
  }
};

}  // namespace

extern "C" gsa_status gsa_prepare(const uint8_t *bytes, int64_t batch, int64_t seq_len,
                                  int32_t block, int32_t n_threads, int32_t *c_out) {
  using gsa::fail;
  gsa::clear_error();
  if (batch < 0 || seq_len < 0) return fail(GSA_ERR_ARG, "negative batch or seq_len");
  if (block <= 0) return fail(GSA_ERR_ARG, "block %d must be > 0", block);
  if (seq_len % block)
    return fail(GSA_ERR_SHAPE, "seq_len %lld is not a multiple of block %d", (long long)seq_len, block);
  if (batch == 0 || seq_len == 0) return GSA_OK;
  if (!bytes || !c_out) return fail(GSA_ERR_ARG, "bytes or c_out is NULL");

  const int64_t n_blocks = seq_len / block;
  const int64_t total = batch * n_blocks;
  int64_t workers = n_threads > 0 ? n_threads : (int64_t)std::thread::hardware_concurrency();
  workers = std::max<int64_t>(1, std::min<int64_t>(workers, total));

  std::atomic<int> first_err{Z_OK};
  auto run = [&](int64_t lo, int64_t hi) {
    BlockDeflater d((uLong)block);
    if (d.init_err != Z_OK) {
      int expect = Z_OK;
      first_err.compare_exchange_strong(expect, d.init_err);
      return;
    }
    for (int64_t t = lo; t < hi; ++t) {
      if (first_err.load(std::memory_order_relaxed) != Z_OK) return;
      const int64_t s = t / n_blocks, i = t % n_blocks;
      int64_t len = d.member_size(bytes + s * seq_len + i * block, (uInt)block);
      if (len < 0 || len > INT32_MAX) {
        int expect = Z_OK;
        first_err.compare_exchange_strong(expect, len < 0 ? (int)len : Z_BUF_ERROR);
        return;
      }
      c_out[t] = (int32_t)len;
    }
  };

  if (workers == 1) {
    run(0, total);
  } else {
    std::vector<std::thread> pool;
    pool.reserve((size_t)workers);
    for (int64_t w = 0; w < workers; ++w) {
      const int64_t lo = total * w / workers, hi = total * (w + 1) / workers;
      pool.emplace_back(run, lo, hi);
    }
    for (auto &th : pool) th.join();
  }
  const int e = first_err.load();
  if (e != Z_OK) return fail(GSA_ERR_ZLIB, "zlib error %d (%s)", e, zError(e));
  return GSA_OK;
}

// ---------------------------------------------------------------------------------------
// Persistent pool.
// ---------------------------------------------------------------------------------------
struct gsa_prep_pool {
  std::vector<std::thread> threads;
  std::mutex mu;
  std::condition_variable cv_job, cv_done;
  // Current job (valid while busy).
  const uint8_t *bytes = nullptr;
  int64_t seq_len = 0, n_blocks = 0, total = 0;
  int32_t block = 0;
  int32_t *c_out = nullptr;
  std::atomic<int64_t> next{0};
  std::atomic<int> err{Z_OK};
  uint64_t generation = 0;
  int active = 0;
  bool busy = false, stop = false;
  int last_err = Z_OK;   // status of the last finished job
};

namespace {

constexpr int64_t kPoolChunk = 16;   // blocks claimed per step

void pool_worker(gsa_prep_pool *p) {
  std::unique_ptr<BlockDeflater> d;
  int32_t d_block = 0;
  uint64_t seen = 0;
  for (;;) {
    {
      std::unique_lock<std::mutex> lock(p->mu);
      p->cv_job.wait(lock, [&] { return p->stop || p->generation != seen; });
      if (p->stop) return;
      seen = p->generation;
    }
    if (!d || d_block < p->block) {
      d.reset(new BlockDeflater((uLong)p->block));
      d_block = p->block;
    }
    if (d->init_err != Z_OK) {
      int expect = Z_OK;
      p->err.compare_exchange_strong(expect, d->init_err);
      d.reset();
      d_block = 0;
    } else {
      for (;;) {
        const int64_t lo = p->next.fetch_add(kPoolChunk);
        if (lo >= p->total || p->err.load(std::memory_order_relaxed) != Z_OK) break;
        const int64_t hi = std::min(lo + kPoolChunk, p->total);
        for (int64_t t = lo; t < hi; ++t) {
          const int64_t s = t / p->n_blocks, i = t % p->n_blocks;
          const int64_t len = d->member_size(p->bytes + s * p->seq_len + i * p->block, (uInt)p->block);
          if (len < 0 || len > INT32_MAX) {
            int expect = Z_OK;
            p->err.compare_exchange_strong(expect, len < 0 ? (int)len : Z_BUF_ERROR);
            break;
          }
          p->c_out[t] = (int32_t)len;
        }
      }
    }
    std::lock_guard<std::mutex> lock(p->mu);
    if (--p->active == 0) {
      p->busy = false;
      p->last_err = p->err.load();
      p->cv_done.notify_all();
    }
  }
}

gsa_status pool_status(int e) {
  if (e != Z_OK) return gsa::fail(GSA_ERR_ZLIB, "zlib error %d (%s)", e, zError(e));
  return GSA_OK;
}

}  // namespace

extern "C" gsa_status gsa_prep_pool_create(int32_t n_threads, gsa_prep_pool **pool) {
  gsa::clear_error();
  if (!pool) return gsa::fail(GSA_ERR_ARG, "pool is NULL");
  *pool = nullptr;
  int64_t workers = n_threads > 0 ? n_threads : (int64_t)std::thread::hardware_concurrency();
  workers = std::max<int64_t>(1, std::min<int64_t>(workers, 1024));
  gsa_prep_pool *p = new (std::nothrow) gsa_prep_pool;
  if (!p) return gsa::fail(GSA_ERR_ARG, "out of host memory");
  try {
    for (int64_t w = 0; w < workers; ++w) p->threads.emplace_back(pool_worker, p);
  } catch (...) {
    {
      std::lock_guard<std::mutex> lock(p->mu);
      p->stop = true;
    }
    p->cv_job.notify_all();
    for (auto &th : p->threads) th.join();
    delete p;
    return gsa::fail(GSA_ERR_ARG, "could not start %lld worker threads", (long long)workers);
  }
  *pool = p;
  return GSA_OK;
}

extern "C" gsa_status gsa_prep_pool_submit(gsa_prep_pool *p, const uint8_t *bytes, int64_t batch,
                                           int64_t seq_len, int32_t block, int32_t *c_out) {
  using gsa::fail;
  gsa::clear_error();
  if (!p) return fail(GSA_ERR_ARG, "pool is NULL");
  if (batch < 0 || seq_len < 0) return fail(GSA_ERR_ARG, "negative batch or seq_len");
  if (block <= 0) return fail(GSA_ERR_ARG, "block %d must be > 0", block);
  if (seq_len % block)
    return fail(GSA_ERR_SHAPE, "seq_len %lld is not a multiple of block %d", (long long)seq_len, block);
  if (batch > 0 && seq_len > 0 && (!bytes || !c_out)) return fail(GSA_ERR_ARG, "bytes or c_out is NULL");
  std::unique_lock<std::mutex> lock(p->mu);
  p->cv_done.wait(lock, [&] { return !p->busy; });
  if (p->last_err != Z_OK) {
    const int e = p->last_err;
    p->last_err = Z_OK;
    return pool_status(e);
  }
  if (batch == 0 || seq_len == 0) return GSA_OK;
  p->bytes = bytes;
  p->seq_len = seq_len;
  p->block = block;
  p->n_blocks = seq_len / block;
  p->total = batch * p->n_blocks;
  p->c_out = c_out;
  p->next.store(0);
  p->err.store(Z_OK);
  p->active = (int)p->threads.size();
  p->busy = true;
  ++p->generation;
  p->cv_job.notify_all();
  return GSA_OK;
}

extern "C" gsa_status gsa_prep_pool_wait(gsa_prep_pool *p) {
  gsa::clear_error();
  if (!p) return gsa::fail(GSA_ERR_ARG, "pool is NULL");
  std::unique_lock<std::mutex> lock(p->mu);
  p->cv_done.wait(lock, [&] { return !p->busy; });
  const int e = p->last_err;
  p->last_err = Z_OK;
  return pool_status(e);
}

extern "C" gsa_status gsa_prep_pool_destroy(gsa_prep_pool *p) {
  gsa::clear_error();
  if (!p) return GSA_OK;
  {
    std::unique_lock<std::mutex> lock(p->mu);
    p->cv_done.wait(lock, [&] { return !p->busy; });
    p->stop = true;
  }
  p->cv_job.notify_all();
  for (auto &th : p->threads) th.join();
  delete p;
  return GSA_OK;
}
