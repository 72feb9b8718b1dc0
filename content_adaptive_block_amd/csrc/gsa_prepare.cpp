// Host stage of gzip-guided sparse attention: the compressed size of every fixed
// block, as the flowchart of "Gzip-guided Sparse Attention" (daiwk.github.io
// reproduction note, 背景与主要改动) and the ratio formula of its 核心公式 section
// define it: gzip at level 1 applied to each block x_{ib:(i+1)b} on its own.
//
// Each worker thread owns one deflate stream, initialised once and reset per block
// (a reset costs far less than a fresh init), and compresses a contiguous range of
// (sample, block) pairs into a private output buffer.
#include <zlib.h>

#include <algorithm>
#include <atomic>
#include <thread>
#include <vector>

#include "gsa_internal.hpp"

namespace {

struct BlockDeflater {
  z_stream zs{};
  int init_err = Z_OK;
  std::vector<unsigned char> out;

  explicit BlockDeflater(uLong max_in) {
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
