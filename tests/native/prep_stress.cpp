// Stress driver of the host gzip stage for the CPU sanitizer builds (ThreadSanitizer,
// AddressSanitizer + UndefinedBehaviorSanitizer): gsa_prepare at several thread counts,
// the persistent pool with back-to-back (overlapping) submits whose block size changes
// between batches, destroy while a batch runs, and the zlib failure path reached through
// the test-only allocator hook.  Prints "OK" and exits 0 when every check holds.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "gsa.h"

extern "C" void gsa_test_fail_zalloc_after(long n);

static int g_fail = 0;
#define CHECK(cond)                                                          \
  do {                                                                       \
    if (!(cond)) {                                                           \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++g_fail;                                                              \
    }                                                                        \
  } while (0)

static std::vector<uint8_t> make_bytes(int64_t batch, int64_t seq, unsigned seed) {
  std::mt19937 rng(seed);
  std::vector<uint8_t> x((size_t)(batch * seq));
  // alternating runs of random bytes and of a repeated letter, so sizes vary per block
  size_t pos = 0;
  bool random_run = true;
  while (pos < x.size()) {
    size_t n = 16 + rng() % 200;
    for (size_t t = 0; t < n && pos < x.size(); ++t, ++pos)
      x[pos] = random_run ? (uint8_t)(rng() & 255) : (uint8_t)('a' + (rng() % 3 == 0 ? rng() % 26 : 4));
    random_run = !random_run;
  }
  return x;
}

static std::vector<int32_t> serial_sizes(const std::vector<uint8_t> &x, int64_t batch, int64_t seq, int32_t block) {
  std::vector<int32_t> c((size_t)(batch * (seq / block)), -1);
  CHECK(gsa_prepare(x.data(), batch, seq, block, 1, c.data()) == GSA_OK);
  return c;
}

int main() {
  const int64_t batch = 6, seq = 8192;
  const int32_t blocks[3] = {64, 128, 16};
  std::vector<uint8_t> xs[3];
  std::vector<int32_t> refs[3];
  for (int v = 0; v < 3; ++v) {
    xs[v] = make_bytes(batch, seq, 11u + v);
    refs[v] = serial_sizes(xs[v], batch, seq, blocks[v]);
  }
  // gsa_prepare at several thread counts equals the one-thread result.
  for (int threads : {2, 3, 8, 0}) {
    for (int v = 0; v < 3; ++v) {
      std::vector<int32_t> c(refs[v].size(), -1);
      CHECK(gsa_prepare(xs[v].data(), batch, seq, blocks[v], threads, c.data()) == GSA_OK);
      CHECK(c == refs[v]);
    }
  }
  // Pool: back-to-back submits into two alternating output buffers; every batch is
  // checked after the next one has been started (submit waits for the previous batch).
  {
    gsa_prep_pool *pool = nullptr;
    CHECK(gsa_prep_pool_create(4, &pool) == GSA_OK && pool);
    std::vector<int32_t> out[2];
    int pending_v = -1, pending_buf = -1;
    for (int k = 0; k < 60; ++k) {
      const int v = k % 3, buf = k % 2;
      out[buf].assign(refs[v].size(), -1);
      CHECK(gsa_prep_pool_submit(pool, xs[v].data(), batch, seq, blocks[v], out[buf].data()) == GSA_OK);
      // the submit above waited for the previous batch, so its buffer is final now
      if (pending_v >= 0) CHECK(out[pending_buf] == refs[pending_v]);
      pending_v = v;
      pending_buf = buf;
    }
    CHECK(gsa_prep_pool_wait(pool) == GSA_OK);
    CHECK(out[pending_buf] == refs[pending_v]);
    // destroy while a batch is running: it waits for the batch
    std::vector<int32_t> last(refs[0].size(), -1);
    CHECK(gsa_prep_pool_submit(pool, xs[0].data(), batch, seq, blocks[0], last.data()) == GSA_OK);
    CHECK(gsa_prep_pool_destroy(pool) == GSA_OK);
    CHECK(last == refs[0]);
  }
  // zlib failures: every deflate allocation fails, then only the third one, then none.
  for (long after : {0L, 2L}) {
    std::vector<int32_t> c(refs[0].size(), -1);
    gsa_test_fail_zalloc_after(after);
    CHECK(gsa_prepare(xs[0].data(), batch, seq, blocks[0], 3, c.data()) == GSA_ERR_ZLIB);
    CHECK(std::strstr(gsa_last_error(), "zlib") != nullptr);
    gsa_test_fail_zalloc_after(-1);
  }
  {
    gsa_prep_pool *pool = nullptr;
    CHECK(gsa_prep_pool_create(3, &pool) == GSA_OK);
    std::vector<int32_t> c(refs[1].size(), -1);
    gsa_test_fail_zalloc_after(1);
    CHECK(gsa_prep_pool_submit(pool, xs[1].data(), batch, seq, blocks[1], c.data()) == GSA_OK);
    CHECK(gsa_prep_pool_wait(pool) == GSA_ERR_ZLIB);
    gsa_test_fail_zalloc_after(-1);
    // the pool recovers: failed workers rebuild their streams on the next batch
    c.assign(refs[1].size(), -1);
    CHECK(gsa_prep_pool_submit(pool, xs[1].data(), batch, seq, blocks[1], c.data()) == GSA_OK);
    CHECK(gsa_prep_pool_wait(pool) == GSA_OK);
    CHECK(c == refs[1]);
    // a failure reported by the next submit instead of a wait
    gsa_test_fail_zalloc_after(0);
    std::vector<int32_t> big(refs[0].size() * 2, -1);
    const std::vector<uint8_t> x2 = make_bytes(batch, 2 * seq, 99u);
    CHECK(gsa_prep_pool_submit(pool, x2.data(), batch, 2 * seq, 256, big.data()) == GSA_OK);
    gsa_status st = gsa_prep_pool_submit(pool, xs[0].data(), batch, seq, blocks[0], c.data());
    CHECK(st == GSA_ERR_ZLIB);
    gsa_test_fail_zalloc_after(-1);
    CHECK(gsa_prep_pool_wait(pool) == GSA_OK);
    CHECK(gsa_prep_pool_destroy(pool) == GSA_OK);
  }
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("OK\n");
  return 0;
}
