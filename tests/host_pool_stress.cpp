// Stress check of the host worker pool (bit_expert_ffn_router_amd/csrc/host_pool.hpp),
// built by tests/test_host_pool_cpu.py with g++, with and without
// -fsanitize=thread.  Jobs alternate between a few items and many, the
// pattern of the host miss path (phase 1: misses x 32 items, phase 2: 192),
// and every item adds into a plain (non-atomic) accumulator: an item run
// twice, or run with another job's function, shows as a wrong count (and,
// under the thread sanitizer, as a data race).
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "host_pool.hpp"

int main(int argc, char** argv) {
  const int threads = argc > 1 ? atoi(argv[1]) : 8;
  const int rounds = argc > 2 ? atoi(argv[2]) : 20000;
  moe_host_pool pool;
  for (int i = 0; i + 1 < threads; ++i) pool.threads.emplace_back([&pool] { pool.worker(); });
  std::vector<long> acc(4096, 0);
  long expect_total = 0;
  int bad = 0;
  for (int r = 0; r < rounds && !bad; ++r) {
    const int n = (r % 2) ? 192 + r % 61 : 1 + r % 5;
    const long tag = r + 1;
    std::vector<long> hit(n, 0);
    pool.run(n, [&acc, &hit, tag](int i) {
      hit[i] += 1;           // plain store: a second run of item i is a race
      acc[i] += tag;
    });
    for (int i = 0; i < n; ++i)
      if (hit[i] != 1) {
        fprintf(stderr, "round %d: item %d ran %ld times\n", r, i, hit[i]);
        bad = 1;
      }
    expect_total += tag * n;
  }
  long total = 0;
  for (long v : acc) total += v;
  if (!bad && total != expect_total) {
    fprintf(stderr, "accumulated %ld, expected %ld\n", total, expect_total);
    bad = 1;
  }
  {
    std::lock_guard<std::mutex> lk(pool.mu);
    pool.stop = true;
  }
  pool.cv.notify_all();
  for (auto& t : pool.threads) t.join();
  printf("%s: %d threads, %d rounds\n", bad ? "FAIL" : "ok", threads, rounds);
  return bad;
}
