// Caller-owned pool of host worker threads for the CPU half of the slot-mode
// layer (see moe_host_pool_create in moe.h).  Plain C++: no HIP types, so a
// host-only build (the thread-sanitizer stress test) can include it.
//
// A layer call runs two short parallel phases, so waking sleeping threads
// would cost more than the work: workers poll for a new job for a while
// (kSpin polls with a pause instruction between them, a few milliseconds:
// longer than the GPU half of a layer between two host phases) before they
// sleep on the condition variable, and the caller waits for the items, not
// for every worker.  Items are claimed by
// compare-and-swap on one word, (generation << 32 | next item).
//
// Publication order of a job (run): first the word moves to the new
// generation with its item index exhausted, which closes every claim a late
// worker of an older generation could still attempt (its compare-and-swap
// expects its own generation); only then are the job, its item count and the
// done counter written; then the word opens item 0 and the generation is
// announced.  A worker therefore reads a job and its item count only after
// it has seen that job's generation, and never runs an item of one job with
// the count or function of another.
#pragma once

#include <atomic>
#include <condition_variable>
#include <cstdint>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

struct moe_host_pool {
  static constexpr int kSpin = 1 << 16;         // polls of the generation before sleeping
  static constexpr uint32_t kClosed = 0xFFFFFFFFu;  // item index of a generation not yet open
  std::vector<std::thread> threads;
  std::mutex mu;
  std::condition_variable cv;
  std::function<void(int)> job;        // written only while no item can be claimed
  std::atomic<uint64_t> state{0};      // generation << 32 | next item
  std::atomic<uint32_t> n_items{0};
  std::atomic<uint32_t> done{0};
  std::atomic<uint32_t> gen{0};
  bool stop = false;                   // under mu

  // Claims and runs items of generation g until none is left.  Called only
  // after gen == g was read (acquire), so n_items and job are g's.
  void drain(uint32_t g) {
    const uint32_t n = n_items.load(std::memory_order_acquire);
    uint64_t v = state.load(std::memory_order_acquire);
    for (;;) {
      if ((uint32_t)(v >> 32) != g || (uint32_t)v >= n) return;
      if (state.compare_exchange_weak(v, v + 1, std::memory_order_acq_rel,
                                      std::memory_order_acquire)) {
        job((int)(uint32_t)v);
        done.fetch_add(1, std::memory_order_release);
        v = state.load(std::memory_order_acquire);
      }
    }
  }
  void worker() {
    uint32_t seen = 0;
    for (;;) {
      uint32_t g;
      int polls = 0;
      while ((g = gen.load(std::memory_order_acquire)) == seen) {
        if (++polls < kSpin) {
#if defined(__x86_64__)
          __builtin_ia32_pause();  // yields the core's issue slots while polling
#endif
          continue;
        }
        std::unique_lock<std::mutex> lk(mu);
        cv.wait(lk, [&] { return stop || gen.load(std::memory_order_acquire) != seen; });
        if (stop) return;
        polls = 0;
      }
      seen = g;
      drain(g);
    }
  }
  // Items 0..n-1 of fn over the workers and the calling thread; returns when
  // all are done.  Items must write disjoint outputs.  One run at a time.
  void run(int n, std::function<void(int)> fn) {
    if (threads.empty() || n <= 0) {
      for (int i = 0; i < n; ++i) fn(i);
      return;
    }
    const uint32_t g = gen.load(std::memory_order_relaxed) + 1;
    // 1. close: late workers of older generations can no longer claim.
    state.store((uint64_t)g << 32 | kClosed, std::memory_order_seq_cst);
    // 2. the job itself.
    job = std::move(fn);
    done.store(0, std::memory_order_relaxed);
    n_items.store((uint32_t)n, std::memory_order_release);
    // 3. open item 0, then announce the generation.
    state.store((uint64_t)g << 32, std::memory_order_release);
    {
      std::lock_guard<std::mutex> lk(mu);  // a worker about to sleep sees g or is woken
      gen.store(g, std::memory_order_release);
    }
    cv.notify_all();
    drain(g);
    while (done.load(std::memory_order_acquire) < (uint32_t)n) {
    }
  }
};
