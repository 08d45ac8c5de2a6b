// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_ext.h>

#include <atomic>

#include "common.hpp"

namespace moe {

// A non-resident (token, rank) pair; same layout as moe_miss in moe.h.
struct MissRec {
  int32_t token, rank, expert;
  float gate;
};

// ---------------------------------------------------------------- timing hook
// Events set by moe_set_kernel_timer, consumed by the next forward call.
struct KernelTimer {
  hipEvent_t before = nullptr, after = nullptr;
};
KernelTimer& kernel_timer();  // the layer's dominant kernel
KernelTimer& router_timer();  // the router projection kernel
KernelTimer& route_event();   // `before` only: recorded once the routing and miss list are written

// Launch `kernel` on st.  When the calling thread has armed the timer `tm`,
// the launch carries its two events (hipExtLaunchKernel), which then take the
// kernel's own start and end timestamps, and the timer is disarmed.  A timed
// launch is refused while st is capturing a graph.
template <typename... P, typename... A>
hipError_t launch_timed_by(KernelTimer& tm, void (*kernel)(P...), dim3 grid, dim3 block,
                           uint32_t lds, hipStream_t st, A... args) {
  static_assert(sizeof...(P) == sizeof...(A), "argument count");
  if (tm.before == nullptr) {
    kernel<<<grid, block, lds, st>>>(args...);
    return hipGetLastError();
  }
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(st, &cs);
  if (e != hipSuccess) return e;
  if (cs != hipStreamCaptureStatusNone) return hipErrorStreamCaptureUnsupported;
  void* argv[] = {(void*)&args...};
  e = hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, lds, st,
                         tm.before, tm.after, 0);
  tm.before = tm.after = nullptr;
  return e;
}
template <typename... P, typename... A>
hipError_t launch_timed(void (*kernel)(P...), dim3 grid, dim3 block, uint32_t lds, hipStream_t st,
                        A... args) {
  return launch_timed_by(kernel_timer(), kernel, grid, block, lds, st, args...);
}

// ---------------------------------------------------------------- LDS limit
// Raise `kernel`'s dynamic-LDS limit on the current device to at least
// `bytes` when a launch needs more than the default 64 KiB (gfx950 has
// 160 KiB per CU).  `cur` remembers, per device, the largest value set;
// two threads that race on a first call may both set it, which is harmless.
constexpr int kMaxDevices = 64;
template <typename K>
hipError_t allow_lds(K kernel, size_t bytes, std::atomic<size_t> (&cur)[kMaxDevices]) {
  if (bytes <= 65536) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (bytes <= cur[dev].load(std::memory_order_acquire)) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess) return e;
  size_t v = cur[dev].load(std::memory_order_relaxed);
  while (v < bytes && !cur[dev].compare_exchange_weak(v, bytes, std::memory_order_acq_rel)) {
  }
  return hipSuccess;
}

// ---------------------------------------------------------------- packing
hipError_t launch_pack(int fmt, int D, int F, int n, const void* codes, const uint16_t* scale,
                       const uint16_t* mins, void* dst, size_t dst_stride, hipStream_t st);
hipError_t launch_unpack(int fmt, int D, int F, int n, const void* src, size_t src_stride,
                         void* codes, uint16_t* scale, uint16_t* mins, hipStream_t st);

// ---------------------------------------------------------------- routing
hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* idx, float* gate,
                        hipStream_t st);

// ---------------------------------------------------------------- permutation
struct PermWs {
  int32_t* chunk_counts;  // [E][nchunks] (expert-major)
  int32_t* totals;        // [E]
  int nchunks;
};
constexpr int kPermChunk = 256;
size_t perm_ws_bytes(int T, int k, int E);
PermWs perm_ws_carve(void* ws, int T, int k, int E);
hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* offsets,
                          int32_t* sorted_pairs, int32_t* inv, const PermWs& w, hipStream_t st);

// ---------------------------------------------------------------- decode path (T <= 4)
constexpr int kDecodeMaxT = 4;

struct DecodeWs {
  int32_t* idx;        // [T*k] routing of the call (written by block 0)
  float* gate;         // [T*k]
  int32_t* nwork;      // [1] listed experts (distinct resident + shared)
  int32_t* work_ref;   // [Wmax] routed index (expert or slot) or -1 = shared
  float* work_gate;    // [Wmax][4] gate of each token for each listed expert
  uint16_t* hh;        // [Wmax][T][Fp] bf16 hi of h
  uint16_t* hl;        // [Wmax][T][Fp] bf16 lo of h
  float2* hs;          // [Wmax][T][Fp/32][2] block sums of h, per 16-row half
  float* rinv;         // [kDecodeMaxT] RMS input factors (2..4 tokens, from the list kernel)
  int Wmax;            // routed work capacity + 1 (shared)
  int Fp;              // padded FFN width of the h rows
};

// The routing outcome of a decode call copied into page-locked host memory
// by the kernel that publishes it (the host half of a slot layer): the miss
// records, their count and the layer input, then `flag` = seq, stored with a
// system-scope release.  flag == NULL: no copy.
struct HostPub {
  MissRec* miss;
  int32_t* count;
  void* x;
  uint32_t* flag;
  uint32_t seq;
};
HostPub& host_pub();  // armed by the caller (thread-local) for its next decode call

struct DecodeArgs {
  int T, D, F, Fs, E, k, fmt;
  const void* x;
  int x_bf16;       // 1: x is bf16, 0: fp32
  int rmsnorm;      // MOE_FLAG_RMSNORM_INPUT
  const float* logits;  // read by the routing (written first by the router, if any)
  const uint8_t* routed;
  size_t stride;
  const int32_t* slot_of;  // NULL = all resident
  int n_slots;             // slots behind `routed` when slot_of != NULL
  const uint8_t* shared;   // NULL = no shared expert
  void* out;
  int out_bf16;
  MissRec* miss;
  int32_t* miss_count;
  uint32_t* use_count;  // NULL, or [E]: +1 per routed pair (slot policy statistics)
  int planned;          // 1: the routing and list are already in the workspace
                        // (decode_plan_kernel); the RMS rule is applied in-block
                        // (one token) or from rms_in (2..4 tokens)
  // Decode stack, 2..4 tokens: rms_out (or NULL) receives, per down block
  // rt (16 output rows) and token t, the sum of squares of the stored
  // outputs at [rt][T]; rms_in holds the previous layer's, from which a
  // planned RMS call takes its factors.
  float* rms_out;
  const float* rms_in;
  HostPub pub;
};

size_t decode_ws_bytes(int T, int D, int F, int Fs, int E, int k);

// Static per-device scratch of moe_layer_forward_noalloc (noalloc.hip): the
// decode workspace of the largest decode request (4 tokens, top-32, d_ff
// 512) is about 1.2 MiB.
constexpr size_t kNoAllocScratchBytes = (size_t)2 << 20;
// Device address of the current device's scratch (looked up once per device).
hipError_t noalloc_scratch(void** ptr);
DecodeWs decode_ws_carve(void* ws, int T, int D, int F, int Fs, int E, int k);
hipError_t launch_decode(const DecodeArgs& a, const DecodeWs& w, hipStream_t st);

// Decode through a stack of layers whose logits are all known up front: one
// launch routes every layer (decode_plan_kernel), then each layer runs its
// gate/up and down kernels on its precomputed list.  Per layer the
// workspace holds a plan area (routing, list, gates); the h buffers are
// shared by the layers.
constexpr int kPlanLayers = 64;  // layers per plan launch (kernel-argument size)
struct PlanArgs {
  int T, E, k, n;                // n: layers of this launch
  const float* logits;           // [n][T][E]
  MissRec* miss;                 // [n][T*k] or NULL (no slot tables)
  int32_t* miss_count;           // [n] or NULL
  uint8_t* plan;                 // [n][plan_bytes]
  size_t plan_bytes;
  const int32_t* slot_of[kPlanLayers];
  uint32_t* use_count[kPlanLayers];
  int n_slots[kPlanLayers];
  int has_shared[kPlanLayers];
};
size_t decode_plan_bytes(int T, int E, int k);
// The plan area of one layer as the routing part of a DecodeWs (idx, gate,
// nwork, work_ref, work_gate); the other fields are left unset.
__host__ __device__ inline void decode_plan_carve(void* plan, int T, int E, int k, DecodeWs& w) {
  const int Wmax = (E < T * k ? E : T * k) + 1;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  uint8_t* q = (uint8_t*)plan;
  w.idx = (int32_t*)q;
  q += al(4 * (size_t)T * k);
  w.gate = (float*)q;
  q += al(4 * (size_t)T * k);
  w.nwork = (int32_t*)q;
  q += 256;
  w.work_ref = (int32_t*)q;
  q += al(4 * (size_t)Wmax);
  w.work_gate = (float*)q;
}
hipError_t launch_decode_plan(const PlanArgs& p, hipStream_t st);

// ---------------------------------------------------------------- host miss path
}  // namespace moe
struct moe_host_pool;
moe_host_pool* moe_host_pool_new(int n_threads);
void moe_host_pool_delete(moe_host_pool* p);
namespace moe {
void host_prepare_x(int T, int D, const void* x, bool x_bf16, bool rms, float* out);
void host_miss_ffn(int D, int F, int fmt, int T, const float* xhat, const MissRec* miss, int nm,
                   const uint8_t* const* experts, float* y, moe_host_pool* pool);
hipError_t launch_add_rows(void* out, int out_bf16, const float* y, size_t n, hipStream_t st);
const char* host_simd_name();  // "avx512", "avx2" or "sse2"

// ---------------------------------------------------------------- router projection
struct RouterArgs {
  int T, D, E;
  const void* x;
  int x_bf16;
  int rmsnorm;
  const uint16_t* w;  // bf16 [E][D]
  float* logits;      // fp32 [T][E]
};
bool router_uses_gemv(int T, int D);
hipError_t launch_router(const RouterArgs& a, hipStream_t st);

// ---------------------------------------------------------------- prefill path
struct PrefillArgs {
  int T, D, F, Fs, E, k, fmt;
  const void* x;
  int x_bf16;
  int rmsnorm;
  float* logits;           // input, or the router's output when `router` is set
  const uint8_t* routed;
  size_t stride;
  const uint8_t* shared;
  void* out;
  int out_bf16;
  const uint16_t* router;  // bf16 [E][D] or null: then `logits` is computed first
  // slot table (all null without one): expert e at routed + slot_of[e]*stride
  // or not resident (-1); non-resident pairs go to `miss` in (token, rank)
  // order with their number in *miss_count; use_count[e] += routed pairs
  const int32_t* slot_of;
  int n_slots;
  MissRec* miss;
  int32_t* miss_count;
  uint32_t* use_count;
};
size_t prefill_ws_bytes(int T, int D, int F, int Fs, int E, int k);
hipError_t launch_prefill(const PrefillArgs& a, void* ws, hipStream_t st);

// ---------------------------------------------------------------- slot table
struct SlotEdit {
  int32_t slot, expert, old_expert, pad;
};
constexpr int kSlotEditsPerLaunch = 32;
// Applies all n edits (any n): the evictions of every edit first, then the
// installs, in launches of kSlotEditsPerLaunch edits.
hipError_t launch_slot_edits(int32_t* slot_of, int32_t* expert_of_slot, const SlotEdit* edits,
                             int n, hipStream_t st);
hipError_t launch_counts_halve(uint32_t* counts, int n, hipStream_t st);
hipError_t launch_slot_init(int32_t* slot_of, int E, int32_t* expert_of_slot, int S,
                            hipStream_t st);

}  // namespace moe
