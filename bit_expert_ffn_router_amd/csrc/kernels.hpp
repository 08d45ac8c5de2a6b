// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_ext.h>

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

struct DecodeArgs {
  int T, D, F, Fs, E, k, fmt;
  const void* x;
  int x_bf16;       // 1: x is bf16, 0: fp32
  int rmsnorm;      // MOE_FLAG_RMSNORM_INPUT
  const float* logits;
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
};

size_t decode_ws_bytes(int T, int D, int F, int Fs, int E, int k);
DecodeWs decode_ws_carve(void* ws, int T, int D, int F, int Fs, int E, int k);
hipError_t launch_decode(const DecodeArgs& a, const DecodeWs& w, hipStream_t st);

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
  const float* logits;
  const uint8_t* routed;
  size_t stride;
  const uint8_t* shared;
  void* out;
  int out_bf16;
  const uint16_t* router;  // bf16 [E][D] or null: then `logits` is computed first
};
size_t prefill_ws_bytes(int T, int D, int F, int Fs, int E, int k);
hipError_t launch_prefill(const PrefillArgs& a, void* ws, hipStream_t st);

// ---------------------------------------------------------------- slot table
struct SlotEdit {
  int32_t slot, expert, old_expert, pad;
};
constexpr int kSlotEditsPerLaunch = 32;
hipError_t launch_slot_edits(int32_t* slot_of, int32_t* expert_of_slot, const SlotEdit* edits,
                             int n, hipStream_t st);
hipError_t launch_counts_halve(uint32_t* counts, int n, hipStream_t st);
hipError_t launch_slot_init(int32_t* slot_of, int E, int32_t* expert_of_slot, int S,
                            hipStream_t st);

}  // namespace moe
