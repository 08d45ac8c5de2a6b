// C ABI of libmoe: argument validation, workspace sizing and dispatch.
// Every entry point validates on the host, returns a negative status with a
// message (moe_last_error) on a bad call and launches nothing in that case.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <vector>

#include "../../include/moe.h"
#include "kernels.hpp"

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

moe_status ok() {
  g_err[0] = '\0';
  return MOE_OK;
}

moe_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned256(const void* p) { return ((uintptr_t)p & 255u) == 0; }

// Shape checks shared by every entry point.
moe_status check_shape(const moe_shape* s) {
  if (!s) return fail(MOE_EINVAL, "shape is NULL");
  if (s->qfmt != MOE_Q2SM32 && s->qfmt != MOE_Q3S32 && s->qfmt != MOE_Q2S32)
    return fail(MOE_EINVAL, "unknown qfmt %d", (int)s->qfmt);
  if (s->d_model <= 0 || s->d_model % 256 != 0)
    return fail(MOE_EINVAL, "d_model %d must be a positive multiple of 256", (int)s->d_model);
  if (s->d_ff <= 0 || s->d_ff % 32 != 0)
    return fail(MOE_EINVAL, "d_ff %d must be a positive multiple of 32", (int)s->d_ff);
  if (s->d_ff_shared < 0 || s->d_ff_shared % 32 != 0)
    return fail(MOE_EINVAL, "d_ff_shared %d must be a non-negative multiple of 32",
                (int)s->d_ff_shared);
  if (s->n_experts <= 0 || s->n_experts > 2048)
    return fail(MOE_EINVAL, "n_experts %d must be in 1..2048", (int)s->n_experts);
  if (s->top_k < 1 || s->top_k > 32 || s->top_k > s->n_experts)
    return fail(MOE_EINVAL, "top_k %d must be in 1..min(32, n_experts)", (int)s->top_k);
  return ok();
}

bool use_decode_path(int T) { return T <= moe::kDecodeMaxT; }

size_t forward_ws_bytes(const moe_shape* s, int T) {
  if (T <= 0) return 0;
  if (use_decode_path(T))
    return moe::decode_ws_bytes(T, s->d_model, s->d_ff, s->d_ff_shared, s->n_experts, s->top_k);
  return moe::prefill_ws_bytes(T, s->d_model, s->d_ff, s->d_ff_shared, s->n_experts, s->top_k);
}

}  // namespace

namespace moe {

KernelTimer& kernel_timer() {
  thread_local KernelTimer t;
  return t;
}
KernelTimer& router_timer() {
  thread_local KernelTimer t;
  return t;
}
KernelTimer& route_event() {
  thread_local KernelTimer t;
  return t;
}
HostPub& host_pub() {
  thread_local HostPub p = {};
  return p;
}

}  // namespace moe

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

moe_status moe_set_kernel_timer(void* before, void* after) {
  if ((before == nullptr) != (after == nullptr))
    return fail(MOE_EINVAL, "before and after must both be set or both be NULL");
  moe::kernel_timer().before = (hipEvent_t)before;
  moe::kernel_timer().after = (hipEvent_t)after;
  return ok();
}

moe_status moe_set_router_timer(void* before, void* after) {
  if ((before == nullptr) != (after == nullptr))
    return fail(MOE_EINVAL, "before and after must both be set or both be NULL");
  moe::router_timer().before = (hipEvent_t)before;
  moe::router_timer().after = (hipEvent_t)after;
  return ok();
}

moe_status moe_set_route_event(void* event) {
  moe::route_event().before = (hipEvent_t)event;
  return ok();
}

const char* moe_host_simd(void) { return moe::host_simd_name(); }

const char* moe_last_error(void) { return g_err; }

size_t moe_packed_expert_bytes(const moe_shape* shape, int32_t d_ff) {
  if (check_shape(shape) != MOE_OK) return 0;
  if (d_ff <= 0 || d_ff % 32 != 0) return 0;
  return moe::packed_bytes(shape->d_model, d_ff, shape->qfmt);
}

moe_status moe_pack_weights(const moe_shape* shape, int32_t n, int32_t d_ff, const void* codes,
                            const uint16_t* scale, const uint16_t* min, void* dst,
                            size_t dst_stride, moe_stream_t stream) {
  moe_status s = check_shape(shape);
  if (s != MOE_OK) return s;
  if (n < 0) return fail(MOE_EINVAL, "n %d < 0", (int)n);
  if (d_ff <= 0 || d_ff % 32 != 0) return fail(MOE_EINVAL, "d_ff %d must be a multiple of 32", (int)d_ff);
  if (n == 0) return ok();
  if (!codes || !scale || !dst) return fail(MOE_EINVAL, "codes, scale and dst are required");
  if (shape->qfmt == MOE_Q2SM32 && !min) return fail(MOE_EINVAL, "Q2SM needs min");
  const size_t need = moe::packed_bytes(shape->d_model, d_ff, shape->qfmt);
  if (dst_stride < need || dst_stride % 256 != 0)
    return fail(MOE_EINVAL, "dst_stride %zu must be >= %zu and a multiple of 256", dst_stride, need);
  if (!aligned256(dst)) return fail(MOE_EINVAL, "dst must be 256-byte aligned");
  if (((uintptr_t)codes & 7u) || ((uintptr_t)scale & 1u) || (min && ((uintptr_t)min & 1u)))
    return fail(MOE_EINVAL, "codes must be 8-byte aligned, scale/min 2-byte aligned");
  return hip_status(moe::launch_pack(shape->qfmt, shape->d_model, d_ff, n, codes, scale,
                                     shape->qfmt == MOE_Q2SM32 ? min : nullptr, dst, dst_stride,
                                     (hipStream_t)stream),
                    "pack launch");
}

moe_status moe_unpack_weights(const moe_shape* shape, int32_t n, int32_t d_ff, const void* src,
                              size_t src_stride, void* codes, uint16_t* scale, uint16_t* min,
                              moe_stream_t stream) {
  moe_status s = check_shape(shape);
  if (s != MOE_OK) return s;
  if (n < 0) return fail(MOE_EINVAL, "n %d < 0", (int)n);
  if (d_ff <= 0 || d_ff % 32 != 0) return fail(MOE_EINVAL, "d_ff %d must be a multiple of 32", (int)d_ff);
  if (n == 0) return ok();
  if (!src || !codes || !scale) return fail(MOE_EINVAL, "src, codes and scale are required");
  if (shape->qfmt == MOE_Q2SM32 && !min) return fail(MOE_EINVAL, "Q2SM needs min");
  const size_t need = moe::packed_bytes(shape->d_model, d_ff, shape->qfmt);
  if (src_stride < need || src_stride % 256 != 0)
    return fail(MOE_EINVAL, "src_stride %zu must be >= %zu and a multiple of 256", src_stride, need);
  if (!aligned256(src)) return fail(MOE_EINVAL, "src must be 256-byte aligned");
  if (((uintptr_t)codes & 7u) || ((uintptr_t)scale & 1u) || (min && ((uintptr_t)min & 1u)))
    return fail(MOE_EINVAL, "codes must be 8-byte aligned, scale/min 2-byte aligned");
  return hip_status(moe::launch_unpack(shape->qfmt, shape->d_model, d_ff, n, src, src_stride,
                                       codes, scale, min, (hipStream_t)stream),
                    "unpack launch");
}

size_t moe_workspace_bytes(const moe_shape* shape, int32_t tokens) {
  if (check_shape(shape) != MOE_OK || tokens < 0) return 0;
  return forward_ws_bytes(shape, tokens);
}

}  // extern "C"

namespace {

// Checks of one expert table against the shape (shared by the layer and the
// stack entry points).
moe_status check_table(const moe_shape* shape, const moe_expert_table* table) {
  if (!table) return fail(MOE_EINVAL, "table is NULL");
  const size_t need_e = moe::packed_bytes(shape->d_model, shape->d_ff, shape->qfmt);
  if (!table->routed) return fail(MOE_EINVAL, "table->routed is NULL");
  if (table->expert_stride < need_e || table->expert_stride % 256 != 0)
    return fail(MOE_EINVAL, "expert_stride %zu must be >= %zu and a multiple of 256",
                table->expert_stride, need_e);
  if (!aligned256(table->routed)) return fail(MOE_EINVAL, "table->routed must be 256-byte aligned");
  if ((shape->d_ff_shared > 0) != (table->shared != nullptr))
    return fail(MOE_EINVAL, "table->shared must be given iff d_ff_shared > 0");
  if (table->shared && !aligned256(table->shared))
    return fail(MOE_EINVAL, "table->shared must be 256-byte aligned");
  if (table->router && ((uintptr_t)table->router & 15u))
    return fail(MOE_EINVAL, "table->router must be 16-byte aligned");
  if (table->use_count && ((uintptr_t)table->use_count & 3u))
    return fail(MOE_EINVAL, "table->use_count must be 4-byte aligned");
  if (table->slot_of && table->n_slots <= 0)
    return fail(MOE_EINVAL, "n_slots must be > 0 with a slot table");
  return ok();
}

// RMS partials of the stack with 2..4 tokens: two buffers of [d_model/16][T]
// floats, written by layer l's down kernel and read by layer l+1's gate/up.
size_t stack_rms_bytes(const moe_shape* s, int T) {
  return T > 1 ? 2 * (((size_t)(s->d_model / 16) * T * 4 + 255) / 256 * 256) : 0;
}

size_t stack_ws_bytes(const moe_shape* s, int L, int T) {
  if (L <= 0 || T <= 0) return 0;
  const size_t plan = moe::decode_plan_bytes(T, s->n_experts, s->top_k);
  return (size_t)L * plan + stack_rms_bytes(s, T) +
         moe::decode_ws_bytes(T, s->d_model, s->d_ff, s->d_ff_shared, s->n_experts, s->top_k);
}

// The layer call behind both entry points.  ws == nullptr with noalloc:
// the decode path's workspace is the library's per-device static scratch.
moe_status layer_forward_impl(const moe_shape* shape, int32_t tokens, const void* x,
                              int32_t x_dtype, uint32_t flags, float* router_logits,
                              const moe_expert_table* table, void* out, int32_t out_dtype,
                              moe_miss* miss, int32_t miss_cap, int32_t* miss_count, void* ws,
                              size_t ws_bytes, bool noalloc, moe_stream_t stream) {
  moe_status s = check_shape(shape);
  if (s != MOE_OK) return s;
  const int T = tokens;
  if (T < 0) return fail(MOE_EINVAL, "tokens %d < 0", T);
  if (!table) return fail(MOE_EINVAL, "table is NULL");
  if (x_dtype != MOE_BF16 && x_dtype != MOE_F32) return fail(MOE_EINVAL, "bad x_dtype %d", (int)x_dtype);
  if (out_dtype != MOE_BF16 && out_dtype != MOE_F32)
    return fail(MOE_EINVAL, "bad out_dtype %d", (int)out_dtype);
  if (flags & ~(uint32_t)MOE_FLAG_RMSNORM_INPUT) return fail(MOE_EINVAL, "unknown flags 0x%x", flags);
  const size_t need_e = moe::packed_bytes(shape->d_model, shape->d_ff, shape->qfmt);
  if (!table->routed) return fail(MOE_EINVAL, "table->routed is NULL");
  if (table->expert_stride < need_e || table->expert_stride % 256 != 0)
    return fail(MOE_EINVAL, "expert_stride %zu must be >= %zu and a multiple of 256",
                table->expert_stride, need_e);
  if (!aligned256(table->routed)) return fail(MOE_EINVAL, "table->routed must be 256-byte aligned");
  if ((shape->d_ff_shared > 0) != (table->shared != nullptr))
    return fail(MOE_EINVAL, "table->shared must be given iff d_ff_shared > 0");
  if (table->shared && !aligned256(table->shared))
    return fail(MOE_EINVAL, "table->shared must be 256-byte aligned");
  if (table->router && ((uintptr_t)table->router & 15u))
    return fail(MOE_EINVAL, "table->router must be 16-byte aligned");
  if (table->use_count && ((uintptr_t)table->use_count & 3u))
    return fail(MOE_EINVAL, "table->use_count must be 4-byte aligned");
  const bool slots = table->slot_of != nullptr;
  if (slots) {
    if (table->n_slots <= 0) return fail(MOE_EINVAL, "n_slots must be > 0 with a slot table");
    if (!miss || !miss_count) return fail(MOE_EINVAL, "slot mode needs miss and miss_count");
    if ((int64_t)miss_cap < (int64_t)T * shape->top_k)
      return fail(MOE_ENOSPACE, "miss_cap %d < tokens*top_k = %lld", (int)miss_cap,
                  (long long)T * shape->top_k);
  }
  if (noalloc && !use_decode_path(T))
    return fail(MOE_EUNSUPPORTED,
                "moe_layer_forward_noalloc runs the decode path only (tokens <= %d), got %d",
                moe::kDecodeMaxT, T);
  if (T == 0) return ok();
  if (!x || !router_logits || !out) return fail(MOE_EINVAL, "x, router_logits and out are required");
  if (((uintptr_t)x & 15u) || ((uintptr_t)router_logits & 3u) || ((uintptr_t)out & 15u))
    return fail(MOE_EINVAL, "x and out must be 16-byte aligned, router_logits 4-byte aligned");
  const size_t need_ws = forward_ws_bytes(shape, T);
  if (noalloc) {
    if (need_ws > moe::kNoAllocScratchBytes)
      return fail(MOE_ENOSPACE, "workspace of %zu bytes exceeds the static scratch (%zu bytes)",
                  need_ws, moe::kNoAllocScratchBytes);
    moe_status ss = hip_status(moe::noalloc_scratch(&ws), "static scratch address");
    if (ss != MOE_OK) return ss;
    ws_bytes = moe::kNoAllocScratchBytes;
  }
  if (!ws) return fail(MOE_EINVAL, "ws is required");
  if (!aligned256(ws)) return fail(MOE_EINVAL, "ws must be 256-byte aligned");
  if (ws_bytes < need_ws) return fail(MOE_ENOSPACE, "ws_bytes %zu < %zu", ws_bytes, need_ws);
  if (use_decode_path(T)) {
    if (shape->d_model > 4096 || shape->d_ff > 512 || shape->d_ff_shared > 512)
      return fail(MOE_EUNSUPPORTED, "decode path supports d_model <= 4096, d_ff <= 512");
    moe::DecodeArgs a = {};
    a.T = T;
    a.D = shape->d_model;
    a.F = shape->d_ff;
    a.Fs = shape->d_ff_shared;
    a.E = shape->n_experts;
    a.k = shape->top_k;
    a.fmt = shape->qfmt;
    a.x = x;
    a.x_bf16 = x_dtype == MOE_BF16;
    a.rmsnorm = (flags & MOE_FLAG_RMSNORM_INPUT) != 0;
    a.logits = router_logits;
    a.routed = (const uint8_t*)table->routed;
    a.stride = table->expert_stride;
    a.slot_of = table->slot_of;
    a.n_slots = table->n_slots;
    a.shared = (const uint8_t*)table->shared;
    a.out = out;
    a.out_bf16 = out_dtype == MOE_BF16;
    a.miss = (moe::MissRec*)miss;
    a.miss_count = miss_count;
    a.use_count = slots ? table->use_count : nullptr;
    if (slots) {  // an armed copy of the routing outcome to the host (taken once)
      a.pub = moe::host_pub();
      moe::host_pub() = {};
    }
    const moe::DecodeWs w = moe::decode_ws_carve(ws, T, a.D, a.F, a.Fs, a.E, a.k);
    if (table->router) {
      moe::RouterArgs r{T, a.D, a.E, x, a.x_bf16, a.rmsnorm, (const uint16_t*)table->router,
                        router_logits};
      moe_status rs = hip_status(moe::launch_router(r, (hipStream_t)stream), "router launch");
      if (rs != MOE_OK) return rs;
    }
    return hip_status(moe::launch_decode(a, w, (hipStream_t)stream), "decode launch");
  }
  moe::PrefillArgs a = {};
  a.T = T;
  a.D = shape->d_model;
  a.F = shape->d_ff;
  a.Fs = shape->d_ff_shared;
  a.E = shape->n_experts;
  a.k = shape->top_k;
  a.fmt = shape->qfmt;
  a.x = x;
  a.x_bf16 = x_dtype == MOE_BF16;
  a.rmsnorm = (flags & MOE_FLAG_RMSNORM_INPUT) != 0;
  a.logits = router_logits;
  a.routed = (const uint8_t*)table->routed;
  a.stride = table->expert_stride;
  a.shared = (const uint8_t*)table->shared;
  a.out = out;
  a.out_bf16 = out_dtype == MOE_BF16;
  a.router = (const uint16_t*)table->router;
  a.slot_of = slots ? table->slot_of : nullptr;
  a.n_slots = slots ? table->n_slots : 0;
  a.miss = slots ? (moe::MissRec*)miss : nullptr;
  a.miss_count = slots ? miss_count : nullptr;
  a.use_count = slots ? table->use_count : nullptr;
  return hip_status(moe::launch_prefill(a, ws, (hipStream_t)stream), "prefill launch");
}

}  // namespace

extern "C" {

moe_status moe_layer_forward(const moe_shape* shape, int32_t tokens, const void* x,
                             int32_t x_dtype, uint32_t flags, float* router_logits,
                             const moe_expert_table* table, void* out, int32_t out_dtype,
                             moe_miss* miss, int32_t miss_cap, int32_t* miss_count, void* ws,
                             size_t ws_bytes, moe_stream_t stream) {
  return layer_forward_impl(shape, tokens, x, x_dtype, flags, router_logits, table, out, out_dtype,
                            miss, miss_cap, miss_count, ws, ws_bytes, false, stream);
}

size_t moe_decode_stack_workspace_bytes(const moe_shape* shape, int32_t layers, int32_t tokens) {
  if (check_shape(shape) != MOE_OK || layers < 0 || tokens < 0 || tokens > moe::kDecodeMaxT)
    return 0;
  return stack_ws_bytes(shape, layers, tokens);
}

moe_status moe_decode_stack_forward(const moe_shape* shape, int32_t layers, int32_t tokens,
                                    const void* x, int32_t x_dtype, const float* logits,
                                    const moe_expert_table* tables, void* out, int32_t out_dtype,
                                    moe_miss* miss, int32_t* miss_count, void* ws,
                                    size_t ws_bytes, moe_stream_t stream) {
  moe_status s = check_shape(shape);
  if (s != MOE_OK) return s;
  const int L = layers, T = tokens;
  if (L < 0 || T < 0) return fail(MOE_EINVAL, "layers %d and tokens %d must be >= 0", L, T);
  if (T > moe::kDecodeMaxT)
    return fail(MOE_EUNSUPPORTED, "the stack runs the decode path: tokens <= %d", moe::kDecodeMaxT);
  if (x_dtype != MOE_BF16 && x_dtype != MOE_F32) return fail(MOE_EINVAL, "bad x_dtype %d", (int)x_dtype);
  if (out_dtype != MOE_BF16 && out_dtype != MOE_F32)
    return fail(MOE_EINVAL, "bad out_dtype %d", (int)out_dtype);
  if (shape->d_model > 4096 || shape->d_ff > 512 || shape->d_ff_shared > 512)
    return fail(MOE_EUNSUPPORTED, "decode path supports d_model <= 4096, d_ff <= 512");
  if (L == 0 || T == 0) return ok();
  if (!tables) return fail(MOE_EINVAL, "tables is NULL");
  bool any_slots = false;
  for (int l = 0; l < L; ++l) {
    s = check_table(shape, &tables[l]);
    if (s != MOE_OK) {
      char msg[256];
      snprintf(msg, sizeof msg, "%s", g_err);  // fail() rewrites g_err
      return fail(s, "layer %d: %s", l, msg);
    }
    if (tables[l].router)
      return fail(MOE_EUNSUPPORTED, "layer %d: the stack takes logits, not a router", l);
    any_slots = any_slots || tables[l].slot_of != nullptr;
  }
  if (any_slots && (!miss || !miss_count))
    return fail(MOE_EINVAL, "slot tables need miss ([layers][tokens*top_k]) and miss_count ([layers])");
  if (!x || !logits || !out || !ws) return fail(MOE_EINVAL, "x, logits, out and ws are required");
  if (!aligned256(ws)) return fail(MOE_EINVAL, "ws must be 256-byte aligned");
  if (((uintptr_t)x & 15u) || ((uintptr_t)logits & 3u) || ((uintptr_t)out & 15u))
    return fail(MOE_EINVAL, "x and out must be 16-byte aligned, logits 4-byte aligned");
  const size_t need = stack_ws_bytes(shape, L, T);
  if (ws_bytes < need) return fail(MOE_ENOSPACE, "ws_bytes %zu < %zu", ws_bytes, need);

  const int D = shape->d_model, E = shape->n_experts, k = shape->top_k;
  const size_t plan_bytes = moe::decode_plan_bytes(T, E, k);
  uint8_t* plan = (uint8_t*)ws;
  float* rms_part[2] = {nullptr, nullptr};
  if (T > 1) {
    const size_t half = stack_rms_bytes(shape, T) / 2;
    rms_part[0] = (float*)(plan + (size_t)L * plan_bytes);
    rms_part[1] = (float*)(plan + (size_t)L * plan_bytes + half);
  }
  const moe::DecodeWs base = moe::decode_ws_carve(
      plan + (size_t)L * plan_bytes + stack_rms_bytes(shape, T), T, D, shape->d_ff,
      shape->d_ff_shared, E, k);
  hipStream_t st = (hipStream_t)stream;
  // 1. The routing of every layer.
  for (int l0 = 0; l0 < L; l0 += moe::kPlanLayers) {
    moe::PlanArgs p = {};
    p.T = T;
    p.E = E;
    p.k = k;
    p.n = L - l0 < moe::kPlanLayers ? L - l0 : moe::kPlanLayers;
    p.logits = logits + (size_t)l0 * T * E;
    p.miss = any_slots ? (moe::MissRec*)miss + (size_t)l0 * T * k : nullptr;
    p.miss_count = any_slots ? miss_count + l0 : nullptr;
    p.plan = plan + (size_t)l0 * plan_bytes;
    p.plan_bytes = plan_bytes;
    for (int i = 0; i < p.n; ++i) {
      const moe_expert_table& t = tables[l0 + i];
      p.slot_of[i] = t.slot_of;
      p.n_slots[i] = t.n_slots;
      p.use_count[i] = t.slot_of ? t.use_count : nullptr;
      p.has_shared[i] = t.shared != nullptr;
    }
    s = hip_status(moe::launch_decode_plan(p, st), "plan launch");
    if (s != MOE_OK) return s;
  }
  // 2. The layers, each on its own list; layer l > 0 reads layer l - 1's
  // output with the RMS rule (with 2..4 tokens its factors come from the
  // sums of squares that layer l - 1's down kernel left in rms_part).
  const size_t out_row = (size_t)T * D * (out_dtype == MOE_BF16 ? 2 : 4);
  for (int l = 0; l < L; ++l) {
    const moe_expert_table& t = tables[l];
    moe::DecodeArgs a = {};
    a.T = T;
    a.D = D;
    a.F = shape->d_ff;
    a.Fs = shape->d_ff_shared;
    a.E = E;
    a.k = k;
    a.fmt = shape->qfmt;
    a.x = l == 0 ? x : (const void*)((const uint8_t*)out + (size_t)(l - 1) * out_row);
    a.x_bf16 = l == 0 ? x_dtype == MOE_BF16 : out_dtype == MOE_BF16;
    a.rmsnorm = l > 0;
    a.logits = logits + (size_t)l * T * E;
    a.routed = (const uint8_t*)t.routed;
    a.stride = t.expert_stride;
    a.slot_of = t.slot_of;
    a.n_slots = t.n_slots;
    a.shared = (const uint8_t*)t.shared;
    a.out = (uint8_t*)out + (size_t)l * out_row;
    a.out_bf16 = out_dtype == MOE_BF16;
    a.planned = 1;
    if (T > 1) {
      a.rms_in = l > 0 ? rms_part[(l - 1) & 1] : nullptr;
      a.rms_out = l + 1 < L ? rms_part[l & 1] : nullptr;
    }
    moe::DecodeWs w = base;
    moe::decode_plan_carve(plan + (size_t)l * plan_bytes, T, E, k, w);
    s = hip_status(moe::launch_decode(a, w, st), "decode launch");
    if (s != MOE_OK) return s;
  }
  return ok();
}

moe_status moe_layer_forward_noalloc(const moe_shape* shape, int32_t tokens, const void* x,
                                     int32_t x_dtype, uint32_t flags, float* router_logits,
                                     const moe_expert_table* table, void* out, int32_t out_dtype,
                                     moe_miss* miss, int32_t miss_cap, int32_t* miss_count,
                                     moe_stream_t stream) {
  return layer_forward_impl(shape, tokens, x, x_dtype, flags, router_logits, table, out, out_dtype,
                            miss, miss_cap, miss_count, nullptr, 0, true, stream);
}

// Validation shared by stage and commit: `slots` name distinct empty slots,
// `experts` distinct experts that are not resident.
static moe_status check_installs(const moe_slot_table* t, int32_t n, const int32_t* slots,
                                 const int32_t* experts, std::vector<char>& slot_named,
                                 std::vector<char>& expert_named) {
  if (!t) return fail(MOE_EINVAL, "table is NULL");
  if (n < 0) return fail(MOE_EINVAL, "n %d < 0", (int)n);
  if (!t->slot_of || !t->expert_of_slot || !t->host_slot_of || !t->host_expert_of_slot ||
      !t->storage)
    return fail(MOE_EINVAL, "table arrays are required");
  if (t->n_experts <= 0 || t->n_slots <= 0) return fail(MOE_EINVAL, "n_experts and n_slots must be > 0");
  if (n > 0 && (!slots || !experts)) return fail(MOE_EINVAL, "slots and experts are required");
  slot_named.assign(t->n_slots, 0);
  expert_named.assign(t->n_experts, 0);
  for (int i = 0; i < n; ++i) {
    const int sl = slots[i], ex = experts[i];
    if (sl < 0 || sl >= t->n_slots) return fail(MOE_EINVAL, "slot %d out of range", sl);
    if (ex < 0 || ex >= t->n_experts) return fail(MOE_EINVAL, "expert %d out of range", ex);
    if (slot_named[sl]) return fail(MOE_EINVAL, "slot %d named twice", sl);
    if (expert_named[ex]) return fail(MOE_EINVAL, "expert %d named twice", ex);
    slot_named[sl] = 1;
    expert_named[ex] = 1;
    if (t->host_expert_of_slot[sl] >= 0)
      return fail(MOE_EINVAL, "slot %d is not empty (expert %d)", sl, t->host_expert_of_slot[sl]);
    if (t->host_slot_of[ex] >= 0)
      return fail(MOE_EINVAL, "expert %d is already resident in slot %d", ex, t->host_slot_of[ex]);
  }
  return ok();
}

moe_status moe_slot_table_stage(moe_slot_table* t, int32_t n, const int32_t* slots,
                                const int32_t* experts, const void* const* src,
                                moe_stream_t stream) {
  std::vector<char> sn, en;
  moe_status s = check_installs(t, n, slots, experts, sn, en);
  if (s != MOE_OK) return s;
  if (n == 0) return ok();
  if (t->stride % 256 != 0 || t->expert_bytes > t->stride || !aligned256(t->storage))
    return fail(MOE_EINVAL, "storage must be 256-byte aligned, stride a multiple of 256 >= expert_bytes");
  if (!src) return fail(MOE_EINVAL, "src is required");
  for (int i = 0; i < n; ++i)
    if (!src[i]) return fail(MOE_EINVAL, "src[%d] is NULL", i);
  for (int i = 0; i < n; ++i) {
    hipError_t e = hipMemcpyAsync((uint8_t*)t->storage + (size_t)slots[i] * t->stride, src[i],
                                  t->expert_bytes, hipMemcpyDefault, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "slot copy");
  }
  return ok();
}

moe_status moe_slot_table_commit(moe_slot_table* t, int32_t n, const int32_t* slots,
                                 const int32_t* experts, const int32_t* evict,
                                 moe_stream_t stream) {
  std::vector<char> sn, en;
  moe_status s = check_installs(t, n, slots, experts, sn, en);
  if (s != MOE_OK) return s;
  if (n == 0) return ok();
  std::vector<char> evicted(t->n_experts, 0);
  if (evict) {
    for (int i = 0; i < n; ++i) {
      const int v = evict[i];
      if (v < -1 || v >= t->n_experts) return fail(MOE_EINVAL, "evict %d out of range", v);
      if (v < 0) continue;
      if (evicted[v]) return fail(MOE_EINVAL, "expert %d evicted twice", v);
      if (t->host_slot_of[v] < 0) return fail(MOE_EINVAL, "evicted expert %d is not resident", v);
      evicted[v] = 1;
    }
  }
  std::vector<moe::SlotEdit> edits;
  for (int i = 0; i < n; ++i) {
    if (evict && evict[i] >= 0) edits.push_back({t->host_slot_of[evict[i]], -1, evict[i], 0});
    edits.push_back({slots[i], experts[i], -1, 0});
  }
  {
    hipError_t e = moe::launch_slot_edits(t->slot_of, t->expert_of_slot, edits.data(),
                                          (int)edits.size(), (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "slot edit launch");
  }
  for (const auto& ed : edits) {
    if (ed.old_expert >= 0) t->host_slot_of[ed.old_expert] = -1;
    t->host_expert_of_slot[ed.slot] = ed.expert;
    if (ed.expert >= 0) t->host_slot_of[ed.expert] = ed.slot;
  }
  return ok();
}

moe_status moe_slot_counts_take(uint32_t* use_count, int32_t n, uint32_t* host_out,
                                moe_stream_t stream) {
  if (n < 0) return fail(MOE_EINVAL, "n %d < 0", (int)n);
  if (n == 0) return ok();
  if (!use_count || !host_out) return fail(MOE_EINVAL, "use_count and host_out are required");
  if ((uintptr_t)use_count & 3u) return fail(MOE_EINVAL, "use_count must be 4-byte aligned");
  hipError_t e = hipMemcpyAsync(host_out, use_count, (size_t)n * sizeof(uint32_t),
                                hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e, "count copy");
  return hip_status(moe::launch_counts_halve(use_count, n, (hipStream_t)stream), "count halve launch");
}

moe_status moe_slot_policy_plan(const moe_slot_table* t, const uint32_t* counts, int32_t max_swaps,
                                uint32_t margin, int32_t* admit, int32_t* evict, int32_t* slots,
                                int32_t* n_swaps) {
  if (!t || !counts || !n_swaps) return fail(MOE_EINVAL, "table, counts and n_swaps are required");
  if (!t->host_slot_of || !t->host_expert_of_slot) return fail(MOE_EINVAL, "host mirrors are required");
  if (t->n_experts <= 0 || t->n_slots <= 0) return fail(MOE_EINVAL, "n_experts and n_slots must be > 0");
  if (max_swaps < 0) return fail(MOE_EINVAL, "max_swaps %d < 0", (int)max_swaps);
  if (max_swaps > 0 && (!admit || !evict || !slots))
    return fail(MOE_EINVAL, "admit, evict and slots are required");
  const int E = t->n_experts, S = t->n_slots;
  std::vector<int32_t> cand, vict, empty;
  for (int e = 0; e < E; ++e) {
    if (t->host_slot_of[e] >= 0)
      vict.push_back(e);
    else if (counts[e] > 0)
      cand.push_back(e);
  }
  for (int sl = 0; sl < S; ++sl)
    if (t->host_expert_of_slot[sl] < 0) empty.push_back(sl);
  std::sort(cand.begin(), cand.end(), [&](int32_t x, int32_t y) {
    return counts[x] != counts[y] ? counts[x] > counts[y] : x < y;
  });
  std::sort(vict.begin(), vict.end(), [&](int32_t x, int32_t y) {
    return counts[x] != counts[y] ? counts[x] < counts[y] : x < y;
  });
  const size_t lim = std::min({(size_t)max_swaps, cand.size(), vict.size(), empty.size()});
  int32_t m = 0;
  for (size_t i = 0; i < lim; ++i) {
    if ((uint64_t)counts[cand[i]] <= (uint64_t)counts[vict[i]] + margin) break;
    admit[m] = cand[i];
    evict[m] = vict[i];
    slots[m] = empty[i];
    ++m;
  }
  *n_swaps = m;
  return ok();
}

moe_status moe_host_pool_create(int32_t n_threads, moe_host_pool** pool) {
  if (!pool) return fail(MOE_EINVAL, "pool is NULL");
  if (n_threads < 1 || n_threads > 1024) return fail(MOE_EINVAL, "n_threads %d not in 1..1024", (int)n_threads);
  try {
    *pool = moe_host_pool_new(n_threads);
  } catch (...) {
    *pool = nullptr;
    return fail(MOE_EINVAL, "could not start %d threads", (int)n_threads);
  }
  return ok();
}

void moe_host_pool_destroy(moe_host_pool* pool) {
  if (pool) moe_host_pool_delete(pool);
}

moe_status moe_host_miss_ffn(const moe_shape* shape, int32_t tokens, const void* x, int32_t x_dtype,
                             uint32_t flags, const moe_miss* misses, int32_t n_miss,
                             const void* const* experts, float* y, moe_host_pool* pool) {
  moe_status s = check_shape(shape);
  if (s != MOE_OK) return s;
  if (tokens < 0 || n_miss < 0) return fail(MOE_EINVAL, "tokens and n_miss must be >= 0");
  if (x_dtype != MOE_BF16 && x_dtype != MOE_F32) return fail(MOE_EINVAL, "bad x_dtype %d", (int)x_dtype);
  if (flags & ~(uint32_t)MOE_FLAG_RMSNORM_INPUT) return fail(MOE_EINVAL, "unknown flags 0x%x", flags);
  if (tokens == 0) return ok();
  if (!x || !y) return fail(MOE_EINVAL, "x and y are required");
  if (n_miss > 0 && (!misses || !experts)) return fail(MOE_EINVAL, "misses and experts are required");
  for (int i = 0; i < n_miss; ++i) {
    const moe_miss& m = misses[i];
    if (m.token < 0 || m.token >= tokens) return fail(MOE_EINVAL, "miss %d: token %d out of range", i, m.token);
    if (m.expert < 0 || m.expert >= shape->n_experts)
      return fail(MOE_EINVAL, "miss %d: expert %d out of range", i, m.expert);
    if (!experts[m.expert]) return fail(MOE_EINVAL, "miss %d: experts[%d] is NULL", i, m.expert);
    if (i > 0 && (m.token < misses[i - 1].token ||
                  (m.token == misses[i - 1].token && m.rank <= misses[i - 1].rank)))
      return fail(MOE_EINVAL, "misses must be in (token, rank) order");
  }
  try {
    std::vector<float> xhat((size_t)tokens * shape->d_model);
    moe::host_prepare_x(tokens, shape->d_model, x, x_dtype == MOE_BF16,
                        (flags & MOE_FLAG_RMSNORM_INPUT) != 0, xhat.data());
    moe::host_miss_ffn(shape->d_model, shape->d_ff, shape->qfmt, tokens, xhat.data(),
                       reinterpret_cast<const moe::MissRec*>(misses), n_miss,
                       reinterpret_cast<const uint8_t* const*>(experts), y, pool);
  } catch (...) {
    return fail(MOE_EINVAL, "host miss path: out of host memory");
  }
  return ok();
}

moe_status moe_add_rows(void* out, int32_t out_dtype, const float* y, int32_t tokens,
                        int32_t d_model, moe_stream_t stream) {
  if (out_dtype != MOE_BF16 && out_dtype != MOE_F32) return fail(MOE_EINVAL, "bad out_dtype %d", (int)out_dtype);
  if (tokens < 0 || d_model < 0) return fail(MOE_EINVAL, "tokens and d_model must be >= 0");
  if ((size_t)tokens * d_model == 0) return ok();
  if (!out || !y) return fail(MOE_EINVAL, "out and y are required");
  if (((uintptr_t)out & 3u) || ((uintptr_t)y & 3u)) return fail(MOE_EINVAL, "out and y must be 4-byte aligned");
  return hip_status(moe::launch_add_rows(out, out_dtype == MOE_BF16, y, (size_t)tokens * d_model,
                                         (hipStream_t)stream),
                    "add launch");
}

}  // extern "C"

namespace {

// The calling thread's side stream and event on the current device, made on
// first use and kept until the process ends (non-blocking, default priority).
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t ev = nullptr;
};
hipError_t side_stream(SideStream*& out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= moe::kMaxDevices) return hipErrorInvalidDevice;
  thread_local SideStream per[moe::kMaxDevices];
  SideStream& ss = per[dev];
  if (!ss.ev) {
    if (!ss.s && (e = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&ss.ev, hipEventDisableTiming)) != hipSuccess) return e;
  }
  out = &ss;
  return hipSuccess;
}

// Device workspace of moe_slot_layer_forward_host: the layer's workspace,
// the miss records with their count right behind them, the host rows.
struct SlotHostWs {
  size_t miss, y, total;
};
SlotHostWs slot_host_ws(const moe_shape* s, int T) {
  auto a256 = [](size_t n) { return (n + 255) / 256 * 256; };
  const size_t fws = a256(forward_ws_bytes(s, T));
  const size_t miss = a256((size_t)T * s->top_k * sizeof(moe_miss) + 4);
  return {fws, fws + miss, fws + miss + a256((size_t)T * s->d_model * 4)};
}
// Pinned host staging: miss records + count, the layer input (fp32-sized),
// the host rows, and (on a 128-byte line of its own) the flag the decode
// kernel raises once it has written the first two.
struct SlotHostStaging {
  size_t x, y, flag, total;
};
SlotHostStaging slot_host_staging(const moe_shape* s, int T) {
  auto a64 = [](size_t n) { return (n + 63) / 64 * 64; };
  auto a128 = [](size_t n) { return (n + 127) / 128 * 128; };
  const size_t m = a64((size_t)T * s->top_k * sizeof(moe_miss) + 4);
  const size_t row = a64((size_t)T * s->d_model * 4);
  const size_t flag = a128(m + 2 * row);
  return {m, m + row, flag, flag + 128};
}

}  // namespace

extern "C" {

size_t moe_slot_host_workspace_bytes(const moe_shape* shape, int32_t tokens) {
  if (check_shape(shape) != MOE_OK || tokens <= 0) return 0;
  return slot_host_ws(shape, tokens).total;
}

size_t moe_slot_host_staging_bytes(const moe_shape* shape, int32_t tokens) {
  if (check_shape(shape) != MOE_OK || tokens <= 0) return 0;
  return slot_host_staging(shape, tokens).total;
}

moe_status moe_slot_layer_forward_host(const moe_shape* shape, int32_t tokens, const void* x,
                                       int32_t x_dtype, uint32_t flags, float* router_logits,
                                       const moe_expert_table* table, void* out,
                                       int32_t out_dtype, const void* const* host_experts,
                                       int32_t* n_miss, void* ws, size_t ws_bytes,
                                       void* staging, size_t staging_bytes, moe_host_pool* pool,
                                       moe_stream_t stream) {
  moe_status s = check_shape(shape);
  if (s != MOE_OK) return s;
  const int T = tokens;
  if (T < 0) return fail(MOE_EINVAL, "tokens %d < 0", T);
  if (!table || !table->slot_of) return fail(MOE_EINVAL, "a slot table (table->slot_of) is required");
  if (T == 0) {
    if (n_miss) *n_miss = 0;
    return ok();
  }
  if (!host_experts) return fail(MOE_EINVAL, "host_experts is required");
  if (!staging || ((uintptr_t)staging & 63u)) return fail(MOE_EINVAL, "staging must be 64-byte aligned");
  if (!ws || !aligned256(ws)) return fail(MOE_EINVAL, "ws must be given and 256-byte aligned");
  const SlotHostWs L = slot_host_ws(shape, T);
  const SlotHostStaging S = slot_host_staging(shape, T);
  if (ws_bytes < L.total) return fail(MOE_ENOSPACE, "ws_bytes %zu < %zu", ws_bytes, L.total);
  if (staging_bytes < S.total)
    return fail(MOE_ENOSPACE, "staging_bytes %zu < %zu", staging_bytes, S.total);
  hipStream_t st = (hipStream_t)stream;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone)
    return fail(MOE_EUNSUPPORTED, "moe_slot_layer_forward_host waits on the host: not for capture");
  void* stg_dev = nullptr;
  if (hipHostGetDevicePointer(&stg_dev, staging, 0) != hipSuccess || !stg_dev) {
    (void)hipGetLastError();
    return fail(MOE_EINVAL, "staging must be page-locked host memory the device can address (hipHostMalloc)");
  }
  const int k = shape->top_k, D = shape->d_model;
  const size_t mbytes = (size_t)T * k * sizeof(moe_miss);
  uint8_t* wsb = (uint8_t*)ws;
  uint8_t* stg = (uint8_t*)staging;
  moe_miss* miss_d = (moe_miss*)(wsb + L.miss);
  int32_t* cnt_d = (int32_t*)(wsb + L.miss + mbytes);
  float* y_d = (float*)(wsb + L.y);
  hipError_t e;
  if (use_decode_path(T)) {
    // 1-2. The layer on the stream; the kernel that publishes its routing
    // also writes the miss list, its count and the input into the staging
    // and then raises the flag (no event, copy or synchronisation calls,
    // which cost the host tens of microseconds per layer).
    static std::atomic<uint32_t> g_seq{0};
    uint32_t seq = ++g_seq;
    if (seq == 0) seq = ++g_seq;
    volatile uint32_t* flag = reinterpret_cast<volatile uint32_t*>(stg + S.flag);
    *flag = 0u;
    uint8_t* dv = (uint8_t*)stg_dev;
    moe::host_pub() = {(moe::MissRec*)dv, (int32_t*)(dv + mbytes), dv + S.x,
                       (uint32_t*)(dv + S.flag), seq};
    s = layer_forward_impl(shape, T, x, x_dtype, flags, router_logits, table, out, out_dtype,
                           miss_d, T * k, cnt_d, ws, L.miss, false, stream);
    const bool armed = moe::host_pub().flag != nullptr;
    moe::host_pub() = {};
    if (s != MOE_OK) return s;
    if (armed) return fail(MOE_EHIP, "the layer did not take the host copy of its routing");
    const auto t0 = std::chrono::steady_clock::now();
    for (uint32_t polls = 0; __atomic_load_n(flag, __ATOMIC_ACQUIRE) != seq; ++polls) {
#if defined(__x86_64__)
      __builtin_ia32_pause();
#endif
      if ((polls & 4095u) == 4095u && std::chrono::steady_clock::now() - t0 > std::chrono::seconds(10))
        return fail(MOE_EHIP, "the layer's routing did not reach the host within 10 s");
    }
  } else {
    SideStream* side = nullptr;
    s = hip_status(side_stream(side), "side stream");
    if (s != MOE_OK) return s;
    // 1. The layer on the stream; its routing records the side event.
    moe::route_event().before = side->ev;
    s = layer_forward_impl(shape, T, x, x_dtype, flags, router_logits, table, out, out_dtype,
                           miss_d, T * k, cnt_d, ws, L.miss, false, stream);
    const bool recorded = moe::route_event().before == nullptr;
    moe::route_event().before = nullptr;
    if (s != MOE_OK) return s;
    if (!recorded) return fail(MOE_EHIP, "the layer did not record its routing event");
    // 2. Miss list, count and input to the host once the routing is written.
    if ((e = hipStreamWaitEvent(side->s, side->ev, 0)) != hipSuccess ||
        (e = hipMemcpyAsync(stg, miss_d, mbytes + 4, hipMemcpyDeviceToHost, side->s)) != hipSuccess ||
        (e = hipMemcpyAsync(stg + S.x, x, (size_t)T * D * (x_dtype == MOE_BF16 ? 2 : 4),
                            hipMemcpyDeviceToHost, side->s)) != hipSuccess ||
        (e = hipStreamSynchronize(side->s)) != hipSuccess)
      return hip_status(e, "miss list copy");
  }
  const int32_t nm = *reinterpret_cast<const int32_t*>(stg + mbytes);
  if (n_miss) *n_miss = nm;
  if (nm == 0) return ok();
  // 3. The missed experts' rows, while the GPU computes the resident ones.
  s = moe_host_miss_ffn(shape, T, stg + S.x, x_dtype, flags, reinterpret_cast<const moe_miss*>(stg),
                        nm, host_experts, reinterpret_cast<float*>(stg + S.y), pool);
  if (s != MOE_OK) return s;
  // 4. Into the layer output, behind the layer on the stream.
  if ((e = hipMemcpyAsync(y_d, stg + S.y, (size_t)T * D * 4, hipMemcpyHostToDevice, st)) != hipSuccess)
    return hip_status(e, "host rows copy");
  return hip_status(moe::launch_add_rows(out, out_dtype == MOE_BF16, y_d, (size_t)T * D, st),
                    "add launch");
}

moe_status moe_router_logits(const moe_shape* shape, int32_t tokens, const void* x,
                             int32_t x_dtype, uint32_t flags, const void* w_router, float* logits,
                             moe_stream_t stream) {
  moe_status s = check_shape(shape);
  if (s != MOE_OK) return s;
  if (tokens < 0) return fail(MOE_EINVAL, "tokens %d < 0", (int)tokens);
  if (x_dtype != MOE_BF16 && x_dtype != MOE_F32) return fail(MOE_EINVAL, "bad x_dtype %d", (int)x_dtype);
  if (flags & ~(uint32_t)MOE_FLAG_RMSNORM_INPUT) return fail(MOE_EINVAL, "unknown flags 0x%x", flags);
  if (tokens == 0) return ok();
  if (!x || !w_router || !logits) return fail(MOE_EINVAL, "x, w_router and logits are required");
  if (((uintptr_t)x & 15u) || ((uintptr_t)w_router & 15u) || ((uintptr_t)logits & 3u))
    return fail(MOE_EINVAL, "x and w_router must be 16-byte aligned, logits 4-byte aligned");
  moe::RouterArgs r{tokens, shape->d_model, shape->n_experts, x, x_dtype == MOE_BF16,
                    (flags & MOE_FLAG_RMSNORM_INPUT) != 0, (const uint16_t*)w_router, logits};
  return hip_status(moe::launch_router(r, (hipStream_t)stream), "router launch");
}

moe_status moe_slot_table_init(moe_slot_table* t, moe_stream_t stream) {
  if (!t) return fail(MOE_EINVAL, "table is NULL");
  if (t->n_experts <= 0 || t->n_slots <= 0) return fail(MOE_EINVAL, "n_experts and n_slots must be > 0");
  if (!t->slot_of || !t->expert_of_slot || !t->host_slot_of || !t->host_expert_of_slot)
    return fail(MOE_EINVAL, "map arrays and host mirrors are required");
  for (int i = 0; i < t->n_experts; ++i) t->host_slot_of[i] = -1;
  for (int i = 0; i < t->n_slots; ++i) t->host_expert_of_slot[i] = -1;
  return hip_status(moe::launch_slot_init(t->slot_of, t->n_experts, t->expert_of_slot, t->n_slots,
                                          (hipStream_t)stream),
                    "slot init launch");
}

moe_status moe_slot_table_update(moe_slot_table* t, int32_t n, const int32_t* slots,
                                 const int32_t* experts, const void* const* src,
                                 moe_stream_t stream) {
  if (!t) return fail(MOE_EINVAL, "table is NULL");
  if (n < 0) return fail(MOE_EINVAL, "n %d < 0", (int)n);
  if (n == 0) return ok();
  if (!slots || !experts) return fail(MOE_EINVAL, "slots and experts are required");
  if (!t->slot_of || !t->expert_of_slot || !t->host_slot_of || !t->host_expert_of_slot ||
      !t->storage)
    return fail(MOE_EINVAL, "table arrays are required");
  if (t->stride % 256 != 0 || t->expert_bytes > t->stride || !aligned256(t->storage))
    return fail(MOE_EINVAL, "storage must be 256-byte aligned, stride a multiple of 256 >= expert_bytes");
  const int E = t->n_experts, S = t->n_slots;
  std::vector<char> slot_named(S, 0), expert_named(E, 0);
  for (int i = 0; i < n; ++i) {
    const int sl = slots[i], ex = experts[i];
    if (sl < 0 || sl >= S) return fail(MOE_EINVAL, "slot %d out of range", sl);
    if (ex < -1 || ex >= E) return fail(MOE_EINVAL, "expert %d out of range", ex);
    if (slot_named[sl]) return fail(MOE_EINVAL, "slot %d named twice", sl);
    slot_named[sl] = 1;
    if (ex >= 0) {
      if (expert_named[ex]) return fail(MOE_EINVAL, "expert %d named twice", ex);
      expert_named[ex] = 1;
      if (!src || !src[i]) return fail(MOE_EINVAL, "src[%d] is NULL for an install", i);
    }
  }
  for (int i = 0; i < n; ++i) {
    const int ex = experts[i];
    if (ex >= 0) {
      const int cur = t->host_slot_of[ex];
      if (cur >= 0 && !slot_named[cur])
        return fail(MOE_EINVAL, "expert %d is already resident in slot %d", ex, cur);
    }
  }
  // Validated: apply.  Copies first, then the map edits, all stream-ordered.
  std::vector<moe::SlotEdit> edits(n);
  for (int i = 0; i < n; ++i) {
    edits[i].slot = slots[i];
    edits[i].expert = experts[i];
    edits[i].old_expert = t->host_expert_of_slot[slots[i]];
    edits[i].pad = 0;
    if (experts[i] >= 0) {
      hipError_t e = hipMemcpyAsync((uint8_t*)t->storage + (size_t)slots[i] * t->stride, src[i],
                                    t->expert_bytes, hipMemcpyDefault, (hipStream_t)stream);
      if (e != hipSuccess) return hip_status(e, "slot copy");
    }
  }
  {
    hipError_t e = moe::launch_slot_edits(t->slot_of, t->expert_of_slot, edits.data(), n,
                                          (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "slot edit launch");
  }
  // Host mirror: evictions first, then installs.
  for (int i = 0; i < n; ++i)
    if (edits[i].old_expert >= 0) t->host_slot_of[edits[i].old_expert] = -1;
  for (int i = 0; i < n; ++i) {
    t->host_expert_of_slot[slots[i]] = experts[i];
    if (experts[i] >= 0) t->host_slot_of[experts[i]] = slots[i];
  }
  return ok();
}

moe_status moe_route(const float* logits, int32_t tokens, int32_t n_experts, int32_t top_k,
                     int32_t* idx, float* gate, moe_stream_t stream) {
  if (tokens < 0) return fail(MOE_EINVAL, "tokens < 0");
  if (n_experts <= 0 || n_experts > 2048) return fail(MOE_EINVAL, "n_experts must be in 1..2048");
  if (top_k < 1 || top_k > 32 || top_k > n_experts) return fail(MOE_EINVAL, "top_k out of range");
  if (tokens == 0) return ok();
  if (!logits || !idx || !gate) return fail(MOE_EINVAL, "logits, idx, gate are required");
  return hip_status(moe::launch_route(logits, tokens, n_experts, top_k, idx, gate,
                                      (hipStream_t)stream),
                    "route launch");
}

size_t moe_permute_workspace_bytes(int32_t tokens, int32_t top_k, int32_t n_experts) {
  if (tokens < 0 || top_k < 1 || n_experts < 1) return 0;
  return moe::perm_ws_bytes(tokens, top_k, n_experts);
}

moe_status moe_permute(const int32_t* idx, int32_t tokens, int32_t top_k, int32_t n_experts,
                       int32_t* offsets, int32_t* sorted_pairs, int32_t* inv, void* ws,
                       size_t ws_bytes, moe_stream_t stream) {
  if (tokens < 0) return fail(MOE_EINVAL, "tokens < 0");
  if (n_experts <= 0 || n_experts > 2048) return fail(MOE_EINVAL, "n_experts must be in 1..2048");
  if (top_k < 1 || top_k > 32 || top_k > n_experts) return fail(MOE_EINVAL, "top_k out of range");
  if (!offsets) return fail(MOE_EINVAL, "offsets is required");
  if ((int64_t)tokens * top_k > (int64_t)1 << 30) return fail(MOE_EINVAL, "too many pairs");
  if (tokens > 0 && (!idx || !sorted_pairs || !inv || !ws))
    return fail(MOE_EINVAL, "idx, sorted_pairs, inv, ws are required");
  const size_t need = moe::perm_ws_bytes(tokens, top_k, n_experts);
  if (tokens > 0 && ws_bytes < need) return fail(MOE_ENOSPACE, "ws_bytes %zu < %zu", ws_bytes, need);
  const moe::PermWs w = moe::perm_ws_carve(ws, tokens, top_k, n_experts);
  return hip_status(moe::launch_permute(idx, tokens, top_k, n_experts, offsets, sorted_pairs, inv,
                                        w, (hipStream_t)stream),
                    "permute launch");
}

}  // extern "C"
