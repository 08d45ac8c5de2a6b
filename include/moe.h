/*
 * moe.h -- C ABI of libmoe, the routed low-bit mixture-of-experts FFN layer
 * for AMD Instinct MI355X (gfx950).
 *
 * Sources ("the pages"):
 *   [KC-en] "Running Qwen3.8-Flash-Next on a 12GB GPU: Custom Engine Hits 65 tok/s"
 *   [JD]    "5070ti16g单卡跑qwen 3.8 flash next 新方案最高90t/s Hermes调用60t/s"
 *   [AF]    "个人开发者用 AI 十天写出 Strata 引擎，让 12GB 显存跑起 1250 亿参数的
 *            Qwen 3.8 Flash Next"
 *   [SL]    daily.steinslab.io, "一台装着 12GB 显存游戏显卡的家用电脑…"
 *
 * The layer: each of 48 layers has 512 routed experts; a token uses the 10
 * most relevant of them plus one shared expert ([AF] section "1250 亿参数，
 * 每个词只用得上 2%"; [SL] section "12GB 显存装下 1250 亿参数").  Expert
 * weights are low-bit block-quantised ([KC-en] section "Hardware
 * Configuration and Quantization Approach").  Hot experts stay resident on
 * the GPU, the others are computed elsewhere and added into the same layer
 * ([AF] section "命中率七成，代价是答案会变").  The pages give no formulas;
 * the readings this library implements are:
 *   out_t = sum_{j<k} g_tj * FFN_{e_tj}(x_t) + FFN_shared(x_t)
 *   FFN(x) = W_down (silu(W_gate x) * (W_up x)),  silu(a) = a / (1 + e^-a)
 *   e_t0..e_t(k-1): the k largest fp32 logits of token t, ties to the lower
 *   expert id, -0.0 == +0.0;  g_tj = exp(l_j - l_0) / sum_i exp(l_i - l_0).
 *
 * Conventions for every entry point:
 *   - Pointers named "device" are HIP device (HBM) addresses; "host" are
 *     CPU addresses.  The caller allocates and frees every buffer, including
 *     the workspace.  The GPU entry points allocate no device memory and
 *     keep no state between calls, except: moe_last_error's per-thread
 *     message; the per-thread event pairs of the profiling aids; per
 *     device, the largest dynamic-LDS limit already set on a kernel (set
 *     once with hipFuncSetAttribute, thread-safe); and the side stream and
 *     event moe_slot_layer_forward_host keeps per thread and device.  The host half of the
 *     slot-mode layer is different: moe_host_pool_create starts threads,
 *     and moe_host_miss_ffn allocates and frees its own host scratch (the
 *     rearranged activations and the h rows) within each call.
 *   - All device work is enqueued on the caller's stream (NULL = the null
 *     stream); nothing waits on the host, except moe_slot_layer_forward_host,
 *     which waits for its layer's routing.  Device-resident results (outputs,
 *     miss lists, counts) are valid after the caller synchronises the stream.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     rejected call returns a negative moe_status, sets moe_last_error(),
 *     and launches nothing.  A failed launch returns MOE_EHIP.  Faults inside
 *     a kernel surface at the caller's next synchronisation of the stream.
 *   - Calls are re-entrant for distinct buffers; two calls that share a
 *     workspace or output must be ordered by the caller (same stream).
 *   - No C++ exception crosses this interface.
 *
 * ---------------------------------------------------------------------------
 * Quantised formats (one block = 32 consecutive weights along the reduction
 * dimension of one output row; the pages name 2- and 3-bit expert formats,
 * [KC-en] section "Detailed Performance Numbers", but give no layout):
 *   MOE_Q2SM32: u in {0,1,2,3}, fp16 scale s and fp16 min m per block:
 *               w = s*u + m                                (3.0 bits/weight)
 *   MOE_Q3S32:  q in {-4..3}, fp16 scale s per block: w = s*q  (3.5 bits/weight)
 *   MOE_Q2S32:  u in {0,1,2,3}, fp16 scale s per block: w = s*(u - 2)
 *               (2.5 bits/weight).  The pages' fastest tier is a uniform
 *               2-bit format of about this footprint ([KC-en] sections
 *               "Detailed Performance Numbers" and "Memory Requirements
 *               (RAM + VRAM combined)"); they give no formula, and the zero
 *               point in the middle of the four codes is the reading taken
 *               here.
 *
 * Logical (unpacked) expert weights, the input of moe_pack_weights, for an
 * expert of model width D and FFN width F: three matrices in the order
 * W_gate [F][D], W_up [F][D], W_down [D][F], each row-major; codes are one
 * byte per weight ([3][F*D]; Q2SM, Q2S: u; Q3S: q as a signed byte); scales and
 * mins are fp16 bit patterns, one per block ([3][F*D/32], row-major over
 * [rows][K/32]).
 *
 * Packed layout (the "pack" the pages build once before serving, [JD]
 * section "为什么从 18t/s 变成 60-90t/s"; this layout is this library's
 * own).  A matrix with R rows and reduction length K is cut into records of
 * 16 rows x 256 columns (8 blocks, one "octet"); K is padded with zero
 * codes and zero scale/min up to a multiple of 256.  Inside a record, lane
 * L = 16*q + n (n = row within the record, q = 0..3) owns four 32-bit code
 * words; word w covers blocks 2w and 2w+1 of the octet; slot s = 0..7 of a
 * word holds block b = 2w + s/4 and pair j = s%4: the code of column
 * 32*b + 8*q + 2*j is at bits 2s..2s+1 and the code of the next column at
 * bits 16+2s..17+2s.
 *   Q2SM record, 1536 bytes: bytes [0,1024) code words, lane-major (word
 *     (L, w) at byte 16*L + 4*w); bytes [1024,1536): for n in 0..15, b in
 *     0..7, the fp16 scale then the fp16 min of (row n, block b), at byte
 *     1024 + 4*(8*n + b).
 *   Q3S record, 1792 bytes: bytes [0,1024) low-plane words as above holding
 *     (q+4) & 3; bytes [1024,1536): high-plane words, two per lane (word
 *     (L, h) at byte 1024 + 8*L + 4*h); high word h serves low words 2h and
 *     2h+1: the high bit ((q+4) >> 2) of the code at bit p of low word 2h is
 *     bit p+1 of the high word, of low word 2h+1 bit p; bytes [1536,1792):
 *     the fp16 scale of (row n, block b) at byte 1536 + 2*(8*n + b).
 *   Q2S record, 1280 bytes: bytes [0,1024) code words as in Q2SM; bytes
 *     [1024,1280): the fp16 scale of (row n, block b) at byte 1024 + 2*(8*n + b).
 * A packed expert is its gate/up region followed by its down region:
 *   gate/up: for g in 0..F/16-1, for matrix in (W_gate, W_up), for each
 *     octet o of D: the record of rows 16g..16g+15, columns 256o..256o+255;
 *   down: for r in 0..D/16-1, for each octet o of F (padded): the record of
 *     W_down rows 16r..16r+15.
 * Requirements: D % 256 == 0, F % 32 == 0.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* moe_stream_t; /* the same type as hipStream_t */

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,       /* bad argument: null pointer, bad size or shape, conflict */
  MOE_EUNSUPPORTED = -2, /* valid request the library does not implement */
  MOE_EHIP = -3,         /* a HIP runtime call or kernel launch failed */
  MOE_ENOSPACE = -4      /* workspace or miss-list capacity too small */
} moe_status;

typedef enum { MOE_Q2SM32 = 1, MOE_Q3S32 = 2, MOE_Q2S32 = 3 } moe_qfmt;
typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Input flag of moe_layer_forward: normalise each token's input first,
 * x <- bf16(x / sqrt(mean(x^2) + 1e-6)), computed in fp32.  The pages stack
 * 48 layers but print nothing of the rest of a block; this parameter-free
 * RMS step stands in for it when layers are chained. */
#define MOE_FLAG_RMSNORM_INPUT 1u

/* Layer geometry.  d_model % 256 == 0; d_ff and d_ff_shared are multiples
 * of 32 (d_ff_shared may be 0: no shared expert); 1 <= top_k <= min(32,
 * n_experts); n_experts <= 2048. */
typedef struct {
  int32_t d_model;
  int32_t d_ff;
  int32_t n_experts;
  int32_t top_k;
  int32_t d_ff_shared;
  int32_t qfmt; /* moe_qfmt */
} moe_shape;

/* Where the packed experts live.
 *   routed:        device; routed expert (or slot) i starts at
 *                  routed + i*expert_stride.  expert_stride must be at least
 *                  moe_packed_expert_bytes(shape, d_ff) and a multiple of 256.
 *   slot_of:       device int32 [n_experts] or NULL.  NULL: all n_experts
 *                  experts are resident, expert e at index e.  Otherwise
 *                  expert e is at slot slot_of[e] (0 <= slot < n_slots) or not
 *                  resident (-1) -- the hot-expert cache of the pages ([AF]
 *                  section "命中率七成，代价是答案会变").
 *   n_slots:       slots in `routed` when slot_of != NULL.
 *   shared:        device; the packed shared expert (width d_ff_shared), or
 *                  NULL when d_ff_shared == 0.  256-byte aligned.
 *   router:        device bf16 [n_experts][d_model] router projection W_r
 *                  (row e = expert e, contiguous along d_model), 16-byte
 *                  aligned, or NULL.  With it, moe_layer_forward computes the
 *                  logits itself (see moe_router_logits) and `router_logits`
 *                  becomes an output.
 *   use_count:     device uint32 [n_experts], 4-byte aligned, or NULL.  Used
 *                  only with a slot table: every routed (token, rank) pair
 *                  adds 1 to its expert's entry (hit or miss), the usage
 *                  statistics of moe_slot_policy_plan. */
typedef struct {
  const void* routed;
  size_t expert_stride;
  const int32_t* slot_of;
  int32_t n_slots;
  const void* shared;
  const void* router;
  uint32_t* use_count;
} moe_expert_table;

/* One routed (token, rank) pair whose expert is not resident. */
typedef struct {
  int32_t token;
  int32_t rank;
  int32_t expert;
  float gate;
} moe_miss;

/* Size in bytes of one packed expert of FFN width d_ff under shape->qfmt and
 * shape->d_model (0 if the shape is invalid). */
size_t moe_packed_expert_bytes(const moe_shape* shape, int32_t d_ff);

/* Pack n logical experts (layout above) into the packed format: the pages'
 * low-bit block-quantised experts ([KC-en] section "Hardware Configuration
 * and Quantization Approach") in the record layout the kernels stream.
 *   codes:  device, n*3*d_ff*d_model bytes (Q2SM, Q2S: u in 0..3; Q3S:
 *           signed q in -4..3; only the low 2 resp. 3 bits of u resp. q+4
 *           are used).
 *   scale:  device fp16 bits, n*3*d_ff*d_model/32.
 *   min:    device fp16 bits, same size (Q2SM), NULL for Q3S and Q2S.
 *   dst:    device; expert i is written at dst + i*dst_stride
 *           (dst_stride >= moe_packed_expert_bytes, multiple of 256).
 * Deterministic; the output bytes depend only on the inputs. */
moe_status moe_pack_weights(const moe_shape* shape, int32_t n, int32_t d_ff,
                            const void* codes, const uint16_t* scale, const uint16_t* min,
                            void* dst, size_t dst_stride, moe_stream_t stream);

/* Inverse of moe_pack_weights (padding dropped), for round trips and
 * inspection.  Q3S codes come back as signed q; min is not written for Q3S
 * and Q2S (may be NULL). */
moe_status moe_unpack_weights(const moe_shape* shape, int32_t n, int32_t d_ff,
                              const void* src, size_t src_stride,
                              void* codes, uint16_t* scale, uint16_t* min,
                              moe_stream_t stream);

/* Workspace bytes moe_layer_forward needs for `tokens` tokens (device
 * scratch of the steps the pages' layer runs: the routing of each token,
 * the list of the distinct selected experts and their h rows for decode;
 * the routing, the stable permutation and the H and Y rows of the grouped
 * GEMMs for prefill, [AF] sections "1250 亿参数，每个词只用得上 2%" and
 * "等最久的，是它读完你的代码").  0 for an invalid shape or tokens < 0. */
size_t moe_workspace_bytes(const moe_shape* shape, int32_t tokens);

/* One MoE FFN layer: each token's input goes to the 10 (top_k) experts its
 * router logits rank highest plus the shared expert, and their outputs are
 * summed with the renormalised gates ([AF] section "1250 亿参数，每个词只
 * 用得上 2%"; [SL] section "12GB 显存装下 1250 亿参数"); decode (1 token,
 * or 1 + 3 drafts verified together, [AF] section "命中率七成，代价是答案会
 * 变") streams each selected expert's weights once ([JD] section "为什么从
 * 18t/s 变成 60-90t/s"); prefill runs chunks of up to 8192 tokens ([AF]
 * section "等最久的，是它读完你的代码").  The formula is the one in the
 * preamble of this header.
 *   tokens:        T >= 0 (T == 0: nothing is launched, *miss_count is not
 *                  touched).
 *   x:             device [T][d_model], dtype x_dtype (MOE_BF16 or MOE_F32),
 *                  16-byte aligned.
 *   flags:         0 or MOE_FLAG_RMSNORM_INPUT.
 *   router_logits: device fp32 [T][n_experts], 4-byte aligned; must be finite.
 *                  An input when table->router is NULL.  Otherwise an output:
 *                  the layer first writes the router projection of its input
 *                  there (as moe_router_logits, on the input the experts
 *                  see) and routes on it.
 *   table:         where the experts are (see moe_expert_table).
 *   out:           device [T][d_model], dtype out_dtype, 16-byte aligned.
 *                  Written in full.
 *                  Without a slot table: the layer output.  With one: the
 *                  partial output -- the shared expert plus every pair whose
 *                  expert is resident, weighted by the full top-k gates.
 *   miss, miss_cap, miss_count: used only when table->slot_of != NULL
 *                  (then all three are required): device array of capacity
 *                  miss_cap >= T*top_k (else MOE_ENOSPACE), receiving every
 *                  non-resident pair in (token, rank) order, and a device
 *                  int32 receiving their number.  partial + sum over misses
 *                  of gate * FFN_expert(x_token) is the whole layer.
 *   ws, ws_bytes:  device workspace, ws_bytes >= moe_workspace_bytes(shape,
 *                  T), 256-byte aligned.
 * Misaligned pointers are rejected with MOE_EINVAL before any launch.
 * Paths: T <= 4 runs the decode path (dequantising MFMA GEMV that streams
 * each distinct selected expert once); larger T runs the prefill path
 * (routing, stable token permutation, grouped MFMA GEMM, combine).  Both
 * paths take all three formats and slot tables; with a slot table the
 * prefill path leaves the non-resident pairs out of the permuted groups and
 * lists them, in (token, rank) order, as the decode path does.
 * Results are deterministic: the same inputs give the same output bits. */
moe_status moe_layer_forward(const moe_shape* shape, int32_t tokens,
                             const void* x, int32_t x_dtype, uint32_t flags,
                             float* router_logits, const moe_expert_table* table,
                             void* out, int32_t out_dtype,
                             moe_miss* miss, int32_t miss_cap, int32_t* miss_count,
                             void* ws, size_t ws_bytes, moe_stream_t stream);

/* moe_layer_forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, results and errors as
 * moe_layer_forward (the same kernels run), minus ws and ws_bytes.
 *   Decode path only: tokens <= 4; larger tokens return MOE_EUNSUPPORTED
 *   before any launch.  Its workspace is a fixed device array of 2 MiB
 *   inside the library (one per GPU, held until the process ends), enough
 *   for every decode request moe_layer_forward accepts (at most about
 *   1.2 MiB: 4 tokens, top-32, d_ff 512); a request needing more returns
 *   MOE_ENOSPACE.  Allocates nothing: on its first call on a device it looks
 *   up that device's copy of the array (hipGetSymbolAddress).
 *   Every call on one GPU shares that array and finds the last call's
 *   contents there (nothing needs to start cleared): calls that overlap in
 *   time on one GPU -- on different streams or from different threads --
 *   race, and must be ordered by the caller (e.g. one stream). */
moe_status moe_layer_forward_noalloc(const moe_shape* shape, int32_t tokens,
                                     const void* x, int32_t x_dtype, uint32_t flags,
                                     float* router_logits, const moe_expert_table* table,
                                     void* out, int32_t out_dtype,
                                     moe_miss* miss, int32_t miss_cap, int32_t* miss_count,
                                     moe_stream_t stream);

/* Decode through `layers` chained layers in one call, for inputs whose
 * router logits are known for every layer when the call is made (the pages
 * verify 1 + 3 draft tokens through all 48 layers together, [AF] section
 * "命中率七成，代价是答案会变"; here the logits of every layer are inputs).
 * One kernel routes all layers at once (top-k, gates, the list of distinct
 * resident experts, miss lists and usage counts); then each layer runs the
 * same expert kernels as moe_layer_forward on its precomputed list, so a
 * layer no longer starts with a routing step.
 *   tokens:   1..4 (the decode path; 0 or layers == 0: nothing is launched).
 *   x:        device [tokens][d_model], x_dtype, the input of layer 0 (taken
 *             as it is).  Layer l > 0 takes layer l - 1's output with the
 *             RMS rule of MOE_FLAG_RMSNORM_INPUT.
 *   logits:   device fp32 [layers][tokens][n_experts], finite.
 *   tables:   host array of `layers` expert tables (as for
 *             moe_layer_forward; slot tables allowed, routers are not:
 *             MOE_EUNSUPPORTED).
 *   out:      device [layers][tokens][d_model], out_dtype: every layer's
 *             output (with a slot table, its partial output).
 *   miss, miss_count: required when any table has a slot table: device
 *             [layers][tokens*top_k] and [layers], filled per layer as
 *             moe_layer_forward fills them (NULL otherwise).
 *   ws:       device, moe_decode_stack_workspace_bytes(shape, layers,
 *             tokens) bytes, 256-byte aligned.
 * Same results as chaining moe_layer_forward calls with the RMS flag: bit
 * for bit with one token; with 2..4 the RMS factors are summed in another
 * order (a bf16 input value may differ by one unit in rare ties).
 * Validation, errors and determinism as for moe_layer_forward. */
size_t moe_decode_stack_workspace_bytes(const moe_shape* shape, int32_t layers, int32_t tokens);
moe_status moe_decode_stack_forward(const moe_shape* shape, int32_t layers, int32_t tokens,
                                    const void* x, int32_t x_dtype, const float* logits,
                                    const moe_expert_table* tables, void* out, int32_t out_dtype,
                                    moe_miss* miss, int32_t* miss_count, void* ws,
                                    size_t ws_bytes, moe_stream_t stream);

/* Host half of the slot-mode layer.  The pages compute the experts that are
 * not on the GPU with the CPU, at the same time as the GPU computes its own,
 * and add both into the same layer ([AF] section "命中率七成，代价是答案会
 * 变"; [SL] section "12GB 显存装下 1250 亿参数").  These run only for the
 * miss list of a slot-mode moe_layer_forward call; no GPU step falls back to
 * them. */

/* Opaque pool of worker threads for moe_host_miss_ffn, owned by the caller
 * (n_threads counts the calling thread: n_threads - 1 workers are started).
 * One moe_host_miss_ffn call at a time may use a pool.  Between calls the
 * workers poll for new work for about 100 us, then sleep.  Destroy joins the
 * workers. */
typedef struct moe_host_pool moe_host_pool;
moe_status moe_host_pool_create(int32_t n_threads, moe_host_pool** pool);
void moe_host_pool_destroy(moe_host_pool* pool);

/* Event for overlapping the host half with the GPU half.  `event` is a
 * hipEvent_t created by the caller (NULL clears a pending one).  The calling
 * thread's next moe_layer_forward call records it on its stream as soon as
 * the routing, the miss list and its count are written -- after the first
 * kernel (one token), the routing kernel (2..4 tokens) or the permutation
 * and miss-list kernels (more tokens), before the experts' FFNs run or
 * finish -- and then forgets it.  A caller that
 * waits for the event can copy the miss list and run moe_host_miss_ffn while
 * the GPU still computes the resident experts, as the pages' CPU and GPU
 * work on one layer at the same time ([AF] section "命中率七成，代价是答案会
 * 变").  Thread-local; no device work is done by this call itself. */
moe_status moe_set_route_event(void* event);

/* The row kernel moe_host_miss_ffn uses on this CPU: "avx512" (AVX-512F),
 * "avx2" (AVX2 + FMA) or "sse2", chosen from the CPU flags the kernel
 * reports; the environment variable MOE_HOST_SIMD=avx2 or =sse2 caps the
 * choice (read at every call).  The pages' CPU side uses AVX-512/AVX2 ([SL]
 * section "12GB 显存装下 1250 亿参数"). */
const char* moe_host_simd(void);

/* y[t] = sum over the misses of token t, in list order, of
 * gate * FFN_expert(xhat_t), for t < tokens (rows without misses are zero).
 *   x:        host [tokens][d_model], x_dtype MOE_BF16 or MOE_F32; flags as
 *             for moe_layer_forward (xhat = x, or the RMS rule computed on the
 *             host: an fp64 mean square, so a bf16 value may differ by one
 *             unit from the GPU's in rare ties).
 *   misses:   host, n_miss entries in (token, rank) order, as a slot-mode
 *             layer returns them (gates are the full top-k gates).
 *   experts:  host [n_experts] pointers to packed experts (the layout above,
 *             shape->qfmt) in host memory; the entry of every missed expert
 *             must be non-NULL.  The misses of a layer are random experts,
 *             read cold: memory backed by 2 MiB pages (madvise
 *             MADV_HUGEPAGE) spares those reads TLB misses (measured: a
 *             3-miss Q3S layer on 16 threads, 0.137 instead of 0.181 ms).
 *   y:        host fp32 [tokens][d_model], written in full.
 *   pool:     worker threads, or NULL for the calling thread alone.
 * fp32 throughout (weights exact in fp32).  Deterministic: each output
 * element is summed by one thread in a fixed order, whatever the pool size.
 * Synchronous; touches no GPU state. */
moe_status moe_host_miss_ffn(const moe_shape* shape, int32_t tokens, const void* x,
                             int32_t x_dtype, uint32_t flags, const moe_miss* misses,
                             int32_t n_miss, const void* const* experts, float* y,
                             moe_host_pool* pool);

/* out[i] += y[i] for i < tokens * d_model on the stream (out bf16, rounded
 * to nearest even after the add, or fp32; y device fp32): completes a
 * slot-mode layer output once the host's miss rows are on the device. */
moe_status moe_add_rows(void* out, int32_t out_dtype, const float* y, int32_t tokens,
                        int32_t d_model, moe_stream_t stream);

/* A whole slot-mode layer with the host computing the misses, in one call:
 * the pages' GPU computes the resident experts while the CPU computes the
 * others, and both go into the same layer ([AF] section "命中率七成，代价是
 * 答案会变"; [SL] section "12GB 显存装下 1250 亿参数").
 *
 * Enqueues moe_layer_forward on `stream` (partial layer and miss list, into
 * the workspace); as soon as the routing and the miss list are written they
 * reach `staging` with their count and the layer input, and the host
 * computes the missed experts' rows (moe_host_miss_ffn on `pool`) while the
 * GPU still computes the resident experts; then it enqueues their copy to
 * the workspace and their addition into `out` (moe_add_rows) on `stream`.
 * With 1..4 tokens the decode kernel that publishes the routing writes the
 * list, the count and the input into `staging` itself and then raises a
 * flag word there (a system-scope release), which the host polls: no event,
 * copy or synchronisation call stands between the routing and the host
 * rows.  With more tokens the layer records an event once its routing is
 * written, and a side stream of the calling thread copies them.  The call
 * returns once the host rows are computed; `out` holds the whole layer when
 * `stream` reaches that point.  Not for stream capture (it waits on the
 * host).
 *   shape, tokens, x (device), x_dtype, flags, router_logits, out,
 *   out_dtype: as moe_layer_forward; table->slot_of is required.
 *   host_experts: host [n_experts] pointers to every expert packed in host
 *             memory (as moe_host_miss_ffn's experts; NULL allowed for
 *             experts that are never missed).
 *   n_miss:   host int32 receiving the number of misses, or NULL.
 *   ws, ws_bytes: device workspace of moe_slot_host_workspace_bytes(shape,
 *             tokens) bytes, 256-byte aligned.
 *   staging, staging_bytes: page-locked host memory the device can address
 *             (hipHostMalloc; MOE_EINVAL otherwise) of
 *             moe_slot_host_staging_bytes(shape, tokens) bytes, 64-byte
 *             aligned.  Its host rows are read by the copy this call
 *             enqueues; a later call on the same stream overwrites them only
 *             after its own routing, which follows that copy.
 *   pool:     host worker threads, or NULL.
 * The side stream (non-blocking, default priority) and its event are
 * created on a thread's first call with more than 4 tokens on a device and
 * kept until the process ends.  Errors: those of moe_layer_forward;
 * MOE_EINVAL for a miss whose host expert is NULL (then nothing is added:
 * `out` stays the partial) or for pageable staging; MOE_EUNSUPPORTED while
 * `stream` is capturing; MOE_EHIP for a failed copy or wait, or a routing
 * that has not reached the host 10 s after the launch. */
size_t moe_slot_host_workspace_bytes(const moe_shape* shape, int32_t tokens);
size_t moe_slot_host_staging_bytes(const moe_shape* shape, int32_t tokens);
moe_status moe_slot_layer_forward_host(const moe_shape* shape, int32_t tokens, const void* x,
                                       int32_t x_dtype, uint32_t flags, float* router_logits,
                                       const moe_expert_table* table, void* out,
                                       int32_t out_dtype, const void* const* host_experts,
                                       int32_t* n_miss, void* ws, size_t ws_bytes,
                                       void* staging, size_t staging_bytes, moe_host_pool* pool,
                                       moe_stream_t stream);

/* Router projection (the router the pages keep resident on the GPU, [AF]
 * section "命中率七成，代价是答案会变"; they give no formula; reading taken:
 * an unquantised bf16 linear map without bias):
 *   logits[t][e] = sum_d W_r[e][d] * xhat[t][d],  accumulated in fp32,
 * xhat = x (flags 0) or bf16(x / sqrt(mean(x^2) + 1e-6)) (MOE_FLAG_RMSNORM_INPUT).
 *   x:        device [T][d_model], x_dtype MOE_BF16 or MOE_F32, 16-byte aligned.
 *   w_router: device bf16 [n_experts][d_model], 16-byte aligned.
 *   logits:   device fp32 [T][n_experts], 4-byte aligned; written in full.
 * T <= 4 with d_model <= 4096: a GEMV on the activations as given (fp32
 * input stays fp32).  Otherwise a bf16 MFMA
 * GEMM: fp32 input is rounded to bf16
 * first, exactly as the layer's prefill path rounds it, so that the logits
 * moe_layer_forward computes for the same input are the same bits.  Only
 * shape->d_model and shape->n_experts are used (and validated with the rest
 * of the shape).  T == 0 launches nothing. */
moe_status moe_router_logits(const moe_shape* shape, int32_t tokens, const void* x,
                             int32_t x_dtype, uint32_t flags, const void* w_router,
                             float* logits, moe_stream_t stream);

/* Resident-expert slot table (the GPU hot-expert cache of the pages, [AF]
 * section "命中率七成，代价是答案会变"; [JD] section "为什么从 18t/s 变成
 * 60-90t/s").  The caller owns all arrays; the host mirror lets updates be
 * validated without reading device memory. */
typedef struct {
  int32_t n_experts;
  int32_t n_slots;
  int32_t* slot_of;              /* device [n_experts], -1 = not resident */
  int32_t* expert_of_slot;       /* device [n_slots], -1 = empty */
  int32_t* host_slot_of;         /* host mirror of slot_of */
  int32_t* host_expert_of_slot;  /* host mirror of expert_of_slot */
  void* storage;                 /* device [n_slots][stride] packed experts */
  size_t stride;                 /* bytes per slot, multiple of 256 */
  size_t expert_bytes;           /* bytes copied per install (<= stride) */
} moe_slot_table;

/* Mark every slot empty and every expert non-resident (device arrays and
 * host mirror). */
moe_status moe_slot_table_init(moe_slot_table* t, moe_stream_t stream);

/* Install or evict n experts.  For each i: slots[i] is the slot to change;
 * experts[i] >= 0 installs that expert there (copying expert_bytes from
 * src[i], a device or pinned-host pointer, into the slot, and evicting the
 * slot's previous occupant); experts[i] == -1 only evicts.  `slots`,
 * `experts` and `src` are host arrays.  Rejected with MOE_EINVAL (nothing
 * changed): an id out of range, a slot named twice, an expert named twice,
 * an expert that is already resident in a slot this call does not change,
 * a NULL src for an install.  Copies and map edits are ordered on the
 * stream, so a later moe_layer_forward on the same stream sees them; the
 * host mirror is updated before return. */
moe_status moe_slot_table_update(moe_slot_table* t, int32_t n, const int32_t* slots,
                                 const int32_t* experts, const void* const* src,
                                 moe_stream_t stream);

/* Frequency-driven slot policy with fills that overlap the layers.  The pages
 * swap experts while serving, moving an expert onto the GPU once it starts to
 * be used often, and report a higher hit rate for that than for a fixed set
 * chosen from the overall frequency curve ([AF] section "命中率七成，代价是
 * 答案会变").  They give no algorithm; the reading implemented here:
 *   - statistics: use_count (see moe_expert_table) counts routed pairs; each
 *     period the caller takes a snapshot and halves the counts, so the score
 *     of an expert is its usage with a weight of 1/2 per period of age;
 *   - plan: the non-resident experts with a nonzero score, hottest first
 *     (ties: lower id), are paired with the resident experts, coldest first
 *     (ties: lower id), and with the empty slots in ascending order; pair i is
 *     a swap while score(candidate i) > score(victim i) + margin, at most
 *     max_swaps of them;
 *   - fills: the admitted experts are copied into empty (spare) slots, which
 *     no layer reads, on a side stream while later layers run; a map-only
 *     commit on the layer stream then installs them and evicts the victims,
 *     whose slots become the spares of the next period.
 * A table built for this keeps n_slots = resident + spare slots. */

/* Copy use_count [n] to host_out (host memory; pinned for an asynchronous
 * copy), then halve every device count.  Both are ordered on the stream; the
 * caller synchronises before reading host_out. */
moe_status moe_slot_counts_take(uint32_t* use_count, int32_t n, uint32_t* host_out,
                                moe_stream_t stream);

/* Plan up to max_swaps swaps from the scores `counts` (host [n_experts]) and
 * the table's host mirrors (rule above).  Writes admit[i] (expert to
 * install), evict[i] (resident expert to evict) and slots[i] (empty slot for
 * the admitted expert), i < *n_swaps.  Host only; deterministic; changes
 * nothing in the table. */
moe_status moe_slot_policy_plan(const moe_slot_table* t, const uint32_t* counts,
                                int32_t max_swaps, uint32_t margin, int32_t* admit,
                                int32_t* evict, int32_t* slots, int32_t* n_swaps);

/* Copy the packed bytes of experts[i] from src[i] (device or pinned host)
 * into slots[i], for i < n, without touching the maps: the slots must be
 * empty (expert_of_slot == -1 in the host mirror) and stay so until the
 * matching moe_slot_table_commit, so no layer reads them meanwhile.  The
 * experts must be distinct and not resident, the slots distinct
 * (MOE_EINVAL otherwise, nothing enqueued).  The caller must not stage into
 * a slot again before committing it. */
moe_status moe_slot_table_stage(moe_slot_table* t, int32_t n, const int32_t* slots,
                                const int32_t* experts, const void* const* src,
                                moe_stream_t stream);

/* Map-only install of staged experts: experts[i] becomes resident in
 * slots[i] (empty, its bytes already staged and the copy ordered before this
 * call, e.g. by an event), and evict[i] (a resident expert, or -1; evict may
 * be NULL) stops being resident, its slot becoming empty.  Validated as for
 * moe_slot_table_stage, plus: each evicted expert resident and named once.
 * The map edits are ordered on the stream; the host mirror is updated before
 * return. */
moe_status moe_slot_table_commit(moe_slot_table* t, int32_t n, const int32_t* slots,
                                 const int32_t* experts, const int32_t* evict,
                                 moe_stream_t stream);


/* Routing alone (the first step of the layer; each token keeps the k
 * experts its router ranks highest, [AF] section "1250 亿参数，每个词只用得
 * 上 2%"; the pages give no gate formula, the reading is in the preamble):
 * device fp32 logits [T][E] (finite) -> device int32 idx [T][k] (descending
 * logit, ties to the lower id, -0.0 == +0.0) and fp32 gates [T][k] (softmax
 * over the k selected logits).  Rejects T < 0, E outside 1..2048, k outside
 * 1..min(32, E) and NULL buffers (T > 0) with MOE_EINVAL before any launch.
 * The caller owns all three buffers. */
moe_status moe_route(const float* logits, int32_t tokens, int32_t n_experts, int32_t top_k,
                     int32_t* idx, float* gate, moe_stream_t stream);

/* Stable token-to-expert permutation of routed pairs p = t*k + j: the step
 * that groups a prefill chunk's rows by expert so that each expert's weights
 * are read once for all its tokens ([AF] section "等最久的，是它读完你的代码";
 * the pages give no algorithm: histogram, prefix scans, stable scatter):
 *   offsets [E+1]: offsets[e] = number of pairs routed to experts < e;
 *   sorted_pairs [T*k]: pair ids grouped by expert, ascending within a group;
 *   inv [T*k]: inv[p] = position of p in sorted_pairs.
 * All device int32.  ws: moe_permute_workspace_bytes(T, k, E) bytes. */
size_t moe_permute_workspace_bytes(int32_t tokens, int32_t top_k, int32_t n_experts);
moe_status moe_permute(const int32_t* idx, int32_t tokens, int32_t top_k, int32_t n_experts,
                       int32_t* offsets, int32_t* sorted_pairs, int32_t* inv,
                       void* ws, size_t ws_bytes, moe_stream_t stream);

/* Profiling aid: time the dominant kernel of the calling thread's next
 * moe_layer_forward call.  `before` and `after` are hipEvent_t handles
 * created by the caller with timing enabled.  The forward call attaches both
 * to the launch of its dominant kernel (decode path: the gate/up GEMV;
 * prefill path: the gate/up grouped GEMM) through hipExtLaunchKernel, so
 * they take that kernel's own start and end timestamps, then forgets both.
 * A forward call on a stream that is capturing a graph fails while a pair is
 * armed (MOE_EHIP: stream capture unsupported).  NULL, NULL clears a pending
 * pair.  Thread-local; no device work is done by this call itself. */
moe_status moe_set_kernel_timer(void* before, void* after);

/* The same for the router projection kernel: the pair is attached to the
 * next router launch of the calling thread, from moe_router_logits or from a
 * moe_layer_forward call whose table has a router.  Independent of the pair
 * of moe_set_kernel_timer; same rules. */
moe_status moe_set_router_timer(void* before, void* after);

/* The calling thread's message for its last failed call ("" if none). */
const char* moe_last_error(void);

/* ABI version of this header. */
#define MOE_ABI_VERSION 4
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
