// Decode path of the MoE layer (1..4 tokens: single-token decode and the
// 4-token verification batch of multi-token prediction).
//
// The pages: per token only the 10 selected experts plus the shared expert
// are touched ([AF] "个人开发者用 AI 十天写出 Strata 引擎…", section
// "1250 亿参数，每个词只用得上 2%"); speed is set by moving expert weights
// ([JD] "5070ti16g单卡跑qwen 3.8 flash next …", section "为什么从 18t/s 变成
// 60-90t/s"; [KC-en] "Running Qwen3.8-Flash-Next on a 12GB GPU…", section
// "Hardware Configuration and Quantization Approach"); the verification
// batch runs 1 + 3 draft tokens through the layers together ([AF] section
// "命中率七成，代价是答案会变").  So the kernels stream each distinct selected
// expert's packed bytes exactly once for all tokens that chose it.
//
// The list of experts a call computes holds the shared expert first (index
// 0, when there is one), then the distinct resident routed experts in order
// of first occurrence over (token, rank).
//
// Two launches (three with 2..4 tokens):
//   decode_list:    2..4 tokens only, one block: wave t routes token t, wave
//                   0 builds and publishes the list and the miss list.
//   decode_gateup:  blocks [0, d_ff_shared/16) compute 16 FFN rows of the
//                   shared expert each and stream its weights at once.  The
//                   other blocks are (routed list entry, 16 FFN rows).  With
//                   one token they route it themselves first (every wave, so
//                   each wave knows its expert without waiting for another;
//                   the first routed block publishes the list for the down
//                   kernel); with 2..4 tokens they read their entry of the
//                   published list.  Then: dequantising MFMA GEMV of W_gate
//                   and W_up, SwiGLU, h in bf16 hi + lo with per-block sums.
//   decode_down:    one block per 16 output rows: W_down GEMV of every listed
//                   expert, gate-weighted sum in list order, output write.
//
// Dequantisation (see DqConsts): a code word is turned into bf16 operands
// (c + u) with one VALU op per pair of weights plus shared shifts and no
// conversion; the MFMA sums (c + u) * x over one 32-weight block; the block
// result is scaled by the fp16 block scale, and the constant parts (c * x,
// and the block min times sum x) come from per-block activation sums.
#include "route_common.hpp"

namespace moe {

namespace {

constexpr int kGuWaves = 4;        // routing blocks (list and plan kernels): 4 waves
constexpr int kGuThreads = 64 * kGuWaves;
// Gate/up block: 16 FFN rows; the reduction over d_model of each matrix
// (gate, up) is split kGuSplit ways, one wave each.
constexpr int kGuSplit = 4;
constexpr int kGuBlkWaves = 2 * kGuSplit;
constexpr int kGuBlkThreads = 64 * kGuBlkWaves;
constexpr int kDnWaves = 16;       // down block: waves share the expert list
constexpr int kMaxOctPerWave = 16 / kGuSplit;  // d_model <= 4096 on the decode path (16 octets)
constexpr int kMaxDecodeFOct = 2;  // d_ff, d_ff_shared <= 512 on the decode path
// Down-record prefetch loads per gate/up thread (one 64-byte line each):
// 32 KiB per block, a block's whole share up to d_model 4096 in every
// format (at most 28 KiB).
constexpr int kDnPrefetchPerThread = 2;

// Activation modes of the gate/up kernel.
constexpr int kXBf16 = 0;  // bf16 input, used as is
constexpr int kXF32 = 1;   // fp32 input, as bf16 hi + bf16 lo (two MFMAs)
constexpr int kXRms = 2;     // bf16 input normalised to bf16(x / sqrt(mean(x^2) + 1e-6))
constexpr int kXRmsF32 = 3;  // fp32 input, same rule

__host__ __device__ inline size_t align256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

size_t decode_ws_bytes(int T, int D, int F, int Fs, int E, int k) {
  const int Wmax = (E < T * k ? E : T * k) + 1;
  const int Fp = 256 * (octets(F) > octets(Fs) ? octets(F) : octets(Fs));
  size_t b = 0;
  b += align256(4 * (size_t)T * k) * 2;               // idx, gate
  b += 256;                                           // nwork
  b += align256(4 * (size_t)Wmax);                    // work_ref
  b += align256(16 * (size_t)Wmax);                   // work_gate
  b += align256(2 * (size_t)Wmax * T * Fp) * 2;       // hh, hl
  b += align256(16 * (size_t)Wmax * T * (Fp / 32));   // hs
  b += 256;                                           // rinv
  return b;
}

DecodeWs decode_ws_carve(void* ws, int T, int D, int F, int Fs, int E, int k) {
  DecodeWs w;
  w.Wmax = (E < T * k ? E : T * k) + 1;
  w.Fp = 256 * (octets(F) > octets(Fs) ? octets(F) : octets(Fs));
  uint8_t* p = (uint8_t*)ws;
  auto take = [&](size_t n) { uint8_t* r = p; p += align256(n); return (void*)r; };
  w.idx = (int32_t*)take(4 * (size_t)T * k);
  w.gate = (float*)take(4 * (size_t)T * k);
  w.nwork = (int32_t*)take(4);
  w.work_ref = (int32_t*)take(4 * (size_t)w.Wmax);
  w.work_gate = (float*)take(16 * (size_t)w.Wmax);
  w.hh = (uint16_t*)take(2 * (size_t)w.Wmax * T * w.Fp);
  w.hl = (uint16_t*)take(2 * (size_t)w.Wmax * T * w.Fp);
  w.hs = (float2*)take(16 * (size_t)w.Wmax * T * (w.Fp / 32));
  w.rinv = (float*)take(4 * kDecodeMaxT);
  return w;
}

size_t decode_plan_bytes(int T, int E, int k) {
  const int Wmax = (E < T * k ? E : T * k) + 1;
  return align256(4 * (size_t)T * k) * 2 + 256 + align256(4 * (size_t)Wmax) +
         align256(16 * (size_t)Wmax);
}

// ----------------------------------------------------------------------------
// Routing inside a decode block.

// Routing results of 2..4 tokens and the list built from them.
struct RouteLds {
  int32_t e[kDecodeMaxT * kMaxTopK];
  float g[kDecodeMaxT * kMaxTopK];
  int32_t ref[kDecodeMaxT * kMaxTopK + 1];
  float wg[(kDecodeMaxT * kMaxTopK + 1) * 4];
  int32_t nu;
};

// Top-k of token t by the calling wave: lane j < k gets the j-th expert and
// its gate.  The id is clamped into 0..E-1 (it always is for finite logits;
// the clamp keeps a wild id out of the weight addresses).
__device__ __forceinline__ void route_token(const DecodeArgs& a, int t, int lane, TopkScratch& S,
                                            int& e, float& g) {
  float l;
  wave_topk_any(a.logits + (size_t)t * a.E, a.E, a.k, lane, S, e, l);
  g = wave_gate(l, a.k, lane);
  e = e < 0 ? 0 : (e >= a.E ? a.E - 1 : e);
}

// Slot of expert e, or -1 when not resident (a slot outside 0..n_slots-1 in
// the caller's map counts as not resident, so it is never dereferenced).
__device__ __forceinline__ int resident_ref(const DecodeArgs& a, int e) {
  if (a.slot_of == nullptr) return e;
  const int s = a.slot_of[e];
  return (s >= 0 && s < a.n_slots) ? s : -1;
}

// The routing outcome into the caller's page-locked staging (HostPub), by
// the publishing wave once its miss records are written there too: the count
// and the layer input, then -- after a system-scope release fence by every
// lane, so that all the wave's stores are out -- the flag the host polls.
__device__ __forceinline__ void publish_host(const DecodeArgs& a, int lane, int nmiss) {
  const HostPub& p = a.pub;
  if (lane == 0) *p.count = nmiss;
  const int n16 = a.T * a.D * (a.x_bf16 ? 2 : 4) / 16;
  const uint4* src = reinterpret_cast<const uint4*>(a.x);
  uint4* dst = reinterpret_cast<uint4*>(p.x);
  for (int i = lane; i < n16; i += 64) dst[i] = src[i];
  __threadfence_system();  // the wave's stores reach host memory before the flag
  __builtin_amdgcn_wave_barrier();
  if (lane == 0) __hip_atomic_store(p.flag, p.seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

// One token: lane j < k holds expert e, gate g and residency ref (-1 = miss);
// `hits` has bit j set for resident ranks.  Hit i (in rank order) is list
// entry base + i.  Writes the list, the routing and the miss list.
__device__ __forceinline__ void publish_t1(const DecodeArgs& a, const DecodeWs& w, int lane, int e,
                                           float g, int ref, unsigned long long hits, int base) {
  const int k = a.k;
  const unsigned long long below = (1ull << lane) - 1ull;
  const unsigned long long kmask = (1ull << k) - 1ull;  // k <= 32
  if (lane < k) {
    w.idx[lane] = e;
    w.gate[lane] = g;
    if (a.use_count) atomicAdd(&a.use_count[e], 1u);
    if ((hits >> lane) & 1ull) {
      const int i = base + __popcll(hits & below);
      w.work_ref[i] = ref;
      w.work_gate[4 * i] = g;
    } else {
      MissRec r;
      r.token = 0;
      r.rank = lane;
      r.expert = e;
      r.gate = g;
      a.miss[__popcll(~hits & kmask & below)] = r;
      if (a.pub.flag) a.pub.miss[__popcll(~hits & kmask & below)] = r;
    }
  }
  if (lane == 0) {
    if (base) {
      w.work_ref[0] = -1;
      w.work_gate[0] = 1.0f;
    }
    *w.nwork = base + __popcll(hits);
    if (a.miss_count) *a.miss_count = k - __popcll(hits);
  }
  if (a.pub.flag) publish_host(a, lane, k - __popcll(hits));
}

// 2..4 tokens, wave 0, once every token's routing is in R.e / R.g.  The
// first occurrence of each resident expert comes from a table in LDS indexed
// by expert (only the entries of named experts are touched): every pair
// stores INT_MAX, then each hit takes the atomic minimum of its pair index.
// Builds R.ref / R.wg / R.nu (shared entry first when base = 1); `publish`
// also writes them, the routing and the miss list to the workspace.
template <int T>
__device__ __forceinline__ void build_list(const DecodeArgs& a, const DecodeWs& w, RouteLds& R,
                                           int32_t* s_first, int lane, bool publish, int base) {
  const int k = a.k, P = T * k;  // P <= 128: lane handles pairs lane, lane + 64
  int e[2], ref[2], tok[2], first[2];
  bool valid[2], hit[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int p = lane + 64 * h;
    valid[h] = p < P;
    e[h] = valid[h] ? R.e[p] : 0;
    ref[h] = valid[h] ? resident_ref(a, e[h]) : -1;
    hit[h] = valid[h] && ref[h] >= 0;
    tok[h] = (p >= k ? 1 : 0) + (p >= 2 * k ? 1 : 0) + (p >= 3 * k ? 1 : 0);
    if (valid[h]) s_first[e[h]] = 0x7FFFFFFF;
  }
  wave_lds_fence();
#pragma unroll
  for (int h = 0; h < 2; ++h)
    if (hit[h]) atomicMin(&s_first[e[h]], lane + 64 * h);
  wave_lds_fence();
  unsigned long long bf[2], bm[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int p = lane + 64 * h;
    first[h] = hit[h] ? s_first[e[h]] : -1;
    bf[h] = __ballot(hit[h] && first[h] == p);
    bm[h] = __ballot(valid[h] && !hit[h]);
  }
  const int nf0 = __popcll(bf[0]), nm0 = __popcll(bm[0]);
  const int U = nf0 + __popcll(bf[1]);
  const int M = nm0 + __popcll(bm[1]);
  const int nu = base + U;
  for (int i = lane; i < nu * 4; i += 64) R.wg[i] = 0.f;
  wave_lds_fence();
  auto list_index = [&](int fp) {  // list entry of the pair that first named an expert
    const unsigned long long m = fp >= 64 ? bf[1] : bf[0];
    return base + (fp >= 64 ? nf0 : 0) + __popcll(m & ((1ull << (fp & 63)) - 1ull));
  };
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int p = lane + 64 * h;
    if (hit[h] && first[h] == p) R.ref[list_index(p)] = ref[h];
    if (hit[h]) R.wg[list_index(first[h]) * 4 + tok[h]] = R.g[p];
  }
  if (lane == 0) {
    R.nu = nu;
    if (base) R.ref[0] = -1;
  }
  if (base && lane < T) R.wg[lane] = 1.0f;
  wave_lds_fence();
  if (!publish) return;
  for (int i = lane; i < nu; i += 64) w.work_ref[i] = R.ref[i];
  for (int i = lane; i < nu * 4; i += 64) w.work_gate[i] = R.wg[i];
  for (int i = lane; i < P; i += 64) {
    w.idx[i] = R.e[i];
    w.gate[i] = R.g[i];
    if (a.use_count) atomicAdd(&a.use_count[R.e[i]], 1u);
  }
  if (lane == 0) {
    *w.nwork = nu;
    if (a.miss_count) *a.miss_count = M;
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int p = lane + 64 * h;
    if (valid[h] && !hit[h]) {
      MissRec r;
      r.token = tok[h];
      r.rank = p - tok[h] * k;
      r.expert = e[h];
      r.gate = R.g[p];
      a.miss[(h ? nm0 : 0) + __popcll(bm[h] & ((1ull << lane) - 1ull))] = r;
      if (a.pub.flag) a.pub.miss[(h ? nm0 : 0) + __popcll(bm[h] & ((1ull << lane) - 1ull))] = r;
    }
  }
  if (a.pub.flag) publish_host(a, lane, M);
}

// ----------------------------------------------------------------------------
// Block parameter helpers.  Q2SM: the two 16-byte parameter loads of a record
// row hold (scale, min) for blocks 0..3 and 4..7.  Q3S and Q2S: one 16-byte
// load holds the 8 scales.
__device__ __forceinline__ uint32_t sel4(const uint4 v, int i) {
  // word i of v by three byte permutes whose selectors depend only on i
  // (loop-invariant per lane): with a lane-dependent index a chain of
  // compares became divergent branches, and a select could become a load
  // from a stack copy of v
  const uint32_t s1 = (i & 1) ? 0x07060504u : 0x03020100u;
  const uint32_t s2 = (i & 2) ? 0x07060504u : 0x03020100u;
  const uint32_t lo = __builtin_amdgcn_perm(v.y, v.x, s1), hi = __builtin_amdgcn_perm(v.w, v.z, s1);
  return __builtin_amdgcn_perm(hi, lo, s2);
}
// Word i of v for an index known at compile time (after unrolling): a plain
// register pick.
__device__ __forceinline__ uint32_t sel4c(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}
template <int FMT>
__device__ __forceinline__ float blk_scale(const uint4& pa, const uint4& pb, int beta) {
  if (FMT == kQ2) {
    const uint32_t v = beta < 4 ? sel4c(pa, beta) : sel4c(pb, beta - 4);
    return f16_to_f32((uint16_t)(v & 0xFFFFu));
  } else {
    const uint32_t v = sel4c(pa, beta >> 1);
    return f16_to_f32((uint16_t)((beta & 1) ? (v >> 16) : (v & 0xFFFFu)));
  }
}

// One record (16 rows x 8 blocks) of one wave: MFMA over the 8 blocks with
// activation fragments fetched by `xfrag(beta, hi_or_lo)`; accumulates
// scale * block result into acc (lanes 0..15 hold tokens 0..T-1), and the
// lane's share of the constant terms (blocks beta = q and q + 4) into mt.
// The activation fragments of HB blocks at a time are read first (every read
// is in range: the staging regions hold whole octets) and their MFMAs follow,
// so the LDS latencies overlap; HB trades that against registers.  Blocks at
// or past nvalid (a partial last octet) are computed on whatever the region
// holds and dropped by selects, not branches.  FULL: nvalid == 8.
template <int T, int FMT, bool HAS_LO, bool FULL = false, int HB = 8, typename XFrag,
          typename XSum>
__device__ __forceinline__ void record_gemv(const uint4& cw, const uint2& hw, const uint4& pa,
                                            const uint4& pb, int nvalid, const DqConsts& kc,
                                            XFrag xfrag, XSum xsum, float (&acc)[T],
                                            float (&mt)[T], int q) {
  const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
  const uint32_t hws[2] = {hw.x, hw.y};
  static_assert(HB == 1 || HB == 2 || HB == 4 || HB == 8, "blocks per read batch");
  if constexpr (HB == 1) {  // least registers: each block read where it is used
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      uint4 ea, eb;
      if (FMT != kQ3)
        dq_q2(words[wd], kc, ea, eb);
      else
        dq_q3(words[wd], hws[wd >> 1], (wd & 1) != 0, kc, ea, eb);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int beta = 2 * wd + half;
        if (FULL || beta < nvalid) {
          const uint4 bop = half ? eb : ea;
          f32x4_t d = {0.f, 0.f, 0.f, 0.f};
          d = mfma16(xfrag(beta, false), bop, d);
          if (HAS_LO) d = mfma16(xfrag(beta, true), bop, d);
          const float s = blk_scale<FMT>(pa, pb, beta);
#pragma unroll
          for (int r = 0; r < T; ++r) acc[r] += s * d[r];
        }
      }
    }
  } else {
#pragma unroll
    for (int b0 = 0; b0 < 8; b0 += HB) {
      uint4 xh[HB], xl[HB];
#pragma unroll
      for (int j = 0; j < HB; ++j) {
        xh[j] = xfrag(b0 + j, false);
        xl[j] = HAS_LO ? xfrag(b0 + j, true) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int wd = b0 / 2; wd < (b0 + HB) / 2; ++wd) {
        uint4 ea, eb;
        if (FMT != kQ3)
          dq_q2(words[wd], kc, ea, eb);
        else
          dq_q3(words[wd], hws[wd >> 1], (wd & 1) != 0, kc, ea, eb);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int beta = 2 * wd + half;
          const uint4 bop = half ? eb : ea;
          f32x4_t d = {0.f, 0.f, 0.f, 0.f};
          d = mfma16(xh[beta - b0], bop, d);
          if (HAS_LO) d = mfma16(xl[beta - b0], bop, d);
          const float s = blk_scale<FMT>(pa, pb, beta);
          const bool on = FULL || beta < nvalid;
#pragma unroll
          for (int r = 0; r < T; ++r) acc[r] += on ? s * d[r] : 0.f;
        }
      }
    }
  }
  // Constant terms of this lane's two blocks.
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int beta = q + 4 * hb;
    const bool on = FULL || beta < nvalid;
    float s, m;
    if (FMT == kQ2) {
      const uint32_t v = sel4(hb ? pb : pa, q);
      s = f16_to_f32((uint16_t)(v & 0xFFFFu));
      m = f16_to_f32((uint16_t)(v >> 16));
    } else {
      const uint32_t v = sel4(pa, beta >> 1);
      s = f16_to_f32((uint16_t)((beta & 1) ? (v >> 16) : (v & 0xFFFFu)));
      m = 0.f;
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float2 X = xsum(beta, t);
      // Q2SM: s*(sum (c+u)x - sum cx) + m*sum x; Q3S and Q2S: the code offset
      // (4 or 2) folds into the same correction.
      const float c = FMT == kQ2 ? m * X.x - s * X.y
                                 : -s * (X.y + (FMT == kQ3 ? 4.0f : 2.0f) * X.x);
      mt[t] += on ? c : 0.f;
    }
  }
}

template <int FMT>
__device__ __forceinline__ void load_record(const uint8_t* rec, int lane, uint4& cw, uint2& hw,
                                            uint4& pa, uint4& pb) {
  const int n = lane & 15;
  cw = *reinterpret_cast<const uint4*>(rec + 16 * lane);
  if (FMT == kQ2) {
    pa = *reinterpret_cast<const uint4*>(rec + 1024 + 32 * n);
    pb = *reinterpret_cast<const uint4*>(rec + 1024 + 32 * n + 16);
    hw = make_uint2(0, 0);
  } else if (FMT == kQ3) {
    hw = *reinterpret_cast<const uint2*>(rec + 1024 + 8 * lane);
    pa = *reinterpret_cast<const uint4*>(rec + 1536 + 16 * n);
    pb = make_uint4(0, 0, 0, 0);
  } else {
    pa = *reinterpret_cast<const uint4*>(rec + 1024 + 16 * n);
    pb = make_uint4(0, 0, 0, 0);
    hw = make_uint2(0, 0);
  }
}

// Sums over groups of 4 / 8 consecutive lanes (DPP quad swaps, half-row
// mirror); every lane of the group gets the group sum.
__device__ __forceinline__ float dpp_add(float v, uint32_t other) { return v + __uint_as_float(other); }
__device__ __forceinline__ float quad_sum(float v) {
  v = dpp_add(v, dpp_u32<kDppQuadSwap1, 0xF>(0u, __float_as_uint(v)));
  return dpp_add(v, dpp_u32<kDppQuadSwap2, 0xF>(0u, __float_as_uint(v)));
}
__device__ __forceinline__ float oct_sum(float v) {
  v = quad_sum(v);
  return dpp_add(v, dpp_u32<kDppRowHalfMirror, 0xF>(0u, __float_as_uint(v)));
}

// ----------------------------------------------------------------------------
// Direct global -> LDS load: lane l's 16 bytes land at lds + 16 l (`lds` the
// same for the whole wave); counts in vmcnt.
typedef __attribute__((address_space(3))) void dn_lds_t;
__device__ __forceinline__ void dn_dma16(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds(src, (dn_lds_t*)lds, 16, 0, 0);
}
// Wait until no vector-memory operation of this wave is in flight.
__device__ __forceinline__ void dn_wait_vm0() {
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0); expcnt, lgkmcnt not waited
}
// Workgroup barrier over LDS: this wave's LDS stores complete (lgkmcnt(0)),
// then s_barrier, without the release/acquire fences of __syncthreads, which
// count direct global -> LDS loads as LDS writes and would drain the down-
// record prefetch in flight.  The compiler barriers keep LDS accesses on
// their side of it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0) only
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Cache warm-up of an expert's down-projection records for decode_down.
// Down block rt (16 output rows) runs on the XCD of its block index modulo
// 8: every launch sends block i to XCD (i + c) mod 8 with the same c for
// all launches of a stream (measured: c = 0 for launches, c = 7 inside a
// graph replay), so blocks of two launches whose indices agree modulo 8
// share an XCD and its L2.  The gate/up block vb of expert u therefore reads
// the records of the down rows rt with rt = vb (mod 8), shared out among the
// expert's gate/up blocks of that residue class: one 4-byte load per 64-byte
// line.  The L2 copies do not survive to the down kernel (its HBM-side
// fetch, FETCH_SIZE, still equals its records, 6.8 MB per one-token layer:
// the L2s are invalidated between kernels); what the down kernel finds is the
// line in the Infinity Cache (MALL), a shorter round trip than to HBM.  The loaded words are only kept alive to the end of the block (see
// keep_alive), so nothing waits for them before then.  Only where the bytes
// are cached depends on this placement, never a result.
struct DnPrefetch {
  uint32_t v[kDnPrefetchPerThread];
};
__device__ __forceinline__ DnPrefetch prefetch_down_rows(const uint8_t* expert, int D, int Fu,
                                                         int fmt_rec, size_t down_off, int vb,
                                                         int base, int ngroups, int tid,
                                                         int threads) {
  DnPrefetch p;
  const int c = vb & 7;
  const int g = vb - base;                  // this block's 16-row group of the expert
  const int g0 = (c - base % 8 + 8) % 8;    // first group of residue class c
  const int nG = ngroups > g0 ? (ngroups - g0 + 7) / 8 : 0;
  const int j = (g - g0) / 8;               // this block's index in its class
  const int nRt = D / 16, nR = nRt > c ? (nRt - c + 7) / 8 : 0;
  const int mine = nG > 0 && nR > j ? (nR - j + nG - 1) / nG : 0;  // row groups j, j + nG, ...
  const int oF = octets(Fu);
  const int lines = oF * fmt_rec / 64;      // 64-byte lines of one row group's records
  const int total = mine * lines;
  // A fixed number of loads per thread (so the compiler can count them);
  // lines past the block's share repeat its last line, a share larger than
  // kDnPrefetchPerThread * threads lines is cut (this is only a warm-up),
  // and a block without a share reads its own expert's first down line.
  const uint32_t* dn = reinterpret_cast<const uint32_t*>(expert + down_off);
#pragma unroll
  for (int r = 0; r < kDnPrefetchPerThread; ++r) {
    int q = tid + threads * r;
    q = total == 0 ? 0 : (q < total ? q : total - 1);
    const int rt = total == 0 ? 0 : c + 8 * (j + nG * (q / lines));
    p.v[r] = dn[((size_t)rt * oF * fmt_rec + 64 * (q % lines)) / 4];
  }
  return p;
}
// Hold the prefetched words until here, so their loads are waited for at
// the end of the block and nowhere earlier.
__device__ __forceinline__ void keep_alive(const DnPrefetch& p) {
#pragma unroll
  for (int r = 0; r < kDnPrefetchPerThread; ++r) asm volatile("" ::"v"(p.v[r]));
}

// Two fp32 values rounded to nearest even bf16 and packed (lo in bits 0..15):
// one v_cvt_pk_bf16_f32, the same bits as f32_to_bf16 for finite values.
typedef __bf16 dq_bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t rne_pk_bf16(float lo, float hi) {
  const dq_bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// ----------------------------------------------------------------------------
// decode_gateup.  Grid: d_ff_shared/16 shared-expert blocks, then
// (routed list capacity x d_ff/16) blocks, of 512 threads, two blocks per
// CU.  A routed block first routes (see above) and drops out when its list
// entry is not used.  Then every block issues its weight loads -- wave w
// holds matrix w / kGuSplit (gate, up) over the K octets o = w % kGuSplit,
// + kGuSplit, ... of one 16-row h-group -- and, while they are in flight,
// the activation loads, the input rule, the bf16 operand(s) in LDS and the
// per-32-block activation sums.  Splitting each matrix's reduction four ways
// rather than two halves the GEMV work of a wave (at d_model 3072, 3 octets
// instead of 6: the dequantising GEMV of one wave costs a few microseconds
// of issue at one or two waves per SIMD) and doubles the waves that can
// hide one another's waits.
// Static LDS of a gate/up block.
struct GuLds {
  RouteLds R;
  TopkScratch topk[kGuBlkWaves];
  float red[kGuBlkWaves][kDecodeMaxT][16];
  float ss[kGuBlkWaves][kDecodeMaxT];
};

// Gate/up work item vb (the block index of decode_gateup_kernel).  Returns
// early, with the same decision in every wave, when its list entry is unused.
// OPW > 0: every wave has exactly OPW octets (d_model = 512 OPW), so its
// record loads are unconditional.  With conditional loads (OPW = 0, any
// d_model) the compiler cannot count the loads issued after the
// activations, and its wait before staging them drains every record: the
// GEMV then starts only once the last record has landed.  With a fixed
// count the staging waits for the activations alone and each octet's GEMV
// waits for its own record.
template <int T, int FMT, int XM, bool PLANNED, int OPW>
__device__ __forceinline__ void gateup_body(const DecodeArgs& a, const DecodeWs& w, int vb,
                                            GuLds& L, uint4* s_dyn) {
  RouteLds& R = L.R;
  auto& s_topk = L.topk;
  auto& s_red = L.red;
  auto& s_ss = L.ss;
  constexpr bool HAS_LO = XM == kXF32;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int D = a.D, oD = octets(D), nbD = D / 32, D8 = D / 8;
  // Token rows of the staged activations are D8p 16-byte pieces apart: one
  // piece more than a row when T > 1, so that the rows one fragment read
  // touches fall on different LDS banks (D/8 pieces is a multiple of the bank
  // cycle for every supported d_model).
  const int D8p = D8 + (T > 1 ? 1 : 0);
  uint4* s_xhi = s_dyn;                                                          // [T][D8p]
  uint4* s_xlo = s_dyn + T * D8p;                                                // [T][D8p]
  float2* s_xs = reinterpret_cast<float2*>(s_dyn + (HAS_LO ? 2 : 1) * T * D8p);  // [T][D/32]

  // 0. This block's work: shared-expert rows, or a routed list entry.
  const int has_sh = a.shared != nullptr;
  const int nsh = has_sh ? a.Fs / 16 : 0;
  const int gpr = a.F / 16;
  int u, g;
  const uint8_t* eb;
  if (vb < nsh) {
    u = 0;
    g = vb;
    eb = a.shared;
  } else {
    const int rb = vb - nsh;
    const int ui = rb / gpr;
    g = rb % gpr;
    int ref;
    if (T == 1 && !PLANNED) {
      int e;
      float gt;
      route_token(a, 0, lane, s_topk[wv], e, gt);
      const int rl = lane < a.k ? resident_ref(a, e) : -1;
      const unsigned long long hits = __ballot(lane < a.k && rl >= 0);
      if (rb == 0 && wv == 0) publish_t1(a, w, lane, e, gt, rl, hits, has_sh);
      if (ui >= __popcll(hits)) return;  // same in every wave of the block
      const unsigned long long below = (1ull << lane) - 1ull;
      const unsigned long long pick =
          __ballot(((hits >> lane) & 1ull) && __popcll(hits & below) == ui);
      ref = __builtin_amdgcn_readlane(rl, __builtin_ctzll(pick));
    } else {  // the list was built by decode_list_kernel or decode_plan_kernel
      // The entry (has_sh + ui < Wmax for every block of the grid) is read
      // together with the count, not after it: one round trip instead of two.
      const int nu = *w.nwork;
      ref = w.work_ref[has_sh + ui];
      asm volatile("" ::"v"(ref));  // keeps the load ahead of the branch
      if (has_sh + ui >= nu) return;
    }
    u = has_sh + ui;
    eb = a.routed + (size_t)ref * a.stride;
  }

  // 1. Activations first (16-byte pieces; every element defined, so the
  // array stays in registers): loads complete in the order they are issued,
  // so the staging below waits for these and not for the weights.
  constexpr bool in_bf16 = XM == kXBf16 || XM == kXRms;
  constexpr bool RMS = XM == kXRms || XM == kXRmsF32;
  const int nin = in_bf16 ? T * D8 : 2 * T * D8;
  constexpr int XJ = (in_bf16 ? 1 : 2) * T * 512 / kGuBlkThreads;  // pieces per thread, D <= 4096
  uint4 xr[XJ];
#pragma unroll
  for (int j = 0; j < XJ; ++j) {
    const int i = tid + kGuBlkThreads * j;
    const uint4 v = reinterpret_cast<const uint4*>(a.x)[i < nin ? i : 0];
    xr[j] = i < nin ? v : make_uint4(0, 0, 0, 0);
  }
  float rinv[T];
#pragma unroll
  for (int t = 0; t < T; ++t) rinv[t] = 1.f;
  if (RMS && T > 1 && !PLANNED) {  // published by decode_list_kernel
#pragma unroll
    for (int t = 0; t < T; ++t) rinv[t] = w.rinv[t];
  }
  // A planned call with 2..4 tokens (decode stack): the previous layer's
  // down blocks left the sums of squares of their output rows; every wave
  // adds the D/16 partials of each token in the same fixed order, so all
  // blocks agree on the factors without a block-wide pass over x.
  float rpart[T];
  if constexpr (RMS && T > 1 && PLANNED) {
#pragma unroll
    for (int t = 0; t < T; ++t) rpart[t] = 0.f;
    for (int i = lane; i < D / 16; i += 64) {
#pragma unroll
      for (int t = 0; t < T; ++t) rpart[t] += a.rms_in[i * T + t];
    }
  }

  // 2. Weight loads of this wave.
  const int mat = wv / kGuSplit, kh = wv % kGuSplit;
  const int n = lane & 15, q = lane >> 4;
  const uint8_t* tile = eb + (size_t)(g * 2 + mat) * oD * rec_bytes(FMT);
  constexpr int NOCT = OPW > 0 ? OPW : kMaxOctPerWave;
  uint4 cw[NOCT], pa[NOCT], pb[NOCT];
  uint2 hw[NOCT];
#pragma unroll
  for (int i = 0; i < NOCT; ++i) {
    const int o = kh + kGuSplit * i;
    if (OPW > 0 || o < oD)
      load_record<FMT>(tile + (size_t)o * rec_bytes(FMT), lane, cw[i], hw[i], pa[i], pb[i]);
  }
  // 3. The expert's down records for the down blocks of this XCD, last, so
  // that no wait for the loads above covers them.
  const int Fu_pf = vb < nsh ? a.Fs : a.F;
  const DnPrefetch dpf = prefetch_down_rows(eb, D, Fu_pf, rec_bytes(FMT),
                                            down_offset(D, Fu_pf, FMT), vb, vb - g, Fu_pf / 16,
                                            tid, kGuBlkThreads);
  // The RMS factors of the input: in-block with one token; from the
  // previous layer's partials in a planned call with 2..4 tokens; from
  // decode_list_kernel otherwise.
  constexpr bool RMS_IN_BLOCK = RMS && T == 1;
  if constexpr (RMS && T > 1 && PLANNED) {
#pragma unroll
    for (int t = 0; t < T; ++t) rinv[t] = 1.0f / sqrtf(wave_sum_f32(rpart[t]) / (float)D + 1e-6f);
  }
  if constexpr (RMS_IN_BLOCK) {
    float ss[T];
#pragma unroll
    for (int t = 0; t < T; ++t) ss[t] = 0.f;
#pragma unroll
    for (int j = 0; j < XJ; ++j) {
      const int i = tid + kGuBlkThreads * j;
      const int t = in_bf16 ? i / D8 : i / (2 * D8);
      const uint32_t qq[4] = {xr[j].x, xr[j].y, xr[j].z, xr[j].w};
      float q2 = 0.f;
      if (in_bf16) {
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) q2 += bf16_lo(qq[e2]) * bf16_lo(qq[e2]) + bf16_hi(qq[e2]) * bf16_hi(qq[e2]);
      } else {
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) q2 += __uint_as_float(qq[e2]) * __uint_as_float(qq[e2]);
      }
#pragma unroll
      for (int tt = 0; tt < T; ++tt) ss[tt] += tt == t ? q2 : 0.f;  // invalid pieces are 0
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float r = wave_sum_f32(ss[t]);
      if (lane == 0) s_ss[wv][t] = r;
    }
    lds_barrier();
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float ssum = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kGuBlkWaves; ++w2) ssum += s_ss[w2][t];
      rinv[t] = 1.0f / sqrtf(ssum / (float)D + 1e-6f);
    }
  }
  // bf16 operand(s) to LDS, and per-block sums X = sum x, X' = sum c x of the
  // operand values (lanes holding the pieces of one block combine by DPP).
#pragma unroll
  for (int j = 0; j < XJ; ++j) {
    const int i = tid + kGuBlkThreads * j;
    const bool ok = i < nin;
    float X = 0.f, Xc = 0.f;
    if (in_bf16) {  // piece i = bf16 elements 8(i % D8) .. +7 of token i / D8
      const int t = i / D8, pc = i % D8, b = pc >> 2;
      const uint32_t qq[4] = {xr[j].x, xr[j].y, xr[j].z, xr[j].w};
      uint32_t hi[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        if (RMS) {
          const float r = rinv[0] * (t == 0) + (T > 1 ? rinv[T > 1 ? 1 : 0] * (t == 1) : 0.f) +
                          (T > 2 ? rinv[T > 2 ? 2 : 0] * (t == 2) : 0.f) +
                          (T > 3 ? rinv[T > 3 ? 3 : 0] * (t == 3) : 0.f);
          hi[e2] = rne_pk_bf16(bf16_lo(qq[e2]) * r, bf16_hi(qq[e2]) * r);
        } else {
          hi[e2] = qq[e2];
        }
        const float v = bf16_lo(hi[e2]) + bf16_hi(hi[e2]);
        X += v;
        Xc += dq_offset(b & 1, e2) * v;
      }
      if (ok) s_xhi[t * D8p + pc] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      X = quad_sum(X);
      Xc = quad_sum(Xc);
      if (ok && (pc & 3) == 0) s_xs[t * nbD + b] = make_float2(X, Xc);
    } else {  // piece i = fp32 elements 4(i % 2D8) .. +3 of token i / (2 D8)
      const int t = i / (2 * D8), pc = i % (2 * D8), b = pc >> 3, j0 = 2 * (pc & 1);
      const float v4[4] = {__uint_as_float(xr[j].x), __uint_as_float(xr[j].y),
                           __uint_as_float(xr[j].z), __uint_as_float(xr[j].w)};
      uint32_t hi[2], lo[2];
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        float v0 = v4[2 * q2], v1 = v4[2 * q2 + 1];
        if (RMS) {
          const float r = rinv[0] * (t == 0) + (T > 1 ? rinv[T > 1 ? 1 : 0] * (t == 1) : 0.f) +
                          (T > 2 ? rinv[T > 2 ? 2 : 0] * (t == 2) : 0.f) +
                          (T > 3 ? rinv[T > 3 ? 3 : 0] * (t == 3) : 0.f);
          v0 *= r;
          v1 *= r;
        }
        const uint16_t h0 = f32_to_bf16(v0), h1 = f32_to_bf16(v1);
        hi[q2] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        float s = bf16_to_f32(h0) + bf16_to_f32(h1);
        if (HAS_LO) {
          lo[q2] = pack_bf16x2(v0 - bf16_to_f32(h0), v1 - bf16_to_f32(h1));
          s += bf16_lo(lo[q2]) + bf16_hi(lo[q2]);
        }
        X += s;
        Xc += dq_offset(b & 1, j0 + q2) * s;
      }
      if (ok) {
        reinterpret_cast<uint2*>(s_xhi)[t * 2 * D8p + pc] = make_uint2(hi[0], hi[1]);
        if (HAS_LO) reinterpret_cast<uint2*>(s_xlo)[t * 2 * D8p + pc] = make_uint2(lo[0], lo[1]);
      }
      X = oct_sum(X);
      Xc = oct_sum(Xc);
      if (ok && (pc & 7) == 0) s_xs[t * nbD + b] = make_float2(X, Xc);
    }
  }
  lds_barrier();

  // 4. Dequantising MFMA GEMV over this wave's octets.  The MFMA output rows
  // are tokens; rows past T are computed from a copy of token 0's
  // activations and never read (only lanes 0..15 are kept), so the A operand
  // needs no zeroing.
  const DqConsts kc = dq_consts();
  float acc[T], mt[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = mt[t] = 0.f;
  const int xrow = (n < T ? n : 0) * D8p + q;  // this lane's A-operand row
#pragma unroll
  for (int i = 0; i < NOCT; ++i) {
    const int o = kh + kGuSplit * i;
    if (OPW > 0 || o < oD) {
      auto xfrag = [&](int beta, bool lo) -> uint4 {
        const int idx = xrow + 4 * (8 * o + beta);
        return lo ? s_xlo[idx] : s_xhi[idx];
      };
      auto xsum = [&](int beta, int t) -> float2 { return s_xs[t * nbD + 8 * o + beta]; };
      record_gemv<T, FMT, HAS_LO, true, (T > 1 ? 4 : 8)>(cw[i], hw[i], pa[i], pb[i], 8, kc, xfrag, xsum, acc, mt, q);
    }
  }
#pragma unroll
  for (int t = 0; t < T; ++t) {
    mt[t] += __shfl_xor(mt[t], 16, 64);
    mt[t] += __shfl_xor(mt[t], 32, 64);
  }
  if (lane < 16) {
#pragma unroll
    for (int t = 0; t < T; ++t) s_red[wv][t][n] = acc[t] + mt[t];
  }
  lds_barrier();

  // 5. SwiGLU over 16 FFN rows x T tokens; h in bf16 hi + lo; half-block sums.
  if (tid < 16 * T) {
    const int t = tid >> 4, nn = tid & 15;
    float ga = s_red[0][t][nn], ub = s_red[kGuSplit][t][nn];
#pragma unroll
    for (int j = 1; j < kGuSplit; ++j) {
      ga += s_red[j][t][nn];
      ub += s_red[kGuSplit + j][t][nn];
    }
    const float h = silu(ga) * ub;
    const uint16_t hi = f32_to_bf16(h);
    const uint16_t lo = f32_to_bf16(h - bf16_to_f32(hi));
    const size_t hidx = ((size_t)u * T + t) * w.Fp + 16 * g + nn;
    w.hh[hidx] = hi;
    w.hl[hidx] = lo;
    const float v = bf16_to_f32(hi) + bf16_to_f32(lo);
    const int kl = 16 * (g & 1) + nn;  // position inside the 32-row down block
    float X = v, Xc = dq_offset((g >> 1) & 1, (kl & 7) >> 1) * v;
#pragma unroll
    for (int o2 = 8; o2 >= 1; o2 >>= 1) {
      X += __shfl_xor(X, o2, 64);
      Xc += __shfl_xor(Xc, o2, 64);
    }
    if (nn == 0) w.hs[(((size_t)u * T + t) * (w.Fp / 32) + (g >> 1)) * 2 + (g & 1)] = make_float2(X, Xc);
  }
  keep_alive(dpf);
}

// 2..4 tokens: the routing and the expert list, once per layer call.  One
// block: wave t routes token t (and waves 4..7 meanwhile find the RMS factors
// of the input rule), then wave 0 builds and publishes the list (and the
// miss list and usage counts).  The gate/up blocks read their entry
// instead of each routing every token and building the list itself, work
// that at four tokens took as long as their GEMV and ran on the same SIMDs.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));  // stays in registers

template <int T>
__global__ __launch_bounds__(2 * kGuThreads) void decode_list_kernel(DecodeArgs a, DecodeWs w) {
  extern __shared__ int32_t s_first[];  // [E]
  __shared__ RouteLds R;
  __shared__ TopkScratch s_topk[kGuWaves];
  __shared__ float s_ss[kGuWaves][kDecodeMaxT];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  static_assert(T <= kGuWaves, "one wave per token");
  if (wv < kGuWaves) {  // waves 0..3: wave t routes token t
    if (wv < T) {
      int e;
      float gt;
      route_token(a, wv, lane, s_topk[wv], e, gt);
      if (lane < a.k) {
        R.e[wv * a.k + lane] = e;
        R.g[wv * a.k + lane] = gt;
      }
    }
  } else if (a.rmsnorm) {  // waves 4..7 meanwhile: the tokens' RMS factors
    // (every gate/up block needs them); sums by thread, wave, then the four
    // waves in order.  Piece i: 8 bf16 or 4 fp32 values of token i / (pieces
    // per token).
    const int tl = tid - kGuThreads, D = a.D;
    const int ppt = (a.x_bf16 ? 1 : 2) * (D / 8);  // pieces per token
    constexpr int kPP = 2 * 4096 / 8 / kGuThreads;  // pieces per thread and token, max
    // Every piece is requested before any is used: pieces past the token
    // read its piece 0 and are dropped by a select.  (Read under a bounds
    // test, each load sat in its own branch behind a wait for the previous
    // one.)
    u32x4_t v[T][kPP];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int j = 0; j < kPP; ++j) {
        const int i = tl + kGuThreads * j;
        v[t][j] = reinterpret_cast<const u32x4_t*>(a.x)[(size_t)t * ppt + (i < ppt ? i : 0)];
      }
    float ss[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      ss[t] = 0.f;
#pragma unroll
      for (int j = 0; j < kPP; ++j) {
        const uint32_t qq[4] = {v[t][j].x, v[t][j].y, v[t][j].z, v[t][j].w};
        float q2 = 0.f;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          if (a.x_bf16)
            q2 += bf16_lo(qq[e2]) * bf16_lo(qq[e2]) + bf16_hi(qq[e2]) * bf16_hi(qq[e2]);
          else
            q2 += __uint_as_float(qq[e2]) * __uint_as_float(qq[e2]);
        }
        ss[t] += tl + kGuThreads * j < ppt ? q2 : 0.f;
      }
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float r = wave_sum_f32(ss[t]);
      if (lane == 0) s_ss[wv - kGuWaves][t] = r;
    }
  }
  __syncthreads();
  if (a.rmsnorm && tid < T) {
    float ssum = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < kGuWaves; ++w2) ssum += s_ss[w2][tid];
    w.rinv[tid] = 1.0f / sqrtf(ssum / (float)a.D + 1e-6f);
  }
  if (wv == 0) build_list<T>(a, w, R, s_first, lane, true, a.shared != nullptr ? 1 : 0);
}

// One layer of a stack per block: wave t routes token t of the layer, then
// wave 0 builds and publishes the layer's list, routing, miss list and usage
// counts into the layer's plan area, exactly as decode_list_kernel (2..4
// tokens) and the one-token gate/up kernel do for a single layer call.
template <int T>
__global__ __launch_bounds__(kGuThreads) void decode_plan_kernel(PlanArgs p) {
  extern __shared__ int32_t s_first[];  // [E]
  __shared__ RouteLds R;
  __shared__ TopkScratch s_topk[kGuWaves];
  const int l = blockIdx.x, lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  DecodeArgs a = {};
  a.T = T;
  a.E = p.E;
  a.k = p.k;
  a.logits = p.logits + (size_t)l * T * p.E;
  a.slot_of = p.slot_of[l];
  a.n_slots = p.n_slots[l];
  a.use_count = p.use_count[l];
  a.miss = p.miss ? p.miss + (size_t)l * T * p.k : nullptr;
  a.miss_count = p.miss_count ? p.miss_count + l : nullptr;
  DecodeWs w = {};
  decode_plan_carve(p.plan + (size_t)l * p.plan_bytes, T, p.E, p.k, w);
  if (wv < T) {
    int e;
    float gt;
    route_token(a, wv, lane, s_topk[wv], e, gt);
    if (lane < a.k) {
      R.e[wv * a.k + lane] = e;
      R.g[wv * a.k + lane] = gt;
    }
  }
  __syncthreads();
  if (wv == 0) build_list<T>(a, w, R, s_first, lane, true, p.has_shared[l]);
}

template <int T, int FMT, int XM, bool PLANNED, int OPW>
__global__ __launch_bounds__(kGuBlkThreads, 2) void decode_gateup_kernel(DecodeArgs a, DecodeWs w) {
  extern __shared__ uint4 s_dyn[];
  __shared__ GuLds L;
  gateup_body<T, FMT, XM, PLANNED, OPW>(a, w, (int)blockIdx.x, L, s_dyn);
}


// ----------------------------------------------------------------------------
// decode_down.  Grid: D/16 blocks of 1024 threads; wave w handles list
// entries u = w, w + 16, ...; outputs are summed over waves in a fixed order.
// Per entry a wave issues, back to back: the entry's weight records, its h
// rows (bf16 hi and lo of its T tokens) by direct global -> LDS loads into
// the wave's own LDS region, its block sums, and the list slot of its next
// entry; then it waits once.  So an entry costs one HBM round trip (the
// weights), with h (an L2 read: every block reads every entry's h) under it.
// Staging h through registers instead, its second half could only be read
// after the first was stored, behind the weights.
template <int T, int FMT>
__global__ __launch_bounds__(1024) void decode_down_kernel(DecodeArgs a, DecodeWs w) {
  extern __shared__ uint4 s_dyn[];
  __shared__ float s_red[kDnWaves][kDecodeMaxT][16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int rt = blockIdx.x, D = a.D;
  const int n = lane & 15, q = lane >> 4;
  const int Fp = w.Fp, hrow = Fp / 8, nbF = Fp / 32;
  const int nh = T * 2 * hrow;  // uint4 of h per entry: [T][hi row, lo row]
  const int nsum = T * nbF;     // uint4 of sums per entry: both halves of one block each
  uint4* s_hw = s_dyn + (size_t)wv * (nh + nsum / 2);
  float2* s_hs = reinterpret_cast<float2*>(s_hw + nh);  // [T][Fp/32], halves combined
  const DqConsts kc = dq_consts();

  // h of entry u, [T][hi row, lo row] (nh uint4, a multiple of 64 since Fp is
  // a multiple of 256), to this wave's LDS region: one direct load per 64
  // uint4, lane l taking element c0 + l.
  auto dma_h = [&](int u) {
    const uint4* gh = reinterpret_cast<const uint4*>(w.hh) + (size_t)u * T * hrow;
    const uint4* gl = reinterpret_cast<const uint4*>(w.hl) + (size_t)u * T * hrow;
    for (int c0 = 0; c0 < nh; c0 += 64) {
      const int i = c0 + lane;
      const int t = i / (2 * hrow), rem = i % (2 * hrow);
      dn_dma16(rem < hrow ? gh + t * hrow + rem : gl + t * hrow + rem - hrow, s_hw + c0);
    }
  };
  uint4 sv;
  auto load_s = [&](int u) {
    const uint4* gs = reinterpret_cast<const uint4*>(w.hs) + (size_t)u * nsum;
    const uint4 v = gs[lane < nsum ? lane : 0];
    sv = lane < nsum ? v : make_uint4(0, 0, 0, 0);
  };

  // The count and this wave's first entry are read together (the entry
  // index clamped into the list's capacity), not one after the other.
  const int nwork = *w.nwork;
  const int u0 = wv < w.Wmax ? wv : w.Wmax - 1;
  int ref = w.work_ref[u0];
  float4 gt = reinterpret_cast<const float4*>(w.work_gate)[u0];
  asm volatile("" ::"v"(ref));  // keeps the loads ahead of the branches on nwork
  float oacc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) oacc[t] = 0.f;
  for (int u = wv; u < nwork; u += kDnWaves) {
    const bool sh = ref < 0;
    const int Fu = sh ? a.Fs : a.F;
    const int oF = octets(Fu), nb = Fu / 32;
    const uint8_t* base = (sh ? a.shared : a.routed + (size_t)ref * a.stride) +
                          down_offset(D, Fu, FMT) + (size_t)rt * oF * rec_bytes(FMT);
    uint4 cw[kMaxDecodeFOct], pa[kMaxDecodeFOct], pb[kMaxDecodeFOct];
    uint2 hw[kMaxDecodeFOct];
#pragma unroll
    for (int o = 0; o < kMaxDecodeFOct; ++o)
      if (o < oF) load_record<FMT>(base + (size_t)o * rec_bytes(FMT), lane, cw[o], hw[o], pa[o], pb[o]);
    dma_h(u);
    load_s(u);
    int ref_n = 0;
    float4 gt_n = make_float4(0.f, 0.f, 0.f, 0.f);
    if (u + kDnWaves < nwork) {
      ref_n = w.work_ref[u + kDnWaves];
      gt_n = reinterpret_cast<const float4*>(w.work_gate)[u + kDnWaves];
    }
    dn_wait_vm0();  // weights, h (in LDS), sums and the next slot have arrived
    if (lane < nsum)
      s_hs[lane] = make_float2(__uint_as_float(sv.x) + __uint_as_float(sv.z),
                               __uint_as_float(sv.y) + __uint_as_float(sv.w));
    wave_lds_fence();
    float acc[T], mt[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = mt[t] = 0.f;
#pragma unroll
    for (int o = 0; o < kMaxDecodeFOct; ++o) {
      if (o < oF) {
        const int nvalid = nb - 8 * o < 8 ? nb - 8 * o : 8;
        // rows past T read token 0's h: those output rows are never used
        auto xfrag = [&](int beta, bool lo) -> uint4 {
          return s_hw[((n < T ? n : 0) * 2 + (lo ? 1 : 0)) * hrow + (32 * (8 * o + beta) + 8 * q) / 8];
        };
        auto xsum = [&](int beta, int t) -> float2 { return s_hs[t * nbF + 8 * o + beta]; };
        record_gemv<T, FMT, true, false, 1>(cw[o], hw[o], pa[o], pb[o], nvalid, kc, xfrag, xsum, acc,
                                            mt, q);
      }
    }
    const float gg[4] = {gt.x, gt.y, gt.z, gt.w};
#pragma unroll
    for (int t = 0; t < T; ++t) {
      mt[t] += __shfl_xor(mt[t], 16, 64);
      mt[t] += __shfl_xor(mt[t], 32, 64);
      oacc[t] += gg[t] * (acc[t] + mt[t]);
    }
    wave_lds_fence();  // this entry's LDS reads are done before the next entry's h lands
    ref = ref_n;
    gt = gt_n;
  }
  if (lane < 16) {
#pragma unroll
    for (int t = 0; t < T; ++t) s_red[wv][t][n] = oacc[t];
  }
  __syncthreads();
  if (tid < 16 * T) {  // lanes 16t .. 16t+15 of wave 0: token t, rows nn
    const int t = tid >> 4, nn = tid & 15;
    float o = 0.f;
#pragma unroll
    for (int i = 0; i < kDnWaves; ++i) o += s_red[i][t][nn];
    const size_t oi = (size_t)t * D + 16 * rt + nn;
    float stored = o;
    if (a.out_bf16) {
      const uint16_t ob = f32_to_bf16(o);
      reinterpret_cast<uint16_t*>(a.out)[oi] = ob;
      stored = bf16_to_f32(ob);
    } else {
      reinterpret_cast<float*>(a.out)[oi] = o;
    }
    if (a.rms_out) {  // the next layer's RMS partial: sum over this block's 16 rows
      float sq = stored * stored;
      sq += __shfl_xor(sq, 1, 64);
      sq += __shfl_xor(sq, 2, 64);
      sq += __shfl_xor(sq, 4, 64);
      sq += __shfl_xor(sq, 8, 64);
      if (nn == 0) a.rms_out[rt * T + t] = sq;
    }
  }
}

template <int T, int FMT, int XM>
static hipError_t launch_decode_x(const DecodeArgs& a, const DecodeWs& w, hipStream_t st) {
  static std::atomic<size_t> lds_gu[2][kMaxDevices], lds_gp[2][kMaxDevices], lds_dn[kMaxDevices];
  const int D8 = a.D / 8, nbD = a.D / 32;
  const int D8p = D8 + (T > 1 ? 1 : 0);  // padded token rows (see gateup_body)
  const size_t lds = (size_t)T * D8p * 16 * (XM == kXF32 ? 2 : 1) + (size_t)T * nbD * 8;
  const size_t lds_down =
      (size_t)kDnWaves * ((size_t)T * 2 * (w.Fp / 8) + (size_t)T * (w.Fp / 32) / 2) * 16;
  hipError_t e;
  // One token with d_model 3072 (the pages' model): a fixed count of
  // 12 / kGuSplit octets per wave, so the record loads are unconditional
  // (see gateup_body); 105 VGPRs for Q2SM, two blocks per CU.  With 2..4
  // tokens the same form takes 164 (one block per CU, so a 4-token layer's
  // blocks would run in three rounds), so those keep the generic form.
  constexpr int kOpw = T == 1 ? 12 / kGuSplit : 0;
  const bool six = kOpw > 0 && a.D == 3072;
  auto gu_kernel = [&](bool planned) {
    return planned ? (six ? decode_gateup_kernel<T, FMT, XM, true, kOpw>
                          : decode_gateup_kernel<T, FMT, XM, true, 0>)
                   : (six ? decode_gateup_kernel<T, FMT, XM, false, kOpw>
                          : decode_gateup_kernel<T, FMT, XM, false, 0>);
  };
  if ((e = allow_lds(gu_kernel(false), lds, lds_gu[six])) != hipSuccess) return e;
  if ((e = allow_lds(gu_kernel(true), lds, lds_gp[six])) != hipSuccess) return e;
  if ((e = allow_lds(decode_down_kernel<T, FMT>, lds_down, lds_dn)) != hipSuccess) return e;
  const int nblk = (a.shared ? a.Fs / 16 : 0) + (w.Wmax - 1) * (a.F / 16);
  // The caller's route event (moe_set_route_event), recorded as soon as the
  // kernel that writes the routing, the list and the miss list has run.
  auto route_done = [&]() -> hipError_t {
    KernelTimer& re = route_event();
    if (re.before == nullptr) return hipSuccess;
    const hipEvent_t ev = re.before;
    re.before = nullptr;
    return hipEventRecord(ev, st);
  };
  if (T > 1 && !a.planned) {
    decode_list_kernel<T><<<1, 2 * kGuThreads, (size_t)a.E * 4, st>>>(a, w);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = route_done()) != hipSuccess) return e;
  }
  if ((e = launch_timed(gu_kernel(a.planned != 0), dim3(nblk), dim3(kGuBlkThreads), (uint32_t)lds, st,
                        a, w)) != hipSuccess)
    return e;
  if constexpr (T == 1) {
    if ((e = route_done()) != hipSuccess) return e;
  }
  decode_down_kernel<T, FMT><<<a.D / 16, 1024, lds_down, st>>>(a, w);
  return hipGetLastError();
}

template <int T, int FMT>
static hipError_t launch_decode_t(const DecodeArgs& a, const DecodeWs& w, hipStream_t st) {
  if (a.rmsnorm) return a.x_bf16 ? launch_decode_x<T, FMT, kXRms>(a, w, st)
                                 : launch_decode_x<T, FMT, kXRmsF32>(a, w, st);
  if (a.x_bf16) return launch_decode_x<T, FMT, kXBf16>(a, w, st);
  return launch_decode_x<T, FMT, kXF32>(a, w, st);
}

hipError_t launch_decode_plan(const PlanArgs& p, hipStream_t st) {
  if (p.n <= 0) return hipSuccess;
  const size_t lds = (size_t)p.E * 4;
  switch (p.T) {
    case 1: decode_plan_kernel<1><<<p.n, kGuThreads, lds, st>>>(p); break;
    case 2: decode_plan_kernel<2><<<p.n, kGuThreads, lds, st>>>(p); break;
    case 3: decode_plan_kernel<3><<<p.n, kGuThreads, lds, st>>>(p); break;
    case 4: decode_plan_kernel<4><<<p.n, kGuThreads, lds, st>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, const DecodeWs& w, hipStream_t st) {
#define MOE_DEC_CASE(TT)                                                              \
  case TT:                                                                            \
    return a.fmt == kQ2   ? launch_decode_t<TT, kQ2>(a, w, st)                    \
           : a.fmt == kQ3 ? launch_decode_t<TT, kQ3>(a, w, st)                    \
                          : launch_decode_t<TT, kQ2S>(a, w, st);
  switch (a.T) {
    MOE_DEC_CASE(1)
    MOE_DEC_CASE(2)
    MOE_DEC_CASE(3)
    MOE_DEC_CASE(4)
    default:
      return hipErrorInvalidValue;
  }
#undef MOE_DEC_CASE
}

}  // namespace moe
