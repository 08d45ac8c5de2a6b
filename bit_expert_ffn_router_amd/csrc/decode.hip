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
// Two launches:
//   decode_gateup:  one block per (listed expert, 16 FFN rows).  Every block
//                   first routes the tokens itself (top-k + gates, the list of
//                   distinct resident experts in first-occurrence order, the
//                   miss list) while its other waves stage the activations in
//                   LDS; block 0 publishes the list for the second kernel.
//                   Then: dequantising MFMA GEMV of W_gate and W_up, SwiGLU,
//                   h in bf16 hi + lo with per-block sums.
//   decode_down:    one block per 16 output rows: W_down GEMV of every listed
//                   expert, gate-weighted sum in a fixed order, output write.
//
// Dequantisation (see DqConsts): a code word is turned into bf16 operands
// (c + u) with one VALU op per pair of weights plus shared shifts and no
// conversion; the MFMA sums (c + u) * x over one 32-weight block; the block
// result is scaled by the fp16 block scale, and the constant parts (c * x,
// and the block min times sum x) come from per-block activation sums.
#include "route_common.hpp"

namespace moe {

namespace {

constexpr int kGuWaves = 4;        // gate/up block: {gate, up} x 2 K halves, 16 FFN rows
constexpr int kGuThreads = 64 * kGuWaves;
constexpr int kDnWaves = 16;       // down block: waves share the expert list
constexpr int kMaxOctPerWave = 8;  // d_model <= 4096 on the decode path (16 octets / 2 halves)
constexpr int kMaxDecodeFOct = 2;  // d_ff, d_ff_shared <= 512 on the decode path

// Activation modes of the gate/up kernel.
constexpr int kXBf16 = 0;  // bf16 input, used as is
constexpr int kXF32 = 1;   // fp32 input, as bf16 hi + bf16 lo (two MFMAs)
constexpr int kXRms = 2;   // input normalised to bf16(x / sqrt(mean(x^2) + 1e-6))

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
  return w;
}

// ----------------------------------------------------------------------------
// Routing inside a decode block.  Waves 0..T-1 route one token each; then
// wave 0 builds the list of distinct resident experts in (token, rank) order
// of first occurrence with their per-token gates, and the miss list.  Every
// block computes the same list; block 0 also publishes it (and the misses).
struct RouteLds {
  key64* scr;  // T regions of topk_scratch_bytes(E, k) in dynamic LDS
  alignas(16) int32_t e[kDecodeMaxT * kMaxTopK];
  float g[kDecodeMaxT * kMaxTopK];
  int32_t ref[kDecodeMaxT * kMaxTopK + 1];
  float wg[(kDecodeMaxT * kMaxTopK + 1) * 4];
  int32_t nu;
};

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ void decode_route_token(const DecodeArgs& a, RouteLds& R, int t,
                                                   int lane) {
  int my_e;
  float my_l;
  wave_topk_any(a.logits + (size_t)t * a.E, a.E, a.k, lane, my_e, my_l,
                R.scr + t * (topk_scratch_bytes(a.E, a.k) / 8));
  const float g = wave_gate(my_l, a.k, lane);
  if (lane < a.k) {
    // never let an id outside 0..E-1 become an address (cannot happen for
    // finite logits; the clamp keeps a fault out of the weight streams)
    R.e[t * a.k + lane] = my_e < 0 ? 0 : (my_e >= a.E ? a.E - 1 : my_e);
    R.g[t * a.k + lane] = g;
  }
}

// Slot of expert e, or -1 when not resident (a slot outside 0..n_slots-1 in
// the caller's map counts as not resident, so it is never dereferenced).
__device__ __forceinline__ int resident_ref(const DecodeArgs& a, int e) {
  if (a.slot_of == nullptr) return e;
  const int s = a.slot_of[e];
  return (s >= 0 && s < a.n_slots) ? s : -1;
}

// Wave 0 only, after every token's routing is visible in LDS.
template <int T>
__device__ __forceinline__ void decode_build_list(const DecodeArgs& a, const DecodeWs& w,
                                                  RouteLds& R, int lane, bool publish) {
  const int k = a.k, P = T * k;  // P <= 128: lane handles pairs lane, lane + 64
  int first[2];
  bool valid[2], hit[2];
  unsigned long long bf[2], bm[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int p = lane + 64 * h;
    valid[h] = p < P;
    first[h] = -1;
    hit[h] = false;
    if (valid[h]) {
      const int e = R.e[p];
      hit[h] = resident_ref(a, e) >= 0;
      if (hit[h]) {
        // first (token, rank) pair naming the same expert; one token's ids
        // are distinct, so only pairs of earlier tokens can match
        first[h] = p;
        if (T > 1) {
          const int4* e4 = reinterpret_cast<const int4*>(R.e);
          const int nq = (p / k) * k;  // pairs of earlier tokens
          for (int c = 0; c < (nq + 3) / 4; ++c) {
            const int4 v = e4[c];
            const int ids[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q2 = 0; q2 < 4; ++q2) {
              const int idx = 4 * c + q2;
              if (idx < nq && ids[q2] == e && first[h] == p) first[h] = idx;
            }
          }
        }
      }
    }
    bf[h] = __ballot(valid[h] && first[h] == p);
    bm[h] = __ballot(valid[h] && !hit[h]);
  }
  const int nf0 = __popcll(bf[0]), nm0 = __popcll(bm[0]);
  const int U = nf0 + __popcll(bf[1]);
  const int M = nm0 + __popcll(bm[1]);
  const bool has_sh = a.shared != nullptr;
  const int nu = U + (has_sh ? 1 : 0);
  for (int i = lane; i < nu * 4; i += 64) R.wg[i] = 0.f;
  wave_lds_sync();
  auto list_index = [&](int fp) {  // list index of the pair that first named an expert
    const unsigned long long b = fp >= 64 ? bf[1] : bf[0];   // no run-time array index
    return (fp >= 64 ? nf0 : 0) + __popcll(b & ((1ull << (fp & 63)) - 1ull));
  };
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int p = lane + 64 * h;
    if (valid[h] && first[h] == p) R.ref[list_index(p)] = resident_ref(a, R.e[p]);
    if (valid[h] && first[h] >= 0) R.wg[list_index(first[h]) * 4 + p / k] = R.g[p];
  }
  if (lane == 0) {
    R.nu = nu;
    if (has_sh) R.ref[U] = -1;
  }
  if (has_sh && lane < T) R.wg[U * 4 + lane] = 1.0f;
  wave_lds_sync();
  if (!publish) return;
  for (int i = lane; i < nu; i += 64) w.work_ref[i] = R.ref[i];
  for (int i = lane; i < nu * 4; i += 64) w.work_gate[i] = R.wg[i];
  for (int i = lane; i < P; i += 64) {
    w.idx[i] = R.e[i];
    w.gate[i] = R.g[i];
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
      r.token = p / k;
      r.rank = p % k;
      r.expert = R.e[p];
      r.gate = R.g[p];
      a.miss[(h ? nm0 : 0) + __popcll(bm[h] & ((1ull << lane) - 1ull))] = r;
    }
  }
}

// ----------------------------------------------------------------------------
// Block parameter helpers.  Q2SM: the two 16-byte parameter loads of a record
// row hold (scale, min) for blocks 0..3 and 4..7.  Q3S: one 16-byte load holds
// the 8 scales.
__device__ __forceinline__ uint32_t sel4(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}
template <int FMT>
__device__ __forceinline__ float blk_scale(const uint4& pa, const uint4& pb, int beta) {
  if (FMT == kQ2) {
    const uint32_t v = beta < 4 ? sel4(pa, beta) : sel4(pb, beta - 4);
    return f16_to_f32((uint16_t)(v & 0xFFFFu));
  } else {
    const uint32_t v = sel4(pa, beta >> 1);
    return f16_to_f32((uint16_t)((beta & 1) ? (v >> 16) : (v & 0xFFFFu)));
  }
}
template <int FMT>
__device__ __forceinline__ float blk_min(const uint4& pa, const uint4& pb, int beta) {
  const uint32_t v = beta < 4 ? sel4(pa, beta) : sel4(pb, beta - 4);
  return f16_to_f32((uint16_t)(v >> 16));
}

// One record (16 rows x 8 blocks) of one wave: MFMA over the 8 blocks with
// activation fragments fetched by `xfrag(beta, hi_or_lo)`; accumulates
// scale * block result into acc (lanes 0..15 hold tokens 0..T-1), and the
// lane's share of the constant terms (blocks beta = q and q + 4) into mt.
template <int T, int FMT, bool HAS_LO, typename XFrag, typename XSum>
__device__ __forceinline__ void record_gemv(const uint4& cw, const uint2& hw, const uint4& pa,
                                            const uint4& pb, int nvalid, const DqConsts& kc,
                                            XFrag xfrag, XSum xsum, float (&acc)[T],
                                            float (&mt)[T], int q) {
  const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
  const uint32_t hws[2] = {hw.x, hw.y};
#pragma unroll
  for (int wd = 0; wd < 4; ++wd) {
    uint4 ea, eb;
    if (FMT == kQ2)
      dq_q2(words[wd], kc, ea, eb);
    else
      dq_q3(words[wd], hws[wd >> 1], (wd & 1) != 0, kc, ea, eb);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int beta = 2 * wd + half;
      if (beta < nvalid) {
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
  // Constant terms of this lane's two blocks.
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int beta = q + 4 * hb;
    if (beta < nvalid) {
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
        if (FMT == kQ2)
          mt[t] += m * X.x - s * X.y;
        else
          mt[t] -= s * (X.y + 4.0f * X.x);
      }
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
  } else {
    hw = *reinterpret_cast<const uint2*>(rec + 1024 + 8 * lane);
    pa = *reinterpret_cast<const uint4*>(rec + 1536 + 16 * n);
    pb = make_uint4(0, 0, 0, 0);
  }
}

// ----------------------------------------------------------------------------
// decode_gateup.  Grid: (routed capacity x F/16) + Fs/16 blocks of 256
// threads, two blocks per CU.  Every thread first issues its share of the
// activation loads, then waves 0..T-1 route; after the list is known, wave w
// computes matrix w/2 (gate, up) over the K octets o = w%2, w%2 + 2, ... of
// one 16-row h-group.
template <int T, int FMT, int XM>
__global__ __launch_bounds__(kGuThreads, 2) void decode_gateup_kernel(DecodeArgs a, DecodeWs w) {
  extern __shared__ uint4 s_dyn[];
  __shared__ RouteLds R;
  __shared__ float s_red[kGuWaves][kDecodeMaxT][16];
  __shared__ float s_ss[kGuWaves][kDecodeMaxT];
  constexpr bool HAS_LO = XM == kXF32;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int D = a.D, oD = octets(D), nbD = D / 32, D8 = D / 8;
  uint4* s_xhi = s_dyn;                                            // [T][D/8]
  uint4* s_xlo = s_dyn + T * D8;                                   // [T][D/8]
  float2* s_xs = reinterpret_cast<float2*>(s_dyn + (HAS_LO ? 2 : 1) * T * D8);   // [T][D/32]
  float* s_raw = reinterpret_cast<float*>(s_xs + T * nbD);         // [T][D] (XM == kXRms)
  if (tid == 0)
    R.scr = reinterpret_cast<key64*>(reinterpret_cast<uint8_t*>(s_raw) +
                                     (XM == kXRms ? (size_t)T * D * 4 : 0));
  __syncthreads();

  // 0. Activation loads in flight before routing (16-byte pieces of the input).
  const bool in_bf16 = XM == kXBf16 || a.x_bf16;
  const int nin = in_bf16 ? T * D8 : 2 * T * D8;          // 16-byte pieces of x
  constexpr int XJ = (XM == kXBf16 ? 2 : 4) * T;          // pieces per thread, D <= 4096
  uint4 xr[XJ];
#pragma unroll
  for (int j = 0; j < XJ; ++j) {
    const int i = tid + kGuThreads * j;
    // clamped index + select: every element defined, so the array stays in VGPRs
    const uint4 v = reinterpret_cast<const uint4*>(a.x)[i < nin ? i : 0];
    xr[j] = i < nin ? v : make_uint4(0, 0, 0, 0);
  }
  // 1. Routing of token wv (waves 0..T-1).
  if (wv < T) decode_route_token(a, R, wv, lane);
  // 2. Activations to LDS: the bf16 operand (hi, and lo for fp32 input), or
  // fp32 values and per-token sums of squares for the normalised mode.
  float ss[T];
#pragma unroll
  for (int t = 0; t < T; ++t) ss[t] = 0.f;
#pragma unroll
  for (int j = 0; j < XJ; ++j) {
    const int i = tid + kGuThreads * j;
    if (i >= nin) continue;
    if (XM == kXBf16) {
      s_xhi[i] = xr[j];
    } else if (XM == kXF32) {  // piece i = fp32 elements 4i..4i+3
      const float v[4] = {__uint_as_float(xr[j].x), __uint_as_float(xr[j].y),
                          __uint_as_float(xr[j].z), __uint_as_float(xr[j].w)};
      uint32_t hi[2], lo[2];
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        const uint16_t h0 = f32_to_bf16(v[2 * q2]), h1 = f32_to_bf16(v[2 * q2 + 1]);
        hi[q2] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        lo[q2] = pack_bf16x2(v[2 * q2] - bf16_to_f32(h0), v[2 * q2 + 1] - bf16_to_f32(h1));
      }
      reinterpret_cast<uint2*>(s_xhi)[i] = make_uint2(hi[0], hi[1]);
      reinterpret_cast<uint2*>(s_xlo)[i] = make_uint2(lo[0], lo[1]);
    } else {  // kXRms
      float q2 = 0.f;
      int t;
      if (in_bf16) {  // piece i = bf16 elements 8i..8i+7
        const uint32_t qq[4] = {xr[j].x, xr[j].y, xr[j].z, xr[j].w};
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const float v0 = bf16_lo(qq[e2]), v1 = bf16_hi(qq[e2]);
          s_raw[8 * i + 2 * e2] = v0;
          s_raw[8 * i + 2 * e2 + 1] = v1;
          q2 += v0 * v0 + v1 * v1;
        }
        t = i / D8;
      } else {        // piece i = fp32 elements 4i..4i+3
        const float v[4] = {__uint_as_float(xr[j].x), __uint_as_float(xr[j].y),
                            __uint_as_float(xr[j].z), __uint_as_float(xr[j].w)};
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          s_raw[4 * i + e2] = v[e2];
          q2 += v[e2] * v[e2];
        }
        t = i / (2 * D8);
      }
#pragma unroll
      for (int tt = 0; tt < T; ++tt) ss[tt] += tt == t ? q2 : 0.f;
    }
  }
  if (XM == kXRms) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float r = wave_sum(ss[t]);
      if (lane == 0) s_ss[wv][t] = r;
    }
  }
  __syncthreads();
  if (XM == kXRms) {
    for (int i = tid; i < T * D8; i += kGuThreads) {
      const int t = i / D8;
      float ssum = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kGuWaves; ++w2) ssum += s_ss[w2][t];
      const float rinv = 1.0f / sqrtf(ssum / (float)D + 1e-6f);
      uint32_t hi[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        hi[j] = pack_bf16x2(s_raw[8 * i + 2 * j] * rinv, s_raw[8 * i + 2 * j + 1] * rinv);
      s_xhi[i] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    }
  }
  if (wv == 0) decode_build_list<T>(a, w, R, lane, blockIdx.x == 0);
  __syncthreads();

  // 3. This block's work item.
  const int has_sh = a.shared != nullptr;
  const int U = R.nu - has_sh;
  const int Wr = w.Wmax - 1, gpr = a.F / 16;
  int u, g;
  const uint8_t* base;
  if ((int)blockIdx.x < Wr * gpr) {
    u = blockIdx.x / gpr;
    g = blockIdx.x % gpr;
    if (u >= U) return;
    base = a.routed + (size_t)R.ref[u] * a.stride;
  } else {
    if (!has_sh) return;
    g = blockIdx.x - Wr * gpr;
    u = U;
    base = a.shared;
  }
  const int mat = wv >> 1, kh = wv & 1;
  const int n = lane & 15, q = lane >> 4;
  const uint8_t* tile = base + (size_t)(g * 2 + mat) * oD * rec_bytes(FMT);
  uint4 cw[kMaxOctPerWave], pa[kMaxOctPerWave], pb[kMaxOctPerWave];
  uint2 hw[kMaxOctPerWave];
#pragma unroll
  for (int i = 0; i < kMaxOctPerWave; ++i) {
    const int o = kh + 2 * i;
    if (o < oD) load_record<FMT>(tile + (size_t)o * rec_bytes(FMT), lane, cw[i], hw[i], pa[i], pb[i]);
  }
  // Per-block activation sums X = sum x and X' = sum c x (while the weights arrive).
  for (int i = tid; i < T * nbD; i += kGuThreads) {
    const int t = i / nbD, b = i % nbD;
    float X = 0.f, Xc = 0.f;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const uint4 vh = s_xhi[t * D8 + 4 * b + qq];
      const uint4 vl = HAS_LO ? s_xlo[t * D8 + 4 * b + qq] : make_uint4(0, 0, 0, 0);
      const uint32_t hh[4] = {vh.x, vh.y, vh.z, vh.w}, ll[4] = {vl.x, vl.y, vl.z, vl.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float v = bf16_lo(hh[j]) + bf16_lo(ll[j]) + bf16_hi(hh[j]) + bf16_hi(ll[j]);
        X += v;
        Xc += dq_offset(b & 1, j) * v;
      }
    }
    s_xs[i] = make_float2(X, Xc);
  }
  __syncthreads();

  // 4. Dequantising MFMA GEMV over this wave's octets.
  const DqConsts kc = dq_consts();
  float acc[T], mt[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = mt[t] = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxOctPerWave; ++i) {
    const int o = kh + 2 * i;
    if (o < oD) {
      auto xfrag = [&](int beta, bool lo) -> uint4 {
        if (n >= T) return make_uint4(0, 0, 0, 0);
        const int idx = n * D8 + 4 * (8 * o + beta) + q;
        return lo ? s_xlo[idx] : s_xhi[idx];
      };
      auto xsum = [&](int beta, int t) -> float2 { return s_xs[t * nbD + 8 * o + beta]; };
      record_gemv<T, FMT, HAS_LO>(cw[i], hw[i], pa[i], pb[i], 8, kc, xfrag, xsum, acc, mt, q);
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
  __syncthreads();

  // 5. SwiGLU over 16 FFN rows x T tokens; h in bf16 hi + lo; half-block sums.
  if (tid < 16 * T) {
    const int t = tid >> 4, nn = tid & 15;
    const float ga = s_red[0][t][nn] + s_red[1][t][nn];
    const float ub = s_red[2][t][nn] + s_red[3][t][nn];
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
}

// ----------------------------------------------------------------------------
// decode_down.  Grid: D/16 blocks of 1024 threads; wave w handles the listed
// experts u = w, w + 16, ...; outputs are summed over waves in a fixed order.
// Each wave stages its expert's h rows (bf16 hi and lo) in a private LDS
// region, so the weight loads of all its octets are in flight together.
template <int T, int FMT>
__global__ __launch_bounds__(1024) void decode_down_kernel(DecodeArgs a, DecodeWs w) {
  extern __shared__ uint4 s_dyn[];
  __shared__ float s_red[kDnWaves][kDecodeMaxT][16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int rt = blockIdx.x, D = a.D;
  const int n = lane & 15, q = lane >> 4;
  const int nwork = *w.nwork;
  const int Fp = w.Fp;
  const int hrow = Fp / 8;                 // uint4 per h row
  uint4* s_hw = s_dyn + (size_t)wv * T * 2 * hrow;   // [T][hi row, lo row]
  const DqConsts kc = dq_consts();
  float oacc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) oacc[t] = 0.f;
  for (int u = wv; u < nwork; u += kDnWaves) {
    const int ref = w.work_ref[u];
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
    // h rows of this expert -> LDS (T rows of hi then lo, each Fp bf16), in
    // chunks of four 16-byte loads per lane to bound register use.
    const uint4* gh = reinterpret_cast<const uint4*>(w.hh) + (size_t)u * T * hrow;
    const uint4* gl = reinterpret_cast<const uint4*>(w.hl) + (size_t)u * T * hrow;
    const int nh = T * 2 * hrow;
    for (int j0 = 0; j0 < nh; j0 += 4 * 64) {
      uint4 hv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i0 = j0 + lane + 64 * j;  // i over [T][2][hrow]
        const int i = i0 < nh ? i0 : 0;     // clamped: all four loads issue unconditionally
        const int t = i / (2 * hrow), rem = i % (2 * hrow);
        const uint4* src = rem < hrow ? gh + t * hrow + rem : gl + t * hrow + rem - hrow;
        hv[j] = *src;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = j0 + lane + 64 * j;
        if (i < nh) s_hw[i] = hv[j];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float acc[T], mt[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = mt[t] = 0.f;
#pragma unroll
    for (int o = 0; o < kMaxDecodeFOct; ++o) {
      if (o < oF) {
        const int nvalid = nb - 8 * o < 8 ? nb - 8 * o : 8;
        auto xfrag = [&](int beta, bool lo) -> uint4 {
          if (n >= T) return make_uint4(0, 0, 0, 0);
          return s_hw[(n * 2 + (lo ? 1 : 0)) * hrow + (32 * (8 * o + beta) + 8 * q) / 8];
        };
        auto xsum = [&](int beta, int t) -> float2 {
          const size_t hi = (((size_t)u * T + t) * (Fp / 32) + 8 * o + beta) * 2;
          const float2 h0 = w.hs[hi], h1 = w.hs[hi + 1];
          return make_float2(h0.x + h1.x, h0.y + h1.y);
        };
        record_gemv<T, FMT, true>(cw[o], hw[o], pa[o], pb[o], nvalid, kc, xfrag, xsum, acc, mt, q);
      }
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      mt[t] += __shfl_xor(mt[t], 16, 64);
      mt[t] += __shfl_xor(mt[t], 32, 64);
      oacc[t] += w.work_gate[u * 4 + t] * (acc[t] + mt[t]);
    }
    __builtin_amdgcn_wave_barrier();   // LDS region reused by the next expert
  }
  if (lane < 16) {
#pragma unroll
    for (int t = 0; t < T; ++t) s_red[wv][t][n] = oacc[t];
  }
  __syncthreads();
  if (tid < 16 * T) {
    const int t = tid >> 4, nn = tid & 15;
    float o = 0.f;
#pragma unroll
    for (int i = 0; i < kDnWaves; ++i) o += s_red[i][t][nn];
    const size_t oi = (size_t)t * D + 16 * rt + nn;
    if (a.out_bf16)
      reinterpret_cast<uint16_t*>(a.out)[oi] = f32_to_bf16(o);
    else
      reinterpret_cast<float*>(a.out)[oi] = o;
  }
}

// ----------------------------------------------------------------------------
// Raise a kernel's dynamic-LDS limit when a launch needs more than the
// default 64 KiB (gfx950 has 160 KiB per CU).  `cur` caches the value set.
template <typename K>
static hipError_t allow_lds(K kernel, size_t bytes, size_t& cur) {
  if (bytes <= 65536 || bytes <= cur) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) cur = bytes;
  return e;
}

template <int T, int FMT, int XM>
static hipError_t launch_decode_x(const DecodeArgs& a, const DecodeWs& w, hipStream_t st) {
  static size_t lds_gu = 0, lds_dn = 0;
  const int D8 = a.D / 8, nbD = a.D / 32;
  const size_t lds = (size_t)T * D8 * 16 * (XM == kXF32 ? 2 : 1) + (size_t)T * nbD * 8 +
                     (XM == kXRms ? (size_t)T * a.D * 4 : 0) + T * topk_scratch_bytes(a.E, a.k);
  const size_t lds_down = (size_t)kDnWaves * T * 2 * w.Fp * 2;
  hipError_t e;
  if ((e = allow_lds(decode_gateup_kernel<T, FMT, XM>, lds, lds_gu)) != hipSuccess) return e;
  if ((e = allow_lds(decode_down_kernel<T, FMT>, lds_down, lds_dn)) != hipSuccess) return e;
  const int Wr = w.Wmax - 1;
  const int nblk = Wr * (a.F / 16) + (a.shared ? a.Fs / 16 : 0);
  if ((e = launch_timed(decode_gateup_kernel<T, FMT, XM>, dim3(nblk), dim3(kGuThreads),
                        (uint32_t)lds, st, a, w)) != hipSuccess)
    return e;
  decode_down_kernel<T, FMT><<<a.D / 16, 1024, lds_down, st>>>(a, w);
  return hipGetLastError();
}

template <int T, int FMT>
static hipError_t launch_decode_t(const DecodeArgs& a, const DecodeWs& w, hipStream_t st) {
  if (a.rmsnorm) return launch_decode_x<T, FMT, kXRms>(a, w, st);
  if (a.x_bf16) return launch_decode_x<T, FMT, kXBf16>(a, w, st);
  return launch_decode_x<T, FMT, kXF32>(a, w, st);
}

hipError_t launch_decode(const DecodeArgs& a, const DecodeWs& w, hipStream_t st) {
#define MOE_DEC_CASE(TT)                                                              \
  case TT:                                                                            \
    return a.fmt == kQ2 ? launch_decode_t<TT, kQ2>(a, w, st) : launch_decode_t<TT, kQ3>(a, w, st);
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
