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
// Three launches:
//   decode_prep:    top-k + gates per token, the list of distinct resident
//                   experts (first-occurrence order) with per-token gates,
//                   the miss list, and the bf16 activation operand with its
//                   per-block sums.
//   decode_gateup:  one block per (expert, 32 FFN rows): dequantising MFMA
//                   GEMV of W_gate and W_up, SwiGLU, h in bf16 hi + lo.
//   decode_down:    one block per 16 output rows: W_down GEMV of every listed
//                   expert, gate-weighted sum in a fixed order, output write.
//
// Dequantisation (see DqConsts): a code word is turned into bf16 operands
// (c + u) with two VALU ops per pair of weights and no conversion; the MFMA
// sums (c + u) * x over one 32-weight block; the block result is scaled by
// the fp16 block scale, and the constant parts (c * x, and the block min
// times sum x) are subtracted/added from per-block activation sums.
#include "route_common.hpp"

namespace moe {

namespace {

constexpr int kGuWaves = 8;      // gate/up block: 2 h-groups x {gate, up} x 2 K halves
constexpr int kDnWaves = 16;     // down block: waves share the expert list
constexpr int kMaxOctPerWave = 8;  // d_model <= 4096 on the decode path
constexpr int kMaxDecodeFOct = 2;  // d_ff, d_ff_shared <= 512 on the decode path

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
  b += align256(2 * (size_t)T * D) * 2;               // xa_hi, xa_lo
  b += align256(8 * (size_t)T * (D / 32));            // xs
  b += align256(2 * (size_t)Wmax * T * Fp) * 2;       // hh, hl
  b += align256(8 * (size_t)Wmax * T * (Fp / 32));    // hs
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
  w.xa_hi = (uint16_t*)take(2 * (size_t)T * D);
  w.xa_lo = (uint16_t*)take(2 * (size_t)T * D);
  w.xs = (float2*)take(8 * (size_t)T * (D / 32));
  w.hh = (uint16_t*)take(2 * (size_t)w.Wmax * T * w.Fp);
  w.hl = (uint16_t*)take(2 * (size_t)w.Wmax * T * w.Fp);
  w.hs = (float2*)take(8 * (size_t)w.Wmax * T * (w.Fp / 32));
  return w;
}

// ----------------------------------------------------------------------------
// decode_prep: one block of 256 threads.
template <int T>
__global__ __launch_bounds__(256) void decode_prep_kernel(DecodeArgs a, DecodeWs w) {
  __shared__ int32_t s_e[kDecodeMaxT * kMaxTopK];
  __shared__ float s_g[kDecodeMaxT * kMaxTopK];
  __shared__ int32_t s_first[kDecodeMaxT * kMaxTopK];
  __shared__ int32_t s_u[kDecodeMaxT * kMaxTopK];
  __shared__ int32_t s_cnt[4];
  __shared__ float s_rinv[kDecodeMaxT];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int k = a.k, P = T * k, D = a.D;

  // 1. routing of token wv; RMS factor of its activations.
  if (wv < T) {
    int my_e;
    float my_l;
    wave_topk(a.logits + (size_t)wv * a.E, a.E, k, lane, my_e, my_l);
    const float g = wave_gate(my_l, k, lane);
    if (lane < k) {
      s_e[wv * k + lane] = my_e;
      s_g[wv * k + lane] = g;
      w.idx[wv * k + lane] = my_e;
      w.gate[wv * k + lane] = g;
    }
    if (a.rmsnorm) {
      float ss = 0.f;
      for (int i = lane; i < D; i += 64) {
        const float v = a.x_bf16 ? bf16_to_f32(((const uint16_t*)a.x)[(size_t)wv * D + i])
                                 : ((const float*)a.x)[(size_t)wv * D + i];
        ss += v * v;
      }
      ss = wave_sum(ss);
      if (lane == 0) s_rinv[wv] = 1.0f / sqrtf(ss / (float)D + 1e-6f);
    }
  }
  for (int i = tid; i < w.Wmax * 4; i += 256) w.work_gate[i] = 0.f;
  __syncthreads();

  // 2. distinct resident experts in (token, rank) order of first occurrence.
  if (tid < P) {
    const int e = s_e[tid];
    const bool hit = a.slot_of == nullptr || a.slot_of[e] >= 0;
    int first = -1;
    if (hit) {
      first = tid;
      for (int p2 = 0; p2 < tid; ++p2)
        if (s_e[p2] == e) {
          first = p2;
          break;
        }
    }
    s_first[tid] = first;
  }
  __syncthreads();
  unsigned long long bf = 0, bm = 0;
  if (wv < 2) {
    const int p = tid;
    const bool isf = p < P && s_first[p] == p;
    const bool ism = p < P && s_first[p] < 0;
    bf = __ballot(isf);
    bm = __ballot(ism);
    if (lane == 0) {
      s_cnt[wv] = __popcll(bf);
      s_cnt[2 + wv] = __popcll(bm);
    }
  }
  __syncthreads();
  const int U = s_cnt[0] + s_cnt[1];
  const int M = s_cnt[2] + s_cnt[3];
  if (tid < P) {
    const unsigned long long lt = (1ull << lane) - 1ull;
    const int t = tid / k, j = tid % k, e = s_e[tid];
    if (s_first[tid] == tid) {
      const int u = (wv == 1 ? s_cnt[0] : 0) + __popcll(bf & lt);
      s_u[tid] = u;
      w.work_ref[u] = a.slot_of ? a.slot_of[e] : e;
    } else if (s_first[tid] < 0) {
      const int mi = (wv == 1 ? s_cnt[2] : 0) + __popcll(bm & lt);
      MissRec r;
      r.token = t;
      r.rank = j;
      r.expert = e;
      r.gate = s_g[tid];
      a.miss[mi] = r;
    }
  }
  __syncthreads();
  if (tid < P && s_first[tid] >= 0) {
    const int u = s_u[s_first[tid]];
    w.work_gate[u * 4 + tid / k] = s_g[tid];
  }
  if (tid == 0) {
    const int has_sh = a.shared != nullptr;
    *w.nwork = U + has_sh;
    if (has_sh) {
      w.work_ref[U] = -1;
      for (int t = 0; t < T; ++t) w.work_gate[U * 4 + t] = 1.0f;
    }
    if (a.miss_count) *a.miss_count = M;
  }

  // 3. activation operand (bf16 hi [+ lo]) and per-block sums (X, X').
  const int nb = D / 32;
  for (int i = tid; i < T * nb; i += 256) {
    const int t = i / nb, b = i % nb;
    float X = 0.f, Xc = 0.f;
    for (int kk = 0; kk < 32; ++kk) {
      const size_t ei = (size_t)t * D + 32 * b + kk;
      uint16_t hi, lo = 0;
      if (a.rmsnorm) {
        const float v = a.x_bf16 ? bf16_to_f32(((const uint16_t*)a.x)[ei]) : ((const float*)a.x)[ei];
        hi = f32_to_bf16(v * s_rinv[t]);
      } else if (a.x_bf16) {
        hi = ((const uint16_t*)a.x)[ei];
      } else {
        const float v = ((const float*)a.x)[ei];
        hi = f32_to_bf16(v);
        lo = f32_to_bf16(v - bf16_to_f32(hi));
      }
      w.xa_hi[ei] = hi;
      w.xa_lo[ei] = lo;
      const float v = bf16_to_f32(hi) + bf16_to_f32(lo);
      X += v;
      Xc += dq_offset(b & 1, (kk & 7) >> 1) * v;
    }
    w.xs[(size_t)t * nb + b] = make_float2(X, Xc);
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
// decode_gateup.  Grid: (routed capacity x F/32) + Fs/32 blocks of 512 threads.
// Wave w: h-group hs = w/4 (16 FFN rows), matrix = (w/2)%2 (gate, up), K half
// = w%2 (octets o = half, half+2, ...).
template <int T, int FMT, bool HAS_LO>
__global__ __launch_bounds__(512) void decode_gateup_kernel(DecodeArgs a, DecodeWs w) {
  extern __shared__ uint4 s_dyn[];
  __shared__ float s_red[kGuWaves][kDecodeMaxT][16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int D = a.D, oD = octets(D), nbD = D / 32;
  const int has_sh = a.shared != nullptr;
  const int nwork = *w.nwork;
  const int U = nwork - has_sh;
  const int Wr = w.Wmax - 1;
  const int gpr = a.F / 32;
  int u, g, Fi;
  const uint8_t* base;
  if ((int)blockIdx.x < Wr * gpr) {
    u = blockIdx.x / gpr;
    g = blockIdx.x % gpr;
    if (u >= U) return;
    Fi = a.F;
    base = a.routed + (size_t)w.work_ref[u] * a.stride;
  } else {
    if (!has_sh) return;
    g = blockIdx.x - Wr * gpr;
    u = U;
    Fi = a.Fs;
    base = a.shared;
  }
  (void)Fi;
  const int hs = wv >> 2, mat = (wv >> 1) & 1, kh = wv & 1;
  const int n = lane & 15, q = lane >> 4;
  const uint8_t* tile = base + (size_t)((2 * g + hs) * 2 + mat) * oD * rec_bytes(FMT);

  // Issue every weight load of this wave first.
  uint4 cw[kMaxOctPerWave], pa[kMaxOctPerWave], pb[kMaxOctPerWave];
  uint2 hw[kMaxOctPerWave];
#pragma unroll
  for (int i = 0; i < kMaxOctPerWave; ++i) {
    const int o = kh + 2 * i;
    if (o < oD) load_record<FMT>(tile + (size_t)o * rec_bytes(FMT), lane, cw[i], hw[i], pa[i], pb[i]);
  }

  // Stage the activation operand and its block sums in LDS.
  uint4* s_xhi = s_dyn;
  uint4* s_xlo = s_dyn + T * D / 8;
  float2* s_xs = reinterpret_cast<float2*>(s_dyn + (HAS_LO ? 2 : 1) * T * D / 8);
  for (int i = tid; i < T * D / 8; i += 512) {
    s_xhi[i] = reinterpret_cast<const uint4*>(w.xa_hi)[i];
    if (HAS_LO) s_xlo[i] = reinterpret_cast<const uint4*>(w.xa_lo)[i];
  }
  for (int i = tid; i < T * nbD; i += 512) s_xs[i] = w.xs[i];
  __syncthreads();

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
        const int idx = (n * D + 32 * (8 * o + beta) + 8 * q) / 8;
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

  // SwiGLU over 32 FFN rows x T tokens; h in bf16 hi + lo; block sums of h.
  if (tid < 32 * T) {
    const int t = tid >> 5, f = tid & 31, hq = f >> 4, nn = f & 15;
    const float ga = s_red[hq * 4 + 0][t][nn] + s_red[hq * 4 + 1][t][nn];
    const float ub = s_red[hq * 4 + 2][t][nn] + s_red[hq * 4 + 3][t][nn];
    const float h = silu(ga) * ub;
    const uint16_t hi = f32_to_bf16(h);
    const uint16_t lo = f32_to_bf16(h - bf16_to_f32(hi));
    const size_t hidx = ((size_t)u * T + t) * w.Fp + 32 * g + f;
    w.hh[hidx] = hi;
    w.hl[hidx] = lo;
    const float v = bf16_to_f32(hi) + bf16_to_f32(lo);
    float X = v, Xc = dq_offset(g & 1, (f & 7) >> 1) * v;
#pragma unroll
    for (int o2 = 16; o2 >= 1; o2 >>= 1) {
      X += __shfl_xor(X, o2, 64);
      Xc += __shfl_xor(Xc, o2, 64);
    }
    if (f == 0) w.hs[((size_t)u * T + t) * (w.Fp / 32) + g] = make_float2(X, Xc);
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
        const int i = j0 + lane + 64 * j;  // i over [T][2][hrow]
        if (i < nh) {
          const int t = i / (2 * hrow), rem = i % (2 * hrow);
          hv[j] = rem < hrow ? gh[t * hrow + rem] : gl[t * hrow + rem - hrow];
        }
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
          return w.hs[((size_t)u * T + t) * (Fp / 32) + 8 * o + beta];
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

template <int T, int FMT>
static hipError_t launch_decode_t(const DecodeArgs& a, const DecodeWs& w, hipStream_t st) {
  static size_t lds_gu_lo = 0, lds_gu = 0, lds_dn = 0;
  const bool has_lo = !a.x_bf16 && !a.rmsnorm;
  const size_t lds = (size_t)T * a.D * 2 * (has_lo ? 2 : 1) + (size_t)T * (a.D / 32) * 8;
  const size_t lds_down = (size_t)kDnWaves * T * 2 * w.Fp * 2;
  hipError_t e;
  if (has_lo) {
    if ((e = allow_lds(decode_gateup_kernel<T, FMT, true>, lds, lds_gu_lo)) != hipSuccess) return e;
  } else {
    if ((e = allow_lds(decode_gateup_kernel<T, FMT, false>, lds, lds_gu)) != hipSuccess) return e;
  }
  if ((e = allow_lds(decode_down_kernel<T, FMT>, lds_down, lds_dn)) != hipSuccess) return e;
  decode_prep_kernel<T><<<1, 256, 0, st>>>(a, w);
  const int Wr = w.Wmax - 1;
  const int nblk = Wr * (a.F / 32) + (a.shared ? a.Fs / 32 : 0);
  KernelTimer& tm = kernel_timer();
  if ((e = record_timer_event(tm.before, st)) != hipSuccess) return e;
  if (has_lo)
    decode_gateup_kernel<T, FMT, true><<<nblk, 512, lds, st>>>(a, w);
  else
    decode_gateup_kernel<T, FMT, false><<<nblk, 512, lds, st>>>(a, w);
  if ((e = record_timer_event(tm.after, st)) != hipSuccess) return e;
  tm.before = tm.after = nullptr;
  decode_down_kernel<T, FMT><<<a.D / 16, 1024, lds_down, st>>>(a, w);
  return hipGetLastError();
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
