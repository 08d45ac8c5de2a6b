// Router projection: logits[t][e] = sum_d W_r[e][d] * xhat[t][d], fp32.
//
// The pages keep the router on the GPU together with attention and the
// shared expert, since every token needs it ([AF] "个人开发者用 AI 十天写出
// Strata 引擎…", section "命中率七成，代价是答案会变").  They give neither
// its precision nor its form; the reading taken here is a plain bf16
// projection W_r [n_experts][d_model] (one expert's row contiguous, no bias)
// applied to the input the experts see: xhat = x, or bf16(x / sqrt(mean(x^2)
// + 1e-6)) under the RMS input rule.
//
// Two kernels:
//   * router_gemv_kernel, T <= 4 tokens: the step is one 3 MB read of W_r
//     (d_model 3072, 512 experts), so it is latency- and HBM-bound.  One wave
//     per expert row; every lane's row pieces are requested before the
//     activations are staged into LDS, so the weight reads overlap the
//     staging; then a wave-wide sum per token.
//   * router_gemm_kernel, more tokens: a bf16 MFMA GEMM (16x16x32) over
//     tiles of 64 tokens x 256 experts with k-steps of 64 staged through LDS
//     (next k-step prefetched into registers while the current one runs).
//     Both operands are rows contiguous along d, which is exactly the
//     per-lane layout of the MFMA A and B operands, so LDS holds plain
//     row-major tiles (rows padded by 16 bytes: the 16 rows one instruction
//     reads fall on distinct banks).  fp32 activations and the RMS rule are
//     applied while staging (rounded to bf16, as in the prefill path).
#include "kernels.hpp"

namespace moe {

namespace {

// RMS factor 1 / sqrt(mean(x^2) + 1e-6) of one D-long row, computed by one
// wave in the order of the prefill path's input preparation (a 256-thread
// pass: thread i sums elements i, i+256, ... in turn; a wave-wide tree per
// group of 64 threads; the four group sums added in order), so that both give
// the same bits.  Lane l plays threads l, l+64, l+128, l+192.  Every lane
// returns the factor.
__device__ __forceinline__ float wave_rinv(const void* x, bool x_bf16, size_t base, int D, int lane) {
  float p[4] = {0.f, 0.f, 0.f, 0.f};
  for (int i0 = 0; i0 < D; i0 += 256) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int i = i0 + 64 * g + lane;
      if (i < D) {
        const float v = x_bf16 ? bf16_to_f32(((const uint16_t*)x)[base + i]) : ((const float*)x)[base + i];
        p[g] += v * v;
      }
    }
  }
  float tot = wave_sum(p[0]);
#pragma unroll
  for (int g = 1; g < 4; ++g) tot += wave_sum(p[g]);
  return 1.0f / sqrtf(tot / (float)D + 1e-6f);
}

// ---------------------------------------------------------------------------
// GEMV, T <= 4.  Block: 4 waves, expert rows 4 b .. 4 b + 3.  Dynamic LDS:
// the T x D activation values (fp32) the dot products use.  Every global load
// of the block is issued before the first one is waited for: the row pieces,
// then the activation pieces (16 bytes each, at most kRvX per thread).
constexpr int kRvJ = 8;  // row pieces (16 bytes) per lane: d_model <= 4096
constexpr int kRvX = 8;  // activation pieces (8 values) per thread: T * d_model <= 16384

template <int T, bool X_BF16, bool RMS>
__global__ __launch_bounds__(256) void router_gemv_kernel(const void* __restrict__ x,
                                                          const uint16_t* __restrict__ W,
                                                          float* __restrict__ logits, int D, int E) {
  extern __shared__ float s_x[];  // [T][D]
  __shared__ float s_ss[4][T];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int e = blockIdx.x * 4 + wv;
  const int nch = D / 8, npc = T * nch;
  // 1. This wave's row pieces c = lane + 64 j (rows past E read row E-1).
  const uint4* wrow = reinterpret_cast<const uint4*>(W + (size_t)(e < E ? e : E - 1) * D);
  uint4 wr[kRvJ];
#pragma unroll
  for (int j = 0; j < kRvJ; ++j) {
    const int c = lane + 64 * j;
    wr[j] = c < nch ? wrow[c] : make_uint4(0, 0, 0, 0);
  }
  // 2. Activation pieces p = tid + 256 i: values 8 p .. 8 p + 7 of the
  // row-major [T][D] input (a piece never straddles two tokens).
  float xv[kRvX][8];
#pragma unroll
  for (int i = 0; i < kRvX; ++i) {
    const int pc = tid + 256 * i;
    if (X_BF16) {
      const uint4 u = pc < npc ? reinterpret_cast<const uint4*>(x)[pc] : make_uint4(0, 0, 0, 0);
      const uint32_t uu[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        xv[i][2 * h] = bf16_lo(uu[h]);
        xv[i][2 * h + 1] = bf16_hi(uu[h]);
      }
    } else {
      const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 a = pc < npc ? reinterpret_cast<const float4*>(x)[2 * pc] : z;
      const float4 b = pc < npc ? reinterpret_cast<const float4*>(x)[2 * pc + 1] : z;
      xv[i][0] = a.x; xv[i][1] = a.y; xv[i][2] = a.z; xv[i][3] = a.w;
      xv[i][4] = b.x; xv[i][5] = b.y; xv[i][6] = b.z; xv[i][7] = b.w;
    }
  }
  // 3. RMS rule: per-token sums of squares (thread, then wave, then the four
  // waves in order), the same in every block.
  float rinv[T];
#pragma unroll
  for (int t = 0; t < T; ++t) rinv[t] = 1.f;
  if (RMS) {
    float ss[T];
#pragma unroll
    for (int t = 0; t < T; ++t) ss[t] = 0.f;
#pragma unroll
    for (int i = 0; i < kRvX; ++i) {
      const int pc = tid + 256 * i;
      float q = 0.f;
#pragma unroll
      for (int h = 0; h < 8; ++h) q = fmaf(xv[i][h], xv[i][h], q);
#pragma unroll
      for (int t = 0; t < T; ++t) ss[t] += (pc < npc && pc / nch == t) ? q : 0.f;
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float r = wave_sum(ss[t]);
      if (lane == 0) s_ss[wv][t] = r;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float tot = s_ss[0][t] + s_ss[1][t] + s_ss[2][t] + s_ss[3][t];
      rinv[t] = 1.0f / sqrtf(tot / (float)D + 1e-6f);
    }
  }
#pragma unroll
  for (int i = 0; i < kRvX; ++i) {
    const int pc = tid + 256 * i;
    if (pc < npc) {
      float v[8];
      if (RMS) {
        const int t = pc / nch;
        float r = rinv[0];
#pragma unroll
        for (int tt = 1; tt < T; ++tt) r = t == tt ? rinv[tt] : r;
#pragma unroll
        for (int h = 0; h < 8; ++h) v[h] = bf16_to_f32(f32_to_bf16(xv[i][h] * r));
      } else {
#pragma unroll
        for (int h = 0; h < 8; ++h) v[h] = xv[i][h];
      }
      float4* d = reinterpret_cast<float4*>(&s_x[8 * (size_t)pc]);
      d[0] = make_float4(v[0], v[1], v[2], v[3]);
      d[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
  __syncthreads();
  // 4. Dot products over the lane's pieces, then a wave-wide sum per token.
  float acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = 0.f;
#pragma unroll
  for (int j = 0; j < kRvJ; ++j) {
    const int c = lane + 64 * j;
    if (c < nch) {
      const uint32_t ww[4] = {wr[j].x, wr[j].y, wr[j].z, wr[j].w};
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const float4 xa = *reinterpret_cast<const float4*>(&s_x[(size_t)t * D + 8 * c]);
        const float4 xb = *reinterpret_cast<const float4*>(&s_x[(size_t)t * D + 8 * c + 4]);
        const float xs[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
        float s = acc[t];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s = fmaf(bf16_lo(ww[i]), xs[2 * i], s);
          s = fmaf(bf16_hi(ww[i]), xs[2 * i + 1], s);
        }
        acc[t] = s;
      }
    }
  }
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const float v = wave_sum(acc[t]);
    if (lane == 0 && e < E) logits[(size_t)t * E + e] = v;
  }
}

// ---------------------------------------------------------------------------
// GEMM, any T.  Block: 4 waves, tile of 64 tokens (m) x 256 experts (n);
// wave w computes experts 64 w .. 64 w + 63 of the tile for all 64 tokens
// (4 x 4 MFMA tiles of 16 x 16), k-steps of 64.  The activation tile is
// shared by the four waves and goes through LDS (two buffers); each wave's
// W_r rows are its own and go straight from memory into MFMA B registers.
// Both are fetched two k-steps ahead.
constexpr int kRgM = 64, kRgN = 256, kRgK = 64;
constexpr int kRgLd = kRgK + 8;  // bf16 per LDS row: 144 bytes

template <bool X_BF16>
struct RgA;  // one thread's share of an activation k-step, as loaded
template <>
struct RgA<true> {
  uint4 v[2];
};
template <>
struct RgA<false> {
  float4 v[2][2];
};

template <bool X_BF16, bool RMS>
__global__ __launch_bounds__(256) void router_gemm_kernel(const void* __restrict__ x,
                                                          const uint16_t* __restrict__ W,
                                                          float* __restrict__ logits, int T, int D,
                                                          int E) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kRgM * kRgLd];
  __shared__ float s_rinv[kRgM];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int m0 = blockIdx.x * kRgM, n0 = blockIdx.y * kRgN;
  const int n = lane & 15, q = lane >> 4;
  const int nk = D / kRgK;  // even: d_model is a multiple of 256

  if (RMS) {  // wave w: the factors of tile rows w, w + 4, ...
    for (int r = wv; r < kRgM; r += 4) {
      const int row = m0 + r < T ? m0 + r : T - 1;
      const float v = wave_rinv(x, X_BF16, (size_t)row * D, D, lane);
      if (lane == 0) s_rinv[r] = v;
    }
    __syncthreads();
  }
  // Activation piece q' = tid + 256 i (i < 2): tile row q' / 8 = tid / 8 + 32 i,
  // columns 8 (tid % 8) .. +7 of the k-step.  Rows past T read row T-1.
  const int kc = 8 * (tid & 7);
  size_t aoff[2];
  float ar[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (tid >> 3) + 32 * i;
    aoff[i] = (size_t)(m0 + r < T ? m0 + r : T - 1) * D + kc;
    ar[i] = RMS ? s_rinv[r] : 1.f;
  }
  // B operand of tile j: W_r row n0 + 64 w + 16 j + n (rows past E read row
  // E-1), columns 32 kk + 8 q .. +7 of the k-step.
  const uint16_t* bptr[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = n0 + 64 * wv + 16 * j + n;
    bptr[j] = W + (size_t)(e < E ? e : E - 1) * D + 8 * q;
  }

  auto load_a = [&](RgA<X_BF16>& R, int s) __attribute__((always_inline)) {
    const int k0 = kRgK * s;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if constexpr (X_BF16) {
        R.v[i] = *reinterpret_cast<const uint4*>((const uint16_t*)x + aoff[i] + k0);
      } else {
        const float4* p = reinterpret_cast<const float4*>((const float*)x + aoff[i] + k0);
        R.v[i][0] = p[0];
        R.v[i][1] = p[1];
      }
    }
  };
  auto store_a = [&](const RgA<X_BF16>& R, uint16_t* L) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      uint4 u;
      if constexpr (X_BF16) {
        if (RMS) {
          const uint32_t uu[4] = {R.v[i].x, R.v[i].y, R.v[i].z, R.v[i].w};
          uint32_t o[4];
#pragma unroll
          for (int h = 0; h < 4; ++h) o[h] = pack_bf16x2(bf16_lo(uu[h]) * ar[i], bf16_hi(uu[h]) * ar[i]);
          u = make_uint4(o[0], o[1], o[2], o[3]);
        } else {
          u = R.v[i];
        }
      } else {
        const float4 a = R.v[i][0], b = R.v[i][1];
        u = make_uint4(pack_bf16x2(a.x * ar[i], a.y * ar[i]), pack_bf16x2(a.z * ar[i], a.w * ar[i]),
                       pack_bf16x2(b.x * ar[i], b.y * ar[i]), pack_bf16x2(b.z * ar[i], b.w * ar[i]));
      }
      *reinterpret_cast<uint4*>(&L[((tid >> 3) + 32 * i) * kRgLd + kc]) = u;
    }
  };
  auto load_b = [&](uint4 (&B)[4][2], int s) __attribute__((always_inline)) {
    const int k0 = kRgK * s;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) B[j][kk] = *reinterpret_cast<const uint4*>(bptr[j] + k0 + 32 * kk);
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const uint16_t* L, const uint4 (&B)[4][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      uint4 af[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const uint4*>(&L[(i * 16 + n) * kRgLd + kk * 32 + 8 * q]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(af[i], B[j][kk], acc[i][j]);
    }
  };

  // Steps s (even) and s + 1 per iteration; buffer 0 / register set X hold
  // even steps, buffer 1 / set Y odd ones.  Loads past the last step reload it.
  RgA<X_BF16> aX, aY;
  uint4 bX[4][2], bY[4][2];
  load_a(aX, 0);
  load_b(bX, 0);
  load_a(aY, 1);
  load_b(bY, 1);
  store_a(aX, sA[0]);
  __syncthreads();
  for (int s = 0; s < nk; s += 2) {
    const int s2 = s + 2 < nk ? s + 2 : nk - 1, s3 = s + 3 < nk ? s + 3 : nk - 1;
    load_a(aX, s2);
    compute(sA[0], bX);
    load_b(bX, s2);
    store_a(aY, sA[1]);
    __syncthreads();
    load_a(aY, s3);
    compute(sA[1], bY);
    load_b(bY, s3);
    store_a(aX, sA[0]);
    __syncthreads();
  }
  // D[4 q + r][n] of tile (i, j): token m0 + 16 i + 4 q + r, expert n0 + 64 w + 16 j + n.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = m0 + 16 * i + 4 * q + r;
      if (t < T) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = n0 + 64 * wv + 16 * j + n;
          if (e < E) logits[(size_t)t * E + e] = acc[i][j][r];
        }
      }
    }
}

template <int T>
hipError_t launch_gemv_t(const RouterArgs& a, hipStream_t st) {
  const dim3 grid((a.E + 3) / 4);
  const size_t lds = (size_t)T * a.D * sizeof(float);
  auto k = a.x_bf16 ? (a.rmsnorm ? router_gemv_kernel<T, true, true> : router_gemv_kernel<T, true, false>)
                    : (a.rmsnorm ? router_gemv_kernel<T, false, true> : router_gemv_kernel<T, false, false>);
  return launch_timed_by(router_timer(), k, grid, dim3(256), (uint32_t)lds, st, a.x, a.w, a.logits,
                         a.D, a.E);
}

}  // namespace

// The GEMV holds a lane's whole row share in registers (d_model <= 4096) and
// the T x d_model activations in registers and LDS (at most 60 KB).
bool router_uses_gemv(int T, int D) {
  return T <= 4 && D <= 64 * 8 * kRvJ && T * D <= 15360 && T * D <= 256 * 8 * kRvX;
}

hipError_t launch_router(const RouterArgs& a, hipStream_t st) {
  if (a.T <= 0) return hipSuccess;
  if (router_uses_gemv(a.T, a.D)) {
    switch (a.T) {
      case 1: return launch_gemv_t<1>(a, st);
      case 2: return launch_gemv_t<2>(a, st);
      case 3: return launch_gemv_t<3>(a, st);
      default: return launch_gemv_t<4>(a, st);
    }
  }
  const dim3 grid((a.T + kRgM - 1) / kRgM, (a.E + kRgN - 1) / kRgN);
  auto k = a.x_bf16 ? (a.rmsnorm ? router_gemm_kernel<true, true> : router_gemm_kernel<true, false>)
                    : (a.rmsnorm ? router_gemm_kernel<false, true> : router_gemm_kernel<false, false>);
  return launch_timed_by(router_timer(), k, grid, dim3(256), 0u, st, a.x, a.w, a.logits, a.T, a.D,
                         a.E);
}

}  // namespace moe
