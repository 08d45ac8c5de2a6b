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
//     (d_model 3072, 512 experts), so it is latency- and HBM-bound.  One
//     one-wave block per expert row; each lane requests its row pieces and
//     the matching activation pieces at once, then a wave-wide sum per token.
//   * router_gemm_kernel, more tokens: a bf16 MFMA GEMM (16x16x32) over
//     tiles of 64 tokens x 128 experts with k-steps of 64 staged through LDS
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
// GEMV, T <= 4.  One wave per expert row and one wave per block, so the grid
// has E blocks and every CU reads a share of W_r.  Lane l owns the 16-byte
// pieces c = l + 64 j (8 values each) of the row and, for every token, the
// same pieces of the activations, so the dot products need neither LDS nor a
// block barrier.  Every load of the wave is issued before the first one is
// used.  Piece indices past the row are clamped into it (the same line for
// every lane) and their activation values replaced by zeros with a select,
// so the loads carry no branches and the clamped pieces add exact zeros.
// Under the RMS rule each lane sums the squares of its pieces of a token in
// order, a wave-wide sum completes it, and every activation value is scaled
// and rounded to bf16 before use.
constexpr int kRvJ = 8;  // pieces per lane: d_model <= 4096

template <int T, bool X_BF16, bool RMS>
__global__ __launch_bounds__(64) void router_gemv_kernel(const void* __restrict__ x,
                                                         const uint16_t* __restrict__ W,
                                                         float* __restrict__ logits, int D, int E) {
  const int lane = threadIdx.x, e = blockIdx.x;
  const int nch = D / 8;
  int cc[kRvJ];
  bool ok[kRvJ];
#pragma unroll
  for (int j = 0; j < kRvJ; ++j) {
    const int c = lane + 64 * j;
    ok[j] = c < nch;
    cc[j] = ok[j] ? c : nch - 1;
  }
  const uint4* wrow = reinterpret_cast<const uint4*>(W + (size_t)e * D);
  uint4 wr[kRvJ];
#pragma unroll
  for (int j = 0; j < kRvJ; ++j) wr[j] = wrow[cc[j]];
  // One token's dot product over the lane's pieces (values v[j][0..7]).
  auto dot = [&](const float (&v)[kRvJ][8]) __attribute__((always_inline)) -> float {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kRvJ; ++j) {
      const uint32_t ww[4] = {wr[j].x, wr[j].y, wr[j].z, wr[j].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s = fmaf(bf16_lo(ww[i]), v[j][2 * i], s);
        s = fmaf(bf16_hi(ww[i]), v[j][2 * i + 1], s);
      }
    }
    return s;
  };
  // The RMS rule on one token's values, in place.
  auto rms = [&](float (&v)[kRvJ][8]) __attribute__((always_inline)) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < kRvJ; ++j)
#pragma unroll
      for (int h = 0; h < 8; ++h) ss = fmaf(v[j][h], v[j][h], ss);
    const float r = 1.0f / sqrtf(wave_sum(ss) / (float)D + 1e-6f);
#pragma unroll
    for (int j = 0; j < kRvJ; ++j)
#pragma unroll
      for (int h = 0; h < 8; ++h) v[j][h] = bf16_to_f32(f32_to_bf16(v[j][h] * r));
  };
  float acc[T];
  if constexpr (X_BF16) {
    uint4 xr[T][kRvJ];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int j = 0; j < kRvJ; ++j)
        xr[t][j] = reinterpret_cast<const uint4*>(x)[(size_t)t * nch + cc[j]];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float v[kRvJ][8];
#pragma unroll
      for (int j = 0; j < kRvJ; ++j) {
        const uint32_t uu[4] = {xr[t][j].x, xr[t][j].y, xr[t][j].z, xr[t][j].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[j][2 * i] = ok[j] ? bf16_lo(uu[i]) : 0.f;
          v[j][2 * i + 1] = ok[j] ? bf16_hi(uu[i]) : 0.f;
        }
      }
      if (RMS) rms(v);
      acc[t] = dot(v);
    }
  } else {  // fp32 input: one token's pieces at a time (64 registers each)
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float4* xp = reinterpret_cast<const float4*>(x) + (size_t)t * 2 * nch;
      float4 xa[kRvJ], xb[kRvJ];
#pragma unroll
      for (int j = 0; j < kRvJ; ++j) {
        xa[j] = xp[2 * cc[j]];
        xb[j] = xp[2 * cc[j] + 1];
      }
      float v[kRvJ][8];
#pragma unroll
      for (int j = 0; j < kRvJ; ++j) {
        const float f[8] = {xa[j].x, xa[j].y, xa[j].z, xa[j].w, xb[j].x, xb[j].y, xb[j].z, xb[j].w};
#pragma unroll
        for (int h = 0; h < 8; ++h) v[j][h] = ok[j] ? f[h] : 0.f;
      }
      if (RMS) rms(v);
      acc[t] = dot(v);
    }
  }
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const float s = wave_sum(acc[t]);
    if (lane == t) logits[(size_t)t * E + e] = s;
  }
}

// ---------------------------------------------------------------------------
// GEMM, any T.  Block: 4 waves, tile of 64 tokens (m) x 128 experts (n);
// wave w computes experts 32 w .. 32 w + 31 of the tile for all 64 tokens
// (4 x 2 MFMA tiles of 16 x 16), k-steps of 64.  The activation tile is
// shared by the four waves and goes through LDS (two buffers); each wave's
// W_r rows are its own and go straight from memory into MFMA B registers.
// Both are fetched two k-steps ahead.  Two blocks share a CU (two waves per
// SIMD).  Measured at 8192 tokens: 61 us, against 63 us for tiles of 256
// experts (one block per CU), 70 us for tiles of 64 and 65 us with four
// register sets per operand (loads four k-steps ahead).
constexpr int kRgM = 64, kRgN = 128, kRgK = 64;
constexpr int kRgJ = kRgN / 64;  // column tiles of 16 experts per wave
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
__global__ __launch_bounds__(256, 2) void router_gemm_kernel(const void* __restrict__ x,
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
  // B operand of tile j: W_r row n0 + 16 kRgJ w + 16 j + n (rows past E read
  // row E-1), columns 32 kk + 8 q .. +7 of the k-step.
  const uint16_t* bptr[kRgJ];
#pragma unroll
  for (int j = 0; j < kRgJ; ++j) {
    const int e = n0 + 16 * kRgJ * wv + 16 * j + n;
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
  auto load_b = [&](uint4 (&B)[kRgJ][2], int s) __attribute__((always_inline)) {
    const int k0 = kRgK * s;
#pragma unroll
    for (int j = 0; j < kRgJ; ++j)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) B[j][kk] = *reinterpret_cast<const uint4*>(bptr[j] + k0 + 32 * kk);
  };

  f32x4_t acc[4][kRgJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kRgJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const uint16_t* L, const uint4 (&B)[kRgJ][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      uint4 af[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const uint4*>(&L[(i * 16 + n) * kRgLd + kk * 32 + 8 * q]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < kRgJ; ++j) acc[i][j] = mfma16(af[i], B[j][kk], acc[i][j]);
    }
  };

  // Steps s (even) and s + 1 per iteration; buffer 0 / register set X hold
  // even steps, buffer 1 / set Y odd ones.  Loads past the last step reload it.
  RgA<X_BF16> aX, aY;
  uint4 bX[kRgJ][2], bY[kRgJ][2];
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
  // D[4 q + r][n] of tile (i, j): token m0 + 16 i + 4 q + r, expert n0 + 16 kRgJ w + 16 j + n.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = m0 + 16 * i + 4 * q + r;
      if (t < T) {
#pragma unroll
        for (int j = 0; j < kRgJ; ++j) {
          const int e = n0 + 16 * kRgJ * wv + 16 * j + n;
          if (e < E) logits[(size_t)t * E + e] = acc[i][j][r];
        }
      }
    }
}

template <int T>
hipError_t launch_gemv_t(const RouterArgs& a, hipStream_t st) {
  auto k = a.x_bf16 ? (a.rmsnorm ? router_gemv_kernel<T, true, true> : router_gemv_kernel<T, true, false>)
                    : (a.rmsnorm ? router_gemv_kernel<T, false, true> : router_gemv_kernel<T, false, false>);
  return launch_timed_by(router_timer(), k, dim3(a.E), dim3(64), 0u, st, a.x, a.w, a.logits, a.D,
                         a.E);
}

}  // namespace

// The GEMV holds a lane's share of one row and of the T x d_model
// activations in registers (d_model <= 4096).
bool router_uses_gemv(int T, int D) { return T <= 4 && D <= 64 * 8 * kRvJ; }

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
