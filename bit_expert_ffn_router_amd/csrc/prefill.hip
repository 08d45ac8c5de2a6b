// Prefill path of the MoE layer: many tokens (the pages cut a prompt into
// chunks of at most 8192 tokens and compute layer by layer on the GPU, [AF]
// "个人开发者用 AI 十天写出 Strata 引擎…", section "等最久的，是它读完你的
// 代码"; [SL] section "猜词与校验让速度翻倍").
//
// Steps (all on the caller's stream):
//   route        one wave per token: top-k ids and renormalised gates
//   xprep        (fp32 input or the RMS input rule only) bf16 activations
//   permute      histogram -> scan -> stable scatter of pairs p = t*k + j
//   tiles        the work list of the grouped GEMM: per expert, row tiles of
//                kBM consecutive permuted pairs; the shared expert takes the
//                T tokens as one more group
//   gate/up      grouped GEMM [rows x D] x dequant(W_gate|W_up)^T with the
//                SwiGLU epilogue -> H [rows][F] (bf16)
//   down         grouped GEMM H x dequant(W_down)^T -> Y [rows][D] (bf16)
//   combine      out_t = sum_j g_tj * Y[inv[t*k+j]] + Y[shared row t]
//                (fixed order, no atomics)
//
// The grouped GEMM is the one dense contraction of the layer.  It runs on
// bf16 MFMA (16x16x32) with fp32 accumulation.  Weights stay packed in HBM;
// each pipeline step dequantises one 32-column block of 256 weight rows into
// LDS (one weight row per thread: a 4-entry bf16 table s*u + m built from the
// block's fp16 scale and min, then v_perm byte selects expand the 2-bit codes),
// while the waves run the MFMAs of the previous step.  Row tiles of
// activations are gathered through the permutation into LDS in the MFMA
// operand order.
#include "route_common.hpp"

namespace moe {

namespace {

constexpr int kBM = 128;             // rows (permuted pairs) per tile
constexpr int kBN = 256;             // weight rows per block: 16 MFMA column tiles
constexpr int kPfThreads = 256;      // 4 waves, 2 x 2 over (rows, weight rows)
constexpr int kNT = kBN / 16;        // column tiles per block
constexpr int kRG = kBM / 16;        // row groups per tile

__host__ __device__ inline size_t al256(size_t v) { return (v + 255) / 256 * 256; }

struct PfWs {
  int32_t* idx;       // [T*k]
  float* gate;        // [T*k]
  int32_t* offsets;   // [E+1]
  int32_t* sorted;    // [P]
  int32_t* inv;       // [P]
  PermWs perm;
  int4* tiles;        // [max_tiles] {expert or -1, row0, rows, 0}
  int32_t* ntiles;    // [1]
  uint16_t* xb;       // [T][D] bf16 operand (fp32 or normalised input)
  uint16_t* H;        // [P+T][Fmax] bf16
  uint16_t* Y;        // [P+T][D] bf16
  int max_tiles, Fmax;
};

int pf_max_tiles(int T, int E, int k) {
  const long P = (long)T * k;
  return (int)((P + kBM - 1) / kBM + (E < P ? E : P) + (T + kBM - 1) / kBM);
}

PfWs pf_carve(void* ws, int T, int D, int F, int Fs, int E, int k) {
  PfWs w;
  const size_t P = (size_t)T * k;
  w.max_tiles = pf_max_tiles(T, E, k);
  w.Fmax = F > Fs ? F : Fs;
  uint8_t* p = (uint8_t*)ws;
  auto take = [&](size_t n) { uint8_t* r = p; p += al256(n); return (void*)r; };
  w.idx = (int32_t*)take(4 * P);
  w.gate = (float*)take(4 * P);
  w.offsets = (int32_t*)take(4 * ((size_t)E + 1));
  w.sorted = (int32_t*)take(4 * P);
  w.inv = (int32_t*)take(4 * P);
  void* pw = take(perm_ws_bytes(T, k, E));
  w.perm = perm_ws_carve(pw, T, k, E);
  w.tiles = (int4*)take(16 * (size_t)w.max_tiles);
  w.ntiles = (int32_t*)take(4);
  w.xb = (uint16_t*)take(2 * (size_t)T * D);
  w.H = (uint16_t*)take(2 * (P + T) * (size_t)w.Fmax);
  w.Y = (uint16_t*)take(2 * (P + T) * (size_t)D);
  return w;
}

}  // namespace

size_t prefill_ws_bytes(int T, int D, int F, int Fs, int E, int k) {
  const size_t P = (size_t)T * k;
  const int Fmax = F > Fs ? F : Fs;
  size_t b = al256(4 * P) * 4 + al256(4 * ((size_t)E + 1)) + al256(perm_ws_bytes(T, k, E)) +
             al256(16 * (size_t)pf_max_tiles(T, E, k)) + 256 + al256(2 * (size_t)T * D) +
             al256(2 * (P + T) * (size_t)Fmax) + al256(2 * (P + T) * (size_t)D);
  return b;
}

namespace {

// ----------------------------------------------------------------------------
// bf16 activations for fp32 input and/or the RMS input rule; one block per token.
__global__ __launch_bounds__(256) void pf_xprep_kernel(const void* __restrict__ x, int x_bf16,
                                                       int rms, int D, uint16_t* __restrict__ xb) {
  __shared__ float s_part[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  const size_t base = (size_t)t * D;
  auto val = [&](int i) -> float {
    return x_bf16 ? bf16_to_f32(((const uint16_t*)x)[base + i]) : ((const float*)x)[base + i];
  };
  float rinv = 1.f;
  if (rms) {
    float ss = 0.f;
    for (int i = tid; i < D; i += 256) {
      const float v = val(i);
      ss += v * v;
    }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) s_part[tid >> 6] = ss;
    __syncthreads();
    const float tot = s_part[0] + s_part[1] + s_part[2] + s_part[3];
    rinv = 1.0f / sqrtf(tot / (float)D + 1e-6f);
  }
  for (int i = tid; i < D; i += 256) xb[base + i] = f32_to_bf16(val(i) * rinv);
}

// ----------------------------------------------------------------------------
// Work list of the grouped GEMMs: for each routed expert with M_e pairs,
// ceil(M_e / kBM) tiles over its permuted rows; then the shared expert's tiles
// over rows P .. P+T-1.  One block of 1024 threads.
__global__ __launch_bounds__(1024) void pf_tiles_kernel(const int32_t* __restrict__ offsets, int E,
                                                        int P, int T, int has_shared,
                                                        int4* __restrict__ tiles,
                                                        int32_t* __restrict__ ntiles) {
  __shared__ int32_t s_part[1024];
  const int tid = threadIdx.x;
  const int per = (E + 1023) / 1024;
  int local = 0;
  for (int i = 0; i < per; ++i) {
    const int e = tid * per + i;
    if (e < E) local += (offsets[e + 1] - offsets[e] + kBM - 1) / kBM;
  }
  s_part[tid] = local;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int y = tid >= o ? s_part[tid - o] : 0;
    __syncthreads();
    s_part[tid] += y;
    __syncthreads();
  }
  int run = s_part[tid] - local;
  for (int i = 0; i < per; ++i) {
    const int e = tid * per + i;
    if (e >= E) continue;
    const int r0 = offsets[e], M = offsets[e + 1] - r0;
    for (int m = 0; m < M; m += kBM) tiles[run++] = make_int4(e, r0 + m, M - m < kBM ? M - m : kBM, 0);
  }
  const int nr = s_part[1023];
  if (has_shared) {
    const int ns = (T + kBM - 1) / kBM;
    for (int i = tid; i < ns; i += 1024)
      tiles[nr + i] = make_int4(-1, P + i * kBM, T - i * kBM < kBM ? T - i * kBM : kBM, 0);
    if (tid == 0) *ntiles = nr + ns;
  } else if (tid == 0) {
    *ntiles = nr;
  }
}

// ----------------------------------------------------------------------------
// Dequantisation of one 32-column block of one weight row into the MFMA B
// layout.  Q2SM: w = s*u + m as bf16 via a 4-entry table and byte permutes.
// codes[q] = the record's code word of lane 16q + n covering this block.
__device__ __forceinline__ void dq_row_block_q2(const uint32_t (&codes)[4], int beta,
                                                uint32_t sm, uint4 (&frag)[4]) {
  const float s = f16_to_f32((uint16_t)(sm & 0xFFFFu));
  const float m = f16_to_f32((uint16_t)(sm >> 16));
  const uint32_t lut_lo = pack_bf16x2(m, s + m);                 // u = 0, 1
  const uint32_t lut_hi = pack_bf16x2(fmaf(2.f, s, m), fmaf(3.f, s, m));  // u = 2, 3
  const int sh = 8 * (beta & 1);  // slots 4*(beta%2) .. +3 -> bits 2*slot
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t t = (codes[q] >> (sh + 2 * j)) & 0x00030003u;   // u0 | u1 << 16
      const uint32_t sel = t * 0x202u + 0x01000100u;                 // bytes 2u0,2u0+1,2u1,2u1+1
      v[j] = __builtin_amdgcn_perm(lut_hi, lut_lo, sel);
    }
    frag[q] = make_uint4(v[0], v[1], v[2], v[3]);
  }
}

struct PfArgs {
  int T, D, F, Fs, E, k;
  const uint8_t* routed;
  size_t stride;
  const uint8_t* shared;
  const uint16_t* x;      // bf16 [T][D]
  PfWs w;
  void* out;
  int out_bf16;
};

// Grouped GEMM tile.  MODE 0: gate/up (A = gathered activations, K = D, B =
// the expert's gate/up rows, SwiGLU epilogue into H).  MODE 1: down (A = H
// rows, K = F, B = W_down rows, epilogue into Y).
template <int MODE>
__global__ __launch_bounds__(kPfThreads, 2) void pf_gemm_kernel(PfArgs a, int nN, int nwork) {
  __shared__ uint4 s_a[2][kRG * 4 * 16];   // [stage][row group][q][m]     2 x 8 KB
  __shared__ uint4 s_b[2][kNT * 4 * 16];   // [stage][col tile][q][n]      2 x 16 KB
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  // XCD-aware order: blocks are dispatched round-robin over the 8 XCDs, so
  // block i runs on XCD i % 8; give each XCD a contiguous range of work items
  // (the grid is a multiple of 8, which makes this a bijection).
  const int per_xcd = gridDim.x / 8;
  const int bid = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (bid >= nwork) return;
  const int ti = bid / nN, nb = bid % nN;
  if (ti >= *a.w.ntiles) return;
  const int4 tile = a.w.tiles[ti];
  const int e = tile.x, row0 = tile.y, rows = tile.z;
  const int P = a.T * a.k;
  const bool sh = e < 0;
  const int F = sh ? a.Fs : a.F;
  const uint8_t* base = sh ? a.shared : a.routed + (size_t)e * a.stride;
  const int K = MODE == 0 ? a.D : F;
  const int nkb = K / 32;
  const int oK = octets(K);
  const int NW = MODE == 0 ? 2 * F : a.D;   // weight rows of this GEMM
  if (nb * kBN >= NW) return;

  // A rows of this thread: chunks c = tid, tid + 256 -> (row c/4, quarter c%4)
  const uint16_t* arow[2];
  bool avalid[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = tid + kPfThreads * h, r = c >> 2;
    avalid[h] = r < rows;
    const int pos = row0 + (r < rows ? r : 0);
    if (MODE == 0) {
      const int tok = pos < P ? a.w.sorted[pos] / a.k : pos - P;
      arow[h] = a.x + (size_t)tok * a.D;
    } else {
      arow[h] = a.w.H + (size_t)pos * a.w.Fmax;
    }
  }
  // B row of this thread: column tile tau = tid / 16, row n = tid % 16.
  const int tau = tid >> 4, n = tid & 15;
  const int wrow = nb * kBN + tau * 16;   // first weight row of the tile
  const bool bvalid = wrow < NW;
  const uint8_t* brec = nullptr;          // record of (tile, octet 0)
  if (bvalid) {
    if (MODE == 0) {
      const int hg = wrow / 32, mat = (wrow / 16) & 1;  // h-group, gate/up
      brec = base + (size_t)(hg * 2 + mat) * oK * kRecQ2;
    } else {
      brec = base + down_offset(a.D, F, kQ2) + (size_t)(wrow / 16) * oK * kRecQ2;
    }
  }
  auto load_a = [&](int kb, uint4 (&ra)[2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int q = (tid + kPfThreads * h) & 3;
      ra[h] = avalid[h] ? *reinterpret_cast<const uint4*>(arow[h] + 32 * kb + 8 * q)
                        : make_uint4(0, 0, 0, 0);
    }
  };
  auto load_b = [&](int kb, uint32_t (&rc)[4], uint32_t& rsm) {
    if (bvalid) {
      const uint8_t* rec = brec + (size_t)(kb >> 3) * kRecQ2;
      const int beta = kb & 7;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        rc[q] = *reinterpret_cast<const uint32_t*>(rec + 16 * (16 * q + n) + 4 * (beta >> 1));
      rsm = *reinterpret_cast<const uint32_t*>(rec + 1024 + 4 * (8 * n + beta));
    } else {
      rc[0] = rc[1] = rc[2] = rc[3] = 0u;
      rsm = 0u;
    }
  };
  auto store_stage = [&](int st, int kb, const uint4 (&ra)[2], const uint32_t (&rc)[4],
                         uint32_t rsm) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = tid + kPfThreads * h, r = c >> 2, q = c & 3;
      s_a[st][((r >> 4) * 4 + q) * 16 + (r & 15)] = ra[h];
    }
    uint4 frag[4];
    dq_row_block_q2(rc, kb & 7, rsm, frag);
#pragma unroll
    for (int q = 0; q < 4; ++q) s_b[st][(tau * 4 + q) * 16 + n] = frag[q];
  };

  f32x4_t acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 ra[2];
  uint32_t rc[4], rsm;
  load_a(0, ra);
  load_b(0, rc, rsm);
  store_stage(0, 0, ra, rc, rsm);
  __syncthreads();
  const int m = lane & 15, q = lane >> 4;
  for (int kb = 0; kb < nkb; ++kb) {
    const int st = kb & 1;
    const bool more = kb + 1 < nkb;
    if (more) {
      load_a(kb + 1, ra);
      load_b(kb + 1, rc, rsm);
    }
    uint4 af[4], bf[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = s_a[st][((4 * wm + i) * 4 + q) * 16 + m];
#pragma unroll
    for (int j = 0; j < 8; ++j) bf[j] = s_b[st][((8 * wn + j) * 4 + q) * 16 + m];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = mfma16(af[i], bf[j], acc[i][j]);
    if (more) store_stage(st ^ 1, kb + 1, ra, rc, rsm);
    __syncthreads();
  }

  // Epilogue.  Lane holds D[4*(lane/16) + r][lane % 16] of each 16x16 tile.
  const int rq = 4 * (lane >> 4), cn = lane & 15;
  if (MODE == 0) {
    // tiles 8wn + 2jj (gate) and 8wn + 2jj + 1 (up) belong to h-group
    // (nb*kBN + (8wn + 2jj)*16) / 32 = nb*8 + 4wn + jj
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int hg = nb * (kBN / 32) + 4 * wn + jj;
      if (hg * 16 >= F) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 64 * wm + 16 * i + rq + r;
          if (row < rows) {
            const float h = silu(acc[i][2 * jj][r]) * acc[i][2 * jj + 1][r];
            a.w.H[(size_t)(row0 + row) * a.w.Fmax + 16 * hg + cn] = f32_to_bf16(h);
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = nb * kBN + (8 * wn + j) * 16 + cn;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 64 * wm + 16 * i + rq + r;
          if (row < rows) a.w.Y[(size_t)(row0 + row) * a.D + col] = f32_to_bf16(acc[i][j][r]);
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------
// out_t = sum_j g_tj * Y[inv[t*k + j]] + Y[P + t], in a fixed order.
__global__ __launch_bounds__(256) void pf_combine_kernel(PfArgs a, int has_shared) {
  const int t = blockIdx.x, tid = threadIdx.x;
  const int P = a.T * a.k, D = a.D;
  for (int c = tid; c < D / 8; c += 256) {
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = 0.f;
    for (int j = 0; j < a.k; ++j) {
      const int p = t * a.k + j;
      const float g = a.w.gate[p];
      const uint4 y = reinterpret_cast<const uint4*>(a.w.Y + (size_t)a.w.inv[p] * D)[c];
      const uint32_t yy[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[2 * i] += g * bf16_lo(yy[i]);
        o[2 * i + 1] += g * bf16_hi(yy[i]);
      }
    }
    if (has_shared) {
      const uint4 y = reinterpret_cast<const uint4*>(a.w.Y + (size_t)(P + t) * D)[c];
      const uint32_t yy[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[2 * i] += bf16_lo(yy[i]);
        o[2 * i + 1] += bf16_hi(yy[i]);
      }
    }
    if (a.out_bf16) {
      uint4 v;
      v.x = pack_bf16x2(o[0], o[1]);
      v.y = pack_bf16x2(o[2], o[3]);
      v.z = pack_bf16x2(o[4], o[5]);
      v.w = pack_bf16x2(o[6], o[7]);
      reinterpret_cast<uint4*>(a.out)[(size_t)t * (D / 8) + c] = v;
    } else {
      float4* op = reinterpret_cast<float4*>(a.out) + ((size_t)t * D + 8 * c) / 4;
      op[0] = make_float4(o[0], o[1], o[2], o[3]);
      op[1] = make_float4(o[4], o[5], o[6], o[7]);
    }
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& pa, void* ws, hipStream_t st) {
  const int T = pa.T, D = pa.D, E = pa.E, k = pa.k;
  PfWs w = pf_carve(ws, T, D, pa.F, pa.Fs, E, k);
  hipError_t e;
  if ((e = launch_route(pa.logits, T, E, k, w.idx, w.gate, st)) != hipSuccess) return e;
  const uint16_t* xb = (const uint16_t*)pa.x;
  if (pa.rmsnorm || !pa.x_bf16) {
    pf_xprep_kernel<<<T, 256, 0, st>>>(pa.x, pa.x_bf16, pa.rmsnorm, D, w.xb);
    xb = w.xb;
  }
  if ((e = launch_permute(w.idx, T, k, E, w.offsets, w.sorted, w.inv, w.perm, st)) != hipSuccess)
    return e;
  const int has_sh = pa.shared != nullptr;
  pf_tiles_kernel<<<1, 1024, 0, st>>>(w.offsets, E, T * k, T, has_sh, w.tiles, w.ntiles);
  PfArgs a;
  a.T = T;
  a.D = D;
  a.F = pa.F;
  a.Fs = pa.Fs;
  a.E = E;
  a.k = k;
  a.routed = pa.routed;
  a.stride = pa.stride;
  a.shared = pa.shared;
  a.x = xb;
  a.w = w;
  a.out = pa.out;
  a.out_bf16 = pa.out_bf16;
  const int nN_gu = (2 * w.Fmax + kBN - 1) / kBN;
  const int nN_dn = (D + kBN - 1) / kBN;
  const int nw_gu = w.max_tiles * nN_gu, nw_dn = w.max_tiles * nN_dn;
  if ((e = launch_timed(pf_gemm_kernel<0>, dim3((nw_gu + 7) / 8 * 8), dim3(kPfThreads), 0u, st, a,
                        nN_gu, nw_gu)) != hipSuccess)
    return e;
  pf_gemm_kernel<1><<<(nw_dn + 7) / 8 * 8, kPfThreads, 0, st>>>(a, nN_dn, nw_dn);
  pf_combine_kernel<<<T, 256, 0, st>>>(a, has_sh);
  return hipGetLastError();
}

}  // namespace moe
