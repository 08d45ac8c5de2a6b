// Router (top-k with renormalised gates) and the stable token-to-expert
// permutation (histogram, scan, scatter).
//
// The pages: every token goes to the 10 most relevant of 512 experts plus a
// shared expert, and the router stays resident on the GPU ([AF] "个人开发者
// 用 AI 十天写出 Strata 引擎…", sections "1250 亿参数，每个词只用得上 2%" and
// "命中率七成，代价是答案会变").  They give no gate formula.  Implemented
// reading: rank the raw fp32 logits (larger first, ties to the lower expert
// id, -0.0 equal to +0.0) and take a softmax over the k selected logits.
#include "route_common.hpp"

namespace moe {

__global__ void fill_i32_kernel(int32_t* p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// ----------------------------------------------------------------------------
// One wave per token.
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E,
                                                   int k, int32_t* __restrict__ idx,
                                                   float* __restrict__ gate) {
  __shared__ TopkScratch s_topk[4];
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int my_e;
  float my_l;
  wave_topk_any(logits + (size_t)t * E, E, k, lane, s_topk[threadIdx.x >> 6], my_e, my_l);
  const float g = wave_gate(my_l, k, lane);
  if (lane < k) {
    idx[(size_t)t * k + lane] = my_e;
    gate[(size_t)t * k + lane] = g;
  }
}

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* idx, float* gate,
                        hipStream_t st) {
  if (T == 0) return hipSuccess;
  route_kernel<<<(T + 3) / 4, 256, 0, st>>>(logits, T, E, k, idx, gate);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Permutation.  Pairs p = t*k + j are cut into chunks of kPermChunk.
//  1. hist:        per-chunk expert counts, stored expert-major [E][nchunks];
//  2. chunk_scan:  per expert, exclusive prefix over chunks (one wave/expert)
//                  and the expert's total;
//  3. expert_scan: exclusive prefix over experts -> offsets[E+1];
//  4. scatter:     each pair's position = offsets[e] + earlier chunks' count
//                  + earlier waves' count in its chunk + earlier lanes' count
//                  in its wave.  No atomic decides an order.

size_t perm_ws_bytes(int T, int k, int E) {
  const size_t P = (size_t)T * k;
  const size_t nch = (P + kPermChunk - 1) / kPermChunk;
  return ((size_t)E * nch * 4 + 255) / 256 * 256 + ((size_t)E * 4 + 255) / 256 * 256;
}

PermWs perm_ws_carve(void* ws, int T, int k, int E) {
  const size_t P = (size_t)T * k;
  PermWs w;
  w.nchunks = (int)((P + kPermChunk - 1) / kPermChunk);
  uint8_t* p = (uint8_t*)ws;
  w.chunk_counts = (int32_t*)p;
  p += ((size_t)E * w.nchunks * 4 + 255) / 256 * 256;
  w.totals = (int32_t*)p;
  return w;
}

__global__ __launch_bounds__(kPermChunk) void perm_hist_kernel(const int32_t* __restrict__ idx,
                                                              int P, int E, int nch,
                                                              int32_t* __restrict__ cc) {
  extern __shared__ int32_t s_cnt[];
  const int c = blockIdx.x, tid = threadIdx.x;
  for (int e = tid; e < E; e += blockDim.x) s_cnt[e] = 0;
  __syncthreads();
  const int p = c * kPermChunk + tid;
  if (p < P) atomicAdd(&s_cnt[idx[p]], 1);  // a count: order does not matter
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) cc[(size_t)e * nch + c] = s_cnt[e];
}

__global__ __launch_bounds__(256) void perm_chunk_scan_kernel(int E, int nch,
                                                              int32_t* __restrict__ cc,
                                                              int32_t* __restrict__ totals) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  int32_t* row = cc + (size_t)e * nch;
  int carry = 0;
  for (int base = 0; base < nch; base += 64) {
    const int i = base + lane;
    const int v = i < nch ? row[i] : 0;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (i < nch) row[i] = carry + incl - v;
    carry += __shfl(incl, 63, 64);
  }
  if (lane == 0) totals[e] = carry;
}

// One block of 1024 threads: exclusive scan of totals[E] -> offsets[E+1].
__global__ __launch_bounds__(1024) void perm_expert_scan_kernel(int E,
                                                               const int32_t* __restrict__ totals,
                                                               int32_t* __restrict__ offsets) {
  __shared__ int32_t s_part[1024];
  const int tid = threadIdx.x;
  const int per = (E + 1023) / 1024;
  int local = 0;
  for (int i = 0; i < per; ++i) {
    const int e = tid * per + i;
    if (e < E) local += totals[e];
  }
  s_part[tid] = local;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int y = tid >= o ? s_part[tid - o] : 0;
    __syncthreads();
    s_part[tid] += y;
    __syncthreads();
  }
  int run = s_part[tid] - local;  // exclusive prefix of this thread's range
  for (int i = 0; i < per; ++i) {
    const int e = tid * per + i;
    if (e < E) {
      offsets[e] = run;
      run += totals[e];
    }
  }
  if (tid == 1023) offsets[E] = s_part[1023];
}

__global__ __launch_bounds__(kPermChunk) void perm_scatter_kernel(
    const int32_t* __restrict__ idx, int P, int E, int nch, const int32_t* __restrict__ cc,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ inv) {
  extern __shared__ int32_t s_h[];  // [4 waves][E]
  const int c = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int i = tid; i < 4 * E; i += blockDim.x) s_h[i] = 0;
  __syncthreads();
  const int p = c * kPermChunk + tid;
  const int e = p < P ? idx[p] : -1;
  // Rank among earlier lanes of this wave with the same expert.
  int r = 0;
  for (int i = 0; i < 64; ++i) {
    const int ei = __shfl(e, i, 64);
    r += (i < lane && ei == e) ? 1 : 0;
  }
  if (e >= 0) atomicAdd(&s_h[wv * E + e], 1);  // per-wave count; order-free
  __syncthreads();
  if (e >= 0) {
    int prior = 0;
    for (int w = 0; w < wv; ++w) prior += s_h[w * E + e];
    const int pos = offsets[e] + cc[(size_t)e * nch + c] + prior + r;
    sorted_pairs[pos] = p;
    inv[p] = pos;
  }
}

hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* offsets,
                          int32_t* sorted_pairs, int32_t* inv, const PermWs& w, hipStream_t st) {
  const int P = T * k;
  if (P == 0) {
    fill_i32_kernel<<<(E + 256) / 256, 256, 0, st>>>(offsets, E + 1, 0);
    return hipGetLastError();
  }
  perm_hist_kernel<<<w.nchunks, kPermChunk, E * sizeof(int32_t), st>>>(idx, P, E, w.nchunks,
                                                                        w.chunk_counts);
  perm_chunk_scan_kernel<<<(E + 3) / 4, 256, 0, st>>>(E, w.nchunks, w.chunk_counts, w.totals);
  perm_expert_scan_kernel<<<1, 1024, 0, st>>>(E, w.totals, offsets);
  perm_scatter_kernel<<<w.nchunks, kPermChunk, 4 * E * sizeof(int32_t), st>>>(
      idx, P, E, w.nchunks, w.chunk_counts, offsets, sorted_pairs, inv);
  return hipGetLastError();
}

}  // namespace moe
