// Wave-level top-k selection and gate computation shared by the router
// kernels.  Reading of the pages (which give no formula): experts ranked on the
// raw fp32 logits, larger first, ties to the lower id, -0.0 == +0.0; gates are
// a softmax over the selected logits.
#pragma once

#include "kernels.hpp"

namespace moe {

constexpr int kMaxExperts = 2048;
constexpr int kMaxTopK = 32;

// Monotone map of a float to uint32 (after canonicalising -0.0 to +0.0).
__device__ __forceinline__ uint32_t ord_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ord_key_inv(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// 64-bit composite key (value key << 32 | ~expert id): larger wins, so equal
// values resolve to the lower expert id; 0 marks an empty or taken slot
// (every real key has a nonzero value half).
typedef unsigned long long key64;

__device__ __forceinline__ key64 make_key(uint32_t vk, int e) {
  return ((key64)vk << 32) | (key64)(0xFFFFFFFFu - (uint32_t)e);
}

// LDS entries of wave_topk's scratch for a given slot count and k, and the
// slot count used for E experts.
// (64 lane maxima, up to k*VPL candidates + 2 pad, k ranked outputs; even
// so that consecutive regions stay 16-byte aligned)
__host__ __device__ constexpr int topk_scratch(int vpl, int k) {
  return (64 + (k * vpl + 2) + k + 1) / 2 * 2;
}
__host__ __device__ constexpr int topk_vpl(int E) { return E <= 512 ? 8 : (E <= 1024 ? 16 : 32); }
__host__ __device__ constexpr size_t topk_scratch_bytes(int E, int k) {
  return (size_t)topk_scratch(topk_vpl(E), k) * 8;
}

__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Top-k of row[0..E) by one wave (E <= 64 * VPL), exact.  Expert e lives in
// lane e % 64, slot e / 64; every key is the composite (value, ~id), so all
// keys are distinct and order = value descending, id ascending.
//  1. Each lane takes the maximum of its keys; the lane maxima are ranked
//     against each other through LDS.  The k-th largest lane maximum L is a
//     lower bound of the k-th largest key (at least k keys are >= L), so
//     every top-k key is >= L.  (Fewer than k non-empty lanes: L = 0.)
//  2. The keys >= L -- at most k lanes contribute, so at most k*VPL -- are
//     compacted into LDS and ranked against each other; those of rank < k
//     are stored at their rank.
// Afterwards lane j < k holds the j-th selected expert and its (canonical)
// logit.  `scratch`: topk_scratch(VPL, k) LDS entries private to the wave.
template <int VPL>
__device__ __forceinline__ void wave_topk(const float* __restrict__ row, int E, int k, int lane,
                                          int& my_e, float& my_l, key64* scratch) {
  key64 key[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = i * 64 + lane;
    key[i] = e < E ? make_key(ord_key(row[e]), e) : 0ull;
  }
  key64 m = key[0];
#pragma unroll
  for (int i = 1; i < VPL; ++i) m = key[i] > m ? key[i] : m;
  scratch[lane] = m;
  wave_lds_fence();
  int r = 0;
  {
    const uint4* s4 = reinterpret_cast<const uint4*>(scratch);  // 2 keys per read
    uint4 v[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) v[j] = s4[j];
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const key64 a0 = ((key64)v[j].y << 32) | v[j].x, a1 = ((key64)v[j].w << 32) | v[j].z;
      r += (a0 > m ? 1 : 0) + (a1 > m ? 1 : 0);
    }
  }
  const unsigned long long nonempty = __ballot(m != 0ull);
  key64 L = 0ull;
  if (__popcll(nonempty) >= k) {
    const unsigned long long at = __ballot(m != 0ull && r == k - 1);
    const int src = __builtin_ctzll(at);
    // readlane returns int: widen through uint32_t (no sign extension)
    L = ((key64)(uint32_t)__builtin_amdgcn_readlane((uint32_t)(m >> 32), src) << 32) |
        (key64)(uint32_t)__builtin_amdgcn_readlane((uint32_t)m, src);
  }
  key64* cand = scratch + 64;
  key64* out = scratch + 64 + k * VPL + 2;
  int C = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const bool c = key[i] != 0ull && key[i] >= L;
    const unsigned long long mc = __ballot(c);
    const int pos = C + __builtin_amdgcn_mbcnt_hi((uint32_t)(mc >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)mc, 0u));
    if (c) cand[pos] = key[i];
    C += __popcll(mc);
  }
  wave_lds_fence();
  if (C & 1) cand[C] = 0ull;  // pad to an even count (a 0 key never outranks)
  wave_lds_fence();
  for (int j = lane; j < C; j += 64) {
    const key64 c = cand[j];
    int rank = 0;
    const uint4* c4 = reinterpret_cast<const uint4*>(cand);
    for (int i = 0; i < (C + 1) / 2; ++i) {
      const uint4 v = c4[i];
      const key64 a0 = ((key64)v.y << 32) | v.x, a1 = ((key64)v.w << 32) | v.z;
      rank += (a0 > c ? 1 : 0) + (a1 > c ? 1 : 0);
    }
    if (rank < k) out[rank] = c;
  }
  wave_lds_fence();
  my_e = 0;
  my_l = 0.f;
  if (lane < k) {
    const key64 o = out[lane];
    my_e = (int)(0xFFFFFFFFu - (uint32_t)o);
    my_l = ord_key_inv((uint32_t)(o >> 32));
  }
}

// Dispatch on the number of experts.
__device__ __forceinline__ void wave_topk_any(const float* __restrict__ row, int E, int k, int lane,
                                              int& my_e, float& my_l, key64* scratch) {
  if (E <= 512)
    wave_topk<8>(row, E, k, lane, my_e, my_l, scratch);
  else if (E <= 1024)
    wave_topk<16>(row, E, k, lane, my_e, my_l, scratch);
  else
    wave_topk<32>(row, E, k, lane, my_e, my_l, scratch);
}

// Gate of lane j < k: exp(l_j - l_0) / sum_i exp(l_i - l_0) (0 for other lanes).
__device__ __forceinline__ float wave_gate(float my_l, int k, int lane) {
  const float l0 = __shfl(my_l, 0, 64);
  const float z = lane < k ? expf(my_l - l0) : 0.f;
  float s = z;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
  return lane < k ? z / s : 0.f;
}

}  // namespace moe
