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

// Top-k of row[0..E) by one wave.  Expert e lives in lane e % 64, slot e / 64.
// Afterwards lane j < k holds the j-th selected expert and its (canonical)
// logit.  Composite 64-bit key: (value key << 32) | ~e, so equal values
// resolve to the lower expert id.
__device__ __forceinline__ void wave_topk(const float* __restrict__ row, int E, int k, int lane,
                                          int& my_e, float& my_l) {
  constexpr int VPL = kMaxExperts / 64;
  uint32_t key[VPL];
  uint32_t taken = 0;
  const int nv = (E + 63) / 64;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = i * 64 + lane;
    if (i < nv && e < E) {
      key[i] = ord_key(row[e]);
    } else {
      key[i] = 0u;
      taken |= 1u << i;
    }
  }
  my_e = 0;
  my_l = 0.f;
  for (int r = 0; r < k; ++r) {
    unsigned long long best = 0ull;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      if (i < nv && !((taken >> i) & 1u)) {
        const unsigned long long c = ((unsigned long long)key[i] << 32) |
                                     (unsigned long long)(0xFFFFFFFFu - (uint32_t)(i * 64 + lane));
        best = c > best ? c : best;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const unsigned long long y = __shfl_xor(best, o, 64);
      best = y > best ? y : best;
    }
    const int e = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull));
    if ((e & 63) == lane) taken |= 1u << (e >> 6);
    if (lane == r) {
      my_e = e;
      my_l = ord_key_inv((uint32_t)(best >> 32));
    }
  }
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
