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

// Wave-wide reductions through DPP (GFX9 row/bank controls): quad swaps,
// half-row and row mirrors combine the 16 lanes of a row; row_bcast:15 and
// row_bcast:31 carry row results upwards, so lane 63 ends with the total,
// which readlane makes uniform.
constexpr int kDppQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROWS, 0xF, false);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  constexpr uint32_t ID = 0u;  // identity of max: rows the DPP step skips keep it
  v = max(v, dpp_u32<kDppQuadSwap1, 0xF>(ID, v));
  v = max(v, dpp_u32<kDppQuadSwap2, 0xF>(ID, v));
  v = max(v, dpp_u32<kDppRowHalfMirror, 0xF>(ID, v));
  v = max(v, dpp_u32<kDppRowMirror, 0xF>(ID, v));
  v = max(v, dpp_u32<kDppRowBcast15, 0xA>(ID, v));
  v = max(v, dpp_u32<kDppRowBcast31, 0xC>(ID, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  constexpr uint32_t ID = 0xFFFFFFFFu;  // identity of min
  v = min(v, dpp_u32<kDppQuadSwap1, 0xF>(ID, v));
  v = min(v, dpp_u32<kDppQuadSwap2, 0xF>(ID, v));
  v = min(v, dpp_u32<kDppRowHalfMirror, 0xF>(ID, v));
  v = min(v, dpp_u32<kDppRowMirror, 0xF>(ID, v));
  v = min(v, dpp_u32<kDppRowBcast15, 0xA>(ID, v));
  v = min(v, dpp_u32<kDppRowBcast31, 0xC>(ID, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Sum over the wave (fixed combination order), uniform result.
__device__ __forceinline__ float wave_sum_f32(float v) {
  auto add = [](float a, uint32_t b) { return a + __uint_as_float(b); };
  v = add(v, dpp_u32<kDppQuadSwap1, 0xF>(0u, __float_as_uint(v)));
  v = add(v, dpp_u32<kDppQuadSwap2, 0xF>(0u, __float_as_uint(v)));
  v = add(v, dpp_u32<kDppRowHalfMirror, 0xF>(0u, __float_as_uint(v)));
  v = add(v, dpp_u32<kDppRowMirror, 0xF>(0u, __float_as_uint(v)));
  v = add(v, dpp_u32<kDppRowBcast15, 0xA>(0u, __float_as_uint(v)));
  v = add(v, dpp_u32<kDppRowBcast31, 0xC>(0u, __float_as_uint(v)));
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 63));
}

// Order keys of row[0..E) for one wave: expert e lives in lane e % 64, slot
// e / 64 (0 = empty; no finite logit maps to 0).
template <int VPL>
__device__ __forceinline__ void load_keys(const float* __restrict__ row, int E, int lane,
                                          uint32_t (&key)[VPL]) {
  // Every load is issued (slots past E read entry 0) and the slot test is a
  // select afterwards: as a guarded load, each one sat in its own branch with
  // a wait for it before the next was issued.
  float v[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = i * 64 + lane;
    v[i] = row[e < E ? e : 0];
  }
#pragma unroll
  for (int i = 0; i < VPL; ++i) key[i] = i * 64 + lane < E ? ord_key(v[i]) : 0u;
}

// Exact top-k by a tournament (any k <= 64): each lane keeps its head, its
// largest key (lowest slot on equal keys).  Round r takes the wave maximum of
// the heads; equal maxima in several lanes go to the lowest expert id (lowest
// slot, then lowest lane).  The winning lane drops that key and recomputes its
// head.  After k rounds lane j < k holds the j-th expert and its (canonical)
// logit: larger logits first, equal logits by ascending id.  Consumes `key`.
template <int VPL>
__device__ __forceinline__ void topk_tournament(uint32_t (&key)[VPL], int k, int lane, int& my_e,
                                                float& my_l) {
  uint32_t hv;
  int hs;
  auto head = [&]() {
    hv = key[VPL - 1];
    hs = VPL - 1;
#pragma unroll
    for (int i = VPL - 2; i >= 0; --i) {
      const bool b = key[i] >= hv;
      hv = b ? key[i] : hv;
      hs = b ? i : hs;
    }
  };
  head();
  my_e = 0;
  my_l = 0.f;
  for (int r = 0; r < k; ++r) {
    const uint32_t mv = wave_max_u32(hv);
    const unsigned long long tie = __ballot(hv == mv);
    int win;
    if (__popcll(tie) == 1) {
      win = __builtin_ctzll(tie);
    } else {
      const uint32_t id = hv == mv ? (uint32_t)(hs * 64 + lane) : 0xFFFFFFFFu;
      win = (int)(wave_min_u32(id) & 63u);
    }
    const int wslot = __builtin_amdgcn_readlane(hs, win);
    if (lane == r) {
      my_e = wslot * 64 + win;
      my_l = ord_key_inv(mv);
    }
    if (lane == win) {
#pragma unroll
      for (int i = 0; i < VPL; ++i) key[i] = i == hs ? 0u : key[i];
      head();
    }
  }
}

// LDS scratch of one wave for topk_threshold.
struct __attribute__((aligned(16))) TopkScratch {
  uint32_t g[16];  // maxima of the 16 lane quads
  uint2 cand[64];  // candidates as {~id, key}
  uint2 top[16];   // {id, key} of ranks 0..15
};

// Exact top-k (k <= 16) in a fixed number of steps instead of k dependent
// rounds.  tau = the k-th largest of the 16 lane-quad maxima: those k maxima
// are k distinct keys >= tau, so the top k all have key >= tau, and only the
// keys >= tau (usually a few more than k) stay candidates.  Candidates are
// packed into LDS; each one's rank is the number of candidates before it in
// the order (key descending, id ascending), i.e. of larger 64-bit values
// key << 32 | ~id.  Lane j < k then gets the candidate of rank j, which is the
// tournament's result.  Returns false (nothing decided) when more than 64
// keys pass tau.  Does not change `key`.
template <int VPL>
__device__ __forceinline__ bool topk_threshold(const uint32_t (&key)[VPL], int k, int lane,
                                               TopkScratch& S, int& my_e, float& my_l) {
  uint32_t t[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) t[i] = key[i];
#pragma unroll
  for (int w = VPL / 2; w >= 1; w /= 2)
#pragma unroll
    for (int i = 0; i < w; ++i) t[i] = max(t[i], t[i + w]);
  uint32_t h = t[0];
  h = max(h, dpp_u32<kDppQuadSwap1, 0xF>(0u, h));
  h = max(h, dpp_u32<kDppQuadSwap2, 0xF>(0u, h));
  if ((lane & 3) == 0) S.g[lane >> 2] = h;
  wave_lds_fence();
  uint32_t tc;
  {
    const uint4* g4 = reinterpret_cast<const uint4*>(S.g);
    const uint32_t mine = S.g[lane & 15];
    int c = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 v = g4[j];
      c += (v.x >= mine) + (v.y >= mine) + (v.z >= mine) + (v.w >= mine);
    }
    tc = (lane < 16 && c >= k) ? mine : 0u;
  }
  uint32_t tau = wave_max_u32(tc);
  tau = tau > 0u ? tau : 1u;  // empty slots are never candidates
  int C = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const bool f = key[i] >= tau;
    const unsigned long long m = __ballot(f);
    const int pos = C + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (f && pos < 64) S.cand[pos] = make_uint2(~(uint32_t)(i * 64 + lane), key[i]);
    C += __popcll(m);
  }
  if (C > 64) return false;  // uniform
  wave_lds_fence();
  const uint2 mc = S.cand[lane];
  const uint64_t mv = ((uint64_t)mc.y << 32) | mc.x;
  int r = 0;
  const uint4* c4 = reinterpret_cast<const uint4*>(S.cand);
  for (int j0 = 0; j0 < C; j0 += 8) {  // 8 candidates per pass (4 reads in flight)
    uint4 v[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) v[jj] = c4[j0 / 2 + jj];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint64_t a = ((uint64_t)v[jj].y << 32) | v[jj].x;
      const uint64_t b = ((uint64_t)v[jj].w << 32) | v[jj].z;
      r += (j0 + 2 * jj < C && a > mv) ? 1 : 0;
      r += (j0 + 2 * jj + 1 < C && b > mv) ? 1 : 0;
    }
  }
  if (lane < C && r < k) S.top[r] = make_uint2(~mc.x, mc.y);
  wave_lds_fence();
  if (lane < k) {
    const uint2 tp = S.top[lane];
    my_e = (int)tp.x;
    my_l = ord_key_inv(tp.y);
  } else {
    my_e = 0;
    my_l = 0.f;
  }
  return true;
}

template <int VPL>
__device__ __forceinline__ void wave_topk(const float* __restrict__ row, int E, int k, int lane,
                                          TopkScratch& S, int& my_e, float& my_l) {
  uint32_t key[VPL];
  load_keys<VPL>(row, E, lane, key);
  if (k <= 16 && topk_threshold<VPL>(key, k, lane, S, my_e, my_l)) return;
  topk_tournament<VPL>(key, k, lane, my_e, my_l);
}

// Top-k of row[0..E) by one wave (E <= kMaxExperts, k <= kMaxTopK): lane j < k
// gets the j-th expert and its logit, larger logits first, equal logits by
// ascending id.  S: this wave's LDS scratch.
__device__ __forceinline__ void wave_topk_any(const float* __restrict__ row, int E, int k, int lane,
                                              TopkScratch& S, int& my_e, float& my_l) {
  if (E <= 512)
    wave_topk<8>(row, E, k, lane, S, my_e, my_l);
  else if (E <= 1024)
    wave_topk<16>(row, E, k, lane, S, my_e, my_l);
  else
    wave_topk<32>(row, E, k, lane, S, my_e, my_l);
}

// Gate of lane j < k: exp(l_j - l_0) / sum_i exp(l_i - l_0) (0 for other lanes).
__device__ __forceinline__ float wave_gate(float my_l, int k, int lane) {
  const float l0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_l), 0));
  const float z = lane < k ? expf(my_l - l0) : 0.f;
  const float s = wave_sum_f32(z);
  return lane < k ? z / s : 0.f;
}

}  // namespace moe
