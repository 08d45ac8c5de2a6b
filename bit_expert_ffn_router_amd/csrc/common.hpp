// Device helpers shared by the libmoe kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kQ2 = 1;   // Q2SM: w = s*u + m
constexpr int kQ3 = 2;   // Q3S:  w = s*q
constexpr int kQ2S = 3;  // Q2S:  w = s*(u - 2)
constexpr int kRecQ2 = 1536;  // bytes of a 16-row x 256-column record
constexpr int kRecQ3 = 1792;
constexpr int kRecQ2S = 1280;
constexpr int kWave = 64;

__host__ __device__ constexpr int rec_bytes(int fmt) {
  return fmt == kQ2 ? kRecQ2 : (fmt == kQ3 ? kRecQ3 : kRecQ2S);
}
__host__ __device__ constexpr int octets(int K) { return (K + 255) / 256; }

// Byte offset of the down region inside a packed expert.
__host__ __device__ inline size_t down_offset(int D, int F, int fmt) {
  return (size_t)2 * (F / 16) * octets(D) * rec_bytes(fmt);
}
__host__ __device__ inline size_t packed_bytes(int D, int F, int fmt) {
  return down_offset(D, F, fmt) + (size_t)(D / 16) * octets(F) * rec_bytes(fmt);
}

// D = (A & M) | C.  Written in plain C so that the compiler emits (and
// tracks hazards for) v_and_or_b32 itself; M and C arrive in VGPRs (see
// dq_consts), so no literal operand blocks the fused form.  Inline asm is
// avoided on purpose: the hazard recognizer does not see through it, and an
// asm write to a register still owned by an in-flight MFMA result gets
// overwritten when the MFMA retires.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  return (a & m) | c;
}

// 16x16x32 bf16 MFMA: D = A(16x32) * B(32x16) + C.  Lane l holds A[l%16][8*(l/16)+0..7],
// B[8*(l/16)+0..7][l%16] and D[4*(l/16)+r][l%16] for r = 0..3.
__device__ __forceinline__ f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// Order this wave's LDS accesses around an exchange between its own lanes
// (release / acquire fences at wavefront scope around a wave barrier).
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// fp32 -> bf16, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t b = __float_as_uint(f);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Magic-number constants of the decode dequantiser.  A 2-bit (or 3-bit) code
// field at mantissa bits [2i, 2i+1(+2)] of a bf16 whose exponent is 7-2i reads
// as c_i + u with c_i = 128, 32, 8 for i = 0, 1, 2.
struct DqConsts {
  uint32_t m0, m1, m2;     // 2-bit field masks at positions 0, 2, 4 of each half
  uint32_t h0, h1, h2;     // third-bit masks (Q3S) at positions 2, 4, 6
  uint32_t c0, c1, c2;     // bf16 pairs 128, 32, 8
};
__device__ __forceinline__ DqConsts dq_consts() {
  DqConsts k;
  // Values pass through readfirstlane so the compiler keeps them in registers
  // instead of folding literals the VOP3 and_or cannot take.
  k.m0 = __builtin_amdgcn_readfirstlane(0x00030003u);
  k.m1 = __builtin_amdgcn_readfirstlane(0x000C000Cu);
  k.m2 = __builtin_amdgcn_readfirstlane(0x00300030u);
  k.h0 = __builtin_amdgcn_readfirstlane(0x00040004u);
  k.h1 = __builtin_amdgcn_readfirstlane(0x00100010u);
  k.h2 = __builtin_amdgcn_readfirstlane(0x00400040u);
  k.c0 = __builtin_amdgcn_readfirstlane(0x43004300u);
  k.c1 = __builtin_amdgcn_readfirstlane(0x42004200u);
  k.c2 = __builtin_amdgcn_readfirstlane(0x41004100u);
  // Move to VGPRs once (v_and_or_b32 on gfx9 may read at most one SGPR).
  asm volatile("" : "+v"(k.m0), "+v"(k.m1), "+v"(k.m2), "+v"(k.h0), "+v"(k.h1), "+v"(k.h2),
               "+v"(k.c0), "+v"(k.c1), "+v"(k.c2));
  return k;
}

// Q2SM / Q2S code word -> MFMA operands (c + u) for its two blocks.
// Slots 0..3 (block 2w) -> ea.x..ea.w, slots 4..7 (block 2w+1) -> eb.x..eb.w.
// Offsets c per register: block 2w: 128, 32, 8, 128; block 2w+1: 32, 8, 128, 32.
__device__ __forceinline__ void dq_q2(uint32_t W, const DqConsts& k, uint4& ea, uint4& eb) {
  uint32_t W6 = W >> 6, W12 = W >> 12;
  ea.x = and_or(W, k.m0, k.c0);
  ea.y = and_or(W, k.m1, k.c1);
  ea.z = and_or(W, k.m2, k.c2);
  ea.w = and_or(W6, k.m0, k.c0);
  eb.x = and_or(W6, k.m1, k.c1);
  eb.y = and_or(W6, k.m2, k.c2);
  eb.z = and_or(W12, k.m0, k.c0);
  eb.w = and_or(W12, k.m1, k.c1);
}

// Q3S: low word L and its high word H; `odd` = the low word's index in the
// pair served by H (high bit at p+1 for the even word, at p for the odd one).
__device__ __forceinline__ void dq_q3(uint32_t L, uint32_t H, bool odd, const DqConsts& k,
                                      uint4& ea, uint4& eb) {
  uint32_t L6 = L >> 6, L12 = L >> 12;
  uint32_t H0 = odd ? (H << 2) : (H << 1);
  uint32_t H6 = odd ? (H >> 4) : (H >> 5);
  uint32_t H12 = odd ? (H >> 10) : (H >> 11);
  ea.x = and_or(H0, k.h0, and_or(L, k.m0, k.c0));
  ea.y = and_or(H0, k.h1, and_or(L, k.m1, k.c1));
  ea.z = and_or(H0, k.h2, and_or(L, k.m2, k.c2));
  ea.w = and_or(H6, k.h0, and_or(L6, k.m0, k.c0));
  eb.x = and_or(H6, k.h1, and_or(L6, k.m1, k.c1));
  eb.y = and_or(H6, k.h2, and_or(L6, k.m2, k.c2));
  eb.z = and_or(H12, k.h0, and_or(L12, k.m0, k.c0));
  eb.w = and_or(H12, k.h1, and_or(L12, k.m1, k.c1));
}

// Offset c of register j of a block of parity `par` (see dq_q2).
__host__ __device__ __forceinline__ float dq_offset(int par, int j) {
  const int c = par == 0 ? ((j == 0 || j == 3) ? 128 : (j == 1 ? 32 : 8))
                         : ((j == 2) ? 128 : (j == 1 ? 8 : 32));
  return (float)c;
}

__device__ __forceinline__ float silu(float a) { return a / (1.0f + expf(-a)); }

// Wave-wide sum via DPP-free shuffles (64 lanes).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace moe
