// Device side of the seeded input generator (see synth/__init__.py for the
// recipe).  Produces logical expert weights -- one code byte per weight plus
// fp16 block scales (and mins) -- bit-identical to the numpy host generator,
// so that large stacks of layers can be generated in HBM without crossing the
// host link.  Holds none of the MoE layer's arithmetic.
//
// SplitMix64: G. Steele, D. Lea, C. Flood, "Fast splittable pseudorandom
// number generators" (OOPSLA 2014): output i of the stream at `key` is
// mix64(key + (i + 1) * GAMMA).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t stream_key(uint64_t seed, int layer, int expert, int mat,
                                               int field) {
  uint64_t k = seed;
  k = mix64(k + kGamma * (uint64_t)(layer + 1));
  k = mix64(k + kGamma * (uint64_t)(expert + 1));
  k = mix64(k + kGamma * (uint64_t)(mat + 1));
  k = mix64(k + kGamma * (uint64_t)(field + 1));
  return k;
}

__device__ __forceinline__ uint64_t draw(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1ull) * kGamma);
}

// One thread per 32-weight block.  Blocks of one expert: [3 mats][F*D/32].
__global__ void fill_kernel(uint64_t seed, int layer, int expert0, int n, int nblk, int fmt,
                            const uint16_t* __restrict__ ts, const uint16_t* __restrict__ tm,
                            uint8_t* __restrict__ codes, uint16_t* __restrict__ scale,
                            uint16_t* __restrict__ mins) {
  const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t per_expert = (size_t)3 * nblk;
  if (gid >= per_expert * n) return;
  const int ex = (int)(gid / per_expert);
  const size_t r = gid % per_expert;
  const int mat = (int)(r / nblk);
  const uint64_t blk = r % nblk;
  const int expert = expert0 + ex;
  const uint64_t w = draw(stream_key(seed, layer, expert, mat, 0), blk);
  const uint64_t sm = draw(stream_key(seed, layer, expert, mat, 1), blk);
  uint64_t h = 0;
  if (fmt == 2) h = draw(stream_key(seed, layer, expert, mat, 2), blk);
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t v = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int kk = 4 * i + b;
      uint32_t c = (uint32_t)(w >> (2 * kk)) & 3u;
      if (fmt == 2) c = (c + 4u * ((uint32_t)(h >> kk) & 1u) - 4u) & 0xFFu;  // q as a byte
      v |= c << (8 * b);
    }
    out[i] = v;
  }
  uint4* dst = reinterpret_cast<uint4*>(codes + gid * 32);
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  scale[gid] = ts[sm & 0xFFFFull];
  if (fmt == 1) mins[gid] = tm[(sm >> 16) & 0xFFFFull];
}

}  // namespace

extern "C" int synth_fill_expert_weights(uint64_t seed, int layer, int expert0, int n, int d_model,
                                         int d_ff, int fmt, const uint16_t* tab_scale,
                                         const uint16_t* tab_min, void* codes, uint16_t* scale,
                                         uint16_t* mins, hipStream_t stream) {
  if (n <= 0) return 0;
  if (d_model % 32 || d_ff % 32 || fmt < 1 || fmt > 3 || !codes || !scale || !tab_scale ||
      (fmt == 1 && (!mins || !tab_min)))
    return -1;
  const int nblk = d_ff * d_model / 32;
  const size_t total = (size_t)3 * nblk * n;
  const unsigned grid = (unsigned)((total + 255) / 256);
  fill_kernel<<<grid, 256, 0, stream>>>(seed, layer, expert0, n, nblk, fmt, tab_scale, tab_min,
                                        (uint8_t*)codes, scale, mins);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
