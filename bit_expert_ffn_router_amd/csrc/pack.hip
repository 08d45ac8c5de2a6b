// Packer and unpacker of the expert weight layout (one-off, per load).
//
// The pages repack the downloaded weights once into a "pack" layout before
// serving ([JD] "5070ti16g单卡跑qwen 3.8 flash next …", section
// "为什么从 18t/s 变成 60-90t/s").  The layout here is this library's own and
// is specified in include/moe.h: 16-row x 256-column records whose code words
// are laid out for the 16x16x32 MFMA operand (lane L = 16*q + n holds row n,
// columns 8q..8q+7 of each 32-column block).
#include "kernels.hpp"

namespace moe {

// Which matrix/rows/octet a record index of one expert covers.
struct RecInfo {
  int mat;     // 0 gate, 1 up, 2 down
  int row0;    // first row of the record inside its matrix
  int o;       // octet along the reduction dimension
  int K;       // reduction length of the matrix
};

__device__ __forceinline__ RecInfo rec_info(int r, int D, int F) {
  RecInfo ri;
  const int oD = octets(D), oF = octets(F);
  const int n_gu = 2 * (F / 16) * oD;
  if (r < n_gu) {
    const int g = r / (2 * oD), rem = r % (2 * oD);
    ri.mat = rem / oD;
    ri.o = rem % oD;
    ri.row0 = 16 * g;
    ri.K = D;
  } else {
    const int rr = r - n_gu;
    ri.mat = 2;
    ri.row0 = 16 * (rr / oF);
    ri.o = rr % oF;
    ri.K = F;
  }
  return ri;
}

// grid: (records per expert, n experts); block: 64 threads (one record).
template <int FMT>
__global__ __launch_bounds__(64) void pack_kernel(int D, int F, const uint8_t* __restrict__ codes,
                                                  const uint16_t* __restrict__ scale,
                                                  const uint16_t* __restrict__ mins,
                                                  uint8_t* __restrict__ dst, size_t dst_stride) {
  const int r = blockIdx.x, ex = blockIdx.y, lane = threadIdx.x;
  const RecInfo ri = rec_info(r, D, F);
  const size_t mat_elems = (size_t)F * D;
  const uint8_t* cm = codes + ((size_t)ex * 3 + ri.mat) * mat_elems;
  const uint16_t* sm = scale + ((size_t)ex * 3 + ri.mat) * (mat_elems / 32);
  const uint16_t* mm = FMT == kQ2 ? mins + ((size_t)ex * 3 + ri.mat) * (mat_elems / 32) : nullptr;
  uint8_t* rec = dst + (size_t)ex * dst_stride + (size_t)r * rec_bytes(FMT);

  const int n = lane & 15, q = lane >> 4;
  const int row = ri.row0 + n;
  // The lane's 8 codes of each of the 8 blocks: columns 256o + 32b + 8q + 0..7.
  uint32_t cw[8][2];
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const int col = 256 * ri.o + 32 * b + 8 * q;
    if (col < ri.K) {
      const uint2 v = *reinterpret_cast<const uint2*>(cm + (size_t)row * ri.K + col);
      cw[b][0] = v.x;
      cw[b][1] = v.y;
    } else {
      cw[b][0] = cw[b][1] = (FMT == kQ3) ? 0xFCFCFCFCu : 0u;  // q = -4 -> u3 = 0
    }
  }
  uint32_t lo[4] = {0, 0, 0, 0}, hi[2] = {0, 0};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int b = 2 * w + s / 4, j = s % 4;
      // bytes 2j and 2j+1 of the block's 8-byte group
      const uint32_t word = cw[b][j >> 1];
      uint32_t c0 = (word >> (16 * (j & 1))) & 0xFFu;
      uint32_t c1 = (word >> (16 * (j & 1) + 8)) & 0xFFu;
      if (FMT == kQ3) {
        c0 = (c0 + 4u) & 7u;
        c1 = (c1 + 4u) & 7u;
        const int extra = (w % 2 == 0) ? 1 : 0;
        hi[w / 2] |= ((c0 >> 2) & 1u) << (2 * s + extra);
        hi[w / 2] |= ((c1 >> 2) & 1u) << (16 + 2 * s + extra);
      }
      lo[w] |= (c0 & 3u) << (2 * s);
      lo[w] |= (c1 & 3u) << (16 + 2 * s);
    }
  }
  *reinterpret_cast<uint4*>(rec + 16 * lane) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  if (FMT == kQ3) *reinterpret_cast<uint2*>(rec + 1024 + 8 * lane) = make_uint2(hi[0], hi[1]);

  // Block parameters: entry e = 8n' + b, two per lane.
  const int nblk = ri.K / 32;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int e = 2 * lane + t, np = e / 8, b = e % 8;
    const int blk = 8 * ri.o + b;
    const size_t pi = (size_t)(ri.row0 + np) * nblk + blk;
    const uint16_t s = blk < nblk ? sm[pi] : (uint16_t)0;
    if (FMT == kQ2) {
      const uint16_t m = blk < nblk ? mm[pi] : (uint16_t)0;
      *reinterpret_cast<uint32_t*>(rec + 1024 + 4 * e) = (uint32_t)s | ((uint32_t)m << 16);
    } else {
      *reinterpret_cast<uint16_t*>(rec + (FMT == kQ3 ? 1536 : 1024) + 2 * e) = s;
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(64) void unpack_kernel(int D, int F, const uint8_t* __restrict__ src,
                                                    size_t src_stride, uint8_t* __restrict__ codes,
                                                    uint16_t* __restrict__ scale,
                                                    uint16_t* __restrict__ mins) {
  const int r = blockIdx.x, ex = blockIdx.y, lane = threadIdx.x;
  const RecInfo ri = rec_info(r, D, F);
  const size_t mat_elems = (size_t)F * D;
  uint8_t* cm = codes + ((size_t)ex * 3 + ri.mat) * mat_elems;
  uint16_t* sm = scale + ((size_t)ex * 3 + ri.mat) * (mat_elems / 32);
  const uint8_t* rec = src + (size_t)ex * src_stride + (size_t)r * rec_bytes(FMT);
  const int n = lane & 15, q = lane >> 4;
  const int row = ri.row0 + n;
  const uint4 lo4 = *reinterpret_cast<const uint4*>(rec + 16 * lane);
  const uint32_t lo[4] = {lo4.x, lo4.y, lo4.z, lo4.w};
  uint2 hi2 = make_uint2(0, 0);
  if (FMT == kQ3) hi2 = *reinterpret_cast<const uint2*>(rec + 1024 + 8 * lane);
  const uint32_t hi[2] = {hi2.x, hi2.y};
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const int col = 256 * ri.o + 32 * b + 8 * q;
    if (col >= ri.K) continue;
    uint32_t out[2] = {0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int w = b / 2, s = 4 * (b % 2) + j;
      uint32_t c0 = (lo[w] >> (2 * s)) & 3u, c1 = (lo[w] >> (16 + 2 * s)) & 3u;
      if (FMT == kQ3) {
        const int extra = (w % 2 == 0) ? 1 : 0;
        c0 |= ((hi[w / 2] >> (2 * s + extra)) & 1u) << 2;
        c1 |= ((hi[w / 2] >> (16 + 2 * s + extra)) & 1u) << 2;
        c0 = (c0 - 4u) & 0xFFu;
        c1 = (c1 - 4u) & 0xFFu;
      }
      out[j >> 1] |= (c0 | (c1 << 8)) << (16 * (j & 1));
    }
    *reinterpret_cast<uint2*>(cm + (size_t)row * ri.K + col) = make_uint2(out[0], out[1]);
  }
  const int nblk = ri.K / 32;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int e = 2 * lane + t, np = e / 8, b = e % 8;
    const int blk = 8 * ri.o + b;
    if (blk >= nblk) continue;
    const size_t pi = (size_t)(ri.row0 + np) * nblk + blk;
    if (FMT == kQ2) {
      const uint32_t v = *reinterpret_cast<const uint32_t*>(rec + 1024 + 4 * e);
      sm[pi] = (uint16_t)(v & 0xFFFFu);
      if (mins) mins[((size_t)ex * 3 + ri.mat) * (mat_elems / 32) + pi] = (uint16_t)(v >> 16);
    } else {
      sm[pi] = *reinterpret_cast<const uint16_t*>(rec + (FMT == kQ3 ? 1536 : 1024) + 2 * e);
    }
  }
}

hipError_t launch_pack(int fmt, int D, int F, int n, const void* codes, const uint16_t* scale,
                       const uint16_t* mins, void* dst, size_t dst_stride, hipStream_t st) {
  const int nrec = 2 * (F / 16) * octets(D) + (D / 16) * octets(F);
  dim3 grid(nrec, n);
  if (fmt == kQ2)
    pack_kernel<kQ2><<<grid, 64, 0, st>>>(D, F, (const uint8_t*)codes, scale, mins,
                                          (uint8_t*)dst, dst_stride);
  else if (fmt == kQ3)
    pack_kernel<kQ3><<<grid, 64, 0, st>>>(D, F, (const uint8_t*)codes, scale, nullptr,
                                          (uint8_t*)dst, dst_stride);
  else
    pack_kernel<kQ2S><<<grid, 64, 0, st>>>(D, F, (const uint8_t*)codes, scale, nullptr,
                                           (uint8_t*)dst, dst_stride);
  return hipGetLastError();
}

hipError_t launch_unpack(int fmt, int D, int F, int n, const void* src, size_t src_stride,
                         void* codes, uint16_t* scale, uint16_t* mins, hipStream_t st) {
  const int nrec = 2 * (F / 16) * octets(D) + (D / 16) * octets(F);
  dim3 grid(nrec, n);
  if (fmt == kQ2)
    unpack_kernel<kQ2><<<grid, 64, 0, st>>>(D, F, (const uint8_t*)src, src_stride,
                                            (uint8_t*)codes, scale, mins);
  else if (fmt == kQ3)
    unpack_kernel<kQ3><<<grid, 64, 0, st>>>(D, F, (const uint8_t*)src, src_stride,
                                            (uint8_t*)codes, scale, nullptr);
  else
    unpack_kernel<kQ2S><<<grid, 64, 0, st>>>(D, F, (const uint8_t*)src, src_stride,
                                             (uint8_t*)codes, scale, nullptr);
  return hipGetLastError();
}

}  // namespace moe
