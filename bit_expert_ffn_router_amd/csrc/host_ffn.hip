// Host half of the slot-mode layer: the FFNs of the non-resident pairs,
// computed on the CPU from packed experts kept in host memory, and the GPU
// kernel that adds them into the partial output.
//
// The pages keep the hot experts on the GPU and let the CPU compute the
// experts that are not there, both sides working at the same time and their
// results added into the same layer ([AF] "个人开发者用 AI 十天写出 Strata
// 引擎…", section "命中率七成，代价是答案会变"; [SL] section "12GB 显存装
// 下 1250 亿参数").  Nothing here stands in for the GPU path: it runs only
// for the miss list a slot-mode layer returns.
//
// The packed record layout is the one include/moe.h specifies; this file
// reads it with its own host code.  Arithmetic: exact fp32 weights (an fp16
// scale times a small integer, plus an fp16 min), fp32 activations, fp32
// accumulation, fp32 h and output.
#include <immintrin.h>

#include <cstdlib>
#include <cstring>
#include <fstream>
#include <string>
#include <vector>

#include "kernels.hpp"

#include "host_pool.hpp"

namespace moe {
namespace {

float half_to_float(uint16_t h) {
  const uint32_t s = (uint32_t)(h >> 15) << 31, e = (h >> 10) & 31u, m = h & 1023u;
  uint32_t bits;
  if (e == 0) {
    if (m == 0) {
      bits = s;
    } else {  // subnormal: m * 2^-24, exact in fp32
      float v = (float)m * 5.9604644775390625e-08f;
      bits = s | (__builtin_bit_cast(uint32_t, v) & 0x7FFFFFFFu);
    }
  } else if (e == 31) {
    bits = s | 0x7F800000u | (m << 13);
  } else {
    bits = s | ((e + 112u) << 23) | (m << 13);
  }
  return __builtin_bit_cast(float, bits);
}
float bf16_bits_to_float(uint16_t v) { return __builtin_bit_cast(float, (uint32_t)v << 16); }
uint16_t float_to_bf16_bits(float f) {
  uint32_t b = __builtin_bit_cast(uint32_t, f);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

// The packed row layout, read without unpacking weight by weight: for row n
// of a record, block b and column quarter q, the eight columns
// 32 b + 8 q + 0..7 have their codes in one 32-bit word (lane 16 q + n, word
// b / 2): column 32 b + 8 q + 2 j in bits 8 (b % 2) + 2 j of the low half,
// column 32 b + 8 q + 2 j + 1 in the same bits of the high half.  So the
// byte (W >> 8 (b % 2)) holds the even columns' codes and (W >> (16 +
// 8 (b % 2))) the odd ones'; a 256-entry table turns a byte into its four
// codes.  Q3S's third bit sits in the high-plane word at bit 2 j + extra of
// the same bytes (mask 0x55 after the shift).
struct CodeTables {
  float code[256][4];  // (v >> 2 j) & 3
  float bit[256][4];   // (v >> 2 j) & 1
  CodeTables() {
    for (int v = 0; v < 256; ++v)
      for (int j = 0; j < 4; ++j) {
        code[v][j] = (float)((v >> (2 * j)) & 3);
        bit[v][j] = (float)((v >> (2 * j)) & 1);
      }
  }
};
const CodeTables& tables() {
  static const CodeTables t;
  return t;
}

// A vector of length K (a multiple of 256 after padding) in record order:
// per octet o, block b, quarter q: the 4 even then the 4 odd columns of
// 256 o + 32 b + 8 q; plus the sum of each 32-block.
struct RecVec {
  std::vector<float> v;    // [oK][8][4][8]
  std::vector<float> sum;  // [oK][8]
  void set(const float* x, int K) {
    const int oK = (K + 255) / 256;
    v.assign((size_t)oK * 256, 0.f);
    sum.assign((size_t)oK * 8, 0.f);
    for (int o = 0; o < oK; ++o)
      for (int b = 0; b < 8; ++b) {
        float bs = 0.f;
        for (int q = 0; q < 4; ++q) {
          const int c = 256 * o + 32 * b + 8 * q;
          float* d = &v[(size_t)o * 256 + 32 * b + 8 * q];
          for (int j = 0; j < 4; ++j) {
            d[j] = c + 2 * j < K ? x[c + 2 * j] : 0.f;
            d[4 + j] = c + 2 * j + 1 < K ? x[c + 2 * j + 1] : 0.f;
          }
          for (int j = 0; j < 8; ++j) bs += d[j];
        }
        sum[(size_t)o * 8 + b] = bs;
      }
  }
};

// Four floats as one SSE2 register (every x86-64 CPU has it); the sums stay
// vectors until the end of a block.
typedef float v4f __attribute__((vector_size(16)));
inline v4f ld4(const float* p) {
  v4f v;
  __builtin_memcpy(&v, p, sizeof v);
  return v;
}
inline float hsum(v4f v) { return (v[0] + v[1]) + (v[2] + v[3]); }

// Block scale and offset of row n, block b: w = sc * u + off.
inline void block_params(const uint8_t* rec, int fmt, int n, int b, float& sc, float& off) {
  if (fmt == kQ2) {
    const uint16_t* pp = reinterpret_cast<const uint16_t*>(rec + 1024 + 4 * (8 * n + b));
    sc = half_to_float(pp[0]);
    off = half_to_float(pp[1]);  // w = s u + m
  } else {
    const int base = fmt == kQ3 ? 1536 : 1024;
    sc = half_to_float(*reinterpret_cast<const uint16_t*>(rec + base + 2 * (8 * n + b)));
    off = -(fmt == kQ3 ? 4.f : 2.f) * sc;  // w = s (u - 4) or s (u - 2)
  }
}

// Row n of one record dotted with octet o of a record-order vector (any
// x86-64 CPU: SSE2 and code tables).
float record_row_dot_sse2(const uint8_t* rec, int fmt, int n, const float* xv, const float* xs) {
  const CodeTables& T = tables();
  const uint32_t* lo = reinterpret_cast<const uint32_t*>(rec);           // word (L, w): 4 L + w
  const uint32_t* hi = reinterpret_cast<const uint32_t*>(rec + 1024);    // Q3S: (L, h): 2 L + h
  float s = 0.f;
  for (int b = 0; b < 8; ++b) {
    const int wd = b / 2, sh = 8 * (b % 2);
    const int extra = (wd % 2 == 0) ? 1 : 0;
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < 4; ++q) {
      const int L = 16 * q + n;
      const uint32_t W = lo[4 * L + wd];
      const float* xe = xv + 32 * b + 8 * q;
      v4f ce = ld4(T.code[(W >> sh) & 255u]), co = ld4(T.code[(W >> (16 + sh)) & 255u]);
      if (fmt == kQ3) {  // u3 = u + 4 * (third bit)
        const uint32_t H = hi[2 * L + wd / 2];
        ce += 4.f * ld4(T.bit[(H >> (sh + extra)) & 0x55u]);
        co += 4.f * ld4(T.bit[(H >> (16 + sh + extra)) & 0x55u]);
      }
      acc += ce * ld4(xe) + co * ld4(xe + 4);
    }
    float sc, off;
    block_params(rec, fmt, n, b, sc, off);
    s += sc * hsum(acc) + off * xs[b];
  }
  return s;
}

// Four rows n0 .. n0 + 3 of one record dotted with octet o of a record-order
// vector, with AVX2 and FMA.  The eight codes of a (block, quarter) word come
// out of one broadcast word by per-lane shifts (even columns at bits 0, 2, 4,
// 6 of the block's byte, odd ones 16 bits higher), already in the record
// order of the vector; the four rows are independent FMA chains that share
// each vector load, and each block's sum is scaled into one accumulator per
// row, so a row ends in one horizontal sum.
typedef float v8f __attribute__((vector_size(32)));
typedef uint32_t v8u __attribute__((vector_size(32)));
__attribute__((target("avx2,fma"))) void record_rows4_avx2(const uint8_t* rec, int fmt, int n0,
                                                           const float* xv, const float* xs,
                                                           float* out) {
  const uint32_t* lo = reinterpret_cast<const uint32_t*>(rec);
  const uint32_t* hi = reinterpret_cast<const uint32_t*>(rec + 1024);
  const v8u lanes = {0, 2, 4, 6, 16, 18, 20, 22};
  const v8f zero = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  v8f tot[4] = {zero, zero, zero, zero};
  float offs[4] = {0.f, 0.f, 0.f, 0.f};
  for (int b = 0; b < 8; ++b) {
    const int wd = b / 2, sh = 8 * (b % 2);
    const int extra = (wd % 2 == 0) ? 1 : 0;
    const v8u shc = lanes + (uint32_t)sh, shb = lanes + (uint32_t)(sh + extra);
    v8f acc[4] = {zero, zero, zero, zero};
    for (int q = 0; q < 4; ++q) {
      v8f x;
      __builtin_memcpy(&x, xv + 32 * b + 8 * q, sizeof x);
      for (int r = 0; r < 4; ++r) {
        const int L = 16 * q + n0 + r;
        const uint32_t W = lo[4 * L + wd];
        v8u c = ((v8u){W, W, W, W, W, W, W, W} >> shc) & 3u;
        if (fmt == kQ3) {  // u3 = u + 4 * (third bit)
          const uint32_t H = hi[2 * L + wd / 2];
          c += (((v8u){H, H, H, H, H, H, H, H} >> shb) & 1u) << 2;
        }
        acc[r] = __builtin_convertvector(c, v8f) * x + acc[r];
      }
    }
    for (int r = 0; r < 4; ++r) {
      float sc, off;
      block_params(rec, fmt, n0 + r, b, sc, off);
      tot[r] = (v8f){sc, sc, sc, sc, sc, sc, sc, sc} * acc[r] + tot[r];
      offs[r] += off * xs[b];
    }
  }
  for (int r = 0; r < 4; ++r) {
    const v8f t = tot[r];
    out[r] = (((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]))) + offs[r];
  }
}

// All 16 rows of one record dotted with octet o of a record-order vector,
// with AVX-512F: the rows run across the 16 lanes.  For column quarter q the
// record holds rows 0..15 x code words 0..3 in 256 contiguous bytes (word
// (n, wd) at 4 n + wd); two two-source permutes gather word wd of all 16
// rows into one vector.  Each of the word's 16 columns is then one shift, a
// mask, a conversion and a multiply-add with the column's activation
// broadcast to every row.  A block's sums stay separate per row and are
// scaled once, as 16-row vectors, when the record is done.
__attribute__((target("avx512f,f16c"))) void record_rows16_avx512(const uint8_t* rec, int fmt,
                                                                  const float* xv, const float* xs,
                                                                  float* out) {
  const __m512i m3 = _mm512_set1_epi32(3), m4 = _mm512_set1_epi32(4);
  const __m512i rows4 = _mm512_setr_epi32(0, 4, 8, 12, 16, 20, 24, 28, 0, 4, 8, 12, 16, 20, 24, 28);
  const __m512i rows2 = _mm512_setr_epi32(0, 2, 4, 6, 8, 10, 12, 14, 16, 18, 20, 22, 24, 26, 28, 30);
  __m512 acc[8];
  for (int b = 0; b < 8; ++b) acc[b] = _mm512_setzero_ps();
  for (int q = 0; q < 4; ++q) {
    const uint8_t* slab = rec + 256 * q;
    const __m512i A0 = _mm512_loadu_si512(slab), A1 = _mm512_loadu_si512(slab + 64);
    const __m512i A2 = _mm512_loadu_si512(slab + 128), A3 = _mm512_loadu_si512(slab + 192);
    __m512i H0 = _mm512_setzero_si512(), H1 = _mm512_setzero_si512();
    if (fmt == kQ3) {  // high-plane words (n, h) at 2 n + h: rows 0..7, then 8..15
      H0 = _mm512_loadu_si512(rec + 1024 + 128 * q);
      H1 = _mm512_loadu_si512(rec + 1024 + 128 * q + 64);
    }
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      const __m512i idx = _mm512_add_epi32(rows4, _mm512_set1_epi32(wd));
      const __m512i V = _mm512_mask_blend_epi32((__mmask16)0xFF00, _mm512_permutex2var_epi32(A0, idx, A1),
                                                _mm512_permutex2var_epi32(A2, idx, A3));
      __m512i HW = _mm512_setzero_si512();
      if (fmt == kQ3)
        HW = _mm512_permutex2var_epi32(H0, _mm512_add_epi32(rows2, _mm512_set1_epi32(wd / 2)), H1);
      const int extra = (wd % 2 == 0) ? 1 : 0;  // the third bit sits one higher for even words
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int b = 2 * wd + kk;
        __m512 a = acc[b];
#pragma unroll
        for (int par = 0; par < 2; ++par)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int pos = 8 * kk + 16 * par + 2 * j;  // bits of column 32 b + 8 q + 2 j + par
            __m512i c = _mm512_and_si512(_mm512_srli_epi32(V, pos), m3);
            if (fmt == kQ3) {  // u3 = u + 4 * (third bit)
              const int hp = pos + extra;
              const __m512i hb = hp >= 2 ? _mm512_srli_epi32(HW, hp - 2) : _mm512_slli_epi32(HW, 2 - hp);
              c = _mm512_or_si512(c, _mm512_and_si512(hb, m4));
            }
            a = _mm512_fmadd_ps(_mm512_cvtepi32_ps(c),
                                _mm512_set1_ps(xv[32 * b + 8 * q + 4 * par + j]), a);
          }
        acc[b] = a;
      }
    }
  }
  // Block parameters of the 16 rows (fp16 -> fp32 16 at a time), then the
  // scaled block sums: out[n] = sum over b of s[n][b] acc[b][n] + off[n][b] X[b].
  alignas(64) float S[16 * 8], M[16 * 8];
  if (fmt == kQ2) {  // (scale, min) pairs, row-major [n][b][2]
    alignas(64) float P[16 * 16];
    for (int i = 0; i < 16; ++i)
      _mm512_store_ps(P + 16 * i, _mm512_cvtph_ps(_mm256_loadu_si256(
                                      reinterpret_cast<const __m256i*>(rec + 1024 + 32 * i))));
    for (int i = 0; i < 128; ++i) {
      S[i] = P[2 * i];
      M[i] = P[2 * i + 1];
    }
  } else {  // scales [n][b]
    const int base = fmt == kQ3 ? 1536 : 1024;
    for (int i = 0; i < 8; ++i)
      _mm512_store_ps(S + 16 * i, _mm512_cvtph_ps(_mm256_loadu_si256(
                                      reinterpret_cast<const __m256i*>(rec + base + 32 * i))));
    const float k = fmt == kQ3 ? -4.f : -2.f;  // w = s (u - 4) or s (u - 2)
    for (int i = 0; i < 128; ++i) M[i] = k * S[i];
  }
  const __m512i col8 = _mm512_setr_epi32(0, 8, 16, 24, 32, 40, 48, 56, 64, 72, 80, 88, 96, 104, 112, 120);
  __m512 o = _mm512_setzero_ps();
  for (int b = 0; b < 8; ++b) {
    const __m512i ib = _mm512_add_epi32(col8, _mm512_set1_epi32(b));
    o = _mm512_fmadd_ps(_mm512_i32gather_ps(ib, S, 4), acc[b], o);
    o = _mm512_fmadd_ps(_mm512_i32gather_ps(ib, M, 4), _mm512_set1_ps(xs[b]), o);
  }
  _mm512_storeu_ps(out, o);
}

// All 16 rows of a record with the AVX2 + FMA or the SSE2 four-row kernels.
void record_rows4_sse2(const uint8_t* rec, int fmt, int n0, const float* xv, const float* xs,
                       float* out) {
  for (int r = 0; r < 4; ++r) out[r] = record_row_dot_sse2(rec, fmt, n0 + r, xv, xs);
}
void record_rows16_sse2(const uint8_t* rec, int fmt, const float* xv, const float* xs, float* out) {
  for (int n0 = 0; n0 < 16; n0 += 4) record_rows4_sse2(rec, fmt, n0, xv, xs, out + n0);
}
__attribute__((target("avx2,fma"))) void record_rows16_avx2(const uint8_t* rec, int fmt,
                                                            const float* xv, const float* xs,
                                                            float* out) {
  for (int n0 = 0; n0 < 16; n0 += 4) record_rows4_avx2(rec, fmt, n0, xv, xs, out + n0);
}

// The record dot products this process uses: AVX-512F (with F16C), else
// AVX2 + FMA, where the CPU has them, else SSE2.  MOE_HOST_SIMD=avx2 or
// =sse2 in the environment caps the choice (read at every host layer call).
// They differ only in fp32 rounding order.
typedef void (*Rows16)(const uint8_t*, int, const float*, const float*, float*);
// The CPU's features come from the flags line of /proc/cpuinfo, which lists
// only what the kernel has enabled (AVX state included).
struct CpuSimd {
  bool avx2_fma = false, avx512f = false;
};
CpuSimd cpu_simd() {
  CpuSimd c;
  std::ifstream f("/proc/cpuinfo");
  std::string line;
  while (std::getline(f, line)) {
    if (line.compare(0, 5, "flags") != 0) continue;
    const std::string l = " " + line + " ";
    c.avx2_fma = l.find(" avx2 ") != std::string::npos && l.find(" fma ") != std::string::npos;
    c.avx512f = l.find(" avx512f ") != std::string::npos && l.find(" f16c ") != std::string::npos;
    break;
  }
  return c;
}
Rows16 rows16_impl() {
  static const CpuSimd cpu = cpu_simd();
  const char* e = getenv("MOE_HOST_SIMD");
  const bool cap_sse2 = e && strcmp(e, "sse2") == 0, cap_avx2 = e && strcmp(e, "avx2") == 0;
  if (cap_sse2) return record_rows16_sse2;
  if (cpu.avx512f && !cap_avx2) return record_rows16_avx512;
  return cpu.avx2_fma ? record_rows16_avx2 : record_rows16_sse2;
}
// Which implementation rows16_impl picks (for the callers' reports).
const char* row_dot_name() {
  const Rows16 d = rows16_impl();
  return d == record_rows16_avx512 ? "avx512" : (d == record_rows16_avx2 ? "avx2" : "sse2");
}

}  // namespace

hipError_t launch_add_rows(void* out, int out_bf16, const float* y, size_t n, hipStream_t st);

const char* host_simd_name() { return row_dot_name(); }

}  // namespace moe

namespace {

__global__ void add_rows_kernel(void* out, int out_bf16, const float* __restrict__ y, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  if (out_bf16) {
    uint16_t* o = reinterpret_cast<uint16_t*>(out);
    o[i] = moe::f32_to_bf16(moe::bf16_to_f32(o[i]) + y[i]);
  } else {
    reinterpret_cast<float*>(out)[i] += y[i];
  }
}

}  // namespace

namespace moe {

hipError_t launch_add_rows(void* out, int out_bf16, const float* y, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  add_rows_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(out, out_bf16, y, n);
  return hipGetLastError();
}

// y[t] = sum over the misses of token t, in list order, of gate * FFN_e(xhat_t).
void host_miss_ffn(int D, int F, int fmt, int T, const float* xhat, const MissRec* miss, int nm,
                   const uint8_t* const* experts, float* y, moe_host_pool* pool) {
  const int ng = F / 16, oD = D / 256, oF = (F + 255) / 256, rb = rec_bytes(fmt);
  const Rows16 dot = rows16_impl();
  std::vector<RecVec> xr(T);
  for (int t = 0; t < T; ++t) xr[t].set(xhat + (size_t)t * D, D);
  std::vector<float> h((size_t)nm * F, 0.f);
  // Phase 1: h rows, one item per (miss, 16-row group).
  auto gateup = [&](int it) {
    const int m = it / ng, g = it % ng;
    const uint8_t* ex = experts[miss[m].expert];
    const RecVec& x = xr[miss[m].token];
    const uint8_t* gate = ex + (size_t)(2 * g) * oD * rb;
    const uint8_t* up = ex + (size_t)(2 * g + 1) * oD * rb;
    float a[16] = {}, b[16] = {}, p[16];
    for (int o = 0; o < oD; ++o) {
      dot(gate + (size_t)o * rb, fmt, &x.v[(size_t)o * 256], &x.sum[(size_t)o * 8], p);
      for (int r = 0; r < 16; ++r) a[r] += p[r];
      dot(up + (size_t)o * rb, fmt, &x.v[(size_t)o * 256], &x.sum[(size_t)o * 8], p);
      for (int r = 0; r < 16; ++r) b[r] += p[r];
    }
    for (int r = 0; r < 16; ++r)
      h[(size_t)m * F + 16 * g + r] = a[r] / (1.0f + expf(-a[r])) * b[r];
  };
  if (pool) pool->run(nm * ng, gateup);
  else for (int i = 0; i < nm * ng; ++i) gateup(i);
  std::vector<RecVec> hr(nm);
  for (int m = 0; m < nm; ++m) hr[m].set(&h[(size_t)m * F], F);
  // Phase 2: output rows, one item per kDownGroups 16-row groups of d_model
  // (items of a few microseconds, so that claiming them stays cheap); each
  // y[t][d] sums its token's misses in list order.
  for (size_t i = 0; i < (size_t)T * D; ++i) y[i] = 0.f;
  constexpr int kDownGroups = 4;
  const int nrg = D / 16, nitems = (nrg + kDownGroups - 1) / kDownGroups;
  auto down = [&](int it) {
    for (int rg = it * kDownGroups; rg < nrg && rg < (it + 1) * kDownGroups; ++rg)
      for (int m = 0; m < nm; ++m) {
        const uint8_t* grp =
            experts[miss[m].expert] + down_offset(D, F, fmt) + (size_t)rg * oF * rb;
        float s[16] = {}, p[16];
        for (int o = 0; o < oF; ++o) {
          dot(grp + (size_t)o * rb, fmt, &hr[m].v[(size_t)o * 256], &hr[m].sum[(size_t)o * 8], p);
          for (int r = 0; r < 16; ++r) s[r] += p[r];
        }
        float* yt = y + (size_t)miss[m].token * D + 16 * rg;
        for (int r = 0; r < 16; ++r) yt[r] += miss[m].gate * s[r];
      }
  };
  if (pool) pool->run(nitems, down);
  else for (int i = 0; i < nitems; ++i) down(i);
}

void host_prepare_x(int T, int D, const void* x, bool x_bf16, bool rms, float* out) {
  for (int t = 0; t < T; ++t) {
    const size_t base = (size_t)t * D;
    auto val = [&](int i) {
      return x_bf16 ? bf16_bits_to_float(((const uint16_t*)x)[base + i]) : ((const float*)x)[base + i];
    };
    float r = 1.f;
    if (rms) {
      double ss = 0.0;  // the host's own mean square; the GPU sums in another order
      for (int i = 0; i < D; ++i) ss += (double)val(i) * val(i);
      r = 1.0f / sqrtf((float)(ss / D) + 1e-6f);
    }
    for (int i = 0; i < D; ++i)
      out[base + i] = rms ? bf16_bits_to_float(float_to_bf16_bits(val(i) * r)) : val(i);
  }
}

}  // namespace moe

moe_host_pool* moe_host_pool_new(int n_threads) {
  moe_host_pool* p = new moe_host_pool;
  for (int i = 0; i + 1 < n_threads; ++i) p->threads.emplace_back([p] { p->worker(); });
  return p;
}

void moe_host_pool_delete(moe_host_pool* p) {
  {
    std::lock_guard<std::mutex> lk(p->mu);
    p->stop = true;
  }
  p->cv.notify_all();  // polling workers see stop once they go to sleep
  for (auto& t : p->threads) t.join();
  delete p;
}
