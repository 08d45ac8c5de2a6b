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
// bf16 MFMA (16x16x32) with fp32 accumulation.  A block of 8 waves computes
// 128 rows of one row tile x 512 weight rows; wave w owns weight rows
// 64w .. 64w+63 (four 16-row column tiles) over all 128 rows, so the
// activation tile in LDS serves 512 weight rows.  Operands reach LDS by
// direct global-to-LDS loads of 16 bytes per lane: the 128 gathered
// activation rows (through the permutation) in a ring of four stages of two
// 32-column k-steps, issued three stages ahead; and each wave's own column
// tiles, a whole 256-column octet of packed code words and (scale, min)
// pairs at a time, double-buffered and issued one octet ahead.  Each wave
// dequantises its tiles in registers -- per (row, block) a 4-entry bf16
// table s*u + m, built once per octet into LDS, and v_perm byte selects, two
// weights per select -- straight into MFMA B fragments, so every weight is
// dequantised once per block.  Tiles of at most 64 rows skip the MFMAs of
// their empty row groups.
#include <type_traits>

#include "route_common.hpp"

namespace moe {

namespace {

constexpr int kBM = 128;             // rows (permuted pairs) per tile
constexpr int kBN = 512;             // weight rows per block: 32 MFMA column tiles
constexpr int kPfWaves = 8;          // wave w: column tiles 4w .. 4w+3, all rows
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kRG = kBM / 16;        // row groups per tile

__host__ __device__ inline size_t al256(size_t v) { return (v + 255) / 256 * 256; }

struct PfWs {
  int32_t* idx;       // [T*k]
  float* gate;        // [T*k]
  int32_t* grp;       // [T*k] permutation group of each pair: its expert, or E
                      // for a pair whose expert is not resident (slot table)
  int32_t* offsets;   // [E+2] group offsets (group E: the misses)
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
  w.grp = (int32_t*)take(4 * P);
  w.offsets = (int32_t*)take(4 * ((size_t)E + 2));
  w.sorted = (int32_t*)take(4 * P);
  w.inv = (int32_t*)take(4 * P);
  void* pw = take(perm_ws_bytes(T, k, E + 1));
  w.perm = perm_ws_carve(pw, T, k, E + 1);
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
  size_t b = al256(4 * P) * 5 + al256(4 * ((size_t)E + 2)) + al256(perm_ws_bytes(T, k, E + 1)) +
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
// Slot table: the permutation group of every pair (its expert when resident,
// else the extra group E, which gets no tiles), and the usage counts: every
// routed pair adds 1 to its expert, hit or miss (counted in LDS per block,
// then one atomic add per expert and block; sums of integers, so the result
// does not depend on their order).
__global__ __launch_bounds__(256) void pf_slot_split_kernel(const int32_t* __restrict__ idx, int P,
                                                            int E, const int32_t* __restrict__ slot_of,
                                                            int n_slots, int32_t* __restrict__ grp,
                                                            uint32_t* __restrict__ use_count) {
  extern __shared__ uint32_t s_use[];
  const int tid = threadIdx.x;
  if (use_count) {
    for (int e = tid; e < E; e += 256) s_use[e] = 0;
    __syncthreads();
  }
  const int p0 = blockIdx.x * 4096;
  for (int p = p0 + tid; p < P && p < p0 + 4096; p += 256) {
    const int e = idx[p];
    const int sl = slot_of[e];  // a slot outside 0..n_slots-1 counts as not resident
    grp[p] = sl >= 0 && sl < n_slots ? e : E;
    if (use_count) atomicAdd(&s_use[e], 1u);
  }
  if (use_count) {
    __syncthreads();
    for (int e = tid; e < E; e += 256)
      if (s_use[e]) atomicAdd(&use_count[e], s_use[e]);
  }
}

// The miss list: group E of the stable permutation holds the non-resident
// pairs in increasing pair index p = t*k + j, which is (token, rank) order.
__global__ __launch_bounds__(256) void pf_miss_kernel(const int32_t* __restrict__ offsets, int E,
                                                      int k, const int32_t* __restrict__ sorted,
                                                      const int32_t* __restrict__ idx,
                                                      const float* __restrict__ gate,
                                                      MissRec* __restrict__ miss,
                                                      int32_t* __restrict__ miss_count) {
  const int m0 = offsets[E], n = offsets[E + 1] - m0;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i == 0) *miss_count = n;
  if (i < n) {
    const int p = sorted[m0 + i];
    MissRec r;
    r.token = p / k;
    r.rank = p % k;
    r.expert = idx[p];
    r.gate = gate[p];
    miss[i] = r;
  }
}

// ----------------------------------------------------------------------------
// Q2SM dequantisation into MFMA B fragments.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};  // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}
// The four values s*u + m (u = 0..3) of one block as bf16, in two words:
// bytes 0..3 (u = 0, 1) and 4..7 (u = 2, 3) of the byte-select source.
__device__ __forceinline__ void q2_table(uint32_t sm, uint32_t& lo, uint32_t& hi) {
  const float s = f16_to_f32((uint16_t)(sm & 0xFFFFu));
  const float m = f16_to_f32((uint16_t)(sm >> 16));
  lo = cvt_pk_bf16(m, s + m);
  hi = cvt_pk_bf16(fmaf(2.f, s, m), fmaf(3.f, s, m));
}
// Q2S: the four values s*(u - 2) of a block whose fp16 scale is half `hf` of
// word `sw`.
__device__ __forceinline__ void q2s_table(uint32_t sw, int hf, uint32_t& lo, uint32_t& hi) {
  const float s = f16_to_f32((uint16_t)(hf ? (sw >> 16) : (sw & 0xFFFFu)));
  lo = cvt_pk_bf16(-2.f * s, -s);
  hi = cvt_pk_bf16(0.f, s);
}
// Eight consecutive weights (k = 8q .. 8q+7 of one block) of one weight row:
// code word W of lane (q, n), block half sh / 8; slot j of the half holds the
// codes of columns 2j (bits sh+2j) and 2j+1 (bits 16+sh+2j).
__device__ __forceinline__ uint4 q2_frag(uint32_t W, int sh, uint32_t lo, uint32_t hi) {
  uint32_t v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t t = (W >> (sh + 2 * j)) & 0x00030003u;  // u0 | u1 << 16
    const uint32_t sel = t * 0x202u + 0x01000100u;          // bytes 2u0, 2u0+1, 2u1, 2u1+1
    v[j] = __builtin_amdgcn_perm(hi, lo, sel);
  }
  return make_uint4(v[0], v[1], v[2], v[3]);
}
// Q3S: the eight weights s*(u3 - 4) of block half KK of low-plane word W of
// record word WD, whose high bits are in high-plane word H (for an even WD
// the high bit of the code at bit p sits at bit p + 1 of H, for an odd one
// at bit p).  s*u3 - 4s is exact in fp32 (an fp16 scale times an integer of
// three bits), so each weight is rounded once, to bf16.  A 4-entry byte
// select cannot index eight codes, and tables of both halves would not fit
// the LDS; the codes go through the float converter instead.
template <int WD, int KK>
__device__ __forceinline__ uint4 q3_frag(uint32_t W, uint32_t H, float s) {
  const float m4 = -4.f * s;
  uint32_t v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int p = 8 * KK + 2 * j;
    const int hs = (WD & 1) ? p - 2 : p - 1;  // moves the high bit to bit 2 (and 18)
    const uint32_t hh = hs >= 0 ? (H >> hs) : (H << -hs);
    const uint32_t u = (hh & 0x00040004u) | ((W >> p) & 0x00030003u);  // u3 of columns 2j, 2j+1
    v[j] = cvt_pk_bf16(fmaf(s, (float)(u & 0xFFu), m4), fmaf(s, (float)((u >> 16) & 0xFFu), m4));
  }
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// ----------------------------------------------------------------------------
// Pipeline plumbing.
typedef __attribute__((address_space(3))) void lds_void_t;

// Direct global -> LDS load: lane l's 16 bytes land at lds + 16 l; `lds` is
// the same for the whole wave.  Counts in vmcnt.
__device__ __forceinline__ void dma16(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)lds, 16, 0, 0);
}
// One 16-byte LDS read as a single native-vector load (a uint4 copy is done
// member by member, and the merged read can lose the LDS variable's alias
// scope; without it the compiler drains every direct load in flight first).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 lds128(const uint4* p) {
  const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// Wait until at most N vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt not waited).
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Workgroup barrier without the release/acquire fences of __syncthreads (which
// would also drain the loads in flight for later stages); the ordering it needs
// comes from wait_vm before it and from the compiler barriers around it.
__device__ __forceinline__ void block_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

struct PfArgs {
  int T, D, F, Fs, E, k;
  const uint8_t* routed;
  size_t stride;
  const int32_t* slot_of;  // slot table or null
  const uint8_t* shared;
  const uint16_t* x;      // bf16 [T][D]
  PfWs w;
  void* out;
  int out_bf16;
};

// LDS of the grouped GEMM: 4 x 16 KB activation stages + 2 x 48 KB weight
// octets = 160 KB, the whole LDS of a CU (one block per CU).  A Q3S octet
// would need 7 KB per wave (low plane, high plane, scales) against the 6 KB
// here, so its high plane goes to registers instead (8 bytes per lane per
// tile).
struct PfA {
  uint4 a[2][kRG * 4 * 16];  // [k-step][row group][quarter q][row m]: A fragments
};
struct PfB {
  uint4 code[kPfWaves][4][64];  // [wave][tile][lane]: the lane's 4 code words of the octet
  uint4 sm[kPfWaves][2][64];    // [wave][tile pair][...]: (scale, min) of rows x 8 blocks
};
// vector-memory operations per wave: activations per stage, weights per
// octet (Q3S adds one 8-byte register load of the high plane per tile)
constexpr int kPfDmaA = 2;
__host__ __device__ constexpr int pf_dma_b(int fmt) { return fmt == kQ3 ? 10 : 6; }

// Grouped GEMM tile: rows row0 .. row0 + rows - 1 of the work list, weight
// rows nb * kBN .. of the expert's matrix.  MODE 0: gate/up (A = gathered
// activations, K = D, B = the expert's gate/up rows, SwiGLU epilogue into H).
// MODE 1: down (A = H rows, K = F, B = W_down rows, epilogue into Y).  FMT:
// Q2SM or Q2S weights (the same code words; Q2S records carry scales only)
// or Q3S (low plane as those code words, then the high plane, then scales).
// NG: row groups of 16 that get MFMAs (rows <= 16 NG); the loads and the
// dequantisation are the same for every NG.
template <int MODE, int FMT, int NG>
__device__ __forceinline__ void pf_tile(const PfArgs& a, PfA& sa0, PfA& sa1, PfA& sa2, PfA& sa3,
                                        PfB& sb0, PfB& sb1, int e, int row0, int rows, int nb) {
  constexpr int kRec = rec_bytes(FMT);
  constexpr int kPfDmaB = pf_dma_b(FMT);
  // VALU instructions placed after each MFMA in the schedule (Q3S builds its
  // fragments with about 9 instructions per register instead of 4)
  constexpr int NV = (FMT == kQ3 ? 40 : 12) / NG;
  // wave index as a uniform (scalar) value: the weight addresses stay in SGPRs
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int P = a.T * a.k;
  const bool sh = e < 0;
  const int F = sh ? a.Fs : a.F;
  const uint8_t* base =
      sh ? a.shared : a.routed + (size_t)(a.slot_of ? a.slot_of[e] : e) * a.stride;
  const int K = MODE == 0 ? a.D : F;
  const int nkb = K / 32, nst = (nkb + 1) / 2;
  const int oK = octets(K);
  const int NW = MODE == 0 ? 2 * F : a.D;  // weight rows of this GEMM

  // A: this lane's 16-byte piece (row 16 wv + lane % 16, quarter lane / 16) of
  // the wave's row group; rows past the tile read row 0 (masked later).
  const uint16_t* arow;
  {
    const int r = 16 * wv + (lane & 15);
    const int pos = row0 + (r < rows ? r : 0);
    if (MODE == 0) {
      const int tok = pos < P ? a.w.sorted[pos] / a.k : pos - P;
      arow = a.x + (size_t)tok * a.D + 8 * (lane >> 4);
    } else {
      arow = a.w.H + (size_t)pos * a.w.Fmax + 8 * (lane >> 4);
    }
  }
  // B: record row of each of the wave's column tiles (uniform).  Tiles past
  // the matrix read the pair's first tile or tile 0 (masked in the epilogue).
  const uint8_t* trec[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int w0 = nb * kBN + (4 * wv + j) * 16;
    if (w0 >= NW) w0 = (j & 1) ? nb * kBN + (4 * wv + j - 1) * 16 : 0;
    if (w0 >= NW) w0 = 0;
    trec[j] = base + (MODE == 0 ? 0 : down_offset(a.D, F, FMT)) + (size_t)(w0 / 16) * oK * kRec;
  }
  // (scale, min) pieces: lanes 0..31 / 32..63 take tile 2i / 2i+1 of pair i,
  // 16 bytes each: row lane % 16, blocks 4 h .. 4 h + 3 with h = (lane / 16) % 2
  // (in LDS: [tile of pair][h][row], so a k-step's reads conflict at most 2-way).
  // Q2S and Q3S: the 16 bytes of row lane % 16 hold all 8 scales; both h
  // take them.
  const uint8_t* smp[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const ptrdiff_t d = trec[2 * i + 1] - trec[2 * i];  // uniform; no indexed pointer array
    smp[i] = trec[2 * i] + (lane >= 32 ? d : 0) + (FMT == kQ3 ? 1536 : 1024) +
             (FMT == kQ2 ? 32 * (lane & 15) + 16 * ((lane >> 4) & 1) : 16 * (lane & 15));
  }
  const int n = lane & 15, q = lane >> 4;

  // Loads of activation stage s and weight octet o (past the end: reload
  // stage / octet 0, so every step issues the same loads).
  auto issue_a = [&](PfA& A, int s0) __attribute__((always_inline)) {
    const int s = s0 < nst ? s0 : 0;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int kb = 2 * s + kk;
      dma16(arow + (kb < nkb ? 32 * kb : 0), &A.a[kk][wv * 64]);
    }
  };
  // Q3S high-plane words of the octets in sb0 / sb1: this lane's two words
  // of each tile (they sit lane-major after the low plane)
  uint2 hw0[4], hw1[4];
  auto issue_b = [&](PfB& B, uint2 (&hw)[4], int o0) __attribute__((always_inline)) {
    const size_t ro = (size_t)(o0 < oK ? o0 : 0) * kRec;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dma16(reinterpret_cast<const uint4*>(trec[j] + ro) + lane, &B.code[wv][j][0]);
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(smp[i] + ro, &B.sm[wv][i][0]);
    if constexpr (FMT == kQ3) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        hw[j] = *reinterpret_cast<const uint2*>(trec[j] + ro + 1024 + 8 * lane);
    }
  };

  f32x4_t acc[NG][4];
#pragma unroll
  for (int i = 0; i < NG; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Software pipeline of the dequantisation: while the MFMAs of one k-step
  // run, the B fragments of the next k-step are built (VALU work that the
  // MFMAs hide).  cwo holds the octet's code words (one 16-byte LDS read per
  // tile per octet); bfa / bfb the fragments of k-steps 2s and 2s+1.
  uint4 cwo[4], bfa[4], bfb[4];
  auto load_codes = [&](const PfB& B) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 4; ++j) cwo[j] = lds128(&B.code[wv][j][lane]);
  };
  // The 4-entry bf16 tables of the octet, once per (tile, row, block) rather
  // than once per lane that uses them: lane l builds the 8 tables of tile
  // l / 16, row l % 16 into the wave's code region, which load_codes has
  // just read out (the wave's LDS operations run in order).  Layout
  // [tile][block][row] x (lo, hi) words, 4 KB per wave: the 16 rows a
  // k-step reads are 128 contiguous bytes.  Blocks of octet o past the
  // reduction length get all-zero tables, so their k-steps (an odd last one,
  // the clamped loads past the end) add exact zeros without a mask.
  auto build_tables = [&](PfB& B, int o) __attribute__((always_inline)) {
    const int jt = lane >> 4, nt = lane & 15;
    const uint32_t* smw = reinterpret_cast<const uint32_t*>(&B.sm[wv][0][0]) + (jt >> 1) * 256;
    uint32_t lo[8], hi[8];
    if constexpr (FMT == kQ2) {
      const u32x4_t a0 = *reinterpret_cast<const u32x4_t*>(smw + ((jt & 1) * 32 + nt) * 4);
      const u32x4_t a1 = *reinterpret_cast<const u32x4_t*>(smw + ((jt & 1) * 32 + 16 + nt) * 4);
      const uint32_t wsm[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
      for (int b = 0; b < 8; ++b) q2_table(wsm[b], lo[b], hi[b]);
    } else {
      const u32x4_t a0 = *reinterpret_cast<const u32x4_t*>(smw + ((jt & 1) * 32 + nt) * 4);
      const uint32_t wsc[4] = {a0.x, a0.y, a0.z, a0.w};
#pragma unroll
      for (int b = 0; b < 8; ++b) q2s_table(wsc[b >> 1], b & 1, lo[b], hi[b]);
    }
    uint2* tb = reinterpret_cast<uint2*>(&B.code[wv][0][0]) + jt * 128 + nt;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool in = 8 * o + b < nkb;
      tb[16 * b] = make_uint2(in ? lo[b] : 0u, in ? hi[b] : 0u);
    }
  };
  // fragments of block b = 2 wd + kk (wd, kk compile-time) of the octet in B
  // (and, for Q3S, its high-plane words hw)
  auto dequant = [&](const PfB& B, const uint2 (&hw)[4], auto WD, auto KK,
                     uint4 (&bf)[4]) __attribute__((always_inline)) {
    constexpr int wd = decltype(WD)::value, kk = decltype(KK)::value, b = 2 * wd + kk;
    if constexpr (FMT == kQ3) {
      // scale of (tile j, row n, block b): word wd of row n's 16 bytes
      const uint32_t* scw = reinterpret_cast<const uint32_t*>(&B.sm[wv][0][0]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = wd == 0 ? cwo[j].x : (wd == 1 ? cwo[j].y : (wd == 2 ? cwo[j].z : cwo[j].w));
        const uint32_t sw = scw[(j >> 1) * 256 + ((j & 1) * 32 + n) * 4 + wd];
        const float sc = f16_to_f32((uint16_t)(kk ? (sw >> 16) : (sw & 0xFFFFu)));
        bf[j] = q3_frag<wd, kk>(w, (wd >> 1) ? hw[j].y : hw[j].x, sc);
      }
    } else {
      const uint2* tbl = reinterpret_cast<const uint2*>(&B.code[wv][0][0]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = wd == 0 ? cwo[j].x : (wd == 1 ? cwo[j].y : (wd == 2 ? cwo[j].z : cwo[j].w));
        const uint2 t = tbl[(j * 8 + b) * 16 + n];
        bf[j] = q2_frag(w, 8 * kk, t.x, t.y);
      }
    }
  };
  auto mfmas = [&](const PfA& A, int kk, const uint4 (&bf)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const uint4 af = lds128(&A.a[kk][(i * 4 + q) * 16 + n]);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(af, bf[j], acc[i][j]);
    }
  };

  // Step s = 8 t + I.  Stage s sits in activation buffer s % 4 and octet s / 4
  // in weight buffer (s / 4) % 2.  Loads are issued in the order: prologue
  // B(0), A(0), A(1), A(2); then in step s, after its barrier and its compute
  // (so that the compute's LDS reads never sit behind newer loads), A(s + 3)
  // and, when s % 4 == 0, B(s / 4 + 1).  So when step s waits, the loads
  // issued after A(s) are A(s+1), A(s+2) and -- unless s % 4 == 0 -- one
  // octet B.  Waiting down to 2 kPfDmaA also completes that octet, which the
  // last stage of an octet needs (it prepares the first fragments of the
  // next octet).  Every wave waits for its own loads, then the barrier makes
  // all of them visible and frees buffer (s + 3) % 4.
  auto abuf = [&](int i) __attribute__((always_inline)) -> PfA& {
    return i == 0 ? sa0 : (i == 1 ? sa1 : (i == 2 ? sa2 : sa3));
  };
  auto step = [&](auto I, int s) __attribute__((always_inline)) {
    constexpr int i = decltype(I)::value;
    constexpr int wd = i % 4;
    if constexpr (wd == 0 || wd == 3)
      wait_vm<2 * kPfDmaA>();
    else
      wait_vm<2 * kPfDmaA + kPfDmaB>();
    block_barrier();
    PfB& bc = (i / 4) % 2 == 0 ? sb0 : sb1;  // this octet
    PfB& bn = (i / 4) % 2 == 0 ? sb1 : sb0;  // the next one
    uint2(&hc)[4] = (i / 4) % 2 == 0 ? hw0 : hw1;
    uint2(&hn)[4] = (i / 4) % 2 == 0 ? hw1 : hw0;
    if (s < nst) {
      const PfA& A = abuf(i % 4);
      // k-step 2s (fragments in bfa) || fragments of k-step 2s+1
      dequant(bc, hc, std::integral_constant<int, wd>(), std::integral_constant<int, 1>(), bfb);
      mfmas(A, 0, bfa);
      // k-step 2s+1 (bfb) || fragments of k-step 2s+2 (next stage, maybe next octet)
      uint4 bfn[4];
      if constexpr (wd == 3) {
        load_codes(bn);
        if constexpr (FMT != kQ3) build_tables(bn, s / 4 + 1);
        dequant(bn, hn, std::integral_constant<int, 0>(), std::integral_constant<int, 0>(), bfn);
      } else {
        dequant(bc, hc, std::integral_constant<int, wd + 1>(), std::integral_constant<int, 0>(), bfn);
      }
      mfmas(A, 1, bfb);
#pragma unroll
      for (int j = 0; j < 4; ++j) bfa[j] = bfn[j];
      // Instruction order for the scheduler: the LDS reads first, then each
      // MFMA followed by three VALU instructions of the other k-step's
      // dequantisation, which thereby run in the MFMAs' shadow.
      __builtin_amdgcn_sched_group_barrier(0x100, NG + 4, 0);  // DS reads: A (k-step 2s), tables
#pragma unroll
      for (int t = 0; t < 4 * NG; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);  // VALU
      }
      __builtin_amdgcn_sched_group_barrier(0x100, NG + 4, 0);  // DS reads: A (k-step 2s+1), tables
#pragma unroll
      for (int t = 0; t < 4 * NG; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
      }
    }
    issue_a(abuf((i + 3) % 4), s + 3);
    if constexpr (wd == 0) issue_b(bn, hn, s / 4 + 1);
  };
  issue_b(sb0, hw0, 0);
  issue_a(sa0, 0);
  issue_a(sa1, 1);
  issue_a(sa2, 2);
  wait_vm<3 * kPfDmaA>();  // B(0) has landed (this wave's own weight buffer)
  load_codes(sb0);
  if constexpr (FMT != kQ3) build_tables(sb0, 0);
  dequant(sb0, hw0, std::integral_constant<int, 0>(), std::integral_constant<int, 0>(), bfa);
#pragma unroll 1
  for (int s = 0; s < nst; s += 8) {  // one exit: the register allocator keeps acc in place
    step(std::integral_constant<int, 0>(), s);
    step(std::integral_constant<int, 1>(), s + 1);
    step(std::integral_constant<int, 2>(), s + 2);
    step(std::integral_constant<int, 3>(), s + 3);
    step(std::integral_constant<int, 4>(), s + 4);
    step(std::integral_constant<int, 5>(), s + 5);
    step(std::integral_constant<int, 6>(), s + 6);
    step(std::integral_constant<int, 7>(), s + 7);
  }
  wait_vm<0>();  // the trailing (unused) loads land before the LDS is reused

  // Epilogue through a wave-private 2 KB LDS patch (the stage buffers are
  // free once every wave is past its last stage): per 16-row group the lane's
  // D[4q + r][n] values go in as bf16, and come out as whole row segments,
  // so each lane stores 16 contiguous bytes.
  block_barrier();
  uint16_t* ep = reinterpret_cast<uint16_t*>(&sa0.a[0][0]) + wv * 1024;
  const int rl = lane >> 2;     // row of the group this lane stores
  const int cb = 8 * (lane & 3);
  if (MODE == 0) {
    // tiles 4wv + 2jj (gate) and 4wv + 2jj + 1 (up) form h-group nb*16 + 2wv + jj
    const int hg = nb * (kBN / 32) + 2 * wv + (cb >> 4);
    const bool colok = hg * 16 < F;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          ep[(4 * q + r) * 32 + 16 * jj + n] =
              f32_to_bf16(silu(acc[i][2 * jj][r]) * acc[i][2 * jj + 1][r]);
      wave_lds_fence();
      const uint4 v = *reinterpret_cast<const uint4*>(ep + rl * 32 + cb);
      const int row = 16 * i + rl;
      if (row < rows && colok)
        *reinterpret_cast<uint4*>(a.w.H + (size_t)(row0 + row) * a.w.Fmax + nb * (kBN / 2) +
                                  32 * wv + cb) = v;
      wave_lds_fence();
    }
  } else {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int col = nb * kBN + 64 * wv + 32 * jj + cb;
#pragma unroll
      for (int i = 0; i < NG; ++i) {
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            ep[(4 * q + r) * 32 + 16 * t2 + n] = f32_to_bf16(acc[i][2 * jj + t2][r]);
        wave_lds_fence();
        const uint4 v = *reinterpret_cast<const uint4*>(ep + rl * 32 + cb);
        const int row = 16 * i + rl;
        if (row < rows && col < a.D)
          *reinterpret_cast<uint4*>(a.w.Y + (size_t)(row0 + row) * a.D + col) = v;
        wave_lds_fence();
      }
    }
  }
}

template <int MODE, int FMT>
__global__ __launch_bounds__(kPfThreads, 1) void pf_gemm_kernel(PfArgs a, int nN, int nwork) {
  static_assert(FMT == kQ2 || FMT == kQ2S || FMT == kQ3, "prefill formats");
  __shared__ PfA sa0, sa1, sa2, sa3;
  __shared__ PfB sb0, sb1;
  // XCD-aware order: blocks are dispatched round-robin over the 8 XCDs, so
  // block i runs on XCD i % 8.  Each XCD gets a contiguous eighth of the
  // work items that exist (ntiles * nN, known only here; the grid is sized
  // for the most tiles the routing can make, nwork, and is a multiple of 8),
  // so the column blocks of one tile and the tiles of one expert share an L2
  // and every XCD has work.  Blocks past an XCD's share exit.
  const int nreal = *a.w.ntiles * nN;
  const int per_xcd = (nreal + 7) / 8;
  const int jx = blockIdx.x / 8;
  const int bid = (blockIdx.x % 8) * per_xcd + jx;
  if (jx >= per_xcd || bid >= nreal || bid >= nwork) return;
  const int ti = bid / nN, nb = bid % nN;
  const int4 tile = a.w.tiles[ti];
  const int e = tile.x, row0 = tile.y, rows = tile.z;
  const int F = e < 0 ? a.Fs : a.F;
  if (nb * kBN >= (MODE == 0 ? 2 * F : a.D)) return;
  // Tiles of at most 64 rows (the tails of the expert groups, and whole small
  // groups) skip the MFMAs of their empty row groups.
  if (rows <= 64)
    pf_tile<MODE, FMT, 4>(a, sa0, sa1, sa2, sa3, sb0, sb1, e, row0, rows, nb);
  else
    pf_tile<MODE, FMT, 8>(a, sa0, sa1, sa2, sa3, sb0, sb1, e, row0, rows, nb);
}

// ----------------------------------------------------------------------------
// out_t = sum_j g_tj * Y[inv[t*k + j]] + Y[P + t], in a fixed order.  One
// block per token: the token's rows and gates go to LDS first, then each
// thread has its 16-byte pieces of KJ rows in flight together before it sums
// them in order j = 0..k-1.  With a slot table the sum runs over the resident
// pairs only (the partial layer).  Every one of the KJ loads is issued: a
// slot past k or a non-resident pair reads a row that is there anyway (the
// shared expert's, else row 0) and is left out of the sum by a select.  As
// guarded loads, each sat in a branch of its own behind a wait for the one
// before it, so a token's k rows came in one round trip after another.
template <int KJ>
__global__ __launch_bounds__(512) void pf_combine_kernel(PfArgs a, int has_shared) {
  __shared__ int32_t s_row[kMaxTopK];
  __shared__ float s_g[kMaxTopK];
  const int t = blockIdx.x, tid = threadIdx.x, k = a.k;
  const int P = a.T * k, D = a.D;
  if (tid < k) {
    const size_t p = (size_t)t * k + tid;
    s_row[tid] = a.slot_of && a.w.grp[p] == a.E ? -1 : a.w.inv[p];
    s_g[tid] = a.w.gate[p];
  }
  __syncthreads();
  auto add = [](float (&o)[8], const uint4& y, float g) __attribute__((always_inline)) {
    const uint32_t yy[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] += g * bf16_lo(yy[i]);
      o[2 * i + 1] += g * bf16_hi(yy[i]);
    }
  };
  auto add_if = [](float (&o)[8], const uint4& y, float g, bool on) __attribute__((always_inline)) {
    const uint32_t yy[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = o[2 * i] + g * bf16_lo(yy[i]), hi = o[2 * i + 1] + g * bf16_hi(yy[i]);
      o[2 * i] = on ? lo : o[2 * i];
      o[2 * i + 1] = on ? hi : o[2 * i + 1];
    }
  };
  const size_t fallback = has_shared ? (size_t)(P + t) : 0;
  for (int c = tid; c < D / 8; c += blockDim.x) {
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = 0.f;
    const uint4 ys = reinterpret_cast<const uint4*>(a.w.Y + fallback * D)[c];
    for (int j0 = 0; j0 < k; j0 += KJ) {
      uint4 y[KJ];
      bool on[KJ];
#pragma unroll
      for (int jj = 0; jj < KJ; ++jj) {
        const int j = j0 + jj;  // < kMaxTopK: the host picks KJ with j0 + KJ <= 32
        on[jj] = j < k && s_row[j] >= 0;
        const size_t r = on[jj] ? (size_t)s_row[j] : fallback;
        y[jj] = reinterpret_cast<const uint4*>(a.w.Y + r * D)[c];
      }
#pragma unroll
      for (int jj = 0; jj < KJ; ++jj) add_if(o, y[jj], s_g[j0 + jj], on[jj]);
    }
    if (has_shared) add(o, ys, 1.f);
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
  const uint16_t* xb = (const uint16_t*)pa.x;
  if (pa.rmsnorm || !pa.x_bf16) {
    pf_xprep_kernel<<<T, 256, 0, st>>>(pa.x, pa.x_bf16, pa.rmsnorm, D, w.xb);
    xb = w.xb;
  }
  if (pa.router) {  // logits of the activations the experts see (bf16, after the RMS rule)
    RouterArgs r{T, D, E, xb, 1, 0, pa.router, pa.logits};
    if ((e = launch_router(r, st)) != hipSuccess) return e;
  }
  if ((e = launch_route(pa.logits, T, E, k, w.idx, w.gate, st)) != hipSuccess) return e;
  if (pa.slot_of) {
    // group E collects the misses; the tiles cover groups 0..E-1 only
    const int P = T * k;
    pf_slot_split_kernel<<<(P + 4095) / 4096, 256, pa.use_count ? E * sizeof(uint32_t) : 0, st>>>(
        w.idx, P, E, pa.slot_of, pa.n_slots, w.grp, pa.use_count);
    if ((e = launch_permute(w.grp, T, k, E + 1, w.offsets, w.sorted, w.inv, w.perm, st)) !=
        hipSuccess)
      return e;
    pf_miss_kernel<<<(P + 255) / 256, 256, 0, st>>>(w.offsets, E, k, w.sorted, w.idx, w.gate,
                                                     pa.miss, pa.miss_count);
  } else if ((e = launch_permute(w.idx, T, k, E, w.offsets, w.sorted, w.inv, w.perm, st)) !=
             hipSuccess) {
    return e;
  }
  {  // the caller's route event (moe_set_route_event): routing and miss list are written
    KernelTimer& re = route_event();
    if (re.before != nullptr) {
      const hipEvent_t ev = re.before;
      re.before = nullptr;
      if ((e = hipEventRecord(ev, st)) != hipSuccess) return e;
    }
  }
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
  a.slot_of = pa.slot_of;
  a.shared = pa.shared;
  a.x = xb;
  a.w = w;
  a.out = pa.out;
  a.out_bf16 = pa.out_bf16;
  const int nN_gu = (2 * w.Fmax + kBN - 1) / kBN;
  const int nN_dn = (D + kBN - 1) / kBN;
  const int nw_gu = w.max_tiles * nN_gu, nw_dn = w.max_tiles * nN_dn;
  if (pa.fmt == kQ2) {
    if ((e = launch_timed(pf_gemm_kernel<0, kQ2>, dim3((nw_gu + 7) / 8 * 8), dim3(kPfThreads), 0u,
                          st, a, nN_gu, nw_gu)) != hipSuccess)
      return e;
    pf_gemm_kernel<1, kQ2><<<(nw_dn + 7) / 8 * 8, kPfThreads, 0, st>>>(a, nN_dn, nw_dn);
  } else if (pa.fmt == kQ3) {
    if ((e = launch_timed(pf_gemm_kernel<0, kQ3>, dim3((nw_gu + 7) / 8 * 8), dim3(kPfThreads), 0u,
                          st, a, nN_gu, nw_gu)) != hipSuccess)
      return e;
    pf_gemm_kernel<1, kQ3><<<(nw_dn + 7) / 8 * 8, kPfThreads, 0, st>>>(a, nN_dn, nw_dn);
  } else {
    if ((e = launch_timed(pf_gemm_kernel<0, kQ2S>, dim3((nw_gu + 7) / 8 * 8), dim3(kPfThreads), 0u,
                          st, a, nN_gu, nw_gu)) != hipSuccess)
      return e;
    pf_gemm_kernel<1, kQ2S><<<(nw_dn + 7) / 8 * 8, kPfThreads, 0, st>>>(a, nN_dn, nw_dn);
  }
  // One thread per 16-byte piece of a row (384 for d_model 3072), at least
  // one wave, at most 512 threads.
  const int cthreads = std::min(512, std::max(64, (D / 8 + 63) / 64 * 64));
  // rows in flight per pass: the fewest of 4, 8, 12, 16 that cover k in
  // whole passes with the least slack (k = 10: 12)
  if (k <= 4)
    pf_combine_kernel<4><<<T, cthreads, 0, st>>>(a, has_sh);
  else if (k <= 8)
    pf_combine_kernel<8><<<T, cthreads, 0, st>>>(a, has_sh);
  else if (k <= 12)
    pf_combine_kernel<12><<<T, cthreads, 0, st>>>(a, has_sh);
  else
    pf_combine_kernel<16><<<T, cthreads, 0, st>>>(a, has_sh);
  return hipGetLastError();
}

}  // namespace moe
