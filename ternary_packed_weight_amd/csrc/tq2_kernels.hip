// gfx950 (MI355X, CDNA4) kernels for the TQ2_0 ternary decode matvec.
//
// Method (page "BitCPM ternary (1.58-bit)"): W[n][k] = d[n][k/256]*(q-1),
// q a 2-bit code in {0,1,2}; y = W x is evaluated per block as
// sum_b d_b * sum_{k in b} x_k (q_k - 1), each lane scaling its own block
// partial by its block's d before the cross-lane reduction (kernel paragraph).
// The int8 variant quantizes x with a static scale first (page "gemma4 wNa8o8
// requires int8 activations") and keeps block partials exact.
//
// Mapping on CDNA4 (wave64):
//   * one wave covers 4096 consecutive k of a row per step: lane l takes
//     k = 64*l .. 64*l+63, i.e. one coalesced 16-byte load per row per lane
//     (a wave reads 1 KiB of one row), and a quarter of one 256-block, so the
//     lane's partial is scaled by a single d;
//   * every wave handles R rows per step to keep R KiB in flight per wave;
//   * x is staged once per workgroup in LDS, already rearranged into the
//     operand pairs the decode needs, so the hot loop does no permutation;
//   * no LUT: a 2-bit field masked in place inside a 16-bit half is itself a
//     binary16 subnormal of value q * 4^j * 2^-24 (fp16 path) or a small
//     integer byte (int8 path), consumed directly by v_dot2_f32_f16 /
//     v_dot4_i32_i8.  The zero point (the "-1") is factored out as the
//     block sum of x, which every row shares (page "Custom Metal kernels",
//     affine matvec note: acc += s*(dot - z*sum x)).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "tq2_internal.h"

namespace tq2 {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, a),
                                __builtin_bit_cast(half2v, b), c, false);
}

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

__device__ __forceinline__ float half_to_float(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ int64_t wave_sum64(int64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t lo = (uint32_t)v, hi = (uint32_t)((uint64_t)v >> 32);
    uint32_t lo2 = __shfl_xor(lo, o, 64), hi2 = __shfl_xor(hi, o, 64);
    v += (int64_t)(((uint64_t)hi2 << 32) | lo2);
  }
  return v;
}

// ------------------------------------------------------------------ pack
// Page "BitCPM ternary (1.58-bit)", recovery paragraph: d_block = max|W|,
// code = round(W/d)+1.  One wave per 256-block: lane l owns elements
// 4l..4l+3, so the block's code bytes are written as 64 contiguous bytes.

__global__ void k_zero_i32(int32_t* p) { *p = 0; }

__global__ __launch_bounds__(256) void k_pack(const float* __restrict__ W,
                                              int64_t N, int64_t K,
                                              uint8_t* __restrict__ codes,
                                              uint16_t* __restrict__ scales,
                                              int32_t* bad) {
  const int lane = threadIdx.x & 63;
  const int64_t BK = K / kBlock;
  const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= N * BK) return;  // whole waves leave together
  const int64_t n = blk / BK, b = blk - n * BK;
  const float4 v = *reinterpret_cast<const float4*>(W + n * K + b * kBlock + lane * 4);
  const float w[4] = {v.x, v.y, v.z, v.w};
  float m = 0.0f;
  int nonfinite = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float a = fabsf(w[i]);
    if (!__builtin_isfinite(a)) nonfinite = 1;
    else m = fmaxf(m, a);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    m = fmaxf(m, __shfl_xor(m, o, 64));
    nonfinite |= __shfl_xor(nonfinite, o, 64);
  }
  const _Float16 dh = (_Float16)m;  // round to nearest even
  const uint16_t hb = __builtin_bit_cast(uint16_t, dh);
  const float d = (float)dh;
  uint32_t byte = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int q = 1;
    if (d != 0.0f && __builtin_isfinite(d)) {
      float c = __builtin_rintf(w[i] / d);  // IEEE division, ties to even
      if (__builtin_isnan(c)) c = 0.0f;
      c = fminf(fmaxf(c, -1.0f), 1.0f);
      q = (int)c + 1;
    }
    byte |= (uint32_t)q << (2 * i);
  }
  codes[n * (K / 4) + b * 64 + lane] = (uint8_t)byte;
  if (lane == 0) {
    scales[n * BK + b] = hb;
    if (bad && (nonfinite || hb == 0x7C00)) atomicAdd(bad, 1);
  }
}

hipError_t launch_pack(const float* W, int64_t N, int64_t K, uint8_t* codes,
                       uint16_t* scales, int32_t* bad, hipStream_t s) {
  if (bad) hipLaunchKernelGGL(k_zero_i32, dim3(1), dim3(1), 0, s, bad);
  const int64_t blocks = N * (K / kBlock);
  hipLaunchKernelGGL(k_pack, dim3((unsigned)((blocks + 3) / 4)), dim3(256), 0, s,
                     W, N, K, codes, scales, bad);
  return hipGetLastError();
}

// --------------------------------------------------------------- dequant

__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ codes,
                                                 const uint16_t* __restrict__ scales,
                                                 int64_t N, int64_t K,
                                                 float* __restrict__ W) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t KB = K / 4;
  if (idx >= N * KB) return;
  const int64_t n = idx / KB, kb = idx - n * KB;
  const float d = half_to_float(scales[n * (K / kBlock) + (kb * 4) / kBlock]);
  const uint32_t c = codes[idx];
  float4 o;
  o.x = d * (float)((int)(c & 3) - 1);
  o.y = d * (float)((int)((c >> 2) & 3) - 1);
  o.z = d * (float)((int)((c >> 4) & 3) - 1);
  o.w = d * (float)((int)((c >> 6) & 3) - 1);
  *reinterpret_cast<float4*>(W + n * K + kb * 4) = o;
}

hipError_t launch_dequant(const uint8_t* codes, const uint16_t* scales,
                          int64_t N, int64_t K, float* W, hipStream_t s) {
  const int64_t total = N * (K / 4);
  hipLaunchKernelGGL(k_dequant, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                     codes, scales, N, K, W);
  return hipGetLastError();
}

// ------------------------------------------------------------ fp16 matvec
//
// Work split.  A wave owns one 4096-wide K-chunk c of R consecutive rows
// (lane l covers k = 4096c + 64l .. +63: one 16-byte weight load per row, a
// quarter of one 256-block).  A workgroup holds C = ceil(K/4096) chunk-waves
// for each of S row groups; a row's C partial sums meet in LDS and are added
// in chunk order, so the result is deterministic.
//
// Order of work in a wave: (1) the workgroup's activation loads and this
// wave's weight loads are all issued; (2) the activations are staged once
// per workgroup in LDS, already rearranged for the decode; (3) each wave
// reads its chunk from LDS (conflict-free, lane-contiguous 16-byte reads),
// decodes R rows, reduces them across the wave and stores.
//
// Decode of one 32-bit code word v (16 weights; byte m holds local weights
// 4m+j at bits 2j):
//   v  & (0x00030003 << 2j) -> halves carry weight j (byte 0) and 8+j (byte 2)
//   v8 & (0x00030003 << 2j) -> halves carry weight 4+j and 12+j, v8 = v >> 8
// Each masked half is a binary16 subnormal equal to q * 4^j * 2^-24, exact.
// v_dot2_f32_f16 against the matching x pair gives S_j = sum x q 4^j 2^-24;
// the fields are combined with exact power-of-two weights (below).
// Subtracting the lane's x sum (folded into the seed) turns q into q-1.  The x pairs a lane needs are, per 16-weight group g,
//   pair[8g+2j+0] = (x[16g+j],   x[16g+8+j])
//   pair[8g+2j+1] = (x[16g+4+j], x[16g+12+j]).

constexpr uint32_t kOnesF16x2 = 0x3C003C00u;  // (1.0, 1.0)

// 64 * (lane partial of x(q-1)) * 2^-24, given seed = -(lane x sum) * 2^-24.
// Two independent Horner chains, a = (S0 + seed) * 4 + S1 and
// b = S2 * 4 + S3, give 16a + b = 64 ((S0 + seed) + S1/4 + S2/16 + S3/64):
// field j weighted by 4^(3-j) with exact power-of-two products, the same
// three multiplies as one chain but half its dependency depth (measured on
// MI355X: 0.05-0.1 us faster on the 256- and 4096-row shapes, where a wave
// runs alone on its SIMD).  The factor 64 is removed at the end, together
// with the 2^-24.
__device__ __forceinline__ float lane_dot_f16(const uint4 w, const uint32_t (&xp)[32],
                                              float seed) {
  const uint32_t v[4] = {w.x, w.y, w.z, w.w};
  uint32_t v8[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) v8[g] = v[g] >> 8;
  // first products in the three-source form, so the seed needs no copy
  float a, b;
  asm("v_dot2_f32_f16 %0, %1, %2, %3" : "=v"(a) : "v"(xp[0]), "v"(v[0] & 0x00030003u), "v"(seed));
  b = dot2(xp[4], v[0] & 0x00300030u, 0.0f);
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    if (jj) {
      a *= 4.0f;
      b *= 4.0f;
    }
    const uint32_t ma = 0x00030003u << (2 * jj), mb = 0x00030003u << (2 * (jj + 2));
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (jj || g) a = dot2(xp[8 * g + 2 * jj + 0], v[g] & ma, a);
      if (jj || g) b = dot2(xp[8 * g + 2 * (jj + 2) + 0], v[g] & mb, b);
      a = dot2(xp[8 * g + 2 * jj + 1], v8[g] & ma, a);
      b = dot2(xp[8 * g + 2 * (jj + 2) + 1], v8[g] & mb, b);
    }
  }
  return __builtin_fmaf(a, 16.0f, b);
}

// lane_dot_f16 for M tokens at once: the masked code words are formed once
// and each token runs lane_dot_f16's two chains on them, in the same order,
// so every token's value is bit-equal to lane_dot_f16 on that token's x.
template <int M>
__device__ __forceinline__ void lane_dot_f16_m(const uint4 w, const uint32_t (&xp)[M][32],
                                               const float (&seed)[M], float (&out)[M]) {
  const uint32_t v[4] = {w.x, w.y, w.z, w.w};
  uint32_t v8[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) v8[g] = v[g] >> 8;
  uint32_t ma[2][4][2], mb[2][4][2];  // [jj][g][v or v8]
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const uint32_t ka = 0x00030003u << (2 * jj), kb = 0x00030003u << (2 * (jj + 2));
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      ma[jj][g][0] = v[g] & ka;
      ma[jj][g][1] = v8[g] & ka;
      mb[jj][g][0] = v[g] & kb;
      mb[jj][g][1] = v8[g] & kb;
    }
  }
#pragma unroll
  for (int t = 0; t < M; ++t) {
    float a = dot2(xp[t][0], ma[0][0][0], seed[t]);
    float b = dot2(xp[t][4], mb[0][0][0], 0.0f);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      if (jj) {
        a *= 4.0f;
        b *= 4.0f;
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (jj || g) a = dot2(xp[t][8 * g + 2 * jj + 0], ma[jj][g][0], a);
        if (jj || g) b = dot2(xp[t][8 * g + 2 * (jj + 2) + 0], mb[jj][g][0], b);
        a = dot2(xp[t][8 * g + 2 * jj + 1], ma[jj][g][1], a);
        b = dot2(xp[t][8 * g + 2 * (jj + 2) + 1], mb[jj][g][1], b);
      }
    }
    out[t] = __builtin_fmaf(a, 16.0f, b);
  }
}

// ---- wave64 reduction of R per-lane values (one per row) ----
// Transposed butterfly: v_permlane32_swap folds lanes 32..63 onto 0..31 for
// two rows at once, v_permlane16_swap folds 16-lane rows likewise, and four
// DPP row rotations finish inside each 16-lane row.  On return, out[i] in
// 16-lane row rho (lanes 16rho..16rho+15, all equal) is the full sum of row
//   i + (rho & 1) * (R/4) + (rho >> 1) * (R/2)     for R >= 4,
//   rho >> 1                                         for R == 2.

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}

__device__ __forceinline__ void swap32(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, a),
                                                  __builtin_bit_cast(unsigned, b), false, false);
  a = __builtin_bit_cast(float, (unsigned)r[0]);
  b = __builtin_bit_cast(float, (unsigned)r[1]);
}

__device__ __forceinline__ void swap16(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, a),
                                                  __builtin_bit_cast(unsigned, b), false, false);
  a = __builtin_bit_cast(float, (unsigned)r[0]);
  b = __builtin_bit_cast(float, (unsigned)r[1]);
}

__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<0x128>(v);  // row_ror:8
  v += dpp_f32<0x124>(v);  // row_ror:4
  v += dpp_f32<0x122>(v);  // row_ror:2
  v += dpp_f32<0x121>(v);  // row_ror:1
  return v;
}

template <int R>
constexpr int kOut = R >= 4 ? R / 4 : 1;

template <int R>
__device__ __forceinline__ void reduce_rows_f32(float (&v)[R], float (&out)[kOut<R>]) {
  static_assert(R == 2 || R == 4 || R == 8 || R == 16, "R must be 2, 4, 8 or 16");
  constexpr int H = R / 2;
#pragma unroll
  for (int i = 0; i < H; ++i) {
    float a = v[i], b = v[i + H];
    swap32(a, b);
    v[i] = a + b;  // lanes 0..31: row i, lanes 32..63: row i+H
  }
  if constexpr (R == 2) {
    float a = v[0], b = v[0];
    swap16(a, b);
    out[0] = row16_sum(a + b);
  } else {
    constexpr int Q = R / 4;
#pragma unroll
    for (int i = 0; i < Q; ++i) {
      float a = v[i], b = v[i + Q];
      swap16(a, b);
      out[i] = row16_sum(a + b);
    }
  }
}

// Row of the value out[i] held by 16-lane row rho; -1 if that 16-lane row
// repeats another one (R == 2).
template <int R>
__device__ __forceinline__ int reduced_row(int i, int rho) {
  if constexpr (R == 2) return (rho & 1) ? -1 : rho >> 1;
  else return i + (rho & 1) * (R / 4) + (rho >> 1) * (R / 2);
}

// Row base pointers.  `row` is wave-uniform, and only constant indices into
// the kernel-argument arrays are used, so all of this stays in scalar
// registers: the weight loads do not wait on a pointer fetch.
struct RowPtr {
  const uint8_t* codes;
  const uint16_t* scales;
};

__device__ __forceinline__ RowPtr row_ptr(const MatSet& ms, int row, int64_t row_bytes,
                                          int64_t BK) {
  int lr = row;
  const uint8_t* c = ms.codes[0];
  const uint16_t* s = ms.scales[0];
  if (ms.nmat > 1 && row >= ms.row_begin[1]) {
    lr = row - ms.row_begin[1];
    c = ms.codes[1];
    s = ms.scales[1];
  }
  if (ms.nmat > 2 && row >= ms.row_begin[2]) {
    lr = row - ms.row_begin[2];
    c = ms.codes[2];
    s = ms.scales[2];
  }
  return RowPtr{c + (int64_t)lr * row_bytes, s + (int64_t)lr * BK};
}

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Buffer resource over `bytes` bytes at `base` (raw, untyped access; reads
// past `bytes` return 0).  Built in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

constexpr int kNonTemporal = 2;  // cache policy: streaming, read once

// One wave's weight words and block-scale bits for R rows.  Every load is
// unconditional and in bounds (rows past the end read the last row, lanes
// past K read k = 0) so that nothing waits on a branch; such rows and lanes
// are zeroed later.  Each load is a raw buffer load: scalar descriptor for
// the row, 32-bit lane offset, so there is no per-row vector address work.
//
// Row spaces.  Plain: the wave's rows row0..row0+R-1 index the concatenation
// of the MatSet's matrices.  PAIR (two matrices of N rows, gate and up): row
// group g = row0/R takes gate rows g*R/2 .. g*R/2+R/2-1 as its first R/2
// rows and the up rows with the same indices as its last R/2, so a wave ends
// up holding both factors of each output of a fused SiLU(gate)*up.
template <int R, bool PAIR>
__device__ __forceinline__ bool row_valid(const MatSet& ms, int row0, int r) {
  if constexpr (PAIR) return (row0 / R) * (R / 2) + (r % (R / 2)) < ms.row_begin[1];
  else return row0 + r < ms.rows;
}

template <int R, bool PAIR>
__device__ __forceinline__ RowPtr mapped_row(const MatSet& ms, int row0, int r, int64_t row_bytes,
                                             int64_t BK) {
  if constexpr (PAIR) {
    const int np = ms.row_begin[1];
    int n = (row0 / R) * (R / 2) + (r % (R / 2));
    n = n < np ? n : np - 1;
    const int m = r / (R / 2);
    return RowPtr{ms.codes[m] + (int64_t)n * row_bytes, ms.scales[m] + (int64_t)n * BK};
  } else {
    const int row = row0 + r < ms.rows ? row0 + r : ms.rows - 1;
    return row_ptr(ms, row, row_bytes, BK);
  }
}

// Rows rb..re-1 only (rb, re compile-time after unrolling).
template <int R, bool PAIR = false>
__device__ __forceinline__ void load_rows(const MatSet& ms, int row0, int64_t kk,
                                          int64_t row_bytes, int64_t BK, uint4 (&w)[R],
                                          uint16_t (&hs)[R], int rb, int re) {
  const uint32_t coff = (uint32_t)(kk / 4);                // byte offset in a code row
  const uint32_t soff = (uint32_t)(kk / kBlock) * 2u;      // byte offset in a scale row
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r < rb || r >= re) continue;
    const RowPtr rp = mapped_row<R, PAIR>(ms, row0, r, row_bytes, BK);
    const v4u t = __builtin_bit_cast(
        v4u, __builtin_amdgcn_raw_buffer_load_b128(rsrc(rp.codes, (uint32_t)row_bytes), (int)coff, 0,
                                                   kNonTemporal));
    w[r] = make_uint4(t.x, t.y, t.z, t.w);
    hs[r] = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rsrc(rp.scales, (uint32_t)(BK * 2)),
                                                           (int)soff, 0, 0);
  }
}

// Rows a wave requests before the activations are staged.  The rest follow
// in one burst as soon as the wave has its activations (before its first
// decode), not one row per decoded row: x comes from HBM, so the first decode
// waits ~1.1-1.6 us for it, and by then the first window has mostly arrived;
// requesting the rest only as rows were decoded left HBM idle in that gap
// and sent the last rows to the end of the stream (measured on MI355X, both
// forms on one box: decode step 881 -> 864 us, 16384x4096 5.35 -> 5.21 us,
// 4096x16384 6.29 -> 5.99 us, the int8 down 6.23 -> 6.12 us).  All R rows at
// the start is slower again (4096x16384 +0.7 us): the flood of weight
// requests delays the activations, which come from HBM as well.
template <int R>
constexpr int kRowWindow = R >= 8 ? 4 : (R >= 4 ? 2 : R);

struct Split {
  int C;  // chunk-waves per row group
  int S;  // row groups per workgroup
};

__host__ __device__ constexpr int f16_stage_passes(int CT) { return CT ? 1 : 4; }

// 16 bytes at byte offset `off` of a buffer; zeros past its end.
__device__ __forceinline__ uint4 load_b128(__amdgpu_buffer_rsrc_t r, int off) {
  const v4u v = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  return make_uint4(v.x, v.y, v.z, v.w);
}


// LDS of the fp16 matvec: x pairs [C][8][64] uint4, group sums [C][64] float4,
// a sink [3] uint4 for the stores of threads with no group to stage,
// cross-wave row sums [C*S][R] float.
__host__ __device__ inline size_t f16_lds_bytes(int C, int S, int R) {
  return (size_t)C * 8 * 64 * 16 + (size_t)C * 64 * 16 + 3 * 16 + (size_t)C * S * R * 4;
}

enum Epilogue { kStoreF32 = 0, kSiluMul = 1, kRequant = 2, kSiluMulSlots = 3 };

// h = silu(g) * u with silu(v) = v / (1 + exp(-v)), fp32
__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// CT: chunk-waves per row group as a compile-time constant (1, 2, 4), or 0
// to take it from `sp` at run time.  EPI: kStoreF32 writes y per row;
// kSiluMul runs over PAIR rows and writes silu(gate)*up per output;
// kSiluMulSlots (even S) gives the first S/2 row groups of a workgroup R
// consecutive gate rows each and the last S/2 the up rows with the same
// indices, so every wave streams one contiguous run of rows as in the plain
// matvec, and the pairs meet in LDS (measured on MI355X, 2 x 16384x4096:
// 9.7 us with four gate and four up rows per wave).
template <int R, int CT, int MAXT, int EPI = kStoreF32, bool EAGER = true>
__global__ __launch_bounds__(MAXT) void k_gemv_f16(MatSet ms, int64_t K,
                                                   const uint16_t* __restrict__ x,
                                                   float* __restrict__ y, Split sp) {
  extern __shared__ uint4 lds[];
  // rows requested before x is staged (the rest follow in one burst after
  // it).  Grids of more than two workgroups per CU (not EAGER) with 8 rows
  // per wave request 1: a CU returns loads in request order, so a later
  // workgroup's x waits behind the first windows of the workgroups before it
  // on the CU (measured on MI355X, same box: fused gate+up 2x16384x4096
  // 8.47 -> 8.29 us, with SiLU 8.68 -> 8.36 us; a window of 0 was slower
  // again, and smaller windows for the EAGER grids were slower).
  constexpr int KW = (EAGER || R < 8) ? kRowWindow<R> : 1;
  const int C = CT ? CT : sp.C, S = sp.S;
  uint4* xpairs = lds;                                          // [C][8][64]
  float4* gsum = reinterpret_cast<float4*>(lds + C * 8 * 64);   // [C][64]
  uint4* sink = reinterpret_cast<uint4*>(gsum + C * 64);        // [3]
  float* red = reinterpret_cast<float*>(sink + 3);              // [C*S][R]

  // issue priority: with EAGER, 2 while the wave requests x and its first
  // rows (a wave that is starting gets its requests out ahead of waves that
  // are decoding), then 0 while it waits for x and stages it; always 1 once
  // its last row is requested (the burst after staging).  Measured on
  // MI355X, when rows were still requested one per decoded row, each time both
  // builds on one box: the start priority took the decode step 905-911 ->
  // 884-886 us and the gate/up launches back to back 5.55 -> 5.34 us, but
  // the fused gate+up call (1024 workgroups, twice the CUs' two) 8.95 ->
  // 9.21 us, so the launcher takes EAGER only for grids of at most two
  // workgroups per CU.  (A run-time flag read from the kernel arguments
  // lost most of the step gain.)  The tail priority alone took the step
  // 911-915 -> 904-908 us and left single calls unchanged.
  if constexpr (EAGER) __builtin_amdgcn_s_setprio(2);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform indices, kept in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = __builtin_amdgcn_readfirstlane(wave / C);
  const int c = wave - slot * C;
  constexpr bool SLOTS = EPI == kSiluMulSlots;
  const int half = S / 2;
  const int n0 = SLOTS ? ((int)blockIdx.x * half + (slot < half ? slot : slot - half)) * R : 0;
  // SLOTS: rows of the gate/up concatenation (up starts at row_begin[1])
  const int row0 = SLOTS ? (slot < half ? 0 : ms.row_begin[1]) + n0 : ((int)blockIdx.x * S + slot) * R;
  const int64_t k0 = (int64_t)c * kChunk + (int64_t)lane * kLaneK;
  const bool active = k0 < K;
  const int64_t kk = active ? k0 : 0;
  const int64_t row_bytes = K / 4;
  const int64_t BK = K / kBlock;

  // (1) loads: XP 16-weight groups of x per thread (two 16-byte reads each,
  //     coalesced across the workgroup; clamped, so unconditional), then
  //     the first kRowWindow rows of this wave's weights.  x goes first and
  //     stays first: the wait for it counts loads in issue order, so weights
  //     issued before x would hold the staging (and the barrier) until they
  //     had arrived.
  // staging passes over the C*256 groups: the launcher guarantees
  // XP * blockDim >= C*256 (one pass for C <= 4, four for the runtime-C form)
  //     x is read through a buffer descriptor of exactly K elements, so the
  //     groups past K (a partial last chunk) come back as zeros, with no
  //     masking in the staging.
  constexpr int XP = f16_stage_passes(CT);
  uint4 xa[XP], xb[XP];
  const __amdgpu_buffer_rsrc_t xr = rsrc(x, (uint32_t)(K * 2));
#pragma unroll
  for (int p = 0; p < XP; ++p) {
    const int m = tid + p * (int)blockDim.x;
    xa[p] = load_b128(xr, 32 * m);
    xb[p] = load_b128(xr, 32 * m + 16);
  }
  __builtin_amdgcn_sched_barrier(0);
  // every wave of the workgroup has requested its share of x before any
  // wave requests weights: a CU returns vector loads in request order across
  // its waves, so x requested after another wave's rows waited for those
  // rows to come from HBM (measured on MI355X: 4096x16384 5.93 -> 5.55 us,
  // int8 down 6.06 -> 5.72 us, decode step 864 -> 852 us).  A bare
  // s_barrier: no memory wait, the loads stay in flight.
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  constexpr bool PAIR = EPI == kSiluMul;
  uint4 w[R];
  uint16_t hs[R];
  load_rows<R, PAIR>(ms, row0, kk, row_bytes, BK, w, hs, 0, KW);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (EAGER) __builtin_amdgcn_s_setprio(0);

  // (2) stage: group m covers weights 16m..16m+15 = group (m % 4) of lane
  //     (m / 4) % 64 of chunk m / 256.  Its 8 operand pairs go to slots
  //     2(m%4) and 2(m%4)+1 of that lane; its x sum to gsum[..].(m % 4).
  //     Groups past K (a partial last chunk) are staged as zeros, so lanes
  //     beyond K contribute exactly 0.
  //     Every thread runs the arithmetic and stores; one without a group
  //     stores into the sink.  (A branch around it would let the compiler
  //     sink the x loads behind the weight loads, into the branch.)
#pragma unroll
  for (int p = 0; p < XP; ++p) {
    const int m = tid + p * (int)blockDim.x;
    const bool staged = m < C * 256;
    const uint4 a4 = xa[p], b4 = xb[p];
    const uint32_t xw[8] = {a4.x, a4.y, a4.z, a4.w, b4.x, b4.y, b4.z, b4.w};
    // pair (x[16m + e0], x[16m + e1]): one byte permute of the two dwords
    // holding them, low halves (selector 0x05040100) or high (0x07060302)
    uint32_t pr[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t a = xw[j >> 1], b = xw[4 + (j >> 1)];
      const uint32_t cc = xw[2 + (j >> 1)], d = xw[6 + (j >> 1)];
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
      pr[2 * j + 0] = __builtin_amdgcn_perm(b, a, sel);
      pr[2 * j + 1] = __builtin_amdgcn_perm(d, cc, sel);
    }
    float s0 = dot2(xw[0], kOnesF16x2, 0.0f), s1 = dot2(xw[1], kOnesF16x2, 0.0f);
    s0 = dot2(xw[2], kOnesF16x2, s0); s1 = dot2(xw[3], kOnesF16x2, s1);
    s0 = dot2(xw[4], kOnesF16x2, s0); s1 = dot2(xw[5], kOnesF16x2, s1);
    s0 = dot2(xw[6], kOnesF16x2, s0); s1 = dot2(xw[7], kOnesF16x2, s1);
    const int ch = m >> 8, ln = (m >> 2) & 63, gg = m & 3;
    uint4* d0 = staged ? xpairs + (ch * 8 + 2 * gg) * 64 + ln : sink;
    uint4* d1 = staged ? xpairs + (ch * 8 + 2 * gg + 1) * 64 + ln : sink + 1;
    float* d2 = staged ? reinterpret_cast<float*>(gsum) + (ch * 64 + ln) * 4 + gg
                       : reinterpret_cast<float*>(sink + 2);
    *d0 = make_uint4(pr[0], pr[1], pr[2], pr[3]);
    *d1 = make_uint4(pr[4], pr[5], pr[6], pr[7]);
    *d2 = s0 + s1;
  }
  __syncthreads();

  // (3) this lane's operand pairs and seed -(sum of its 64 x) * 2^-24
  uint32_t xp[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 tt = xpairs[(c * 8 + i) * 64 + lane];
    xp[4 * i + 0] = tt.x; xp[4 * i + 1] = tt.y; xp[4 * i + 2] = tt.z; xp[4 * i + 3] = tt.w;
  }
  const float4 gs = gsum[c * 64 + lane];
  const float seed = -ldexpf((gs.x + gs.y) + (gs.z + gs.w), -24);
  if constexpr (KW < R) {  // the rest of the rows, in one burst
    __builtin_amdgcn_sched_barrier(0);
    load_rows<R, PAIR>(ms, row0, kk, row_bytes, BK, w, hs, KW, R);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_setprio(1);  // every row is requested: only decoding is left

  // lanes past K hold x = 0 and seed 0, so only padding rows need zeroing;
  // the row test is wave-uniform (a scalar select of the mask)
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t keep = row_valid<R, PAIR>(ms, row0, r) ? 0xFFFFu : 0u;
    const _Float16 d = __builtin_bit_cast(_Float16, (uint16_t)(hs[r] & keep));
    acc[r] = __builtin_fmaf((float)d, lane_dot_f16(w[r], xp, seed), 0.0f);  // v_fma_mix
  }
  float out[kOut<R>];
  reduce_rows_f32<R>(acc, out);
  const int rho = lane >> 4;
  if (C == 1 && !SLOTS) {
    if constexpr (EPI == kSiluMul) {
      // rows of the first half (gate) sit in lanes 0..31, their up partners
      // (row + R/2) at lane + 32
#pragma unroll
      for (int i = 0; i < kOut<R>; ++i) {
        float a = out[i], b = out[i];
        swap32(a, b);  // b: lanes 0..31 now hold lanes 32..63
        const int rr = reduced_row<R>(i, rho);
        const int n = (row0 / R) * (R / 2) + rr;
        if ((lane & 15) == 0 && lane < 32 && rr >= 0 && n < ms.row_begin[1])
          y[n] = silu_mul(ldexpf(out[i], 18), ldexpf(b, 18));
      }
    } else {
      if ((lane & 15) == 0) {
#pragma unroll
        for (int i = 0; i < kOut<R>; ++i) {
          const int rr = reduced_row<R>(i, rho);
          if (rr >= 0 && row0 + rr < ms.rows) y[row0 + rr] = ldexpf(out[i], 18);
        }
      }
    }
    return;
  }
  // several chunk-waves per row: add their sums in chunk order
  if ((lane & 15) == 0) {
#pragma unroll
    for (int i = 0; i < kOut<R>; ++i) {
      const int rr = reduced_row<R>(i, rho);
      if (rr >= 0) red[wave * R + rr] = out[i];
    }
  }
  __syncthreads();
  if constexpr (SLOTS) {
    // gate row group `slot` and its up partner `slot + S/2`, chunk sums in order
    if (slot < half && c == 0 && lane < R) {
      const int wu = (slot + half) * C;
      float g = red[wave * R + lane], u = red[wu * R + lane];
      for (int cc = 1; cc < C; ++cc) {
        g += red[(wave + cc) * R + lane];
        u += red[(wu + cc) * R + lane];
      }
      const int n = n0 + lane;
      if (n < ms.row_begin[1]) y[n] = silu_mul(ldexpf(g, 18), ldexpf(u, 18));
    }
  } else if constexpr (EPI == kSiluMul) {
    if (c == 0 && lane < R / 2) {
      float g = red[wave * R + lane], u = red[wave * R + lane + R / 2];
      for (int cc = 1; cc < C; ++cc) {
        g += red[(wave + cc) * R + lane];
        u += red[(wave + cc) * R + lane + R / 2];
      }
      const int n = (row0 / R) * (R / 2) + lane;
      if (n < ms.row_begin[1]) y[n] = silu_mul(ldexpf(g, 18), ldexpf(u, 18));
    }
  } else {
    if (c == 0 && lane < R) {
      float tsum = red[wave * R + lane];
      for (int cc = 1; cc < C; ++cc) tsum += red[(wave + cc) * R + lane];
      if (row0 + lane < ms.rows) y[row0 + lane] = ldexpf(tsum, 18);
    }
  }
}

// The matvec for M = 2..4 tokens (the small-M batched matvec): k_gemv_f16's
// waves, rows, loads and order, with the M tokens' activations staged side
// by side in LDS.  Each code word is masked once and then dotted with every
// token's operand pairs (lane_dot_f16_m), so the weights are streamed and
// decoded once for all M tokens.  Every token's arithmetic is k_gemv_f16's
// on that token: its output equals tq2_gemv's bit for bit.  Output y[M][N].
// staging passes of k_gemv_f16m: every group of 16 activations of the C
// chunks gets a thread (MAXT is the block size the launcher uses)
__host__ __device__ constexpr int f16m_stage_passes(int CT, int MAXT) {
  return CT ? (CT * 256 + MAXT - 1) / MAXT : 4;
}

template <int M>
__host__ __device__ inline size_t f16m_lds_bytes(int C, int S, int R) {
  return (size_t)M * ((size_t)C * 8 * 64 * 16 + (size_t)C * 64 * 16) + 3 * 16 + (size_t)M * C * S * R * 4;
}

template <int R, int M, int CT, int MAXT, bool EAGER>
__global__ __launch_bounds__(MAXT) void k_gemv_f16m(MatSet ms, int64_t K, const uint16_t* __restrict__ x,
                                                    float* __restrict__ y, Split sp) {
  extern __shared__ uint4 lds[];
  constexpr int KW = (EAGER || R < 8) ? kRowWindow<R> : 1;
  const int C = CT ? CT : sp.C, S = sp.S;
  uint4* xpairs = lds;                                            // [M][C][8][64]
  float4* gsum = reinterpret_cast<float4*>(lds + M * C * 8 * 64);  // [M][C][64]
  uint4* sink = reinterpret_cast<uint4*>(gsum + M * C * 64);       // [3]
  float* red = reinterpret_cast<float*>(sink + 3);                 // [M][C*S][R]
  if constexpr (EAGER) __builtin_amdgcn_s_setprio(2);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = __builtin_amdgcn_readfirstlane(wave / C);
  const int c = wave - slot * C;
  const int row0 = ((int)blockIdx.x * S + slot) * R;
  const int64_t k0 = (int64_t)c * kChunk + (int64_t)lane * kLaneK;
  const bool active = k0 < K;
  const int64_t kk = active ? k0 : 0;
  const int64_t row_bytes = K / 4;
  const int64_t BK = K / kBlock;
  const int64_t N = ms.rows;

  // (1) loads: every token's activations (as k_gemv_f16, per token), the
  //     workgroup barrier, then the first KW rows
  constexpr int XP = f16m_stage_passes(CT, MAXT);
  uint4 xa[M][XP], xb[M][XP];
#pragma unroll
  for (int t = 0; t < M; ++t) {
    const __amdgpu_buffer_rsrc_t xr = rsrc(x + t * K, (uint32_t)(K * 2));
#pragma unroll
    for (int p = 0; p < XP; ++p) {
      const int m = tid + p * (int)blockDim.x;
      xa[t][p] = load_b128(xr, 32 * m);
      xb[t][p] = load_b128(xr, 32 * m + 16);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();  // x of every wave ahead of any weight request (see k_gemv_f16)
  __builtin_amdgcn_sched_barrier(0);
  uint4 w[R];
  uint16_t hs[R];
  load_rows<R>(ms, row0, kk, row_bytes, BK, w, hs, 0, KW);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (EAGER) __builtin_amdgcn_s_setprio(0);

  // (2) stage every token as k_gemv_f16 stages its one
#pragma unroll
  for (int t = 0; t < M; ++t) {
#pragma unroll
    for (int p = 0; p < XP; ++p) {
      const int m = tid + p * (int)blockDim.x;
      const bool staged = m < C * 256;
      const uint4 a4 = xa[t][p], b4 = xb[t][p];
      const uint32_t xw[8] = {a4.x, a4.y, a4.z, a4.w, b4.x, b4.y, b4.z, b4.w};
      uint32_t pr[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t a = xw[j >> 1], b = xw[4 + (j >> 1)];
        const uint32_t cc = xw[2 + (j >> 1)], d = xw[6 + (j >> 1)];
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        pr[2 * j + 0] = __builtin_amdgcn_perm(b, a, sel);
        pr[2 * j + 1] = __builtin_amdgcn_perm(d, cc, sel);
      }
      float s0 = dot2(xw[0], kOnesF16x2, 0.0f), s1 = dot2(xw[1], kOnesF16x2, 0.0f);
      s0 = dot2(xw[2], kOnesF16x2, s0); s1 = dot2(xw[3], kOnesF16x2, s1);
      s0 = dot2(xw[4], kOnesF16x2, s0); s1 = dot2(xw[5], kOnesF16x2, s1);
      s0 = dot2(xw[6], kOnesF16x2, s0); s1 = dot2(xw[7], kOnesF16x2, s1);
      const int ch = m >> 8, ln = (m >> 2) & 63, gg = m & 3;
      uint4* d0 = staged ? xpairs + ((t * C + ch) * 8 + 2 * gg) * 64 + ln : sink;
      uint4* d1 = staged ? xpairs + ((t * C + ch) * 8 + 2 * gg + 1) * 64 + ln : sink + 1;
      float* d2 = staged ? reinterpret_cast<float*>(gsum) + ((t * C + ch) * 64 + ln) * 4 + gg
                         : reinterpret_cast<float*>(sink + 2);
      *d0 = make_uint4(pr[0], pr[1], pr[2], pr[3]);
      *d1 = make_uint4(pr[4], pr[5], pr[6], pr[7]);
      *d2 = s0 + s1;
    }
  }
  __syncthreads();

  // (3) this lane's operand pairs and seed per token, then the rest of the rows
  uint32_t xp[M][32];
  float seed[M];
#pragma unroll
  for (int t = 0; t < M; ++t) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 tt = xpairs[((t * C + c) * 8 + i) * 64 + lane];
      xp[t][4 * i + 0] = tt.x; xp[t][4 * i + 1] = tt.y; xp[t][4 * i + 2] = tt.z; xp[t][4 * i + 3] = tt.w;
    }
    const float4 gs = gsum[(t * C + c) * 64 + lane];
    seed[t] = -ldexpf((gs.x + gs.y) + (gs.z + gs.w), -24);
  }
  if constexpr (KW < R) {
    __builtin_amdgcn_sched_barrier(0);
    load_rows<R>(ms, row0, kk, row_bytes, BK, w, hs, KW, R);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_setprio(1);

  float acc[M][R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t keep = row_valid<R, false>(ms, row0, r) ? 0xFFFFu : 0u;
    const _Float16 d = __builtin_bit_cast(_Float16, (uint16_t)(hs[r] & keep));
    // the row's code words pass through an empty asm here, so that its masked
    // words are formed here and not hoisted ahead for all rows at once
    uint4 wr = w[r];
    asm volatile("" : "+v"(wr.x), "+v"(wr.y), "+v"(wr.z), "+v"(wr.w));
    float dt[M];
    lane_dot_f16_m<M>(wr, xp, seed, dt);
#pragma unroll
    for (int t = 0; t < M; ++t) acc[t][r] = __builtin_fmaf((float)d, dt[t], 0.0f);  // v_fma_mix
    // one row's masked words live at a time (M tokens' operands take
    // 32 M registers already)
    __builtin_amdgcn_sched_barrier(0);
  }
  const int rho = lane >> 4;
#pragma unroll
  for (int t = 0; t < M; ++t) {
    float out[kOut<R>];
    reduce_rows_f32<R>(acc[t], out);
    if (C == 1) {
      if ((lane & 15) == 0) {
#pragma unroll
        for (int i = 0; i < kOut<R>; ++i) {
          const int rr = reduced_row<R>(i, rho);
          if (rr >= 0 && row0 + rr < ms.rows) y[t * N + row0 + rr] = ldexpf(out[i], 18);
        }
      }
    } else if ((lane & 15) == 0) {
#pragma unroll
      for (int i = 0; i < kOut<R>; ++i) {
        const int rr = reduced_row<R>(i, rho);
        if (rr >= 0) red[(t * C * S + wave) * R + rr] = out[i];
      }
    }
  }
  if (C == 1) return;
  __syncthreads();
  if (c == 0 && lane < R) {
#pragma unroll
    for (int t = 0; t < M; ++t) {
      float tsum = red[(t * C * S + wave) * R + lane];
      for (int cc = 1; cc < C; ++cc) tsum += red[(t * C * S + wave + cc) * R + lane];
      if (row0 + lane < ms.rows) y[t * N + row0 + lane] = ldexpf(tsum, 18);
    }
  }
}

static int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  return cus;
}

// Waves per workgroup: C chunk-waves for each of S row groups (measured on
// MI355X).  fp16, one chunk (K <= 4096): 4-wave workgroups.  Otherwise 8
// waves when C divides 8, except K = 16384 (C = 4), where 16-wave workgroups
// halve the activation staging per row.  (The int8 launcher may take 4-wave
// workgroups at one chunk as well, by how the row groups fill the CUs.)
static Split pick_split(int64_t K, bool fp16) {
  const int C = (int)chunks_of(K);
  Split sp;
  sp.C = C;
  sp.S = (fp16 && C == 1) ? 4 : (C == 4 ? 4 : (C >= 8 ? 1 : 8 / C));
  return sp;
}

// Rows per wave (measured on MI355X): as many rows per wave (up to rmax) as
// still give waves_per_cu waves per CU; the fp16 matvec does best with 8
// waves per CU for one chunk and 16 otherwise, the int8 matvec with 16.
static int pick_rows_per_wave(int64_t rows, int C, int waves_per_cu, int rmax) {
  const int64_t want_waves = (int64_t)device_cus() * waves_per_cu;
  for (int R = rmax; R > 2; R /= 2) {
    if ((rows + R - 1) / R * C >= want_waves) return R;
  }
  return 2;
}

static hipError_t set_lds_cap(const void* fn) {
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
}

// Launch one instantiation of the fp16 matvec (EAGER: see k_gemv_f16).
template <int R, int EPI, bool EAGER>
static hipError_t launch_f16_kernel(const Split& sp, dim3 grid, dim3 block, size_t lds, hipStream_t s,
                                    const MatSet& m, int64_t K, const uint16_t* x, float* y) {
  if (sp.C == 1) {
    hipLaunchKernelGGL((k_gemv_f16<R, 1, 512, EPI, EAGER>), grid, block, lds, s, m, K, x, y, sp);
  } else if (sp.C == 2) {
    hipLaunchKernelGGL((k_gemv_f16<R, 2, 512, EPI, EAGER>), grid, block, lds, s, m, K, x, y, sp);
  } else if (sp.C == 4) {
    hipLaunchKernelGGL((k_gemv_f16<R, 4, 1024, EPI, EAGER>), grid, block, lds, s, m, K, x, y, sp);
  } else if (block.x <= 512) {
    hipLaunchKernelGGL((k_gemv_f16<R, 0, 512, EPI, EAGER>), grid, block, lds, s, m, K, x, y, sp);
  } else {
    if (lds > 64 * 1024) {
      const hipError_t e = set_lds_cap(reinterpret_cast<const void*>(&k_gemv_f16<R, 0, 1024, EPI, EAGER>));
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_gemv_f16<R, 0, 1024, EPI, EAGER>), grid, block, lds, s, m, K, x, y, sp);
  }
  return hipGetLastError();
}

template <int R, int EPI>
static hipError_t run_gemv_f16(const MatSet& m, int64_t K, const uint16_t* x, float* y,
                               hipStream_t s) {
  const Split sp = pick_split(K, true);
  // PAIR rows: R/2 outputs per row group, each reading one gate and one up row;
  // paired slots: R outputs per gate row group, S/2 of them per workgroup
  const int64_t groups = EPI == kSiluMul ? (m.row_begin[1] + R / 2 - 1) / (R / 2) : (m.rows + R - 1) / R;
  const int64_t nwg = EPI == kSiluMulSlots ? (m.row_begin[1] + (int64_t)(sp.S / 2) * R - 1) / ((int64_t)(sp.S / 2) * R)
                                           : (groups + sp.S - 1) / sp.S;
  if (EPI == kSiluMulSlots && sp.S % 2 != 0) return hipErrorInvalidConfiguration;
  const bool eager = nwg <= 2LL * device_cus();
  const dim3 grid((unsigned)nwg);
  const size_t lds = f16_lds_bytes(sp.C, sp.S, R);
  const dim3 block(64 * sp.C * sp.S);
  const int ct = sp.C <= 4 && sp.C != 3 ? sp.C : 0;
  if ((int64_t)f16_stage_passes(ct) * block.x < (int64_t)sp.C * 256) return hipErrorInvalidConfiguration;
  if (eager) return launch_f16_kernel<R, EPI, true>(sp, grid, block, lds, s, m, K, x, y);
  return launch_f16_kernel<R, EPI, false>(sp, grid, block, lds, s, m, K, x, y);
}


static int f16_waves_per_cu(int64_t K) { return chunks_of(K) == 1 ? 8 : 16; }

hipError_t launch_gemv_f16(const MatSet& m, int64_t K, const uint16_t* x, float* y,
                           hipStream_t s) {
  switch (pick_rows_per_wave(m.rows, (int)chunks_of(K), f16_waves_per_cu(K), 8)) {
    case 8: return run_gemv_f16<8, kStoreF32>(m, K, x, y, s);
    case 4: return run_gemv_f16<4, kStoreF32>(m, K, x, y, s);
    default: return run_gemv_f16<2, kStoreF32>(m, K, x, y, s);
  }
}

// The matvec for M = 2..4 tokens: k_gemv_f16m with fewer rows per wave
// than tq2_gemv (4 for two tokens, 2 for three or four; M tokens' operands
// take 32 M registers) and, for K = 16384, 8-wave workgroups, so that every
// wave stays within 256 registers without spilling.  The results do not
// depend on either choice: a row's 64 lane partials are added in the same
// order for every rows-per-wave (lanes l and l+32, then l and l+16, then the
// 16-lane rotations), and chunk sums in chunk order, so every token's output
// still equals tq2_gemv's.  For K of 1, 2 or 4 chunks (the caller checks).
template <int R, int M>
static hipError_t run_gemv_f16m(const MatSet& m, int64_t K, const uint16_t* x, float* y, hipStream_t s) {
  Split sp = pick_split(K, true);
  if (sp.C != 1 && sp.C != 2 && sp.C != 4) return hipErrorInvalidConfiguration;
  if (sp.C == 4) sp.S = 2;  // 512 threads: 256 registers per wave
  const int64_t groups = (m.rows + R - 1) / R;
  const int64_t nwg = (groups + sp.S - 1) / sp.S;
  const bool eager = nwg <= 2LL * device_cus();
  const dim3 grid((unsigned)nwg);
  const size_t lds = f16m_lds_bytes<M>(sp.C, sp.S, R);
  const dim3 block(64 * sp.C * sp.S);
  // every instantiation below has MAXT = 512 and the block is exactly 512
  // threads for C = 2 and 4, 256 for C = 1 (256 groups)
  if ((int64_t)f16m_stage_passes(sp.C, 512) * block.x < (int64_t)sp.C * 256 || block.x > 512 ||
      lds > 160 * 1024)
    return hipErrorInvalidConfiguration;
  auto go = [&](auto kfn) -> hipError_t {
    if (lds > 64 * 1024) {
      const hipError_t e = set_lds_cap(reinterpret_cast<const void*>(kfn));
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kfn, grid, block, lds, s, m, K, x, y, sp);
    return hipGetLastError();
  };
  if (eager) {
    if (sp.C == 1) return go(k_gemv_f16m<R, M, 1, 512, true>);
    if (sp.C == 2) return go(k_gemv_f16m<R, M, 2, 512, true>);
    return go(k_gemv_f16m<R, M, 4, 512, true>);
  }
  if (sp.C == 1) return go(k_gemv_f16m<R, M, 1, 512, false>);
  if (sp.C == 2) return go(k_gemv_f16m<R, M, 2, 512, false>);
  return go(k_gemv_f16m<R, M, 4, 512, false>);
}

// rows per wave of k_gemv_f16m for M tokens (see run_gemv_f16m)
static int f16m_rows_per_wave(int64_t rows, int64_t K, int64_t M) {
  return pick_rows_per_wave(rows, (int)chunks_of(K), f16_waves_per_cu(K), M == 2 ? 4 : 2);
}

// Activation bytes k_gemv_f16m stages over all its workgroups (each stages
// every token's whole x).  Measured on MI355X against the matrix-core path:
// the one-pass kernel wins while this stays at or below 32 MiB (4096x4096
// at 4 tokens 5.2 against 7.5 us, 16384x4096 at 2 tokens 8.1 against 9.1,
// 4096x16384 at 2 tokens 9.9 against 11.7) and loses above (16384x4096 at
// 3 and 4 tokens, 48 and 64 MiB: 11.8 and 14.0 against 9.3 us; 4096x16384
// at 4 tokens, 128 MiB: 23.5 against 11.9).
static int64_t f16m_staging_bytes(int64_t rows, int64_t K, int64_t M) {
  const int R = f16m_rows_per_wave(rows, K, M);
  Split sp = pick_split(K, true);
  if (sp.C == 4) sp.S = 2;
  const int64_t nwg = ((rows + R - 1) / R + sp.S - 1) / sp.S;
  return nwg * M * K * 2;
}

template <int M>
static hipError_t launch_gemv_f16m(const MatSet& m, int64_t K, const uint16_t* x, float* y, hipStream_t s) {
  if (f16m_rows_per_wave(m.rows, K, M) == 4 && M == 2) return run_gemv_f16m<4, M>(m, K, x, y, s);
  return run_gemv_f16m<2, M>(m, K, x, y, s);
}

hipError_t launch_gemv_silu_mul(const MatSet& m, int64_t K, const uint16_t* x, float* h,
                                hipStream_t s) {
  const bool slots = pick_split(K, true).S % 2 == 0;  // paired row groups need an even S
  switch (pick_rows_per_wave(m.rows, (int)chunks_of(K), f16_waves_per_cu(K), 8)) {
    case 8: return slots ? run_gemv_f16<8, kSiluMulSlots>(m, K, x, h, s) : run_gemv_f16<8, kSiluMul>(m, K, x, h, s);
    case 4: return slots ? run_gemv_f16<4, kSiluMulSlots>(m, K, x, h, s) : run_gemv_f16<4, kSiluMul>(m, K, x, h, s);
    default: return slots ? run_gemv_f16<2, kSiluMulSlots>(m, K, x, h, s) : run_gemv_f16<2, kSiluMul>(m, K, x, h, s);
  }
}

// -------------------------------------------- small-M batched matvec (MFMA)
//
// Y[M][N] = X[M][K] . W^T for a few tokens at once (prefill, speculative
// decode): the weight stream is paid once for all M tokens.  Page "BitCPM
// ternary (1.58-bit)", kernel paragraph, applied per token.
//
// A 16 x 32 tile of the masked codes is the A operand of
// v_mfma_f32_16x16x32_f16 (the same subnormal binary16 decode as the
// matvec); the B operand carries the x values of 16 tokens, one per column,
// so the matrix cores do useful work in every column.  Lane (G = l/16,
// i = l%16) supplies row i's codes at k-slots 8G..8G+7 and token i's x
// values at the same slots, and receives D[rows 4G..4G+3][token i].
//
//   gemm   : a wave owns U row groups (16U rows) and a K range; per 256-block
//            step it builds the B operands of its token from X (one byte
//            permute per pair, then a power-of-two scale, below) and the
//            block zero point -sum(x) * 2^(-18-sh), then runs 8 MFMAs per row
//            group starting from the zero point and does
//            acc += d_row * 2^sh * D;
//   reduce : when K is split across workgroups, the split partials are added
//            in split order.
//
// Operand scale.  The mask at position j makes a code worth q * 4^j * 2^-24,
// so the x paired with it is scaled by 4^(3-j) * 2^-sh, which makes every
// product q * x * 2^(-18-sh).  For a (token, block) whose sum of x^2 is
// below 2^16 (so every |x| < 256), sh = 0: the scale is up by 1..64, exact
// in binary16 (no overflow below 16384, and scaling up never drops a bit).
// Otherwise sh = 6 (scale 4^-j): x values tiny enough to be rounded lose at
// most 2^-19 each, under 2^-10 |d| per block, against this block's share
// 2e-3 |d| sum|x| >= 2e-3 |d| 256 of the tolerance.  (A plain 4^-j scale
// for every block would round tiny activations, x near 2^-14, by up to 3%.)

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kTok = 16;        // tokens per tile (MFMA columns)
constexpr int kTileRows16 = 16;  // rows per MFMA tile

struct GemmArgs {
  const uint8_t* codes;
  const uint16_t* scales;
  const uint16_t* x;  // X[M][K]
  float* out;         // y[M][N], or the split partials [splits][M][N]
  int64_t N, K, M;
  int32_t steps_per_split;  // multiple of C*T
};

constexpr int kStepTile = kTok * kBlock * 2;  // x of one step for one tile: 8 KiB

// Load order of a batch: with two or more row groups per wave the scales go
// before the code words, so that a wave's first row group can be scaled
// once its codes arrive rather than after all its codes.  Measured on MI355X
// (same box, alternating passes, µs per call): 16384x4096 int8 at 16/32
// tokens 10.47 -> 9.88 / 15.73 -> 14.93, fp16 at 64 tokens 21.28 -> 20.87;
// with one row group it loses (4096x16384 int8 at 16 tokens 12.11 -> 12.23,
// 4096x4096 fp16 at 8 tokens 5.81 -> 5.96), so that order stays there.
template <int U>
constexpr bool kScalesFirstFor = U >= 2;

// wait until at most N vector-memory operations of this wave are in flight
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// the same for an n that is a constant once the caller's loops are unrolled
template <int N = 63>
__device__ __forceinline__ void wait_vm_at(int n) {
  if (n == N) wait_vm<N>();
  else if constexpr (N > 0) wait_vm_at<N - 1>(n);
}
// 16 bytes per lane from a buffer straight to LDS: lane l's bytes land at
// lds + 16 l (lds wave-uniform)
__device__ __forceinline__ void load_b128_lds(__amdgpu_buffer_rsrc_t r, int off, uint8_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off, 0,
                                           0, 0);
}

// Workgroup: C waves, the C chunks of one K-split of one row set (U row
// groups) and TT token tiles; their sums meet in LDS and are added in chunk
// order.  A wave decodes each code word once for all TT tiles (the A
// operand is shared; each tile brings its own B operands).  Grid: (row sets,
// K-splits, token tiles / TT).
//
// x reaches the lanes one of two ways.  XL: straight to LDS, each load
// instruction bringing two tokens' 512 contiguous bytes of a step (every
// cache line read by one instruction), then read back in operand order.
// Otherwise: each lane loads its own token's 64 values of the step, so one
// instruction touches 64 cache lines and each line is touched by eight
// instructions, which stalls issue once the tile is full; with few tokens
// there is little to stall and the LDS round trip costs more.
template <int U, int T, int C, int TT, bool XL>
__global__ __launch_bounds__(64 * C) void k_gemm_mfma(GemmArgs a) {
  constexpr bool kScalesFirst = kScalesFirstFor<U>;
  // XL: per wave, the x of its load batch (T steps x TT tiles of 8 KiB);
  // after the loop the same memory holds the chunk sums
  constexpr int kXBytes = XL ? C * T * TT * kStepTile : 0;
  constexpr int kRedBytes = C * TT * U * 4 * 64 * 4;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kXBytes > kRedBytes ? kXBytes : kRedBytes];
  float(*red)[TT][U][4][64] = reinterpret_cast<float(*)[TT][U][4][64]>(smem);
  const int lane = threadIdx.x & 63;
  const int G = lane >> 4, i = lane & 15;
  const int c = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rset = blockIdx.x;
  const int split = blockIdx.y, tt0 = blockIdx.z * TT;
  const int64_t row_bytes = a.K / 4, BK = a.K / kBlock;
  const int spw = a.steps_per_split / C;  // steps per wave
  const int s_begin = split * a.steps_per_split + c * spw;
  const int s_lim = s_begin + spw;
  const int s_end = (int64_t)s_lim < BK ? s_lim : (int)BK;

  // per row group: scalar descriptors over its valid rows (zeros past N)
  __amdgpu_buffer_rsrc_t rc[U], rs[U];
  int valid[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int gi = rset * U + u;
    int v = (int)(a.N - (int64_t)gi * kTileRows16);
    v = v < 0 ? 0 : (v > kTileRows16 ? kTileRows16 : v);
    v = __builtin_amdgcn_readfirstlane(v);
    valid[u] = v;
    const int64_t r0 = v > 0 ? (int64_t)gi * kTileRows16 : 0;
    rc[u] = rsrc(a.codes + r0 * row_bytes, (uint32_t)(v * row_bytes));
    rs[u] = rsrc(a.scales + r0 * BK, (uint32_t)(v * BK * 2));
  }

  v4f acc[TT][U];
#pragma unroll
  for (int q = 0; q < TT; ++q)
#pragma unroll
    for (int u = 0; u < U; ++u) acc[q][u] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  // token tiles past M (the last of a pair) read zeros and store nothing
  __amdgpu_buffer_rsrc_t xr[TT];
#pragma unroll
  for (int q = 0; q < TT; ++q) {
    int64_t tv = a.M - (int64_t)(tt0 + q) * kTok;
    tv = tv > kTok ? kTok : (tv < 0 ? 0 : tv);
    const int64_t base = tv > 0 ? (int64_t)(tt0 + q) * kTok * a.K : 0;
    xr[q] = rsrc(a.x + base, (uint32_t)(tv * a.K * 2));
  }

  for (int s0 = s_begin; s0 < s_end; s0 += T) {
    // issue, in this order (loads complete in issue order): the x of up to
    // T steps for each tile (L2; XL: into LDS, two tokens per load,
    // otherwise this lane's token's 64 values per step into registers), then
    // the code words (HBM) and the scales, the scales first when the wave
    // holds two or more row groups (kScalesFirst).  Steps past the range read
    // zeros (or are not used); tokens past M read zeros through their tile's
    // descriptor.
    uint4 xv[TT][T][8];
    uint8_t* xs = smem + c * (T * TT * kStepTile);  // XL: this wave's x
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int s = s0 + t < s_end ? s0 + t : s0;  // in range
      if constexpr (XL) {
        // load n of a step-tile: tokens 2n + (lane >> 5); lane l stores chunk
        // (l & 31) ^ token (16 bytes) of its token at position l & 31, which
        // puts the 16 tokens of one later read in distinct banks
#pragma unroll
        for (int q = 0; q < TT; ++q)
#pragma unroll
          for (int n = 0; n < 8; ++n) {
            const int tok = 2 * n + (lane >> 5);
            const int ch = (lane & 31) ^ tok;
            const int off = (int)((tok * a.K + 256 * (int64_t)s + 8 * ch) * 2);
            load_b128_lds(xr[q], off, xs + (t * TT + q) * kStepTile + 1024 * n);
          }
      } else {
        const int xoff = (int)((i * a.K + 256 * (int64_t)s + 64 * G) * 2);
#pragma unroll
        for (int q = 0; q < TT; ++q)
#pragma unroll
          for (int k = 0; k < 8; ++k) xv[q][t][k] = load_b128(xr[q], xoff + 16 * k);
      }
    }
    if constexpr (XL) __builtin_amdgcn_sched_barrier(0);  // keeps the order the wait counts on
    uint4 w[T][U];
    uint16_t d[T][U][4];
    if constexpr (kScalesFirst) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int s = s0 + t;
        const bool ok = s < s_end;
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t so = ok ? (uint32_t)(((4 * G + r) * BK + s) * 2) : 0x7FFFFFF0u;
            d[t][u][r] = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rs[u], (int)so, 0, 0);
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int s = s0 + t;
      const bool ok = s < s_end;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t off = ok ? (uint32_t)(i * row_bytes + 64 * s + 16 * G) : 0x7FFFFFF0u;
        const v4u v = __builtin_bit_cast(
            v4u, __builtin_amdgcn_raw_buffer_load_b128(rc[u], (int)off, 0, kNonTemporal));
        w[t][u] = make_uint4(v.x, v.y, v.z, v.w);
      }
    }
    if constexpr (!kScalesFirst) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int s = s0 + t;
        const bool ok = s < s_end;
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t so = ok ? (uint32_t)(((4 * G + r) * BK + s) * 2) : 0x7FFFFFF0u;
            d[t][u][r] = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rs[u], (int)so, 0, 0);
          }
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < T; ++t) {
      if (s0 + t >= s_end) break;  // uniform
      uint4 bo[TT][8];
      float zt[TT], fsh[TT];
      bool any_sh[TT];
#pragma unroll
      for (int q = 0; q < TT; ++q) {
        uint32_t xw[32];
        if constexpr (XL) {
          // this step's x is in LDS once the loads issued after it are all
          // that is left in flight (its later steps, the codes, the scales).
          // The compiler also orders LDS reads after the LDS-bound loads (it
          // waits for all of them), so this is the bound, not the only guard.
          if (q == 0) wait_vm_at((T - 1 - t) * TT * 8 + 5 * T * U);
          const uint8_t* xl = xs + (t * TT + q) * kStepTile + 512 * i;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const uint4 e = *reinterpret_cast<const uint4*>(xl + 16 * ((8 * G + k) ^ i));
            xw[4 * k] = e.x; xw[4 * k + 1] = e.y; xw[4 * k + 2] = e.z; xw[4 * k + 3] = e.w;
          }
        } else {
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            xw[4 * k] = xv[q][t][k].x; xw[4 * k + 1] = xv[q][t][k].y;
            xw[4 * k + 2] = xv[q][t][k].z; xw[4 * k + 3] = xv[q][t][k].w;
          }
        }
        // block sums of x and x^2 (the four lanes of a token hold its block)
        float s0f = 0.0f, s1f = 0.0f, q0f = 0.0f, q1f = 0.0f;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          s0f = dot2(xw[2 * k], kOnesF16x2, s0f);
          s1f = dot2(xw[2 * k + 1], kOnesF16x2, s1f);
          q0f = dot2(xw[2 * k], xw[2 * k], q0f);
          q1f = dot2(xw[2 * k + 1], xw[2 * k + 1], q1f);
        }
        float bsum = s0f + s1f, bsq = q0f + q1f;
        bsum += __shfl_xor(bsum, 16, 64);
        bsq += __shfl_xor(bsq, 16, 64);
        bsum += __shfl_xor(bsum, 32, 64);
        bsq += __shfl_xor(bsq, 32, 64);
        const int sh = bsq < 65536.0f ? 0 : 6;  // not finite: 6
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t hb = (uint32_t)(21 - 2 * j - sh) << 10;  // binary16 2^(6-2j-sh)
          const half2v sc = __builtin_bit_cast(half2v, hb | (hb << 16));
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            uint32_t pr[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int e0 = 16 * g + 4 * h + j, e1 = e0 + 8;
              const uint32_t sel = ((e0 & 1) ? 0x0302u : 0x0100u) | ((e1 & 1) ? 0x07060000u : 0x05040000u);
              pr[g] = __builtin_amdgcn_perm(xw[e1 >> 1], xw[e0 >> 1], sel);
              pr[g] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, pr[g]) * sc);
            }
            bo[q][2 * j + h] = make_uint4(pr[0], pr[1], pr[2], pr[3]);
          }
        }
        zt[q] = -ldexpf(bsum, -18 - sh);
        any_sh[q] = __builtin_amdgcn_ballot_w64(sh != 0) != 0;  // wave-uniform
        fsh[q] = sh ? 64.0f : 1.0f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t v[4] = {w[t][u].x, w[t][u].y, w[t][u].z, w[t][u].w};
        uint32_t v8[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) v8[g] = v[g] >> 8;
        v4f D[TT];
#pragma unroll
        for (int q = 0; q < TT; ++q) D[q] = v4f{zt[q], zt[q], zt[q], zt[q]};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t mask = 0x00030003u << (2 * j);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t* src = h ? v8 : v;
            const uint4 av = make_uint4(src[0] & mask, src[1] & mask, src[2] & mask, src[3] & mask);
#pragma unroll
            for (int q = 0; q < TT; ++q)
              D[q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, av),
                                                            __builtin_bit_cast(v8h, bo[q][2 * j + h]),
                                                            D[q], 0, 0, 0);
          }
        }
#pragma unroll
        for (int q = 0; q < TT; ++q) {
          if (any_sh[q]) D[q] *= fsh[q];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[q][u][r] = __builtin_fmaf(half_to_float(d[t][u][r]), D[q][r], acc[q][u][r]);
        }
      }
    }
  }

  // chunk sums meet in LDS; wave 0 adds them in chunk order and stores
  if (C > 1) {
    if constexpr (XL) __syncthreads();  // all x reads done before the sums overwrite it
#pragma unroll
    for (int q = 0; q < TT; ++q)
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[c][q][u][r][lane] = acc[q][u][r];
    __syncthreads();
    if (c != 0) return;
#pragma unroll
    for (int q = 0; q < TT; ++q)
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float sum = red[0][q][u][r][lane];
          for (int cc = 1; cc < C; ++cc) sum += red[cc][q][u][r][lane];
          acc[q][u][r] = sum;
        }
  }
  // lane (G, i): rows 4G..4G+3 of each group, token (tt0 + q)*16 + i
#pragma unroll
  for (int q = 0; q < TT; ++q) {
    const int64_t tok = (int64_t)(tt0 + q) * kTok + i;
    if (tok >= a.M) continue;
    float* o = a.out + ((int64_t)split * a.M + tok) * a.N;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t gi = (int64_t)rset * U + u;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * G + r < valid[u]) o[gi * kTileRows16 + 4 * G + r] = ldexpf(acc[q][u][r], 18);
    }
  }
}

// y = sum over splits of the partials, in split order.
__global__ __launch_bounds__(256) void k_gemm_reduce(const float* __restrict__ part, int splits,
                                                     int64_t MN, float* __restrict__ y) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= MN) return;
  float s = part[id];
  for (int p = 1; p < splits; ++p) s += part[(int64_t)p * MN + id];
  y[id] = s;
}

GemmPlan plan_gemm(int64_t N, int64_t K, int64_t M) {
  GemmPlan p;
  p.U = 4;
  p.mt = (M + kTok - 1) / kTok;
  const int64_t steps = K / kBlock;
  const int64_t groups = (N + kTileRows16 - 1) / kTileRows16;
  int64_t rsets = (groups + p.U - 1) / p.U;
  // Two token tiles per wave (one decode of the weights for 32 tokens, one
  // step per load batch to bound the registers) once there are two tiles and
  // the matrix is large (>= 2^26 weights: the gate/up and down shapes).
  // Measured on MI355X: 16384x4096 at 64 tokens 41 -> 28 us, 4096x16384 at
  // 48 tokens 39 -> 29 us; smaller matrices lose more parallelism than they
  // save (256x4096 at 32 tokens 7.2 -> 9.2 us), so they keep one tile.
  p.TT = (p.mt >= 2 && rsets * steps >= 4096) ? 2 : 1;
  p.zt = (p.mt + p.TT - 1) / p.TT;
  // x through LDS once the tile holds enough tokens for the scattered
  // per-lane loads to stall (measured on MI355X, same box: 16384x4096 at 16
  // tokens 12.2 -> 10.1 us, 4096x16384 at 16 14.6 -> 12.9, at 4 tokens
  // 10.2 -> 9.6 and 12.6 -> 12.3; 4096x4096 and 256x4096 lose 0.1-0.3 us
  // at up to 8 tokens, and every shape loses at 1-2 tokens).  Two-tile waves
  // (more than 16 tokens) always take it.
  p.xl = M > 8 || (M >= 4 && rsets * steps >= 4096);
  // Row groups per wave: below 64 steps (K < 16384), with one token tile
  // per wave, the most of 4, 2, 1 that still leaves more row sets than half
  // the CUs, where K is then not split: the split's partials and second
  // launch cost more than decoding each step's x for fewer rows (measured
  // on MI355X, same box: 4096x4096 at 5/16/32 tokens 7.56/8.10/9.20 ->
  // 5.23/5.86/6.94 us with 1; 4608x4096 at 8 tokens 8.81 -> 7.50 with 2;
  // 4096x12288 at 8 tokens 19.7 -> 12.3; 256x4096 at 16 tokens 7.84 ->
  // 6.50 with 1 and the split kept; no case slower).  At 64 steps and more
  // each CU would decode 4x the x steps for the same rows: 4096x16384 at
  // 16 tokens 12.4 us with 4 row groups, 13.1 with 2, 15.0 with 1.
  if (p.TT == 1 && steps < 64) {
    for (int u = 4; u >= 1; u /= 2) {
      p.U = u;
      rsets = (groups + u - 1) / u;
      if (2 * rsets * p.zt > device_cus()) break;
    }
  }
  // Measured on MI355X: when the row sets alone fill the CUs, or K is long
  // (>= 8192), 8 chunk-waves per workgroup with 2 steps per load batch;
  // otherwise (few rows, short K: K is split across workgroups anyway) 4
  // chunk-waves with 1 step per batch, which keeps each wave's
  // load-then-compute chain short.
  //
  // K splits (each adds its partials to the workspace traffic and needs the
  // reduce launch) double while the workgroups still fit one per CU and
  // every wave keeps at least T steps.  Measured on MI355X, same box: the
  // former rule (double until 8 waves per CU) split 16384x4096 at 17-32
  // tokens into 512 workgroups, 15.8-17.6 us against 13.9-14.1 unsplit;
  // 4096x16384 at 17-32 tokens 18.8-19.3 (512) against 16.6-17.6 (256);
  // 4096x4096 at 48 tokens 11.5 (768) against 9.6 (192).  Below one
  // workgroup per CU splitting pays: 4096x16384 at 16 tokens 24.6 us
  // unsplit, 17.2 at 2 splits, 11.9 at 4.
  const bool wide = rsets * p.zt >= device_cus() || steps >= 32;
  p.T = (wide && p.TT == 1) ? 2 : 1;
  p.S = (wide && steps >= 16 && p.TT == 1) ? 8 : 4;  // two tiles: 4 waves (registers)
  const int64_t per_split = (int64_t)p.S * p.T;
  int64_t max_splits = steps / per_split;
  if (max_splits < 1) max_splits = 1;
  int64_t splits = 1;
  while (splits * 2 <= max_splits && rsets * p.zt * splits * 2 <= device_cus()) splits *= 2;
  int64_t sps = (steps + splits - 1) / splits;
  sps = (sps + per_split - 1) / per_split * per_split;
  p.splits = (steps + sps - 1) / sps;
  p.steps_per_split = sps;
  p.wgs = rsets;
  p.part_bytes = p.splits > 1 ? p.splits * M * N * 4 : 0;
  return p;
}

// 2 to 4 tokens with K of 1, 2 or 4 chunks take the one-pass VALU matvec
// (k_gemv_f16m) while its activation staging stays within 32 MiB: the
// weights are then decoded once for the few tokens, where the matrix-core
// tile computes 16 tokens whatever M is (9.1-9.7 us at 16384x4096 for 2 to
// 16 tokens).
constexpr int64_t kValuTokens = 4;
constexpr int64_t kValuStagingBytes = (int64_t)32 << 20;
static bool gemm_on_valu(int64_t N, int64_t K, int64_t M) {
  const int64_t c = chunks_of(K);
  return M >= 2 && M <= kValuTokens && (c == 1 || c == 2 || c == 4) &&
         f16m_staging_bytes(N, K, M) <= kValuStagingBytes;
}

// One token tile per wave, U row groups: the instantiation for the plan's
// steps per load batch, chunk-waves and x path.
template <int U>
static void launch_gemm_tile(const GemmPlan& p, dim3 grid, hipStream_t st, const GemmArgs& a) {
  if (p.T == 2 && p.S == 8 && p.xl)
    hipLaunchKernelGGL((k_gemm_mfma<U, 2, 8, 1, true>), grid, dim3(64 * 8), 0, st, a);
  else if (p.T == 2 && p.S == 8)
    hipLaunchKernelGGL((k_gemm_mfma<U, 2, 8, 1, false>), grid, dim3(64 * 8), 0, st, a);
  else if (p.T == 2 && p.xl)
    hipLaunchKernelGGL((k_gemm_mfma<U, 2, 4, 1, true>), grid, dim3(64 * 4), 0, st, a);
  else if (p.T == 2)
    hipLaunchKernelGGL((k_gemm_mfma<U, 2, 4, 1, false>), grid, dim3(64 * 4), 0, st, a);
  else if (p.xl)
    hipLaunchKernelGGL((k_gemm_mfma<U, 1, 4, 1, true>), grid, dim3(64 * 4), 0, st, a);
  else
    hipLaunchKernelGGL((k_gemm_mfma<U, 1, 4, 1, false>), grid, dim3(64 * 4), 0, st, a);
}

size_t gemm_workspace_bytes(int64_t N, int64_t K, int64_t M) {
  if (M == 1 || gemm_on_valu(N, K, M)) return 0;  // the matvec kernels (see launch_gemm)
  const GemmPlan p = plan_gemm(N, K, M);
  return (size_t)p.part_bytes;
}

hipError_t launch_gemm(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K,
                       const uint16_t* x, int64_t M, float* y, void* ws, hipStream_t st) {
  if (M == 1) {
    // one token: the VALU matvec, which streams the weights without the
    // matrix-core tile's per-step x staging (measured on MI355X: 16384x4096
    // one token 9.4-9.6 us through k_gemm_mfma, 5.2-5.3 us through
    // k_gemv_f16)
    MatSet m{};
    m.codes[0] = codes;
    m.scales[0] = scales;
    m.nmat = 1;
    m.rows = (int32_t)N;
    return launch_gemv_f16(m, K, x, y, st);
  }
  if (gemm_on_valu(N, K, M)) {
    MatSet m{};
    m.codes[0] = codes;
    m.scales[0] = scales;
    m.nmat = 1;
    m.rows = (int32_t)N;
    if (M == 2) return launch_gemv_f16m<2>(m, K, x, y, st);
    if (M == 3) return launch_gemv_f16m<3>(m, K, x, y, st);
    return launch_gemv_f16m<4>(m, K, x, y, st);
  }
  const GemmPlan p = plan_gemm(N, K, M);
  float* part = static_cast<float*>(ws);
  GemmArgs a;
  a.codes = codes;
  a.scales = scales;
  a.x = x;
  a.out = p.splits > 1 ? part : y;
  a.N = N;
  a.K = K;
  a.M = M;
  a.steps_per_split = (int32_t)p.steps_per_split;
  const dim3 grid((unsigned)p.wgs, (unsigned)p.splits, (unsigned)p.zt);
  if (p.TT == 2)  // implies xl and 4 row groups
    hipLaunchKernelGGL((k_gemm_mfma<4, 1, 4, 2, true>), grid, dim3(64 * 4), 0, st, a);
  else if (p.U == 4)
    launch_gemm_tile<4>(p, grid, st, a);
  else if (p.U == 2)
    launch_gemm_tile<2>(p, grid, st, a);
  else
    launch_gemm_tile<1>(p, grid, st, a);
  if (p.splits > 1) {
    const int64_t MN = M * N;
    hipLaunchKernelGGL(k_gemm_reduce, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, st, part,
                       (int)p.splits, MN, y);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------ int8 path
// Static int8 activation quantization (page "gemma4 wNa8o8 requires int8
// activations"): x_q = clamp(rint(x / s), -128, 127) with x/s one IEEE fp32
// division and ties to even.
//
// Fast exact evaluation: with rs = RN(1/s) and v = RN(x * rs), v lies within
// 3u|x/s| of RN(x/s) (u = 2^-24).  rint only changes value at half-integers,
// so when |v| is farther than 8u|v| from the nearest half-integer, rint(v)
// equals rint(RN(x/s)); otherwise (near a tie, or v not finite) the IEEE
// division is evaluated.  Saturation at +-127.5/-128.5 gives the same clamped
// value on either side, so it needs no special case.
__device__ __forceinline__ int quantize_one(uint16_t xh, float s, float rs) {
  const float xf = half_to_float(xh);
  const float v = xf * rs;
  const float a = fabsf(v);
  const float frac = a - floorf(a);  // exact: Sterbenz, or a < 1
  float r;
  if (fabsf(frac - 0.5f) > a * 0x1p-21f) r = __builtin_rintf(v);
  else r = __builtin_rintf(xf / s);
  if (__builtin_isnan(r)) r = 0.0f;
  r = fminf(fmaxf(r, -128.0f), 127.0f);
  return (int)r;
}

// The same rule split for bulk use: the fast part gives the code and whether
// it can be trusted (near = too close to a half-integer, or v not finite);
// the exact part is the IEEE division, taken for `near` values only.
// v = RN(x * rs) is clamped first, c = clamp(v) in [-128, 127]: beyond 127
// (below -128) both sides of a tie clamp to the same code, so clamped values
// never need the division.  c + 1.5*2^23 rounds c to an integer (ties to
// even) in the low mantissa bits, so the low byte of that float is x_q (two's
// complement), and subtracting 1.5*2^23 again gives r = rint(c) exactly.
// t = c - r is exact with |t| <= 1/2, and c (when not clamped) is farther
// than 8u|c| (u = 2^-24) from every half-integer exactly when
// |t| + |c| 2^-21 < 1/2.  The test uses |v| for the margin, so NaN, the
// infinities and |v| >= 2^20 also land on the exact path.
__device__ __forceinline__ uint32_t quantize_fast_bits(uint16_t xh, float rs, bool& near) {
  const float v = __builtin_fmaf(half_to_float(xh), rs, 0.0f);  // RN(x * rs)
  const float c = __builtin_amdgcn_fmed3f(v, -128.0f, 127.0f);
  const float m = c + 0x1.8p23f;
  const float t = c - (m - 0x1.8p23f);
  near = !(__builtin_fmaf(fabsf(v), 0x1p-21f, fabsf(t)) < 0.5f);
  return __builtin_bit_cast(uint32_t, m);
}

__device__ __forceinline__ int quantize_exact(uint16_t xh, float s) {
  float r = __builtin_rintf(half_to_float(xh) / s);
  if (__builtin_isnan(r)) r = 0.0f;
  return (int)fminf(fmaxf(r, -128.0f), 127.0f);
}

__global__ __launch_bounds__(256) void k_quantize_i8(const uint16_t* __restrict__ x, int64_t K,
                                                     float s, int8_t* __restrict__ xq) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const float rs = 1.0f / s;
  if (k < K) xq[k] = (int8_t)quantize_one(x[k], s, rs);
}

hipError_t launch_quantize_i8(const uint16_t* x, int64_t K, float scale, int8_t* xq,
                              hipStream_t s) {
  hipLaunchKernelGGL(k_quantize_i8, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, s,
                     x, K, scale, xq);
  return hipGetLastError();
}

// Exact lane partial sum_{64 weights} x_q (q-1), from one 16-byte code load.
// xq[4g+j] holds bytes (x_q[16g+j], x_q[16g+4+j], x_q[16g+8+j], x_q[16g+12+j]),
// the order in which (v >> 2j) & 0x03030303 lays out a code word's fields.
__device__ __forceinline__ int lane_dot_i8(const uint4 w, const uint32_t (&xq)[16], int seed) {
  int a = seed, b = 0, c = 0;
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t v = ws[g];
    a = dot4(xq[4 * g + 0], v & 0x03030303u, a);
    b = dot4(xq[4 * g + 1], v & 0x0C0C0C0Cu, b);
    c = dot4(xq[4 * g + 2], v & 0x30303030u, c);
    a = dot4(xq[4 * g + 3], (v >> 6) & 0x03030303u, a);
  }
  // b and c carry the factors 4 and 16 of their field positions (exact shifts)
  return a + (b >> 2) + (c >> 4);
}

// (d * 2^24) * P as an exact int64, from the binary16 bits of d.
__device__ __forceinline__ int64_t scaled_partial(uint16_t h, int P) {
  const int e = (h >> 10) & 31;
  const int f = h & 1023;
  const int m = e ? (f | 1024) : f;
  const int sh = e ? e - 1 : 0;
  // |m| < 2^11 and |P| <= 2^13: both fit 24-bit operands, which the sign
  // extension makes visible to the compiler (one v_mul_i32_i24 instead of a
  // quarter-rate 32-bit multiply); the product is exact
  const int P24 = (int)((uint32_t)P << 8) >> 8;
  int t = m * P24;
  if (h & 0x8000) t = -t;
  // times 2^sh as a multiply (a left shift of a negative value is undefined
  // in C++17); |t| 2^sh < 2^40, so it cannot overflow, and it compiles to
  // the same 64-bit shift
  return (int64_t)t * ((int64_t)1 << sh);
}

// ---- the same transposed reduction for exact int64 sums ----
__device__ __forceinline__ void swap32_i64(int64_t& a, int64_t& b) {
  const auto lo = __builtin_amdgcn_permlane32_swap((unsigned)a, (unsigned)b, false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap((unsigned)((uint64_t)a >> 32),
                                                   (unsigned)((uint64_t)b >> 32), false, false);
  a = (int64_t)(((uint64_t)(unsigned)hi[0] << 32) | (unsigned)lo[0]);
  b = (int64_t)(((uint64_t)(unsigned)hi[1] << 32) | (unsigned)lo[1]);
}

__device__ __forceinline__ void swap16_i64(int64_t& a, int64_t& b) {
  const auto lo = __builtin_amdgcn_permlane16_swap((unsigned)a, (unsigned)b, false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap((unsigned)((uint64_t)a >> 32),
                                                   (unsigned)((uint64_t)b >> 32), false, false);
  a = (int64_t)(((uint64_t)(unsigned)hi[0] << 32) | (unsigned)lo[0]);
  b = (int64_t)(((uint64_t)(unsigned)hi[1] << 32) | (unsigned)lo[1]);
}

template <int CTRL>
__device__ __forceinline__ int64_t dpp_i64(int64_t v) {
  const unsigned lo = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)v, CTRL, 0xF, 0xF, false);
  const unsigned hi = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)((uint64_t)v >> 32), CTRL,
                                                            0xF, 0xF, false);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int64_t row16_sum_i64(int64_t v) {
  v += dpp_i64<0x128>(v);
  v += dpp_i64<0x124>(v);
  v += dpp_i64<0x122>(v);
  v += dpp_i64<0x121>(v);
  return v;
}

template <int R>
__device__ __forceinline__ void reduce_rows_i64(int64_t (&v)[R], int64_t (&out)[kOut<R>]) {
  static_assert(R == 2 || R == 4 || R == 8 || R == 16, "R must be 2, 4, 8 or 16");
  constexpr int H = R / 2;
#pragma unroll
  for (int i = 0; i < H; ++i) {
    int64_t a = v[i], b = v[i + H];
    swap32_i64(a, b);
    v[i] = a + b;
  }
  if constexpr (R == 2) {
    int64_t a = v[0], b = v[0];
    swap16_i64(a, b);
    out[0] = row16_sum_i64(a + b);
  } else {
    constexpr int Q = R / 4;
#pragma unroll
    for (int i = 0; i < Q; ++i) {
      int64_t a = v[i], b = v[i + Q];
      swap16_i64(a, b);
      out[i] = row16_sum_i64(a + b);
    }
  }
}

// y = fl32(fl64(fl64(A) * s) * 2^-24); fl64(A) is formed as hi*2^32 + lo in
// one rounding.
__device__ __forceinline__ float i8_epilogue(int64_t A, float s) {
  const double hi = (double)(int32_t)((uint64_t)A >> 32);
  const double lo = (double)(uint32_t)((uint64_t)A & 0xFFFFFFFFu);
  const double a = hi * 4294967296.0 + lo;
  return (float)((a * (double)s) * 0x1p-24);
}

// LDS of the int8 matvec: x_q dwords [C][4][64] uint4, x_q group sums
// [C][64][4] int32, a sink uint4 for the stores of threads with no group to
// stage, cross-wave sums [C*S][R] int64.
__host__ __device__ inline size_t i8_lds_bytes(int C, int S, int R) {
  return (size_t)C * 4 * 64 * 16 + (size_t)C * 64 * 16 + 16 + (size_t)C * S * R * 8;
}

// Same work split as the fp16 matvec.  The workgroup quantizes the
// activations itself (QUANT: from fp16 x with scale s) or takes them
// pre-quantized, and stages them in LDS in the dword order of lane_dot_i8.
// Partials are exact and so is the cross-wave sum: the output does not depend
// on the reduction order at all.
// Output requantization (page "gemma4 wNa8o8 requires int8 activations",
// recipe paragraph): y_q = clamp(rint(y / s_out), -128, 127) from the exact
// fp32 y, one IEEE division; y_deq = y_q * s_out (fp32), when requested.
struct Requant {
  float s_out;
  int8_t* y_q;
  float* y_deq;  // nullable
};

__device__ __forceinline__ void store_i8(float* y, const Requant& rq, int64_t row, float v,
                                         bool requant) {
  if (!requant) {
    y[row] = v;
    return;
  }
  float r = __builtin_rintf(v / rq.s_out);
  if (__builtin_isnan(r)) r = 0.0f;
  r = fminf(fmaxf(r, -128.0f), 127.0f);
  rq.y_q[row] = (int8_t)(int)r;
  if (rq.y_deq) rq.y_deq[row] = r * rq.s_out;
}

template <int R, bool QUANT, bool PARTIALS, int CT, int MAXT, bool REQUANT = false>
__global__ __launch_bounds__(MAXT) void k_gemv_i8(MatSet ms, int64_t K,
                                                  const uint16_t* __restrict__ x,
                                                  const int8_t* __restrict__ xq_in, float s,
                                                  float rs, float* __restrict__ y,
                                                  int32_t* __restrict__ partials, Split sp,
                                                  Requant rq) {
  extern __shared__ uint4 lds[];
  const int C = CT ? CT : sp.C, S = sp.S;
  uint4* xs = lds;                                                // [C][4][64]
  int* gsum = reinterpret_cast<int*>(lds + C * 4 * 64);           // [C][64][4] group sums of x_q
  uint4* sink = lds + C * 4 * 64 + C * 64;                        // [1]
  int64_t* red = reinterpret_cast<int64_t*>(sink + 1);            // [C*S][R]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = __builtin_amdgcn_readfirstlane(wave / C);
  const int c = wave - slot * C;
  const int row0 = ((int)blockIdx.x * S + slot) * R;
  const int64_t k0 = (int64_t)c * kChunk + (int64_t)lane * kLaneK;
  const bool active = k0 < K;
  const int64_t kk = active ? k0 : 0;
  const int64_t row_bytes = K / 4;
  const int64_t BK = K / kBlock;
  const int ngroups = (int)(K / 16);

  // (1) loads: the activations first (XP groups of 16 per thread, clamped),
  //     then the first kRowWindow rows of weights; x stays first so that
  //     waiting for it does not wait for the weights (loads complete in
  //     issue order).
  constexpr int XP = f16_stage_passes(CT);
  uint4 xa[XP], xb[XP];
  // range-checked: groups past K load as zeros (and quantize to 0)
  const __amdgpu_buffer_rsrc_t xr =
      QUANT ? rsrc(x, (uint32_t)(K * 2)) : rsrc(xq_in, (uint32_t)K);
#pragma unroll
  for (int p = 0; p < XP; ++p) {
    const int m = tid + p * (int)blockDim.x;
    if (QUANT) {
      xa[p] = load_b128(xr, 32 * m);
      xb[p] = load_b128(xr, 32 * m + 16);
    } else {
      xa[p] = load_b128(xr, 16 * m);
      xb[p] = make_uint4(0, 0, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();  // x of every wave ahead of any weight request (see k_gemv_f16)
  __builtin_amdgcn_sched_barrier(0);
  uint4 w[R];
  uint16_t hs[R];
  load_rows<R>(ms, row0, kk, row_bytes, BK, w, hs, 0, kRowWindow<R>);
  __builtin_amdgcn_sched_barrier(0);

  // (2) stage: group m (weights 16m..16m+15) = group m % 4 of lane
  //     (m / 4) % 64 of chunk m / 256.  Every thread quantizes and stores;
  //     one without a group stores into the sink (no branch for the x
  //     loads to sink into).
#pragma unroll
  for (int p = 0; p < XP; ++p) {
    const int m = tid + p * (int)blockDim.x;
    const bool staged = m < ngroups;
    const uint4 a4 = xa[p], b4 = xb[p];
    // mb[e]: a float whose low byte is x_q of element e
    uint32_t mb[16];
    if (QUANT) {
      const uint32_t hw[8] = {a4.x, a4.y, a4.z, a4.w, b4.x, b4.y, b4.z, b4.w};
      // fast path for all 16; the IEEE division only for values near a tie,
      // behind a wave-uniform branch (almost never taken on real data: the
      // compiler would otherwise evaluate the division for every value)
      bool any_near = false;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint16_t h = (uint16_t)((e & 1) ? hw[e >> 1] >> 16 : hw[e >> 1] & 0xFFFFu);
        bool nr;
        mb[e] = quantize_fast_bits(h, rs, nr);
        any_near |= nr;
      }
      if (__builtin_amdgcn_ballot_w64(any_near)) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const uint16_t h = (uint16_t)((e & 1) ? hw[e >> 1] >> 16 : hw[e >> 1] & 0xFFFFu);
          bool nr;
          (void)quantize_fast_bits(h, rs, nr);
          if (nr) mb[e] = (uint32_t)quantize_exact(h, s) & 0xFFu;
        }
      }
    } else {
      const uint32_t bw[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
      for (int i = 0; i < 16; ++i) mb[i] = bw[i >> 2] >> (8 * (i & 3));
    }
    // dword j holds x_q of elements j, 4+j, 8+j, 12+j (low bytes, one permute
    // per pair and one for the halves)
    uint32_t dw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = __builtin_amdgcn_perm(mb[4 + j], mb[j], 0x0C0C0400u);
      const uint32_t hi = __builtin_amdgcn_perm(mb[12 + j], mb[8 + j], 0x04000C0Cu);
      dw[j] = lo | hi;
    }
    const int ch = m >> 8, ln = (m >> 2) & 63, gg = m & 3;
    *(staged ? xs + (ch * 4 + gg) * 64 + ln : sink) = make_uint4(dw[0], dw[1], dw[2], dw[3]);
    int gs = dot4(dw[0], 0x01010101u, 0);
    gs = dot4(dw[1], 0x01010101u, gs);
    gs = dot4(dw[2], 0x01010101u, gs);
    gs = dot4(dw[3], 0x01010101u, gs);
    *(staged ? gsum + (ch * 64 + ln) * 4 + gg : reinterpret_cast<int*>(sink)) = gs;
  }
  __syncthreads();

  // (3) this lane's activations and seed -(sum of its 64 x_q), from the
  //     four group sums its stagers wrote
  uint32_t xq[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 tt = xs[(c * 4 + i) * 64 + lane];
    xq[4 * i + 0] = tt.x; xq[4 * i + 1] = tt.y; xq[4 * i + 2] = tt.z; xq[4 * i + 3] = tt.w;
  }
  const int4 gs4 = reinterpret_cast<const int4*>(gsum)[c * 64 + lane];
  const int seed = -((gs4.x + gs4.y) + (gs4.z + gs4.w));
  if constexpr (kRowWindow<R> < R) {  // the rest of the rows, in one burst
    __builtin_amdgcn_sched_barrier(0);
    load_rows<R>(ms, row0, kk, row_bytes, BK, w, hs, kRowWindow<R>, R);
    __builtin_amdgcn_sched_barrier(0);
  }

  int64_t acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int P = lane_dot_i8(w[r], xq, seed);
    const uint32_t keep = (row0 + r < ms.rows ? 0xFFFFu : 0u) & (0u - (uint32_t)active);
    acc[r] = scaled_partial((uint16_t)(hs[r] & keep), P);
    if (PARTIALS) {
      // a 256-block spans lanes 4i..4i+3 of this chunk
      int bp = P + __shfl_xor(P, 1, 64);
      bp += __shfl_xor(bp, 2, 64);
      const int row = row0 + r;
      if (active && (lane & 3) == 0 && row < ms.rows) partials[(int64_t)row * BK + k0 / kBlock] = bp;
    }
  }
  int64_t out[kOut<R>];
  reduce_rows_i64<R>(acc, out);
  const int rho = lane >> 4;
  if (C == 1) {
    if ((lane & 15) == 0) {
#pragma unroll
      for (int i = 0; i < kOut<R>; ++i) {
        const int rr = reduced_row<R>(i, rho);
        if (rr >= 0 && row0 + rr < ms.rows) store_i8(y, rq, row0 + rr, i8_epilogue(out[i], s), REQUANT);
      }
    }
    return;
  }
  if ((lane & 15) == 0) {
#pragma unroll
    for (int i = 0; i < kOut<R>; ++i) {
      const int rr = reduced_row<R>(i, rho);
      if (rr >= 0) red[wave * R + rr] = out[i];
    }
  }
  __syncthreads();
  if (c == 0 && lane < R) {
    int64_t tsum = red[wave * R + lane];
    for (int cc = 1; cc < C; ++cc) tsum += red[(wave + cc) * R + lane];
    if (row0 + lane < ms.rows) store_i8(y, rq, row0 + lane, i8_epilogue(tsum, s), REQUANT);
  }
}

// The int8 matvec for M = 2..4 tokens of pre-quantized activations (the
// small-M batched int8 matvec): k_gemv_i8's waves, rows, loads and order,
// with the M tokens' x_q staged side by side in LDS.  Each code word is
// masked once and then dotted with every token's x_q (the same v_dot4 sums
// as lane_dot_i8), so the weights are streamed and decoded once for all M
// tokens.  The sums are exact integers: every token's output equals
// tq2_gemv_i8q's bit for bit.  Output y[M][N].
template <int M>
__host__ __device__ inline size_t i8m_lds_bytes(int C, int S, int R) {
  return (size_t)M * ((size_t)C * 4 * 64 * 16 + (size_t)C * 64 * 16) + 16 + (size_t)M * C * S * R * 8;
}

template <int R, int M, int CT, int MAXT>
__global__ __launch_bounds__(MAXT) void k_gemv_i8m(MatSet ms, int64_t K, const int8_t* __restrict__ xq_in,
                                                   float s, float* __restrict__ y, Split sp) {
  extern __shared__ uint4 lds[];
  const int C = CT ? CT : sp.C, S = sp.S;
  uint4* xs = lds;                                                  // [M][C][4][64]
  int* gsum = reinterpret_cast<int*>(lds + M * C * 4 * 64);         // [M][C][64][4]
  uint4* sink = lds + M * C * 4 * 64 + M * C * 64;                  // [1]
  int64_t* red = reinterpret_cast<int64_t*>(sink + 1);              // [M][C*S][R]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = __builtin_amdgcn_readfirstlane(wave / C);
  const int c = wave - slot * C;
  const int row0 = ((int)blockIdx.x * S + slot) * R;
  const int64_t k0 = (int64_t)c * kChunk + (int64_t)lane * kLaneK;
  const bool active = k0 < K;
  const int64_t kk = active ? k0 : 0;
  const int64_t row_bytes = K / 4;
  const int64_t BK = K / kBlock;
  const int64_t N = ms.rows;
  const int ngroups = (int)(K / 16);

  // (1) loads: every token's x_q (16 bytes per group of 16, clamped), the
  //     workgroup barrier, then the first rows
  constexpr int XP = f16m_stage_passes(CT, MAXT);
  uint4 xa[M][XP];
#pragma unroll
  for (int t = 0; t < M; ++t) {
    const __amdgpu_buffer_rsrc_t xr = rsrc(xq_in + t * K, (uint32_t)K);
#pragma unroll
    for (int p = 0; p < XP; ++p) xa[t][p] = load_b128(xr, 16 * (tid + p * (int)blockDim.x));
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();  // x_q of every wave ahead of any weight request (see k_gemv_f16)
  __builtin_amdgcn_sched_barrier(0);
  uint4 w[R];
  uint16_t hs[R];
  load_rows<R>(ms, row0, kk, row_bytes, BK, w, hs, 0, kRowWindow<R>);
  __builtin_amdgcn_sched_barrier(0);

  // (2) stage every token as k_gemv_i8 stages its one
#pragma unroll
  for (int t = 0; t < M; ++t) {
#pragma unroll
    for (int p = 0; p < XP; ++p) {
      const int m = tid + p * (int)blockDim.x;
      const bool staged = m < ngroups;
      const uint32_t bw[4] = {xa[t][p].x, xa[t][p].y, xa[t][p].z, xa[t][p].w};
      uint32_t mb[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) mb[i] = bw[i >> 2] >> (8 * (i & 3));
      uint32_t dw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = __builtin_amdgcn_perm(mb[4 + j], mb[j], 0x0C0C0400u);
        const uint32_t hi = __builtin_amdgcn_perm(mb[12 + j], mb[8 + j], 0x04000C0Cu);
        dw[j] = lo | hi;
      }
      const int ch = m >> 8, ln = (m >> 2) & 63, gg = m & 3;
      *(staged ? xs + ((t * C + ch) * 4 + gg) * 64 + ln : sink) = make_uint4(dw[0], dw[1], dw[2], dw[3]);
      int gs = dot4(dw[0], 0x01010101u, 0);
      gs = dot4(dw[1], 0x01010101u, gs);
      gs = dot4(dw[2], 0x01010101u, gs);
      gs = dot4(dw[3], 0x01010101u, gs);
      *(staged ? gsum + ((t * C + ch) * 64 + ln) * 4 + gg : reinterpret_cast<int*>(sink)) = gs;
    }
  }
  __syncthreads();

  // (3) this lane's x_q and seed per token, then the rest of the rows
  uint32_t xq[M][16];
  int seed[M];
#pragma unroll
  for (int t = 0; t < M; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 tt = xs[((t * C + c) * 4 + i) * 64 + lane];
      xq[t][4 * i + 0] = tt.x; xq[t][4 * i + 1] = tt.y; xq[t][4 * i + 2] = tt.z; xq[t][4 * i + 3] = tt.w;
    }
    const int4 gs4 = reinterpret_cast<const int4*>(gsum)[(t * C + c) * 64 + lane];
    seed[t] = -((gs4.x + gs4.y) + (gs4.z + gs4.w));
  }
  if constexpr (kRowWindow<R> < R) {
    __builtin_amdgcn_sched_barrier(0);
    load_rows<R>(ms, row0, kk, row_bytes, BK, w, hs, kRowWindow<R>, R);
    __builtin_amdgcn_sched_barrier(0);
  }

  int64_t acc[M][R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t keep = (row0 + r < ms.rows ? 0xFFFFu : 0u) & (0u - (uint32_t)active);
    const uint16_t h = (uint16_t)(hs[r] & keep);
    // the fields of bit pairs 0..3 in bytes, once for all tokens (as lane_dot_i8)
    const uint32_t ws[4] = {w[r].x, w[r].y, w[r].z, w[r].w};
    uint32_t mk[4][4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      mk[g][0] = ws[g] & 0x03030303u;
      mk[g][1] = ws[g] & 0x0C0C0C0Cu;
      mk[g][2] = ws[g] & 0x30303030u;
      mk[g][3] = (ws[g] >> 6) & 0x03030303u;
    }
#pragma unroll
    for (int t = 0; t < M; ++t) {
      int a = seed[t], b = 0, cc = 0;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        a = dot4(xq[t][4 * g + 0], mk[g][0], a);
        b = dot4(xq[t][4 * g + 1], mk[g][1], b);
        cc = dot4(xq[t][4 * g + 2], mk[g][2], cc);
        a = dot4(xq[t][4 * g + 3], mk[g][3], a);
      }
      acc[t][r] = scaled_partial(h, a + (b >> 2) + (cc >> 4));
    }
    __builtin_amdgcn_sched_barrier(0);  // one row's masked words live at a time
  }
  const int rho = lane >> 4;
#pragma unroll
  for (int t = 0; t < M; ++t) {
    int64_t out[kOut<R>];
    reduce_rows_i64<R>(acc[t], out);
    if (C == 1) {
      if ((lane & 15) == 0) {
#pragma unroll
        for (int i = 0; i < kOut<R>; ++i) {
          const int rr = reduced_row<R>(i, rho);
          if (rr >= 0 && row0 + rr < ms.rows) y[t * N + row0 + rr] = i8_epilogue(out[i], s);
        }
      }
    } else if ((lane & 15) == 0) {
#pragma unroll
      for (int i = 0; i < kOut<R>; ++i) {
        const int rr = reduced_row<R>(i, rho);
        if (rr >= 0) red[(t * C * S + wave) * R + rr] = out[i];
      }
    }
  }
  if (C == 1) return;
  __syncthreads();
  if (c == 0 && lane < R) {
#pragma unroll
    for (int t = 0; t < M; ++t) {
      int64_t tsum = red[(t * C * S + wave) * R + lane];
      for (int cc = 1; cc < C; ++cc) tsum += red[(t * C * S + wave + cc) * R + lane];
      if (row0 + lane < ms.rows) y[t * N + row0 + lane] = i8_epilogue(tsum, s);
    }
  }
}

// Launch of k_gemv_i8m: 4 row groups per workgroup for K of 1 and 2 chunks,
// 2 for 4 chunks (512 threads), as k_gemv_f16m.
static Split i8m_split(int64_t K) {
  Split sp = pick_split(K, false);
  sp.S = sp.C == 4 ? 2 : 4;
  return sp;
}
static int i8m_rows_per_wave(int64_t rows, int64_t K, int64_t M) {
  return pick_rows_per_wave(rows, (int)chunks_of(K), 16, M == 2 ? 4 : 2);
}
// x_q bytes k_gemv_i8m stages over all its workgroups (each stages every token)
static int64_t i8m_staging_bytes(int64_t rows, int64_t K, int64_t M) {
  const int R = i8m_rows_per_wave(rows, K, M);
  const Split sp = i8m_split(K);
  const int64_t nwg = ((rows + R - 1) / R + sp.S - 1) / sp.S;
  return nwg * M * K;
}

template <int R, int M>
static hipError_t run_gemv_i8m(const MatSet& m, int64_t K, const int8_t* xq, float s, float* y, hipStream_t st) {
  const Split sp = i8m_split(K);
  if (sp.C != 1 && sp.C != 2 && sp.C != 4) return hipErrorInvalidConfiguration;
  const int64_t groups = (m.rows + R - 1) / R;
  const dim3 grid((unsigned)((groups + sp.S - 1) / sp.S));
  const size_t lds = i8m_lds_bytes<M>(sp.C, sp.S, R);
  const dim3 block(64 * sp.C * sp.S);
  // MAXT 512: the block is 512 threads for C = 2 and 4, 256 for C = 1
  if ((int64_t)f16m_stage_passes(sp.C, 512) * block.x < K / 16 || block.x > 512 || lds > 160 * 1024)
    return hipErrorInvalidConfiguration;
  auto go = [&](auto kfn) -> hipError_t {
    if (lds > 64 * 1024) {
      const hipError_t e = set_lds_cap(reinterpret_cast<const void*>(kfn));
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kfn, grid, block, lds, st, m, K, xq, s, y, sp);
    return hipGetLastError();
  };
  if (sp.C == 1) return go(k_gemv_i8m<R, M, 1, 512>);
  if (sp.C == 2) return go(k_gemv_i8m<R, M, 2, 512>);
  return go(k_gemv_i8m<R, M, 4, 512>);
}

template <int M>
static hipError_t launch_gemv_i8m(const MatSet& m, int64_t K, const int8_t* xq, float s, float* y, hipStream_t st) {
  if constexpr (M == 2)
    if (i8m_rows_per_wave(m.rows, K, M) == 4) return run_gemv_i8m<4, M>(m, K, xq, s, y, st);
  return run_gemv_i8m<2, M>(m, K, xq, s, y, st);
}

template <int R, bool QUANT, bool PARTIALS, bool REQUANT>
static hipError_t run_gemv_i8(const MatSet& m, int64_t K, const uint16_t* x, const int8_t* xq,
                              float s, float* y, int32_t* partials, const Requant& rq,
                              hipStream_t st) {
  Split sp = pick_split(K, false);
  const int64_t groups = (m.rows + R - 1) / R;
  if (sp.C == 1) {
    // 8 or 4 row groups per workgroup, whichever leaves fewer on the
    // busiest CU (8 on a tie).  Measured on MI355X, same box: q/k/v fused
    // (4608 rows, 288 workgroups of 8) 4.30 -> 3.92 us with 4; 256 rows
    // 3.04 -> 2.87; 4096 rows (256 workgroups of 8) 3.33 against 3.55.
    const int64_t cus = device_cus(), w8 = (groups + 7) / 8, w4 = (groups + 3) / 4;
    if ((w4 + cus - 1) / cus * 4 < (w8 + cus - 1) / cus * 8) sp.S = 4;
  }
  const int64_t grid = (groups + sp.S - 1) / sp.S;
  const size_t lds = i8_lds_bytes(sp.C, sp.S, R);
  const dim3 g((unsigned)grid), b(64 * sp.C * sp.S);
  const int ct = sp.C <= 4 && sp.C != 3 ? sp.C : 0;
  if ((int64_t)f16_stage_passes(ct) * b.x < K / 16) return hipErrorInvalidConfiguration;
  if (sp.C == 1)
    hipLaunchKernelGGL((k_gemv_i8<R, QUANT, PARTIALS, 1, 512, REQUANT>), g, b, lds, st, m, K, x, xq, s, 1.0f / s, y,
                       partials, sp, rq);
  else if (sp.C == 2)
    hipLaunchKernelGGL((k_gemv_i8<R, QUANT, PARTIALS, 2, 512, REQUANT>), g, b, lds, st, m, K, x, xq, s, 1.0f / s, y,
                       partials, sp, rq);
  else if (sp.C == 4)
    hipLaunchKernelGGL((k_gemv_i8<R, QUANT, PARTIALS, 4, 1024, REQUANT>), g, b, lds, st, m, K, x, xq, s, 1.0f / s,
                       y, partials, sp, rq);
  else if (b.x <= 512)
    hipLaunchKernelGGL((k_gemv_i8<R, QUANT, PARTIALS, 0, 512, REQUANT>), g, b, lds, st, m, K, x, xq, s, 1.0f / s, y,
                       partials, sp, rq);
  else
    hipLaunchKernelGGL((k_gemv_i8<R, QUANT, PARTIALS, 0, 1024, REQUANT>), g, b, lds, st, m, K, x, xq, s, 1.0f / s,
                       y, partials, sp, rq);
  return hipGetLastError();
}

template <int R>
static hipError_t run_gemv_i8_r(const MatSet& m, int64_t K, const uint16_t* x, const int8_t* xq,
                                float s, float* y, int32_t* partials, const Requant* rq,
                                hipStream_t st) {
  const Requant none = {1.0f, nullptr, nullptr};
  if (rq) return run_gemv_i8<R, true, false, true>(m, K, x, xq, s, y, partials, *rq, st);
  if (x) {
    if (partials) return run_gemv_i8<R, true, true, false>(m, K, x, xq, s, y, partials, none, st);
    return run_gemv_i8<R, true, false, false>(m, K, x, xq, s, y, partials, none, st);
  }
  if (partials) return run_gemv_i8<R, false, true, false>(m, K, x, xq, s, y, partials, none, st);
  return run_gemv_i8<R, false, false, false>(m, K, x, xq, s, y, partials, none, st);
}

hipError_t launch_gemv_i8(const MatSet& m, int64_t K, const uint16_t* x, const int8_t* xq,
                          float s, float* y, int32_t* partials, hipStream_t st) {
  switch (pick_rows_per_wave(m.rows, (int)chunks_of(K), 16, 8)) {
    case 8: return run_gemv_i8_r<8>(m, K, x, xq, s, y, partials, nullptr, st);
    case 4: return run_gemv_i8_r<4>(m, K, x, xq, s, y, partials, nullptr, st);
    default: return run_gemv_i8_r<2>(m, K, x, xq, s, y, partials, nullptr, st);
  }
}

hipError_t launch_gemv_i8_requant(const MatSet& m, int64_t K, const uint16_t* x, float s,
                                  float s_out, int8_t* y_q, float* y_deq, hipStream_t st) {
  const Requant rq = {s_out, y_q, y_deq};
  switch (pick_rows_per_wave(m.rows, (int)chunks_of(K), 16, 8)) {
    case 8: return run_gemv_i8_r<8>(m, K, x, nullptr, s, nullptr, nullptr, &rq, st);
    case 4: return run_gemv_i8_r<4>(m, K, x, nullptr, s, nullptr, nullptr, &rq, st);
    default: return run_gemv_i8_r<2>(m, K, x, nullptr, s, nullptr, nullptr, &rq, st);
  }
}

// ------------------------------------- small-M batched int8 matvec (MFMA)
//
// Y[M][N] for M tokens of int8 activations x_q sharing the scale s: per
// token the int8 matvec of tq2_gemv_i8q (page "gemma4 wNa8o8 requires int8
// activations", Implemented section), with each 256-block's exact sum
// P = sum_k x_q(k) (q(k) - 1) formed on the matrix cores
// (v_mfma_i32_16x16x64_i8: 16 rows x 16 tokens x 64 k, int32 exact), then
// the same exact A = sum_b (d_b 2^24) P_b in int64 and the same epilogue.
// Integer sums give the same A in any order, so every token's output equals
// tq2_gemv_i8q's bit for bit.
//
// Operands.  Lane (G = l/16, i = l%16) loads row i's 16 code bytes of block
// quarter G (codes k = 64G + 4b + f of the block in byte b, bit pair f).
// (v >> 2f) & 0x03030303 puts the 16 codes k = 64G + 4b + f (b = 0..15) in
// 16 bytes, the A operand of MFMA f; its B operand is token i's x_q at the
// same k: byte f of each of the lane's 16 x_q dwords, gathered by a 4 x 4
// byte transpose of every 4 dwords.  A and B put the same k in the same lane
// group and byte, so each MFMA sums the block's k = f mod 4 (the order inside
// the instruction is the hardware's and does not matter for integers).
// D: lane (G, i) gets rows 4G..4G+3 of token i.  The zero point sum_k x_q
// is the lane's 64 bytes (4 v_dot4 per 16) summed over its lane group.

struct GemmI8Args {
  const uint8_t* codes;
  const uint16_t* scales;
  const int8_t* xq;  // X_q[M][K]
  float s;
  float* y;          // y[M][N] (no split)
  int64_t* part;     // the split sums A [splits][M][N] (split K)
  int64_t N, K, M;
  int32_t steps_per_split;  // multiple of C*T
};

typedef int v4i __attribute__((ext_vector_type(4)));

// byte f of a, b, c, d as the dword {a_f, b_f, c_f, d_f}, for f = 0..3
__device__ __forceinline__ void transpose4x4_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d,
                                                   uint32_t (&o)[4]) {
  const uint32_t t0 = __builtin_amdgcn_perm(b, a, 0x05010400u);  // a0 b0 a1 b1
  const uint32_t t1 = __builtin_amdgcn_perm(b, a, 0x07030602u);  // a2 b2 a3 b3
  const uint32_t t2 = __builtin_amdgcn_perm(d, c, 0x05010400u);  // c0 d0 c1 d1
  const uint32_t t3 = __builtin_amdgcn_perm(d, c, 0x07030602u);  // c2 d2 c3 d3
  o[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
  o[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
  o[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  o[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

constexpr int kStepTileI8 = kTok * kBlock;  // x_q of one step for one tile: 4 KiB

// Workgroup: C waves, the C chunks of steps of one K-split of one row set
// (U row groups of 16) for one tile of 16 tokens; their int64 sums meet in
// LDS.  Grid: (row sets, K-splits, token tiles).
//
// x_q reaches the lanes one of two ways.  XL: straight to LDS, each load
// instruction bringing four tokens' 256 contiguous bytes of a step, token t's
// 16-byte chunk c stored at position c ^ t of its 256 bytes, so that the 16
// tokens of a later ds_read_b128 fall in distinct banks; then read back in
// operand order.  Otherwise each lane loads its own token's 64 bytes.
template <int U, int T, int C, bool XL>
__global__ __launch_bounds__(64 * C) void k_gemm_i8(GemmI8Args a) {
  constexpr bool kScalesFirst = kScalesFirstFor<U>;
  constexpr int kXBytes = XL ? C * T * kStepTileI8 : 0;
  constexpr int kRedBytes = C * U * 4 * 64 * 8;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kXBytes > kRedBytes ? kXBytes : kRedBytes];
  int64_t(*red)[U][4][64] = reinterpret_cast<int64_t(*)[U][4][64]>(smem);
  const int lane = threadIdx.x & 63;
  const int G = lane >> 4, i = lane & 15;
  const int c = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rset = blockIdx.x;
  const int split = blockIdx.y, tile = blockIdx.z;
  const int64_t row_bytes = a.K / 4, BK = a.K / kBlock;
  const int spw = a.steps_per_split / C;  // steps per wave
  const int s_begin = split * a.steps_per_split + c * spw;
  const int s_lim = s_begin + spw;
  const int s_end = (int64_t)s_lim < BK ? s_lim : (int)BK;

  // per row group: scalar descriptors over its valid rows (zeros past N)
  __amdgpu_buffer_rsrc_t rc[U], rs[U];
  int valid[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int gi = rset * U + u;
    int v = (int)(a.N - (int64_t)gi * kTileRows16);
    v = v < 0 ? 0 : (v > kTileRows16 ? kTileRows16 : v);
    v = __builtin_amdgcn_readfirstlane(v);
    valid[u] = v;
    const int64_t r0 = v > 0 ? (int64_t)gi * kTileRows16 : 0;
    rc[u] = rsrc(a.codes + r0 * row_bytes, (uint32_t)(v * row_bytes));
    rs[u] = rsrc(a.scales + r0 * BK, (uint32_t)(v * BK * 2));
  }
  // this tile's tokens (past M: zeros, nothing stored)
  int64_t tv = a.M - (int64_t)tile * kTok;
  tv = tv > kTok ? kTok : (tv < 0 ? 0 : tv);
  const __amdgpu_buffer_rsrc_t xr =
      rsrc(a.xq + (tv > 0 ? (int64_t)tile * kTok * a.K : 0), (uint32_t)(tv * a.K));

  int64_t acc[U][4];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[u][r] = 0;

  for (int s0 = s_begin; s0 < s_end; s0 += T) {
    // issue, in this order (loads complete in issue order): this lane's 64
    // x_q bytes of each step (L2), then the code words (HBM) and the scales,
    // ordered as in k_gemm_mfma (kScalesFirst)
    uint4 xv[T][4];
    uint8_t* xs = smem + c * (T * kStepTileI8);  // XL: this wave's x_q
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int s = s0 + t < s_end ? s0 + t : s0;  // in range
      if constexpr (XL) {
        // load n: tokens 4n + (lane >> 4); lane l stores chunk (l & 15) ^ token
        // of its token at position l & 15
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const int tk = 4 * n + (lane >> 4);
          const int ch = (lane & 15) ^ tk;
          const int off = (int)(tk * a.K + 256 * (int64_t)s + 16 * ch);
          load_b128_lds(xr, off, xs + t * kStepTileI8 + 1024 * n);
        }
      } else {
        const int xoff = (int)(i * a.K + 256 * (int64_t)s + 64 * G);
#pragma unroll
        for (int n = 0; n < 4; ++n) xv[t][n] = load_b128(xr, xoff + 16 * n);
      }
    }
    if constexpr (XL) __builtin_amdgcn_sched_barrier(0);  // keeps the order the wait counts on
    uint4 w[T][U];
    uint16_t d[T][U][4];
    if constexpr (kScalesFirst) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const bool ok = s0 + t < s_end;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t so = ok ? (uint32_t)(((4 * G + r) * BK + s0 + t) * 2) : 0x7FFFFFF0u;
            d[t][u][r] = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rs[u], (int)so, 0, 0);
          }
      }
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const bool ok = s0 + t < s_end;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t off = ok ? (uint32_t)(i * row_bytes + 64 * (s0 + t) + 16 * G) : 0x7FFFFFF0u;
        const v4u v = __builtin_bit_cast(
            v4u, __builtin_amdgcn_raw_buffer_load_b128(rc[u], (int)off, 0, kNonTemporal));
        w[t][u] = make_uint4(v.x, v.y, v.z, v.w);
      }
    }
    if constexpr (!kScalesFirst) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const bool ok = s0 + t < s_end;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t so = ok ? (uint32_t)(((4 * G + r) * BK + s0 + t) * 2) : 0x7FFFFFF0u;
            d[t][u][r] = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rs[u], (int)so, 0, 0);
          }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < T; ++t) {
      if (s0 + t >= s_end) break;  // uniform
      if constexpr (XL) {
        // this step's x_q is in LDS once the loads issued after it are all
        // that is left in flight (its later steps, the codes, the scales)
        wait_vm_at((T - 1 - t) * 4 + 5 * T * U);
        const uint8_t* xl = xs + t * kStepTileI8 + 256 * i;
#pragma unroll
        for (int k = 0; k < 4; ++k) xv[t][k] = *reinterpret_cast<const uint4*>(xl + 16 * ((4 * G + k) ^ i));
      }
      const uint32_t xw[16] = {xv[t][0].x, xv[t][0].y, xv[t][0].z, xv[t][0].w,
                               xv[t][1].x, xv[t][1].y, xv[t][1].z, xv[t][1].w,
                               xv[t][2].x, xv[t][2].y, xv[t][2].z, xv[t][2].w,
                               xv[t][3].x, xv[t][3].y, xv[t][3].z, xv[t][3].w};
      // B operands (one per bit pair f) and the block's sum of x_q for token i
      uint32_t bo[4][4];
      int zx = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t o[4];
        transpose4x4_bytes(xw[4 * e], xw[4 * e + 1], xw[4 * e + 2], xw[4 * e + 3], o);
#pragma unroll
        for (int f = 0; f < 4; ++f) bo[f][e] = o[f];
#pragma unroll
        for (int n = 0; n < 4; ++n) zx = dot4(xw[4 * e + n], 0x01010101u, zx);
      }
      zx += __shfl_xor(zx, 16, 64);
      zx += __shfl_xor(zx, 32, 64);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t v[4] = {w[t][u].x, w[t][u].y, w[t][u].z, w[t][u].w};
        v4i D = {0, 0, 0, 0};
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const v4i av = {(int)((v[0] >> (2 * f)) & 0x03030303u), (int)((v[1] >> (2 * f)) & 0x03030303u),
                          (int)((v[2] >> (2 * f)) & 0x03030303u), (int)((v[3] >> (2 * f)) & 0x03030303u)};
          const v4i bv = {(int)bo[f][0], (int)bo[f][1], (int)bo[f][2], (int)bo[f][3]};
          D = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, D, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[u][r] += scaled_partial(d[t][u][r], D[r] - zx);
      }
    }
  }

  // chunk sums meet in LDS (int64: exact in any order); wave 0 stores
  if (C > 1) {
    if constexpr (XL) __syncthreads();  // all x_q reads done before the sums overwrite it
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[c][u][r][lane] = acc[u][r];
    __syncthreads();
    if (c != 0) return;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // rolled: unrolled, every chunk's value would be loaded at once
        int64_t sum = red[0][u][r][lane];
#pragma unroll 1
        for (int cc = 1; cc < C; ++cc) sum += red[cc][u][r][lane];
        acc[u][r] = sum;
      }
  }
  // lane (G, i): rows 4G..4G+3 of each group, token tile*16 + i
  const int64_t tok = (int64_t)tile * kTok + i;
  if (tok >= a.M) return;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t gi = (int64_t)rset * U + u;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (4 * G + r >= valid[u]) continue;
      const int64_t n = gi * kTileRows16 + 4 * G + r;
      if (a.part) a.part[((int64_t)split * a.M + tok) * a.N + n] = acc[u][r];
      else a.y[tok * a.N + n] = i8_epilogue(acc[u][r], a.s);
    }
  }
}

// y = the epilogue of the sum over splits of the int64 partials
__global__ __launch_bounds__(256) void k_gemm_i8_reduce(const int64_t* __restrict__ part, int splits,
                                                        int64_t MN, float s, float* __restrict__ y) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= MN) return;
  int64_t A = part[id];
  for (int p = 1; p < splits; ++p) A += part[(int64_t)p * MN + id];
  y[id] = i8_epilogue(A, s);
}

GemmPlan plan_gemm_i8(int64_t N, int64_t K, int64_t M) {
  GemmPlan p;
  p.TT = 1;
  // x_q through LDS from 8 tokens (16384x4096 at 16 tokens 14.2 -> 13.7 us,
  // 4096x16384 15.6 -> 12.1; at 2 and 4 tokens the per-lane loads are
  // 0.05-0.3 us faster, at 8 they tie)
  p.xl = M >= 8;
  p.mt = (M + kTok - 1) / kTok;
  p.zt = p.mt;
  const int64_t steps = K / kBlock;
  const int64_t groups = (N + kTileRows16 - 1) / kTileRows16;
  // row groups per wave: the most of 4, 2, 1 that still gives two
  // workgroups per CU, then 4-wave workgroups; otherwise 1 row group and
  // 8-wave workgroups.  (Building a step's B operands costs ~50
  // instructions and a row group's decode ~30 per step, so fewer rows per
  // wave cost little; what counts is that each wave's work comes in more
  // than one load batch, so that its compute overlaps its later loads.)
  // Measured on MI355X, same box, against 4 row groups in 8-wave
  // workgroups: 16384x4096 at 8/16/32 tokens 13.4/13.7/20.9 ->
  // 9.7/10.4/15.7 us, 4608x4096 at 8 8.2 -> 7.1; 4096x16384 at 16 (1 row
  // group, 8 waves) 12.1 either way; 8-wave against 4-wave workgroups for
  // 4096x4096 at 4/8 tokens 5.57/5.78 against 5.90/5.92.
  int64_t rsets = groups;
  bool two = false;
  for (int u = 4; u >= 1; u /= 2) {
    p.U = u;
    rsets = (groups + u - 1) / u;
    if (rsets * p.zt >= 2 * device_cus()) {
      two = true;
      break;
    }
  }
  const bool wide = rsets * p.zt >= device_cus() || steps >= 32;
  p.T = wide ? 2 : 1;
  p.S = (!two && wide && steps >= 16) ? 8 : 4;
  const int64_t per_split = (int64_t)p.S * p.T;
  int64_t max_splits = steps / per_split;
  if (max_splits < 1) max_splits = 1;
  int64_t splits = 1;
  while (splits * 2 <= max_splits && rsets * p.zt * splits * 2 <= device_cus()) splits *= 2;
  int64_t sps = (steps + splits - 1) / splits;
  sps = (sps + per_split - 1) / per_split * per_split;
  p.splits = (steps + sps - 1) / sps;
  p.steps_per_split = sps;
  p.wgs = rsets;
  p.part_bytes = p.splits > 1 ? p.splits * M * N * 8 : 0;
  return p;
}

// 2 to 4 tokens with K of 1, 2 or 4 chunks take the one-pass int8 matvec
// (k_gemv_i8m) while its x_q staging stays within 24 MiB.  Measured on
// MI355X against the matrix cores (us): 4096x4096 at 2/3/4 tokens
// 5.44/5.52/5.56 -> 3.55/3.95/4.44, 256x4096 at 2 5.56 -> 2.82, 16384x4096
// at 2 and 3 (8 and 24 MiB) 9.05/9.09 -> 6.33/8.57, 4096x16384 at 2 10.46 ->
// 6.70; past the cap it loses: 16384x4096 at 4 (32 MiB) 10.1 against 9.2,
// 4096x16384 at 3 (48 MiB) 11.2 against 10.6.
constexpr int64_t kValuStagingBytesI8 = (int64_t)24 << 20;
static bool gemm_i8_on_valu(int64_t N, int64_t K, int64_t M) {
  const int64_t c = chunks_of(K);
  return M >= 2 && M <= kValuTokens && (c == 1 || c == 2 || c == 4) &&
         i8m_staging_bytes(N, K, M) <= kValuStagingBytesI8;
}

size_t gemm_i8_workspace_bytes(int64_t N, int64_t K, int64_t M) {
  if (M == 1 || gemm_i8_on_valu(N, K, M)) return 0;  // the matvec kernels (see launch_gemm_i8)
  return (size_t)plan_gemm_i8(N, K, M).part_bytes;
}

template <int U, bool XL>
static void launch_gemm_i8_tile(const GemmPlan& p, dim3 grid, hipStream_t st, const GemmI8Args& a) {
  if (p.T == 2 && p.S == 8)
    hipLaunchKernelGGL((k_gemm_i8<U, 2, 8, XL>), grid, dim3(64 * 8), 0, st, a);
  else if (p.T == 2)
    hipLaunchKernelGGL((k_gemm_i8<U, 2, 4, XL>), grid, dim3(64 * 4), 0, st, a);
  else
    hipLaunchKernelGGL((k_gemm_i8<U, 1, 4, XL>), grid, dim3(64 * 4), 0, st, a);
}
template <int U>
static void launch_gemm_i8_tile(const GemmPlan& p, dim3 grid, hipStream_t st, const GemmI8Args& a) {
  if (p.xl) launch_gemm_i8_tile<U, true>(p, grid, st, a);
  else launch_gemm_i8_tile<U, false>(p, grid, st, a);
}

hipError_t launch_gemm_i8(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K,
                          const int8_t* xq, int64_t M, float s, float* y, void* ws, hipStream_t st) {
  if (M == 1) {
    // one token: the int8 matvec kernel itself (its output, bit for bit)
    MatSet m{};
    m.codes[0] = codes;
    m.scales[0] = scales;
    m.nmat = 1;
    m.rows = (int32_t)N;
    return launch_gemv_i8(m, K, nullptr, xq, s, y, nullptr, st);
  }
  if (gemm_i8_on_valu(N, K, M)) {
    MatSet m{};
    m.codes[0] = codes;
    m.scales[0] = scales;
    m.nmat = 1;
    m.rows = (int32_t)N;
    if (M == 2) return launch_gemv_i8m<2>(m, K, xq, s, y, st);
    if (M == 3) return launch_gemv_i8m<3>(m, K, xq, s, y, st);
    return launch_gemv_i8m<4>(m, K, xq, s, y, st);
  }
  const GemmPlan p = plan_gemm_i8(N, K, M);
  GemmI8Args a;
  a.codes = codes;
  a.scales = scales;
  a.xq = xq;
  a.s = s;
  a.y = y;
  a.part = p.splits > 1 ? static_cast<int64_t*>(ws) : nullptr;
  a.N = N;
  a.K = K;
  a.M = M;
  a.steps_per_split = (int32_t)p.steps_per_split;
  const dim3 grid((unsigned)p.wgs, (unsigned)p.splits, (unsigned)p.zt);
  if (p.U == 4)
    launch_gemm_i8_tile<4>(p, grid, st, a);
  else if (p.U == 2)
    launch_gemm_i8_tile<2>(p, grid, st, a);
  else
    launch_gemm_i8_tile<1>(p, grid, st, a);
  if (p.splits > 1) {
    const int64_t MN = M * N;
    hipLaunchKernelGGL(k_gemm_i8_reduce, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, st, a.part,
                       (int)p.splits, MN, s, y);
  }
  return hipGetLastError();
}

// ------------------------------------------- static scratch (no allocation)
// For callers that cannot allocate (graph capture, serving loops that forbid
// hipMalloc): tq2_gemm's split partials live in this file-scope device array
// instead of a caller workspace.  Every GPU the library runs on holds its own
// copy, at its own address, until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory, so its device address is
// taken once per device with hipGetSymbolAddress (that device current) and
// only that address is passed to kernels.
static __device__ __align__(256) uint8_t scratch[kGemmScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t gemm_scratch(hipStream_t st, void** out) {
  int dev = -1;
  hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace tq2
