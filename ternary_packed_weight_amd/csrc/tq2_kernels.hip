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
// Work split: a wave owns one 4096-wide K-chunk c of R consecutive rows
// (lane l covers k = 4096c + 64l .. +63, a quarter of one 256-block).  A
// workgroup holds C chunk-waves for each of S row groups (C = ceil(K/4096),
// S = max(1, 4/C)), so a row's C partial sums meet in LDS and are added in
// chunk order: the result is deterministic.  Each wave first issues all its
// weight loads (R x 16 B per lane), then loads and rearranges its x chunk
// while they are in flight.
//
// Decode of one 32-bit code word v (16 weights; byte m holds local weights
// 4m+j at bits 2j):
//   v  & (0x00030003 << 2j) -> halves carry weight j (byte 0) and 8+j (byte 2)
//   v8 & (0x00030003 << 2j) -> halves carry weight 4+j and 12+j, v8 = v >> 8
// Each masked half is a binary16 subnormal equal to q * 4^j * 2^-24, exact.
// v_dot2_f32_f16 against the matching x pair gives sum x q * 4^j * 2^-24;
// four accumulators (one per j) are combined with the exact power-of-two
// weights 4^-j.  Subtracting the lane's x sum (folded into the seed) turns q
// into q-1.  The x pairs a lane needs are, per 16-weight group g,
//   pair[8g+2j+0] = (x[16g+j],   x[16g+8+j])
//   pair[8g+2j+1] = (x[16g+4+j], x[16g+12+j]).

constexpr uint32_t kOnesF16x2 = 0x3C003C00u;  // (1.0, 1.0)

// Rearrange a lane's 64 fp16 activations (natural order, 32 dwords) into the
// decode's operand pairs, and return -(sum of the 64 values) * 2^-24.
__device__ __forceinline__ float x_pairs_f16(const uint32_t (&xw)[32], uint32_t (&xp)[32]) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t a = xw[8 * g + (j >> 1)], b = xw[8 * g + 4 + (j >> 1)];
      const uint32_t c = xw[8 * g + 2 + (j >> 1)], d = xw[8 * g + 6 + (j >> 1)];
      if (j & 1) {
        xp[8 * g + 2 * j + 0] = (a >> 16) | (b & 0xFFFF0000u);
        xp[8 * g + 2 * j + 1] = (c >> 16) | (d & 0xFFFF0000u);
      } else {
        xp[8 * g + 2 * j + 0] = (a & 0xFFFFu) | (b << 16);
        xp[8 * g + 2 * j + 1] = (c & 0xFFFFu) | (d << 16);
      }
    }
  }
  float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; i += 4) {
    s0 = dot2(xw[i + 0], kOnesF16x2, s0);
    s1 = dot2(xw[i + 1], kOnesF16x2, s1);
    s2 = dot2(xw[i + 2], kOnesF16x2, s2);
    s3 = dot2(xw[i + 3], kOnesF16x2, s3);
  }
  return -ldexpf((s0 + s1) + (s2 + s3), -24);
}

// sum_{64 weights} x * q * 2^-24 + seed, i.e. (lane partial of x(q-1)) * 2^-24
__device__ __forceinline__ float lane_dot_f16(const uint4 w, const uint32_t (&xp)[32],
                                              float seed) {
  float a0 = seed, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t v = ws[g], v8 = v >> 8;
    a0 = dot2(xp[8 * g + 0], v & 0x00030003u, a0);
    a0 = dot2(xp[8 * g + 1], v8 & 0x00030003u, a0);
    a1 = dot2(xp[8 * g + 2], v & 0x000C000Cu, a1);
    a1 = dot2(xp[8 * g + 3], v8 & 0x000C000Cu, a1);
    a2 = dot2(xp[8 * g + 4], v & 0x00300030u, a2);
    a2 = dot2(xp[8 * g + 5], v8 & 0x00300030u, a2);
    a3 = dot2(xp[8 * g + 6], v & 0x00C000C0u, a3);
    a3 = dot2(xp[8 * g + 7], v8 & 0x00C000C0u, a3);
  }
  // field j sits 2j bits up, so accumulator j carries a factor 4^j: undo it
  return fmaf(a3, 0.015625f, fmaf(a2, 0.0625f, fmaf(a1, 0.25f, a0)));
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
__device__ __forceinline__ void reduce_rows_f32(float (&v)[R], float (&out)[R >= 4 ? R / 4 : 1]) {
  static_assert(R == 2 || R == 4 || R == 8, "R must be 2, 4 or 8");
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

template <int R>
__device__ __forceinline__ int reduced_row(int i, int rho) {
  if constexpr (R == 2) return rho >> 1;
  else return i + (rho & 1) * (R / 4) + (rho >> 1) * (R / 2);
}

// Row base pointers.  `row` is wave-uniform, and only constant indices into
// the kernel-argument arrays are used, so all of this stays in scalar
// registers: the weight loads do not wait on a pointer fetch.
struct RowPtr {
  const uint8_t* codes;
  const uint16_t* scales;
};

__device__ __forceinline__ RowPtr row_ptr(const MatSet& ms, int64_t row, int64_t row_bytes,
                                          int64_t BK) {
  int64_t lr = row;
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
  return RowPtr{c + lr * row_bytes, s + lr * BK};
}

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Weights are read exactly once: stream them past the caches.
__device__ __forceinline__ uint4 load_codes(const uint8_t* p) {
  const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

template <int R, int MAXT>
__global__ __launch_bounds__(MAXT) void k_gemv_f16(MatSet ms, int64_t K,
                                                   const uint16_t* __restrict__ x,
                                                   float* __restrict__ y, int C, int S) {
  __shared__ float red[16][R];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = wave % C;
  const int slot = wave / C;
  const int64_t row0 = ((int64_t)blockIdx.x * S + slot) * R;
  const int64_t k0 = (int64_t)c * kChunk + (int64_t)lane * kLaneK;
  const bool active = k0 < K;
  const int64_t row_bytes = K / 4;
  const int64_t BK = K / kBlock;

  // 1. every load is unconditional and in bounds (rows past the end read the
  //    last row, lanes past K read k = 0) so that nothing waits on a branch;
  //    those lanes and rows are zeroed afterwards through their scale.
  //    The activations are requested first: memory counters retire in
  //    order, so x can be rearranged while the weights are still in flight.
  const int64_t kk = active ? k0 : 0;
  uint32_t xw[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 t = *reinterpret_cast<const uint4*>(x + kk + 8 * i);
    xw[4 * i + 0] = t.x; xw[4 * i + 1] = t.y; xw[4 * i + 2] = t.z; xw[4 * i + 3] = t.w;
  }
  uint4 w[R];
  uint16_t hs[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = row0 + r < ms.rows ? row0 + r : ms.rows - 1;
    const RowPtr rp = row_ptr(ms, row, row_bytes, BK);
    w[r] = load_codes(rp.codes + kk / 4);
    hs[r] = rp.scales[kk / kBlock];
  }
  __builtin_amdgcn_sched_barrier(0);  // keep every load ahead of the math
  // 2. rearrange this lane's 64 activations into the decode's operand pairs
  uint32_t xp[32];
  const float seed = x_pairs_f16(xw, xp);
  // 3. decode, block partial times its scale
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    // binary16 +0 for padding lanes and rows, by masking the bits (a select
    // here would let the compiler sink the scale load into a branch)
    const uint32_t keep = 0u - (uint32_t)(active && row0 + r < ms.rows);
    const float d = half_to_float((uint16_t)(hs[r] & keep));
    acc[r] = d * lane_dot_f16(w[r], xp, seed);
  }
  // 4. reduce over the wave
  float out[R >= 4 ? R / 4 : 1];
  reduce_rows_f32<R>(acc, out);
  const int rho = lane >> 4;
  constexpr int NOUT = R >= 4 ? R / 4 : 1;
  if (C == 1) {
    if ((lane & 15) == 0) {
#pragma unroll
      for (int i = 0; i < NOUT; ++i) {
        const int64_t row = row0 + reduced_row<R>(i, rho);
        if (R != 2 || (rho & 1) == 0)
          if (row < ms.rows) y[row] = ldexpf(out[i], 24);
      }
    }
    return;
  }
  // 5. several chunk-waves per row: add their sums in chunk order
  if ((lane & 15) == 0) {
#pragma unroll
    for (int i = 0; i < NOUT; ++i)
      if (R != 2 || (rho & 1) == 0) red[wave][reduced_row<R>(i, rho)] = out[i];
  }
  __syncthreads();
  if (c == 0 && lane < R) {
    float t = red[wave][lane];
    for (int cc = 1; cc < C; ++cc) t += red[wave + cc][lane];
    const int64_t row = row0 + lane;
    if (row < ms.rows) y[row] = ldexpf(t, 24);
  }
}

static int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  return cus;
}

// Rows per wave: as many as keep at least ~8 waves per CU busy (all weight
// bytes are then in flight at once), at most 8.
static int pick_rows_per_wave(int64_t rows, int C) {
  const int64_t want_waves = (int64_t)device_cus() * 8;
  for (int R : {8, 4}) {
    if ((rows + R - 1) / R * C >= want_waves) return R;
  }
  return 2;
}

template <int R>
static hipError_t run_gemv_f16(const MatSet& m, int64_t K, const uint16_t* x, float* y,
                               hipStream_t s) {
  const int C = (int)chunks_of(K);
  const int S = C >= 4 ? 1 : 4 / C;
  const int64_t groups = (m.rows + R - 1) / R;
  const int64_t grid = (groups + S - 1) / S;
  if (C * S <= 4)
    hipLaunchKernelGGL((k_gemv_f16<R, 256>), dim3((unsigned)grid), dim3(64 * C * S), 0, s, m, K, x, y, C, S);
  else
    hipLaunchKernelGGL((k_gemv_f16<R, 1024>), dim3((unsigned)grid), dim3(64 * C * S), 0, s, m, K, x, y, C, S);
  return hipGetLastError();
}

hipError_t launch_gemv_f16(const MatSet& m, int64_t K, const uint16_t* x, float* y,
                           hipStream_t s) {
  switch (pick_rows_per_wave(m.rows, (int)chunks_of(K))) {
    case 8: return run_gemv_f16<8>(m, K, x, y, s);
    case 4: return run_gemv_f16<4>(m, K, x, y, s);
    default: return run_gemv_f16<2>(m, K, x, y, s);
  }
}

// ------------------------------------------------------------ int8 path
// Static int8 activation quantization (page "gemma4 wNa8o8 requires int8
// activations"): x_q = clamp(rint(x / s), -128, 127), x/s one IEEE fp32
// division (HIP's default division is correctly rounded), ties to even.

__device__ __forceinline__ int quantize_one(uint16_t xh, float s) {
  float r = __builtin_rintf(half_to_float(xh) / s);
  if (__builtin_isnan(r)) r = 0.0f;
  r = fminf(fmaxf(r, -128.0f), 127.0f);
  return (int)r;
}

__global__ __launch_bounds__(256) void k_quantize_i8(const uint16_t* __restrict__ x, int64_t K,
                                                     float s, int8_t* __restrict__ xq) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k < K) xq[k] = (int8_t)quantize_one(x[k], s);
}

hipError_t launch_quantize_i8(const uint16_t* x, int64_t K, float scale, int8_t* xq,
                              hipStream_t s) {
  hipLaunchKernelGGL(k_quantize_i8, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, s,
                     x, K, scale, xq);
  return hipGetLastError();
}

// Staged int8 activations for one lane-chunk (64 weights): 4 uint4 slots,
// slot g holding dwords j=0..3 = bytes (x_q[16g+j], x_q[16g+4+j],
// x_q[16g+8+j], x_q[16g+12+j]), the byte order that (v >> 2j) & 0x03030303
// produces from a code word; plus an int32 seed -(sum of the 64 x_q).
// Workspace layout: slots [chunks][4][64] uint4, then seeds [chunks][64].

__global__ __launch_bounds__(256) void k_i8_stage(const uint16_t* __restrict__ x,
                                                  const int8_t* __restrict__ xq_in,
                                                  int64_t K, float s, uint4* __restrict__ slots,
                                                  int32_t* __restrict__ seeds) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= K / kLaneK) return;
  const int64_t c = idx >> 6;
  const int lane = (int)(idx & 63);
  int v[64];
  if (x) {
    const uint4* src = reinterpret_cast<const uint4*>(x + idx * kLaneK);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 t = src[i];
      const uint32_t ww[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        v[8 * i + 2 * h] = quantize_one((uint16_t)(ww[h] & 0xFFFFu), s);
        v[8 * i + 2 * h + 1] = quantize_one((uint16_t)(ww[h] >> 16), s);
      }
    }
  } else {
    const uint4* src = reinterpret_cast<const uint4*>(xq_in + idx * kLaneK);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 t = src[i];
      const uint32_t ww[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int b = 0; b < 4; ++b) v[16 * i + 4 * h + b] = (int)(int8_t)((ww[h] >> (8 * b)) & 0xFFu);
    }
  }
  int sum = 0;
#pragma unroll
  for (int t = 0; t < 64; ++t) sum += v[t];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    uint32_t d[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      d[j] = ((uint32_t)(v[16 * g + j] & 0xFF)) | ((uint32_t)(v[16 * g + 4 + j] & 0xFF) << 8) |
             ((uint32_t)(v[16 * g + 8 + j] & 0xFF) << 16) | ((uint32_t)(v[16 * g + 12 + j] & 0xFF) << 24);
    slots[(c * 4 + g) * 64 + lane] = make_uint4(d[0], d[1], d[2], d[3]);
  }
  seeds[c * 64 + lane] = -sum;
}

hipError_t launch_i8_stage(const uint16_t* x, const int8_t* xq, int64_t K, float scale,
                           void* ws, hipStream_t s) {
  const int64_t chunks = chunks_of(K);
  uint4* slots = reinterpret_cast<uint4*>(ws);
  int32_t* seeds = reinterpret_cast<int32_t*>(slots + chunks * 4 * 64);
  const int64_t n = K / kLaneK;
  hipLaunchKernelGGL(k_i8_stage, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     x, xq, K, scale, slots, seeds);
  return hipGetLastError();
}

// Exact lane partial sum_{64 weights} x_q (q-1), from one 16-byte code load.
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
  int t = m * P;  // |m| < 2^11, |P| <= 2^13
  if (h & 0x8000) t = -t;
  return (int64_t)t << sh;
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
__device__ __forceinline__ void reduce_rows_i64(int64_t (&v)[R], int64_t (&out)[R >= 4 ? R / 4 : 1]) {
  static_assert(R == 2 || R == 4 || R == 8, "R must be 2, 4 or 8");
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

// Same work split as the fp16 matvec.  Activations come pre-arranged from the
// staging kernel (4 x 16 B + one seed per lane and chunk), so a wave needs no
// permutation.  Partials are exact, the cross-wave sum is exact, hence the
// output does not depend on the reduction order at all.
template <int R, bool PARTIALS, int MAXT>
__global__ __launch_bounds__(MAXT) void k_gemv_i8(MatSet ms, int64_t K,
                                                  const uint4* __restrict__ slots,
                                                  const int32_t* __restrict__ seeds, float s,
                                                  float* __restrict__ y,
                                                  int32_t* __restrict__ partials, int C, int S) {
  __shared__ int64_t red[16][R];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = wave % C;
  const int slot = wave / C;
  const int64_t row0 = ((int64_t)blockIdx.x * S + slot) * R;
  const int64_t k0 = (int64_t)c * kChunk + (int64_t)lane * kLaneK;
  const bool active = k0 < K;
  const int64_t row_bytes = K / 4;
  const int64_t BK = K / kBlock;

  // unconditional in-bounds loads, masked afterwards (see the fp16 matvec)
  const int64_t kk = active ? k0 : 0;
  uint32_t xq[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 t = slots[((int64_t)c * 4 + i) * 64 + lane];
    xq[4 * i + 0] = t.x; xq[4 * i + 1] = t.y; xq[4 * i + 2] = t.z; xq[4 * i + 3] = t.w;
  }
  const int seed = seeds[(int64_t)c * 64 + lane];
  uint4 w[R];
  uint16_t hs[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = row0 + r < ms.rows ? row0 + r : ms.rows - 1;
    const RowPtr rp = row_ptr(ms, row, row_bytes, BK);
    w[r] = load_codes(rp.codes + kk / 4);
    hs[r] = rp.scales[kk / kBlock];
  }
  __builtin_amdgcn_sched_barrier(0);  // keep every load ahead of the math

  int64_t acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int P = lane_dot_i8(w[r], xq, seed);
    const uint32_t keep = 0u - (uint32_t)(active && row0 + r < ms.rows);
    const uint16_t h = (uint16_t)(hs[r] & keep);
    acc[r] = scaled_partial(h, P);
    if (PARTIALS) {
      // a 256-block spans lanes 4i..4i+3 of this chunk
      int bp = P + __shfl_xor(P, 1, 64);
      bp += __shfl_xor(bp, 2, 64);
      const int64_t row = row0 + r;
      if (active && (lane & 3) == 0 && row < ms.rows) partials[row * BK + k0 / kBlock] = bp;
    }
  }
  int64_t out[R >= 4 ? R / 4 : 1];
  reduce_rows_i64<R>(acc, out);
  const int rho = lane >> 4;
  constexpr int NOUT = R >= 4 ? R / 4 : 1;
  if (C == 1) {
    if ((lane & 15) == 0) {
#pragma unroll
      for (int i = 0; i < NOUT; ++i) {
        const int64_t row = row0 + reduced_row<R>(i, rho);
        if (R != 2 || (rho & 1) == 0)
          if (row < ms.rows) y[row] = i8_epilogue(out[i], s);
      }
    }
    return;
  }
  if ((lane & 15) == 0) {
#pragma unroll
    for (int i = 0; i < NOUT; ++i)
      if (R != 2 || (rho & 1) == 0) red[wave][reduced_row<R>(i, rho)] = out[i];
  }
  __syncthreads();
  if (c == 0 && lane < R) {
    int64_t t = red[wave][lane];
    for (int cc = 1; cc < C; ++cc) t += red[wave + cc][lane];
    const int64_t row = row0 + lane;
    if (row < ms.rows) y[row] = i8_epilogue(t, s);
  }
}

template <int R, bool PARTIALS>
static hipError_t run_gemv_i8(const MatSet& m, int64_t K, const void* ws, float s, float* y,
                              int32_t* partials, hipStream_t st) {
  const int C = (int)chunks_of(K);
  const int S = C >= 4 ? 1 : 4 / C;
  const uint4* slots = reinterpret_cast<const uint4*>(ws);
  const int32_t* seeds = reinterpret_cast<const int32_t*>(slots + (int64_t)C * 4 * 64);
  const int64_t groups = (m.rows + R - 1) / R;
  const int64_t grid = (groups + S - 1) / S;
  if (C * S <= 4)
    hipLaunchKernelGGL((k_gemv_i8<R, PARTIALS, 256>), dim3((unsigned)grid), dim3(64 * C * S), 0, st,
                       m, K, slots, seeds, s, y, partials, C, S);
  else
    hipLaunchKernelGGL((k_gemv_i8<R, PARTIALS, 1024>), dim3((unsigned)grid), dim3(64 * C * S), 0, st,
                       m, K, slots, seeds, s, y, partials, C, S);
  return hipGetLastError();
}

hipError_t launch_gemv_i8(const MatSet& m, int64_t K, const void* ws, float scale, float* y,
                          int32_t* partials, hipStream_t s) {
  const int R = pick_rows_per_wave(m.rows, (int)chunks_of(K));
  if (partials) {
    if (R == 8) return run_gemv_i8<8, true>(m, K, ws, scale, y, partials, s);
    if (R == 4) return run_gemv_i8<4, true>(m, K, ws, scale, y, partials, s);
    return run_gemv_i8<2, true>(m, K, ws, scale, y, partials, s);
  }
  if (R == 8) return run_gemv_i8<8, false>(m, K, ws, scale, y, partials, s);
  if (R == 4) return run_gemv_i8<4, false>(m, K, ws, scale, y, partials, s);
  return run_gemv_i8<2, false>(m, K, ws, scale, y, partials, s);
}

}  // namespace tq2
