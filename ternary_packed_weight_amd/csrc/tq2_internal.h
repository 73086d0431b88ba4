// Internal launch interface between the C ABI (tq2_api.cpp) and the gfx950
// kernels (tq2_kernels.hip).  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tq2 {

constexpr int64_t kBlock = 256;    // weights per block, one fp16 scale each
constexpr int64_t kLaneK = 64;     // weights one lane decodes per 16-byte load
constexpr int64_t kChunk = 4096;   // weights one wave64 covers per step

__host__ __device__ inline int64_t chunks_of(int64_t K) { return (K + kChunk - 1) / kChunk; }

// Up to three weight matrices that share K and the activation vector; their
// outputs are concatenated in y (matrix m, row n -> y[row_begin[m] + n]).
// Row indices are 32-bit (the ABI limits the total row count to < 2^31), so
// every wave-uniform row test is a scalar compare.
struct MatSet {
  const uint8_t* codes[3];
  const uint16_t* scales[3];
  int32_t row_begin[3];
  int32_t nmat;
  int32_t rows;  // total rows over all matrices
};

hipError_t launch_pack(const float* W, int64_t N, int64_t K, uint8_t* codes,
                       uint16_t* scales, int32_t* bad, hipStream_t s);
hipError_t launch_dequant(const uint8_t* codes, const uint16_t* scales,
                          int64_t N, int64_t K, float* W, hipStream_t s);
hipError_t launch_gemv_f16(const MatSet& m, int64_t K, const uint16_t* x,
                           float* y, hipStream_t s);
hipError_t launch_quantize_i8(const uint16_t* x, int64_t K, float scale,
                              int8_t* xq, hipStream_t s);
// fp16 matvec over two matrices of m.row_begin[1] rows each (gate, up),
// writing h[n] = silu(gate_n) * up_n only.
hipError_t launch_gemv_silu_mul(const MatSet& m, int64_t K, const uint16_t* x,
                                float* h, hipStream_t s);
// int8 matvec; the activations come either as fp16 x (quantized inside the
// kernel with scale s) or pre-quantized as xq (exactly one is non-null).
hipError_t launch_gemv_i8(const MatSet& m, int64_t K, const uint16_t* x,
                          const int8_t* xq, float s, float* y, int32_t* partials,
                          hipStream_t st);
// int8 matvec from fp16 x, output requantized with s_out: y_q (int8) and,
// if y_deq is non-null, y_q * s_out (fp32).
hipError_t launch_gemv_i8_requant(const MatSet& m, int64_t K, const uint16_t* x,
                                  float s, float s_out, int8_t* y_q, float* y_deq,
                                  hipStream_t st);

// Small-M batched matvec Y[M][N] = X[M][K] W^T (matrix cores).  The
// workspace holds the split partials when K is split across workgroups
// (otherwise nothing); plan_gemm fixes the tiling.
struct GemmPlan {
  int U, T, S;                // row groups per wave, steps per load batch, chunk-waves per workgroup
  int TT;                     // token tiles per wave
  bool xl;                    // x staged through LDS (see k_gemm_mfma)
  int64_t mt, zt;             // 16-token tiles; groups of TT tiles (grid z)
  int64_t splits, steps_per_split, wgs;
  int64_t part_bytes;
};
GemmPlan plan_gemm(int64_t N, int64_t K, int64_t M);
GemmPlan plan_gemm_i8(int64_t N, int64_t K, int64_t M);
size_t gemm_i8_workspace_bytes(int64_t N, int64_t K, int64_t M);
hipError_t launch_gemm_i8(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K,
                          const int8_t* xq, int64_t M, float s, float* y, void* ws, hipStream_t st);
size_t gemm_workspace_bytes(int64_t N, int64_t K, int64_t M);
hipError_t launch_gemm(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K,
                       const uint16_t* x, int64_t M, float* y, void* ws, hipStream_t st);

// Device address of the library's static scratch array (kGemmScratchBytes,
// 256-byte aligned) on the device of `st` (the current device when st is
// null), looked up with hipGetSymbolAddress on first use per device.
constexpr size_t kGemmScratchBytes = (size_t)4 << 20;
hipError_t gemm_scratch(hipStream_t st, void** out);

}  // namespace tq2
