// C ABI of libtq2 (declared in include/tq2.h): argument validation, then
// launches on the caller's stream.  Every check happens before any launch.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "tq2.h"
#include "tq2_internal.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// [a, a+an) and [b, b+bn) intersect
bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return an && bn && x < y + bn && y < x + an;
}

int32_t check_shape(int64_t N, int64_t K, int64_t kmax) {
  if (N < 1) return TQ2_ERR_ARG;
  if (K < TQ2_BLOCK || K % TQ2_BLOCK != 0 || K > kmax) return TQ2_ERR_SHAPE;
  if (N > TQ2_MAX_ROWS || N > ((int64_t)1 << 40) / K) return TQ2_ERR_SHAPE;
  return TQ2_OK;
}

int32_t check_weights(const uint8_t* codes, const uint16_t* scales) {
  if (!codes || !scales) return TQ2_ERR_ARG;
  if (!aligned(codes, 16) || !aligned(scales, 2)) return TQ2_ERR_ALIGN;
  return TQ2_OK;
}

int32_t check_scale(float s) {
  return (isfinite(s) && s > 0.0f) ? TQ2_OK : TQ2_ERR_SCALE;
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? TQ2_OK : TQ2_ERR_HIP; }

#define TQ2_TRY(expr)              \
  do {                             \
    const int32_t st_ = (expr);    \
    if (st_ != TQ2_OK) return st_; \
  } while (0)

}  // namespace

extern "C" {

int32_t tq2_abi_version(void) { return TQ2_ABI_VERSION; }

const char* tq2_status_string(int32_t status) {
  switch (status) {
    case TQ2_OK: return "ok";
    case TQ2_ERR_ARG: return "invalid argument (null pointer, N < 1, unknown op or aliasing)";
    case TQ2_ERR_SHAPE: return "invalid shape (K must be a multiple of 256 within the limit)";
    case TQ2_ERR_ALIGN: return "misaligned pointer";
    case TQ2_ERR_WORKSPACE: return "workspace missing or too small";
    case TQ2_ERR_SCALE: return "activation scale must be finite and > 0";
    case TQ2_ERR_HIP: return "HIP launch failed";
    case TQ2_ERR_SCRATCH: return "split partials exceed the library's static scratch (TQ2_GEMM_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

size_t tq2_codes_bytes(int64_t N, int64_t K) {
  if (check_shape(N, K, TQ2_MAX_K) != TQ2_OK) return 0;
  return (size_t)(N * (K / 4));
}

size_t tq2_scales_bytes(int64_t N, int64_t K) {
  if (check_shape(N, K, TQ2_MAX_K) != TQ2_OK) return 0;
  return (size_t)(N * (K / TQ2_BLOCK) * 2);
}

size_t tq2_workspace_bytes(int32_t op, int64_t N, int64_t K) {
  switch (op) {
    case TQ2_OP_GEMV:
    case TQ2_OP_GATE_UP:
      return check_shape(N, K, TQ2_MAX_K) == TQ2_OK ? 0 : (size_t)-1;
    case TQ2_OP_GEMV_I8:
    case TQ2_OP_GEMV_I8Q:
      return check_shape(N, K, TQ2_I8_MAX_K) == TQ2_OK ? 0 : (size_t)-1;
    default:
      return (size_t)-1;
  }
}

int32_t tq2_pack(const float* W, int64_t N, int64_t K, uint8_t* codes, uint16_t* scales,
                 int32_t* bad_blocks, tq2_stream_t stream) {
  TQ2_TRY(check_shape(N, K, TQ2_MAX_K));
  if (!W) return TQ2_ERR_ARG;
  TQ2_TRY(check_weights(codes, scales));
  if (!aligned(W, 16) || (bad_blocks && !aligned(bad_blocks, 4))) return TQ2_ERR_ALIGN;
  const size_t wb = (size_t)(N * K) * 4, cb = (size_t)(N * K / 4), sb = (size_t)(N * K / 128);
  if (overlaps(W, wb, codes, cb) || overlaps(W, wb, scales, sb) || overlaps(codes, cb, scales, sb) ||
      (bad_blocks && (overlaps(bad_blocks, 4, W, wb) || overlaps(bad_blocks, 4, codes, cb) ||
                      overlaps(bad_blocks, 4, scales, sb))))
    return TQ2_ERR_ARG;
  (void)hipGetLastError();
  return hip_status(tq2::launch_pack(W, N, K, codes, scales, bad_blocks, (hipStream_t)stream));
}

int32_t tq2_dequant(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K, float* W,
                    tq2_stream_t stream) {
  TQ2_TRY(check_shape(N, K, TQ2_MAX_K));
  TQ2_TRY(check_weights(codes, scales));
  if (!W) return TQ2_ERR_ARG;
  if (!aligned(W, 16)) return TQ2_ERR_ALIGN;
  const size_t wb = (size_t)(N * K) * 4;
  if (overlaps(W, wb, codes, (size_t)(N * K / 4)) || overlaps(W, wb, scales, (size_t)(N * K / 128)))
    return TQ2_ERR_ARG;
  (void)hipGetLastError();
  return hip_status(tq2::launch_dequant(codes, scales, N, K, W, (hipStream_t)stream));
}

// Validate nmat (1..3) matrices of the same K and row counts N[i] sharing x,
// and describe them as one concatenated row space.
static int32_t build_matset(int nmat, const uint8_t* const* codes, const uint16_t* const* scales,
                            const int64_t* N, int64_t K, int64_t kmax, tq2::MatSet* m) {
  if (nmat < 1 || nmat > 3 || !codes || !scales || !N) return TQ2_ERR_ARG;
  int64_t total = 0;
  *m = tq2::MatSet{};
  for (int i = 0; i < nmat; ++i) {
    TQ2_TRY(check_shape(N[i], K, kmax));
    TQ2_TRY(check_weights(codes[i], scales[i]));
    m->codes[i] = codes[i];
    m->scales[i] = scales[i];
    m->row_begin[i] = (int32_t)total;
    total += N[i];
  }
  if (total > TQ2_MAX_ROWS) return TQ2_ERR_SHAPE;
  m->nmat = nmat;
  m->rows = (int32_t)total;
  return TQ2_OK;
}

// Outputs must not overlap any input of the call.
static bool output_clear(const void* out, size_t out_b, const tq2::MatSet& m, int64_t K,
                         const void* x, size_t x_b) {
  if (overlaps(out, out_b, x, x_b)) return false;
  for (int i = 0; i < m.nmat; ++i) {
    const int64_t n = (i + 1 < m.nmat ? m.row_begin[i + 1] : m.rows) - m.row_begin[i];
    if (overlaps(out, out_b, m.codes[i], (size_t)(n * K / 4)) ||
        overlaps(out, out_b, m.scales[i], (size_t)(n * K / 128)))
      return false;
  }
  return true;
}

static int32_t gemv_common(int nmat, const uint8_t* const* codes, const uint16_t* const* scales,
                           const int64_t* N, int64_t K, const uint16_t* x, float* y,
                           tq2_stream_t stream, bool silu_mul) {
  tq2::MatSet m;
  TQ2_TRY(build_matset(nmat, codes, scales, N, K, TQ2_MAX_K, &m));
  if (!x || !y) return TQ2_ERR_ARG;
  if (!aligned(x, 16) || !aligned(y, 4)) return TQ2_ERR_ALIGN;
  const size_t yb = (size_t)(silu_mul ? N[0] : m.rows) * 4;
  if (!output_clear(y, yb, m, K, x, (size_t)K * 2)) return TQ2_ERR_ARG;
  (void)hipGetLastError();
  if (silu_mul) return hip_status(tq2::launch_gemv_silu_mul(m, K, x, y, (hipStream_t)stream));
  return hip_status(tq2::launch_gemv_f16(m, K, x, y, (hipStream_t)stream));
}

int32_t tq2_gemv(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K,
                 const uint16_t* x, float* y, void* ws, size_t ws_bytes, tq2_stream_t stream) {
  (void)ws;
  (void)ws_bytes;
  return gemv_common(1, &codes, &scales, &N, K, x, y, stream, false);
}

int32_t tq2_gemv_gate_up(const uint8_t* codes_g, const uint16_t* scales_g, const uint8_t* codes_u,
                         const uint16_t* scales_u, int64_t N, int64_t K, const uint16_t* x,
                         float* y, void* ws, size_t ws_bytes, tq2_stream_t stream) {
  (void)ws;
  (void)ws_bytes;
  const uint8_t* c[2] = {codes_g, codes_u};
  const uint16_t* s[2] = {scales_g, scales_u};
  const int64_t n[2] = {N, N};
  return gemv_common(2, c, s, n, K, x, y, stream, false);
}

int32_t tq2_gemv_fused(int32_t nmat, const uint8_t* const* codes, const uint16_t* const* scales,
                       const int64_t* N, int64_t K, const uint16_t* x, float* y, void* ws,
                       size_t ws_bytes, tq2_stream_t stream) {
  (void)ws;
  (void)ws_bytes;
  return gemv_common(nmat, codes, scales, N, K, x, y, stream, false);
}

int32_t tq2_gemv_gate_up_silu(const uint8_t* codes_g, const uint16_t* scales_g,
                              const uint8_t* codes_u, const uint16_t* scales_u, int64_t N,
                              int64_t K, const uint16_t* x, float* h, void* ws, size_t ws_bytes,
                              tq2_stream_t stream) {
  (void)ws;
  (void)ws_bytes;
  const uint8_t* c[2] = {codes_g, codes_u};
  const uint16_t* s[2] = {scales_g, scales_u};
  const int64_t n[2] = {N, N};
  return gemv_common(2, c, s, n, K, x, h, stream, true);
}

int32_t tq2_quantize_i8(const uint16_t* x, int64_t K, float s, int8_t* x_q, tq2_stream_t stream) {
  // elementwise: any whole number of 256-blocks up to a full batch of tokens
  if (K < TQ2_BLOCK || K % TQ2_BLOCK != 0 || K > (int64_t)TQ2_MAX_TOKENS * TQ2_MAX_K) return TQ2_ERR_SHAPE;
  if (!x || !x_q) return TQ2_ERR_ARG;
  if (!aligned(x, 16) || !aligned(x_q, 16)) return TQ2_ERR_ALIGN;
  TQ2_TRY(check_scale(s));
  if (overlaps(x, (size_t)K * 2, x_q, (size_t)K)) return TQ2_ERR_ARG;
  (void)hipGetLastError();
  return hip_status(tq2::launch_quantize_i8(x, K, s, x_q, (hipStream_t)stream));
}

// int8 matvec over nmat matrices; activations are fp16 x (quantized with s
// in the kernel) or pre-quantized x_q; optional block partials (nmat == 1)
// or output requantization with s_out.
static int32_t i8_common(int nmat, const uint8_t* const* codes, const uint16_t* const* scales,
                         const int64_t* N, int64_t K, const uint16_t* x, const int8_t* x_q,
                         float s, float* y, int32_t* partials, const float* s_out,
                         int8_t* y_q, float* y_deq, tq2_stream_t stream) {
  tq2::MatSet m;
  TQ2_TRY(build_matset(nmat, codes, scales, N, K, TQ2_I8_MAX_K, &m));
  if (!x && !x_q) return TQ2_ERR_ARG;
  if (s_out ? !y_q : !y) return TQ2_ERR_ARG;
  if ((x && !aligned(x, 16)) || (x_q && !aligned(x_q, 16)) || (y && !aligned(y, 4)) ||
      (partials && !aligned(partials, 4)) || (y_deq && !aligned(y_deq, 4)))
    return TQ2_ERR_ALIGN;
  TQ2_TRY(check_scale(s));
  if (s_out) TQ2_TRY(check_scale(*s_out));
  const void* in_ptr = x ? (const void*)x : (const void*)x_q;
  const size_t in_b = x ? (size_t)K * 2 : (size_t)K;
  const size_t rows = (size_t)m.rows;
  const void* outs[4] = {y, partials, y_q, y_deq};
  const size_t outb[4] = {y ? rows * 4 : 0, partials ? (size_t)(m.rows * (K / 256)) * 4 : 0,
                          y_q ? rows : 0, y_deq ? rows * 4 : 0};
  for (int i = 0; i < 4; ++i) {
    if (!output_clear(outs[i], outb[i], m, K, in_ptr, in_b)) return TQ2_ERR_ARG;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], outb[i], outs[j], outb[j])) return TQ2_ERR_ARG;
  }
  (void)hipGetLastError();
  if (s_out)
    return hip_status(tq2::launch_gemv_i8_requant(m, K, x, s, *s_out, y_q, y_deq, (hipStream_t)stream));
  return hip_status(tq2::launch_gemv_i8(m, K, x, x_q, s, y, partials, (hipStream_t)stream));
}

int32_t tq2_gemv_i8q(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K,
                     const int8_t* x_q, float s, float* y, int32_t* partials, void* ws,
                     size_t ws_bytes, tq2_stream_t stream) {
  (void)ws;
  (void)ws_bytes;
  if (!x_q) return TQ2_ERR_ARG;
  return i8_common(1, &codes, &scales, &N, K, nullptr, x_q, s, y, partials, nullptr, nullptr,
                   nullptr, stream);
}

int32_t tq2_gemv_i8(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K,
                    const uint16_t* x, float s, float* y, void* ws, size_t ws_bytes,
                    tq2_stream_t stream) {
  (void)ws;
  (void)ws_bytes;
  if (!x) return TQ2_ERR_ARG;
  return i8_common(1, &codes, &scales, &N, K, x, nullptr, s, y, nullptr, nullptr, nullptr,
                   nullptr, stream);
}

int32_t tq2_gemv_i8_fused(int32_t nmat, const uint8_t* const* codes, const uint16_t* const* scales,
                          const int64_t* N, int64_t K, const uint16_t* x, float s, float* y,
                          void* ws, size_t ws_bytes, tq2_stream_t stream) {
  (void)ws;
  (void)ws_bytes;
  if (!x) return TQ2_ERR_ARG;
  return i8_common(nmat, codes, scales, N, K, x, nullptr, s, y, nullptr, nullptr, nullptr, nullptr,
                   stream);
}

int32_t tq2_gemv_i8_requant(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K,
                            const uint16_t* x, float s_in, float s_out, int8_t* y_q, float* y_deq,
                            void* ws, size_t ws_bytes, tq2_stream_t stream) {
  (void)ws;
  (void)ws_bytes;
  if (!x) return TQ2_ERR_ARG;
  return i8_common(1, &codes, &scales, &N, K, x, nullptr, s_in, nullptr, nullptr, &s_out, y_q,
                   y_deq, stream);
}

size_t tq2_gemm_workspace_bytes(int64_t N, int64_t K, int64_t M) {
  if (check_shape(N, K, TQ2_MAX_K) != TQ2_OK || M < 1 || M > TQ2_MAX_TOKENS) return (size_t)-1;
  return tq2::gemm_workspace_bytes(N, K, M);
}

}  // extern "C"

// tq2_gemm's checks of everything but the workspace.
static int32_t gemm_args(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K,
                         const uint16_t* x, int64_t M, float* y) {
  TQ2_TRY(check_shape(N, K, TQ2_MAX_K));
  TQ2_TRY(check_weights(codes, scales));
  if (M < 1 || M > TQ2_MAX_TOKENS || !x || !y) return TQ2_ERR_ARG;
  if (M * N > ((int64_t)1 << 40)) return TQ2_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(y, 4)) return TQ2_ERR_ALIGN;
  const size_t xb = (size_t)(M * K) * 2, yb = (size_t)(M * N) * 4;
  const size_t cb = (size_t)(N * (K / 4)), sb = (size_t)(N * (K / TQ2_BLOCK)) * 2;
  if (overlaps(y, yb, x, xb) || overlaps(y, yb, codes, cb) || overlaps(y, yb, scales, sb))
    return TQ2_ERR_ARG;
  return TQ2_OK;
}

static_assert(TQ2_GEMM_SCRATCH_BYTES == tq2::kGemmScratchBytes, "scratch size of the header and the library");

extern "C" {

int32_t tq2_gemm(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K, const uint16_t* x,
                 int64_t M, float* y, void* ws, size_t ws_bytes, tq2_stream_t stream) {
  TQ2_TRY(gemm_args(codes, scales, N, K, x, M, y));
  const size_t need = tq2::gemm_workspace_bytes(N, K, M);
  if (need && (!ws || ws_bytes < need || !aligned(ws, 256))) return TQ2_ERR_WORKSPACE;
  const size_t xb = (size_t)(M * K) * 2, yb = (size_t)(M * N) * 4;
  const size_t cb = (size_t)(N * (K / 4)), sb = (size_t)(N * (K / TQ2_BLOCK)) * 2;
  if (need && (overlaps(ws, need, x, xb) || overlaps(ws, need, y, yb) || overlaps(ws, need, codes, cb) ||
               overlaps(ws, need, scales, sb)))
    return TQ2_ERR_WORKSPACE;
  (void)hipGetLastError();
  return hip_status(tq2::launch_gemm(codes, scales, N, K, x, M, y, ws, (hipStream_t)stream));
}

size_t tq2_gemm_i8q_workspace_bytes(int64_t N, int64_t K, int64_t M) {
  if (check_shape(N, K, TQ2_I8_MAX_K) != TQ2_OK || M < 1 || M > TQ2_MAX_TOKENS) return (size_t)-1;
  return tq2::gemm_i8_workspace_bytes(N, K, M);
}

int32_t tq2_gemm_i8q(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K, const int8_t* x_q,
                     int64_t M, float s, float* y, void* ws, size_t ws_bytes, tq2_stream_t stream) {
  TQ2_TRY(check_shape(N, K, TQ2_I8_MAX_K));
  TQ2_TRY(check_weights(codes, scales));
  if (M < 1 || M > TQ2_MAX_TOKENS || !x_q || !y) return TQ2_ERR_ARG;
  if (M * N > ((int64_t)1 << 40)) return TQ2_ERR_SHAPE;
  if (!aligned(x_q, 16) || !aligned(y, 4)) return TQ2_ERR_ALIGN;
  TQ2_TRY(check_scale(s));
  const size_t xb = (size_t)(M * K), yb = (size_t)(M * N) * 4;
  const size_t cb = (size_t)(N * (K / 4)), sb = (size_t)(N * (K / TQ2_BLOCK)) * 2;
  if (overlaps(y, yb, x_q, xb) || overlaps(y, yb, codes, cb) || overlaps(y, yb, scales, sb)) return TQ2_ERR_ARG;
  const size_t need = tq2::gemm_i8_workspace_bytes(N, K, M);
  if (need && (!ws || ws_bytes < need || !aligned(ws, 256))) return TQ2_ERR_WORKSPACE;
  if (need && (overlaps(ws, need, x_q, xb) || overlaps(ws, need, y, yb) || overlaps(ws, need, codes, cb) ||
               overlaps(ws, need, scales, sb)))
    return TQ2_ERR_WORKSPACE;
  (void)hipGetLastError();
  return hip_status(tq2::launch_gemm_i8(codes, scales, N, K, x_q, M, s, y, ws, (hipStream_t)stream));
}

int32_t tq2_gemm_noalloc(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K,
                         const uint16_t* x, int64_t M, float* y, tq2_stream_t stream) {
  TQ2_TRY(gemm_args(codes, scales, N, K, x, M, y));
  const size_t need = tq2::gemm_workspace_bytes(N, K, M);
  if (need > TQ2_GEMM_SCRATCH_BYTES) return TQ2_ERR_SCRATCH;
  void* ws = nullptr;
  if (need) {
    (void)hipGetLastError();
    if (tq2::gemm_scratch((hipStream_t)stream, &ws) != hipSuccess) return TQ2_ERR_HIP;
  }
  (void)hipGetLastError();
  return hip_status(tq2::launch_gemm(codes, scales, N, K, x, M, y, ws, (hipStream_t)stream));
}

}  // extern "C"
