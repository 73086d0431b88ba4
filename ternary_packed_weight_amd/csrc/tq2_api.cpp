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

static int32_t gemv_common(const uint8_t* const* codes, const uint16_t* const* scales, int nmat,
                           int64_t N, int64_t K, const uint16_t* x, float* y,
                           tq2_stream_t stream) {
  TQ2_TRY(check_shape(N, K, TQ2_MAX_K));
  if (!x || !y) return TQ2_ERR_ARG;
  for (int i = 0; i < nmat; ++i) TQ2_TRY(check_weights(codes[i], scales[i]));
  if (!aligned(x, 16) || !aligned(y, 4)) return TQ2_ERR_ALIGN;
  const size_t yb = (size_t)(nmat * N) * 4;
  if (overlaps(y, yb, x, (size_t)K * 2)) return TQ2_ERR_ARG;
  for (int i = 0; i < nmat; ++i)
    if (overlaps(y, yb, codes[i], (size_t)(N * K / 4)) || overlaps(y, yb, scales[i], (size_t)(N * K / 128)))
      return TQ2_ERR_ARG;
  tq2::MatSet m = {};
  for (int i = 0; i < nmat; ++i) {
    m.codes[i] = codes[i];
    m.scales[i] = scales[i];
    m.row_begin[i] = (int32_t)(i * N);
  }
  m.nmat = nmat;
  m.rows = (int32_t)(nmat * N);
  (void)hipGetLastError();
  return hip_status(tq2::launch_gemv_f16(m, K, x, y, (hipStream_t)stream));
}

int32_t tq2_gemv(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K,
                 const uint16_t* x, float* y, void* ws, size_t ws_bytes, tq2_stream_t stream) {
  (void)ws;
  (void)ws_bytes;
  return gemv_common(&codes, &scales, 1, N, K, x, y, stream);
}

int32_t tq2_gemv_gate_up(const uint8_t* codes_g, const uint16_t* scales_g, const uint8_t* codes_u,
                         const uint16_t* scales_u, int64_t N, int64_t K, const uint16_t* x,
                         float* y, void* ws, size_t ws_bytes, tq2_stream_t stream) {
  (void)ws;
  (void)ws_bytes;
  const uint8_t* c[2] = {codes_g, codes_u};
  const uint16_t* s[2] = {scales_g, scales_u};
  return gemv_common(c, s, 2, N, K, x, y, stream);
}

int32_t tq2_quantize_i8(const uint16_t* x, int64_t K, float s, int8_t* x_q, tq2_stream_t stream) {
  TQ2_TRY(check_shape(1, K, TQ2_MAX_K));
  if (!x || !x_q) return TQ2_ERR_ARG;
  if (!aligned(x, 16) || !aligned(x_q, 16)) return TQ2_ERR_ALIGN;
  TQ2_TRY(check_scale(s));
  if (overlaps(x, (size_t)K * 2, x_q, (size_t)K)) return TQ2_ERR_ARG;
  (void)hipGetLastError();
  return hip_status(tq2::launch_quantize_i8(x, K, s, x_q, (hipStream_t)stream));
}

static int32_t i8_common(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K,
                         const uint16_t* x, const int8_t* x_q, float s, float* y,
                         int32_t* partials, tq2_stream_t stream) {
  TQ2_TRY(check_shape(N, K, TQ2_I8_MAX_K));
  if ((!x && !x_q) || !y) return TQ2_ERR_ARG;
  TQ2_TRY(check_weights(codes, scales));
  if ((x && !aligned(x, 16)) || (x_q && !aligned(x_q, 16)) || !aligned(y, 4) ||
      (partials && !aligned(partials, 4)))
    return TQ2_ERR_ALIGN;
  TQ2_TRY(check_scale(s));
  const size_t yb = (size_t)N * 4, pb = partials ? (size_t)(N * (K / 256)) * 4 : 0;
  const size_t cb = (size_t)(N * K / 4), sb = (size_t)(N * K / 128);
  const void* in_ptr = x ? (const void*)x : (const void*)x_q;
  const size_t in_b = x ? (size_t)K * 2 : (size_t)K;
  const void* outs[2] = {y, partials};
  const size_t outb[2] = {yb, pb};
  for (int i = 0; i < 2; ++i)
    if (overlaps(outs[i], outb[i], codes, cb) || overlaps(outs[i], outb[i], scales, sb) ||
        overlaps(outs[i], outb[i], in_ptr, in_b))
      return TQ2_ERR_ARG;
  if (overlaps(y, yb, partials, pb)) return TQ2_ERR_ARG;
  tq2::MatSet m = {};
  m.codes[0] = codes;
  m.scales[0] = scales;
  m.nmat = 1;
  m.rows = (int32_t)N;
  (void)hipGetLastError();
  return hip_status(tq2::launch_gemv_i8(m, K, x, x_q, s, y, partials, (hipStream_t)stream));
}

int32_t tq2_gemv_i8q(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K,
                     const int8_t* x_q, float s, float* y, int32_t* partials, void* ws,
                     size_t ws_bytes, tq2_stream_t stream) {
  (void)ws;
  (void)ws_bytes;
  if (!x_q) return TQ2_ERR_ARG;
  return i8_common(codes, scales, N, K, nullptr, x_q, s, y, partials, stream);
}

int32_t tq2_gemv_i8(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K,
                    const uint16_t* x, float s, float* y, void* ws, size_t ws_bytes,
                    tq2_stream_t stream) {
  (void)ws;
  (void)ws_bytes;
  if (!x) return TQ2_ERR_ARG;
  return i8_common(codes, scales, N, K, x, nullptr, s, y, nullptr, stream);
}

}  // extern "C"
