/*
 * tq2.h -- C ABI of libtq2, the TQ2_0 ternary decode matvec for MI355X
 * (gfx950).
 *
 * The method (page "BitCPM ternary (1.58-bit)", TQ2_0 paragraph): a weight
 * W[N][K] is stored in blocks of 256 consecutive elements along K; every
 * element is a 2-bit code q in {0,1,2} standing for q-1 in {-1,0,+1}, and
 * every block carries one fp16 scale d, so W[n][k] = d[n][k/256]*(q[n][k]-1).
 * The matvec y = W x is computed per block, sum_b d_b * sum_{k in b} x_k(q_k-1)
 * (same page, kernel paragraph).
 *
 * Byte layout (our own; the pages fix no interleave):
 *   codes  : uint8  [N][K/4], row-major.  Element k of row n is in byte
 *            n*(K/4) + k/4 at bits 2*(k%4) and 2*(k%4)+1, least significant
 *            first.  One block = 64 bytes, one 16-byte word = 64 elements.
 *   scales : uint16 [N][K/256], row-major, IEEE binary16 bit patterns.
 * Codes and scales live in two separate planes so that every code row is
 * 16-byte aligned.  Bytes per block: 64 + 2.
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers that the caller allocates, owns
 *     and keeps alive until the work completes.  The library allocates
 *     nothing and keeps no mutable state; calls are thread-safe.  (One
 *     exception: tq2_gemm_noalloc keeps its split partials in a static
 *     device array per GPU; see there.)
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL = the
 *     default stream) and returns; results are valid once the caller has
 *     synchronized the stream.  Nothing synchronizes inside.
 *   - Arguments are validated before anything is launched; on error nothing
 *     is written and a TQ2_ERR_* status is returned.  Shapes are never padded
 *     or truncated.  Device faults surface at the caller's synchronization.
 *   - Outputs must not alias inputs.
 *   - K must be a positive multiple of 256 and at most TQ2_MAX_K
 *     (TQ2_I8_MAX_K on the int8 path).  N is any value with
 *     1 <= N <= TQ2_MAX_ROWS and N*K < 2^40.
 *   - Alignment: codes, x, x_q and W 16 bytes; scales 2; y, partials 4.
 */
#ifndef TQ2_H
#define TQ2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ2_ABI_VERSION 1
#define TQ2_BLOCK 256
#define TQ2_MAX_K 65536    /* fp16 activations staged on chip: 16 x 4096 */
#define TQ2_MAX_ROWS 1073741823 /* rows of one call (gate+up: both matrices) < 2^31 */
#define TQ2_I8_MAX_K 65280 /* 255 blocks: keeps the exact int64 sum in range */

enum tq2_status {
    TQ2_OK = 0,
    TQ2_ERR_ARG = 1,       /* null pointer, N < 1, unknown op, aliasing    */
    TQ2_ERR_SHAPE = 2,     /* K < 256, K % 256 != 0, K too large           */
    TQ2_ERR_ALIGN = 3,     /* a pointer violates its alignment             */
    TQ2_ERR_WORKSPACE = 4, /* workspace missing or smaller than required   */
    TQ2_ERR_SCALE = 5,     /* int8 activation scale not finite or <= 0     */
    TQ2_ERR_HIP = 6,       /* the HIP runtime refused a launch             */
    TQ2_ERR_SCRATCH = 7    /* more scratch than tq2_gemm_noalloc holds     */
};

enum tq2_op {
    TQ2_OP_GEMV = 0,
    TQ2_OP_GATE_UP = 1,
    TQ2_OP_GEMV_I8 = 2,
    TQ2_OP_GEMV_I8Q = 3
};

typedef void *tq2_stream_t; /* hipStream_t */

/* Version of this header the library was built from (TQ2_ABI_VERSION). */
int32_t tq2_abi_version(void);

/* Static, never-NULL description of a status code. */
const char *tq2_status_string(int32_t status);

/* Sizes in bytes of the code plane (N*K/4) and the scale plane
 * (N*(K/256)*2).  Return 0 for an invalid shape. */
size_t tq2_codes_bytes(int64_t N, int64_t K);
size_t tq2_scales_bytes(int64_t N, int64_t K);

/* Device workspace an operation needs, in bytes.  Every operation of this
 * version needs none (0: pass ws = NULL, ws_bytes = 0); the arguments are
 * kept so that a split-K variant can take scratch without an ABI change.
 * `op` is a tq2_op; for TQ2_OP_GATE_UP, N is the row count of one matrix.
 * Returns (size_t)-1 for an invalid op or shape. */
size_t tq2_workspace_bytes(int32_t op, int64_t N, int64_t K);

/* tq2_pack -- fp32 W[N][K] (row-major) -> codes + scales.
 * Page "BitCPM ternary (1.58-bit)", recovery paragraph: d_block = max|W|
 * over the block, code = round(W/d) + 1.  Precisely: d is max|W| rounded to
 * binary16 (nearest, ties to even); each code is rint(W/d) (IEEE fp32
 * division by that rounded d, ties to even) clamped to [-1,1], plus 1; a
 * block whose d is 0 gets code 1 everywhere.  For W of exact ternary form
 * d*(q-1) the round trip is exact.
 * bad_blocks (nullable, device int32): receives the number of blocks that
 * hold a non-finite value or whose maximum rounds to binary16 infinity; the
 * bytes written for such blocks are unspecified.
 * Enqueues two kernels (counter reset, pack). */
int32_t tq2_pack(const float *W, int64_t N, int64_t K, uint8_t *codes,
                 uint16_t *scales, int32_t *bad_blocks, tq2_stream_t stream);

/* tq2_dequant -- codes + scales -> fp32 W[N][K] = d*(q-1), exact.  A test
 * aid; code 3 (never produced by tq2_pack) decodes as +2*d. */
int32_t tq2_dequant(const uint8_t *codes, const uint16_t *scales, int64_t N,
                    int64_t K, float *W, tq2_stream_t stream);

/* tq2_gemv -- y[N] = W x with fp16 activations x[K] (binary16 bit
 * patterns) and fp32 output.  Page "BitCPM ternary (1.58-bit)", kernel
 * paragraph (block decomposition; per-lane partial times its block's d,
 * then a cross-lane reduction); page "Custom Metal kernels" (tensors cross
 * the kernel boundary in their native dtype, accumulation is fp32 in
 * registers).  Accuracy: |y - y_exact| <= 2e-3 * sum_k |d_b(k) x_k| + 1e-6
 * per output (the accumulation is fp32; the result is deterministic run to
 * run).  One kernel.  Workspace: none (ws may be NULL). */
int32_t tq2_gemv(const uint8_t *codes, const uint16_t *scales, int64_t N,
                 int64_t K, const uint16_t *x, float *y, void *ws,
                 size_t ws_bytes, tq2_stream_t stream);

/* tq2_gemv_gate_up -- two matrices of the same shape [N][K] sharing one x
 * (page "gemma4 wNa8o8 requires int8 activations": gate and up share their
 * input).  y is [2][N]: row 0 = gate, row 1 = up.  Same arithmetic and
 * accuracy as tq2_gemv; one kernel reads x once for both. */
int32_t tq2_gemv_gate_up(const uint8_t *codes_g, const uint16_t *scales_g,
                         const uint8_t *codes_u, const uint16_t *scales_u,
                         int64_t N, int64_t K, const uint16_t *x, float *y,
                         void *ws, size_t ws_bytes, tq2_stream_t stream);

/* tq2_quantize_i8 -- static int8 activation quantization (page "gemma4
 * wNa8o8 requires int8 activations": clamp(round(x/s), -128, 127)).
 * Precisely: v = x/s as one IEEE fp32 division, rint (ties to even),
 * clamped to [-128,127] before conversion.  s must be finite and > 0;
 * non-finite x gives an unspecified x_q.  x_q[K] is int8 in natural order.
 * Elementwise, so K is any positive multiple of 256 up to
 * TQ2_MAX_TOKENS * TQ2_MAX_K: the M tokens of a tq2_gemm_i8q call
 * (x [M][K] row-major) are quantized in one call (TQ2_ERR_SHAPE otherwise). */
int32_t tq2_quantize_i8(const uint16_t *x, int64_t K, float s, int8_t *x_q,
                        tq2_stream_t stream);

/* tq2_gemv_i8q -- int8 matvec on pre-quantized activations x_q[K]
 * (same page: the input scale, then an int8 x integer-weight product).
 * Block partials P[n][b] = sum_{k in b} x_q[k]*(q[n][k]-1) are exact
 * integers; the output is defined order-free as
 *   A_n = sum_b (d_nb * 2^24) * P[n][b]   (exact, int64)
 *   y_n = fp32( fp64( fp64(A_n) * (double)s ) * 2^-24 ),
 * which equals sum_b d_b*s*P[n][b] up to that final rounding and is
 * bit-exact run to run.  K <= TQ2_I8_MAX_K.  partials (nullable): receives
 * P as int32 [N][K/256].  One kernel; no workspace. */
int32_t tq2_gemv_i8q(const uint8_t *codes, const uint16_t *scales,
                     int64_t N, int64_t K, const int8_t *x_q, float s,
                     float *y, int32_t *partials, void *ws, size_t ws_bytes,
                     tq2_stream_t stream);

/* tq2_gemv_i8 -- tq2_quantize_i8 then tq2_gemv_i8q, fused: the matvec
 * kernel quantizes x itself (same definition, bit for bit) and keeps x_q on
 * chip.  One kernel; no workspace. */
int32_t tq2_gemv_i8(const uint8_t *codes, const uint16_t *scales, int64_t N,
                    int64_t K, const uint16_t *x, float s, float *y, void *ws,
                    size_t ws_bytes, tq2_stream_t stream);

/* ---- linears that share one input, and fused epilogues ---- */

/* tq2_gemv_fused -- nmat (1..3) matrices with the same K and row counts
 * N[0..nmat-1] sharing one fp16 x, in one kernel (page "gemma4 wNa8o8
 * requires int8 activations": q, k and v share their input, as do gate and
 * up).  codes/scales/N are HOST arrays of nmat entries (the matrices
 * themselves are device memory).  y is the concatenation [N0 | N1 | N2] of
 * the outputs.  Same arithmetic and accuracy as tq2_gemv; the sum of the
 * N[i] is at most TQ2_MAX_ROWS. */
int32_t tq2_gemv_fused(int32_t nmat, const uint8_t *const *codes,
                       const uint16_t *const *scales, const int64_t *N,
                       int64_t K, const uint16_t *x, float *y, void *ws,
                       size_t ws_bytes, tq2_stream_t stream);

/* tq2_gemv_i8_fused -- the int8 matvec (tq2_gemv_i8) over nmat (1..3)
 * matrices sharing one fp16 x and one activation scale s: x is quantized
 * once per workgroup, as the shared-input rule of the same page allows (the
 * input scales of q/k/v, and of gate/up, are equal).  Each output is
 * bit-identical to tq2_gemv_i8 of its matrix.  Arrays as tq2_gemv_fused. */
int32_t tq2_gemv_i8_fused(int32_t nmat, const uint8_t *const *codes,
                          const uint16_t *const *scales, const int64_t *N,
                          int64_t K, const uint16_t *x, float s, float *y,
                          void *ws, size_t ws_bytes, tq2_stream_t stream);

/* tq2_gemv_gate_up_silu -- h[n] = silu(g[n]) * u[n], silu(v) = v/(1+exp(-v)),
 * where g and u are the fp16-x matvecs of the gate and up matrices ([N][K]
 * each) with a shared x: the MLP activation fused into the gate+up kernel
 * (page "Custom Metal kernels": several graph ops collapsed into one
 * dispatch).  Only h[N] (fp32) is written.  g and u carry the tq2_gemv
 * accuracy; the epilogue is fp32 (expf and one IEEE division). */
int32_t tq2_gemv_gate_up_silu(const uint8_t *codes_g, const uint16_t *scales_g,
                              const uint8_t *codes_u, const uint16_t *scales_u,
                              int64_t N, int64_t K, const uint16_t *x, float *h,
                              void *ws, size_t ws_bytes, tq2_stream_t stream);

/* tq2_gemv_i8_requant -- the whole static-int8 linear of the wNa8o8 page's
 * recipe: quantize x with s_in, int8 x ternary matvec (y exactly as
 * tq2_gemv_i8), then requantize the output with the static output scale:
 * y_q = clamp(rint(y / s_out), -128, 127) (one IEEE fp32 division, ties to
 * even), and, if y_deq is non-NULL, the dequantized y_deq = y_q * s_out
 * (fp32).  s_in and s_out must be finite and > 0.  One kernel. */
int32_t tq2_gemv_i8_requant(const uint8_t *codes, const uint16_t *scales,
                            int64_t N, int64_t K, const uint16_t *x, float s_in,
                            float s_out, int8_t *y_q, float *y_deq, void *ws,
                            size_t ws_bytes, tq2_stream_t stream);

/* ---- several tokens at once ---- */

/* tq2_gemm_workspace_bytes -- device workspace that tq2_gemm needs for this
 * shape and token count: the split partials (4*M*N bytes per split) when the
 * matrix-core plan splits K across workgroups, which it does only when N
 * gives too few row groups to fill the GPU; 0 otherwise, and 0 whenever
 * the call runs a matvec kernel (M = 1, and the few-token calls described
 * at tq2_gemm).  (size_t)-1 for an invalid shape or token count. */
size_t tq2_gemm_workspace_bytes(int64_t N, int64_t K, int64_t M);

/* tq2_gemm -- the matvec of page "BitCPM ternary (1.58-bit)" (kernel
 * paragraph) for M tokens at once: Y[m][n] = sum_k W[n][k] * X[m][k],
 * X [M][K] fp16 (row-major, 16-byte aligned), Y [M][N] fp32 (row-major).
 * The weights are streamed once for all M tokens (prefill, speculative
 * decode; the page runs prefill as one matvec per token).  Per output the
 * accuracy of tq2_gemv: |Y - Y_ref| <= 2e-3 * sum_k |d_b(k) X[m][k]| + 1e-6.
 * 1 <= M <= TQ2_MAX_TOKENS.  ws: when tq2_gemm_workspace_bytes(N, K, M)
 * is non-zero, device memory of at least that many bytes, 256-byte aligned,
 * not overlapping X or Y (TQ2_ERR_WORKSPACE otherwise); its contents on
 * entry do not matter and are overwritten.  Otherwise ws may be NULL.  One
 * kernel on `stream` (two when K is split); deterministic (chunk and split
 * sums are added in a fixed order).  M = 1 runs tq2_gemv's kernel (no
 * workspace; the output equals tq2_gemv's bit for bit).  M = 2 to 4 with K
 * of 1, 2 or 4 chunks of 4096 runs a one-pass matvec that decodes every
 * code word once for all M tokens, while the activations it stages over all
 * its workgroups (workgroups x M x 2K bytes) stay within 32 MiB, which
 * holds for small and medium N: no workspace, and every token's output
 * equals tq2_gemv's bit for bit.  Other calls run on the matrix cores.  A
 * token's output does not depend on the values of the other tokens of the
 * call; calls with different M can take different plans (route, K split,
 * rows per wave), so the same token may differ in its last bits between
 * them, always within the bound above. */
#define TQ2_MAX_TOKENS 65536
int32_t tq2_gemm(const uint8_t *codes, const uint16_t *scales, int64_t N,
                 int64_t K, const uint16_t *x, int64_t M, float *y, void *ws,
                 size_t ws_bytes, tq2_stream_t stream);

/* tq2_gemm_i8q_workspace_bytes -- device workspace that tq2_gemm_i8q
 * needs: the split sums (8*M*N bytes per split, int64) when the plan splits
 * K across workgroups, which it does only when N gives too few row groups
 * to fill the GPU; 0 otherwise, and 0 for M = 1.  (size_t)-1 for an
 * invalid shape or token count. */
size_t tq2_gemm_i8q_workspace_bytes(int64_t N, int64_t K, int64_t M);

/* tq2_gemm_i8q -- the int8 matvec of page "gemma4 wNa8o8 requires int8
 * activations" (Implemented section), tq2_gemv_i8q's, for M tokens at once:
 * x_q [M][K] int8 activations (row-major, 16-byte aligned, already
 * quantized with the activation scale s, for example by tq2_quantize_i8 on
 * each token), Y [M][N] fp32 (row-major).  Row n of token m equals
 * tq2_gemv_i8q(W, x_q[m], s) bit for bit: every 256-block's sum of
 * x_q * (code - 1) is exact (int32 on the matrix cores), the blocks are
 * scaled and summed exactly in int64, and the same epilogue
 * fp32(fp64(A) * s * 2^-24) follows.  1 <= M <= TQ2_MAX_TOKENS, K <=
 * TQ2_I8_MAX_K, s finite and > 0 (TQ2_ERR_SCALE).  ws: when
 * tq2_gemm_i8q_workspace_bytes(N, K, M) is non-zero, device memory of at
 * least that many bytes, 256-byte aligned, not overlapping x_q or Y
 * (TQ2_ERR_WORKSPACE otherwise); its contents on entry do not matter.
 * Otherwise ws may be NULL.  One kernel on `stream` (two when K is split);
 * M = 1 runs tq2_gemv_i8q's kernel; M = 2 to 4 with K of 1, 2 or 4 chunks
 * of 4096 a one-pass VALU matvec while the x_q it stages over all its
 * workgroups (workgroups x M x K bytes) stays within 24 MiB (no workspace);
 * other calls the matrix cores.  The weights are streamed once for all M
 * tokens. */
int32_t tq2_gemm_i8q(const uint8_t *codes, const uint16_t *scales, int64_t N,
                     int64_t K, const int8_t *x_q, int64_t M, float s, float *y,
                     void *ws, size_t ws_bytes, tq2_stream_t stream);

/* tq2_gemm_noalloc -- tq2_gemm for callers that cannot allocate (code
 * under HIP graph capture, serving loops or harnesses that forbid
 * hipMalloc): the same kernels and results (bit-identical to tq2_gemm), but
 * the split partials live in a static device array of the library,
 * TQ2_GEMM_SCRATCH_BYTES per GPU, held by every GPU the library runs on
 * until the process ends.  Allocates nothing (no hipMalloc, no allocating
 * library routine).  Returns TQ2_ERR_SCRATCH, before any launch, when
 * tq2_gemm_workspace_bytes(N, K, M) exceeds TQ2_GEMM_SCRATCH_BYTES (on
 * MI355X no shape needs more than 2 MiB).  The first call on a device looks
 * the array's device address up (hipGetSymbolAddress) on the device of
 * `stream`.  All calls on one GPU share its array and every call overwrites
 * what it uses: calls that can overlap on one GPU (concurrent streams, or
 * other host threads) race and must be serialized by the caller.  Nothing in
 * the array needs to start at zero. */
#define TQ2_GEMM_SCRATCH_BYTES 4194304
int32_t tq2_gemm_noalloc(const uint8_t *codes, const uint16_t *scales,
                         int64_t N, int64_t K, const uint16_t *x, int64_t M,
                         float *y, tq2_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ2_H */
