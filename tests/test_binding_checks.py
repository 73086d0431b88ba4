"""The Python binding refuses a mistyped or mis-sized tensor with ValueError
before anything reaches the library (the C ABI sees only pointers, so such a
buffer would otherwise be read or written past its end).  CPU tensors are
used: every check here fires before the device check, and a well-formed CPU
tensor is refused as not being on the device, so no library call is made."""
import pytest
import torch

from ternary_packed_weight_amd import build


@pytest.fixture(scope="module")
def tq2():
    import os
    if not os.path.exists(build.LIB):
        build.build()
    from ternary_packed_weight_amd import tq2 as mod
    return mod


N, K = 8, 512


def _w(dtype_codes=torch.uint8, dtype_scales=torch.float16, n=N, k=K):
    return torch.zeros((n, k // 4), dtype=dtype_codes), torch.zeros((n, k // 256), dtype=dtype_scales)


def _raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_weights_checked(tq2):
    c, s = _w()
    x = torch.zeros(K, dtype=torch.float16)
    _raises("codes must have dtype uint8", tq2.tq2_gemv, c.to(torch.int8), s, x)
    _raises("scales must have dtype", tq2.tq2_gemv, c, s.to(torch.bfloat16), x)
    _raises("scales must have dtype", tq2.tq2_gemv, c, s.float(), x)
    _raises("scales must hold 16 elements, got 8", tq2.tq2_gemv, c, s[:, :1].contiguous(), x)
    _raises("codes must be a 2-D", tq2.tq2_gemv, c.flatten(), s, x)
    _raises("multiple of 256", tq2.tq2_gemv, torch.zeros((N, 100), dtype=torch.uint8), s, x)


def test_activation_and_output_checked(tq2):
    c, s = _w()
    x = torch.zeros(K, dtype=torch.float16)
    _raises("x must have dtype", tq2.tq2_gemv, c, s, x.float())
    _raises(f"x must hold {K} elements, got {K - 256}", tq2.tq2_gemv, c, s, x[: K - 256])
    _raises(f"y must hold {N} elements, got {N - 1}", tq2.tq2_gemv, c, s, x, y=torch.zeros(N - 1))
    _raises("y must have dtype float32", tq2.tq2_gemv, c, s, x, y=torch.zeros(N, dtype=torch.float64))
    _raises("codes must be a device tensor", tq2.tq2_gemv, c, s, x)   # well-formed, on the CPU
    _raises("x must be contiguous", tq2.tq2_gemv, c, s, torch.zeros((K, 2), dtype=torch.float16)[:, 0])
    _raises("codes must be contiguous", tq2.tq2_gemv, torch.zeros((K // 4, N), dtype=torch.uint8).t(), s, x)


def test_gate_up_and_silu_checked(tq2):
    c, s = _w()
    x = torch.zeros(K, dtype=torch.float16)
    _raises(f"y must hold {2 * N} elements", tq2.tq2_gemv_gate_up, c, s, c, s, x, y=torch.zeros(N))
    c2, s2 = _w(n=N + 1)
    _raises("same shape", tq2.tq2_gemv_gate_up, c, s, c2, s2, x)
    _raises(f"h must hold {N} elements", tq2.tq2_gemv_gate_up_silu, c, s, c, s, x, h=torch.zeros(2 * N))


def test_int8_paths_checked(tq2):
    c, s = _w()
    x = torch.zeros(K, dtype=torch.float16)
    xq = torch.zeros(K, dtype=torch.int8)
    _raises("x_q must have dtype int8", tq2.tq2_gemv_i8q, c, s, xq.to(torch.uint8), 0.1)
    _raises(f"x_q must hold {K} elements", tq2.tq2_gemv_i8q, c, s, xq[:256], 0.1)
    _raises("partials must hold 16 elements", tq2.tq2_gemv_i8q, c, s, xq, 0.1,
            y=torch.zeros(N), partials=torch.zeros(N, dtype=torch.int32))
    _raises("partials must have dtype int32", tq2.tq2_gemv_i8q, c, s, xq, 0.1,
            y=torch.zeros(N), partials=torch.zeros(16, dtype=torch.int64))
    _raises("x must have dtype", tq2.tq2_gemv_i8, c, s, x.float(), 0.1)
    _raises(f"y must hold {N} elements", tq2.tq2_gemv_i8, c, s, x, 0.1, y=torch.zeros(N + 1))
    _raises("x_q must hold 512 elements", tq2.tq2_quantize_i8, x, 0.1, x_q=torch.zeros(511, dtype=torch.int8))
    _raises("x must have dtype", tq2.tq2_quantize_i8, x.float(), 0.1)
    _raises("y_q must have dtype int8", tq2.tq2_gemv_i8_requant, c, s, x, 0.1, 0.1,
            y_q=torch.zeros(N, dtype=torch.uint8))
    _raises(f"y_deq must hold {N} elements", tq2.tq2_gemv_i8_requant, c, s, x, 0.1, 0.1,
            y_q=torch.zeros(N, dtype=torch.int8), y_deq=torch.zeros(N - 1))


def test_fused_checked(tq2):
    c, s = _w()
    x = torch.zeros(K, dtype=torch.float16)
    c2, s2 = _w(k=2 * K)
    _raises("share K", tq2.tq2_gemv_fused, [(c, s), (c2, s2)], x)
    _raises(f"y must hold {3 * N} elements", tq2.tq2_gemv_fused, [(c, s)] * 3, x, y=torch.zeros(2 * N))
    _raises("x must hold", tq2.tq2_gemv_i8_fused, [(c, s)] * 2, x[:256], 0.1)
    _raises("1 to 3 matrices", tq2.tq2_gemv_fused, [(c, s)] * 4, x)


def test_pack_and_dequant_checked(tq2):
    W = torch.zeros((N, K), dtype=torch.float32)
    _raises("W must have dtype float32", tq2.tq2_pack, W.half())
    _raises("W must have dtype float32", tq2.tq2_pack, W.to(torch.bfloat16))
    _raises("W must be a 2-D", tq2.tq2_pack, W.flatten())
    _raises("codes must hold", tq2.tq2_pack, W, codes=torch.zeros((N, K // 8), dtype=torch.uint8))
    _raises("scales must hold", tq2.tq2_pack, W, codes=torch.zeros((N, K // 4), dtype=torch.uint8),
            scales=torch.zeros(N, dtype=torch.float16))
    _raises("bad_blocks must have dtype int32", tq2.tq2_pack, W,
            codes=torch.zeros((N, K // 4), dtype=torch.uint8),
            scales=torch.zeros((N, K // 256), dtype=torch.float16), bad_blocks=torch.zeros(1))
    c, s = _w()
    _raises(f"W must hold {N * K} elements", tq2.tq2_dequant, c, s, W=torch.zeros(N * K - 1))


def test_gemm_checked(tq2):
    c, s = _w()
    X = torch.zeros((3, K), dtype=torch.float16)
    _raises("x must be a", tq2.tq2_gemm, c, s, torch.zeros((3, K + 256), dtype=torch.float16))
    _raises("x must have dtype", tq2.tq2_gemm, c, s, X.float())
    _raises(f"y must hold {3 * N} elements", tq2.tq2_gemm, c, s, X, y=torch.zeros(3 * N - 1))


def test_gemm_i8q_checked(tq2):
    c, s = _w()
    XQ = torch.zeros((3, K), dtype=torch.int8)
    _raises("x_q must be a", tq2.tq2_gemm_i8q, c, s, torch.zeros((3, K + 256), dtype=torch.int8), 0.1)
    _raises("x_q must have dtype", tq2.tq2_gemm_i8q, c, s, XQ.to(torch.uint8), 0.1)
    _raises("x_q must have dtype", tq2.tq2_gemm_i8q, c, s, XQ.half(), 0.1)
    _raises(f"y must hold {3 * N} elements", tq2.tq2_gemm_i8q, c, s, XQ, 0.1, y=torch.zeros(3 * N - 1))
    _raises("y must have dtype", tq2.tq2_gemm_i8q, c, s, XQ, 0.1, y=torch.zeros(3 * N, dtype=torch.float16))
