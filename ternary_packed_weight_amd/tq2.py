"""Thin ctypes binding of libtq2 (include/tq2.h), same names as the C ABI.

Argument marshalling only: every step runs in the library's HIP kernels.
Tensors are torch device tensors; binary16 data (x, scales) may be passed as
torch.float16 (the bit patterns are what crosses the ABI).  Calls enqueue on
torch's current stream unless `stream` is given, and raise Tq2Error on a
non-zero status.  There is no fallback: if libtq2.so is missing the import
fails.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq2.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libtq2.so not built at {LIB_PATH}; run __graft_entry__.build()")

# torch is imported first so that libtq2 binds to the HIP runtime torch loaded.
_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
_F = ctypes.c_float

_lib.tq2_abi_version.argtypes = []
_lib.tq2_abi_version.restype = _I32
_lib.tq2_status_string.argtypes = [_I32]
_lib.tq2_status_string.restype = ctypes.c_char_p
_lib.tq2_codes_bytes.argtypes = [_I64, _I64]
_lib.tq2_codes_bytes.restype = _SZ
_lib.tq2_scales_bytes.argtypes = [_I64, _I64]
_lib.tq2_scales_bytes.restype = _SZ
_lib.tq2_workspace_bytes.argtypes = [_I32, _I64, _I64]
_lib.tq2_workspace_bytes.restype = _SZ
_lib.tq2_pack.argtypes = [_P, _I64, _I64, _P, _P, _P, _P]
_lib.tq2_pack.restype = _I32
_lib.tq2_dequant.argtypes = [_P, _P, _I64, _I64, _P, _P]
_lib.tq2_dequant.restype = _I32
_lib.tq2_gemv.argtypes = [_P, _P, _I64, _I64, _P, _P, _P, _SZ, _P]
_lib.tq2_gemv.restype = _I32
_lib.tq2_gemv_gate_up.argtypes = [_P, _P, _P, _P, _I64, _I64, _P, _P, _P, _SZ, _P]
_lib.tq2_gemv_gate_up.restype = _I32
_lib.tq2_quantize_i8.argtypes = [_P, _I64, _F, _P, _P]
_lib.tq2_quantize_i8.restype = _I32
_lib.tq2_gemv_i8q.argtypes = [_P, _P, _I64, _I64, _P, _F, _P, _P, _P, _SZ, _P]
_lib.tq2_gemv_i8q.restype = _I32
_lib.tq2_gemv_i8.argtypes = [_P, _P, _I64, _I64, _P, _F, _P, _P, _SZ, _P]
_lib.tq2_gemv_i8.restype = _I32
_lib.tq2_gemv_fused.argtypes = [_I32, _P, _P, _P, _I64, _P, _P, _P, _SZ, _P]
_lib.tq2_gemv_fused.restype = _I32
_lib.tq2_gemv_i8_fused.argtypes = [_I32, _P, _P, _P, _I64, _P, _F, _P, _P, _SZ, _P]
_lib.tq2_gemv_i8_fused.restype = _I32
_lib.tq2_gemv_gate_up_silu.argtypes = [_P, _P, _P, _P, _I64, _I64, _P, _P, _P, _SZ, _P]
_lib.tq2_gemv_gate_up_silu.restype = _I32
_lib.tq2_gemv_i8_requant.argtypes = [_P, _P, _I64, _I64, _P, _F, _F, _P, _P, _P, _SZ, _P]
_lib.tq2_gemv_i8_requant.restype = _I32
_lib.tq2_gemm_workspace_bytes.argtypes = [_I64, _I64, _I64]
_lib.tq2_gemm_workspace_bytes.restype = _SZ
_lib.tq2_gemm.argtypes = [_P, _P, _I64, _I64, _P, _I64, _P, _P, _SZ, _P]
_lib.tq2_gemm.restype = _I32

TQ2_OK = 0
TQ2_OP_GEMV, TQ2_OP_GATE_UP, TQ2_OP_GEMV_I8, TQ2_OP_GEMV_I8Q = 0, 1, 2, 3
EXPORTED = ("tq2_abi_version", "tq2_status_string", "tq2_codes_bytes", "tq2_scales_bytes",
            "tq2_workspace_bytes", "tq2_pack", "tq2_dequant", "tq2_gemv", "tq2_gemv_gate_up",
            "tq2_quantize_i8", "tq2_gemv_i8q", "tq2_gemv_i8", "tq2_gemv_fused", "tq2_gemv_i8_fused",
            "tq2_gemv_gate_up_silu", "tq2_gemv_i8_requant", "tq2_gemm_workspace_bytes", "tq2_gemm")


class Tq2Error(RuntimeError):
    def __init__(self, fn, status):
        msg = _lib.tq2_status_string(status).decode()
        super().__init__(f"{fn}: status {status} ({msg})")
        self.status = status


def lib():
    return _lib


def _check(fn, status):
    if status != TQ2_OK:
        raise Tq2Error(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, name):
    if t is None or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    return t


def tq2_abi_version():
    return int(_lib.tq2_abi_version())


def tq2_status_string(status):
    return _lib.tq2_status_string(int(status)).decode()


def tq2_codes_bytes(N, K):
    return int(_lib.tq2_codes_bytes(N, K))


def tq2_scales_bytes(N, K):
    return int(_lib.tq2_scales_bytes(N, K))


def tq2_workspace_bytes(op, N, K):
    return int(_lib.tq2_workspace_bytes(op, N, K))


def _shape(codes, scales):
    _dev(codes, "codes")
    _dev(scales, "scales")
    N = codes.shape[0]
    K = codes.shape[-1] * 4 if codes.dim() == 2 else None
    if K is None or scales.numel() != N * (K // 256):
        raise ValueError("codes must be [N][K/4] uint8 and scales [N][K/256] fp16 bits")
    return N, K


def tq2_pack(W, codes=None, scales=None, bad_blocks=None, stream=None):
    _dev(W, "W")
    N, K = W.shape
    if codes is None:
        codes = torch.empty((N, K // 4), dtype=torch.uint8, device=W.device)
    if scales is None:
        scales = torch.empty((N, K // 256), dtype=torch.float16, device=W.device)
    if bad_blocks is None:
        bad_blocks = torch.empty(1, dtype=torch.int32, device=W.device)
    _check("tq2_pack", _lib.tq2_pack(_ptr(W), N, K, _ptr(codes), _ptr(scales), _ptr(bad_blocks),
                                     _stream(stream)))
    return codes, scales, bad_blocks


def tq2_dequant(codes, scales, W=None, stream=None):
    N, K = _shape(codes, scales)
    if W is None:
        W = torch.empty((N, K), dtype=torch.float32, device=codes.device)
    _check("tq2_dequant", _lib.tq2_dequant(_ptr(codes), _ptr(scales), N, K, _ptr(W), _stream(stream)))
    return W


def tq2_gemv(codes, scales, x, y=None, ws=None, stream=None):
    N, K = _shape(codes, scales)
    _dev(x, "x")
    if y is None:
        y = torch.empty(N, dtype=torch.float32, device=codes.device)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check("tq2_gemv", _lib.tq2_gemv(_ptr(codes), _ptr(scales), N, K, _ptr(x), _ptr(y), _ptr(ws),
                                     wsb, _stream(stream)))
    return y


def tq2_gemv_gate_up(codes_g, scales_g, codes_u, scales_u, x, y=None, ws=None, stream=None):
    N, K = _shape(codes_g, scales_g)
    if _shape(codes_u, scales_u) != (N, K):
        raise ValueError("gate and up must have the same shape")
    _dev(x, "x")
    if y is None:
        y = torch.empty((2, N), dtype=torch.float32, device=codes_g.device)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check("tq2_gemv_gate_up", _lib.tq2_gemv_gate_up(
        _ptr(codes_g), _ptr(scales_g), _ptr(codes_u), _ptr(scales_u), N, K, _ptr(x), _ptr(y),
        _ptr(ws), wsb, _stream(stream)))
    return y


def tq2_quantize_i8(x, s, x_q=None, stream=None):
    _dev(x, "x")
    K = x.numel()
    if x_q is None:
        x_q = torch.empty(K, dtype=torch.int8, device=x.device)
    _check("tq2_quantize_i8", _lib.tq2_quantize_i8(_ptr(x), K, float(s), _ptr(x_q), _stream(stream)))
    return x_q


def _workspace(op, N, K, ws, device):
    need = tq2_workspace_bytes(op, N, K)
    if ws is None and need not in (0, 2 ** 64 - 1):
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    return ws, wsb


def tq2_gemv_i8q(codes, scales, x_q, s, y=None, partials=None, ws=None, stream=None):
    N, K = _shape(codes, scales)
    _dev(x_q, "x_q")
    if y is None:
        y = torch.empty(N, dtype=torch.float32, device=codes.device)
    ws, wsb = _workspace(TQ2_OP_GEMV_I8Q, N, K, ws, codes.device)
    _check("tq2_gemv_i8q", _lib.tq2_gemv_i8q(_ptr(codes), _ptr(scales), N, K, _ptr(x_q), float(s),
                                             _ptr(y), _ptr(partials), _ptr(ws), wsb, _stream(stream)))
    return y


def tq2_gemv_i8(codes, scales, x, s, y=None, ws=None, stream=None):
    N, K = _shape(codes, scales)
    _dev(x, "x")
    if y is None:
        y = torch.empty(N, dtype=torch.float32, device=codes.device)
    ws, wsb = _workspace(TQ2_OP_GEMV_I8, N, K, ws, codes.device)
    _check("tq2_gemv_i8", _lib.tq2_gemv_i8(_ptr(codes), _ptr(scales), N, K, _ptr(x), float(s),
                                           _ptr(y), _ptr(ws), wsb, _stream(stream)))
    return y


def _host_arrays(mats):
    """Host pointer/size arrays for the fused entry points: mats is a list
    of (codes, scales) device tensors sharing K."""
    if not 1 <= len(mats) <= 3:
        raise ValueError("1 to 3 matrices")
    shapes = [_shape(c, s) for c, s in mats]
    K = shapes[0][1]
    if any(k != K for _, k in shapes):
        raise ValueError("fused matrices must share K")
    n = len(mats)
    cp = (ctypes.c_void_p * n)(*[c.data_ptr() for c, _ in mats])
    sp = (ctypes.c_void_p * n)(*[s.data_ptr() for _, s in mats])
    Np = (ctypes.c_int64 * n)(*[N for N, _ in shapes])
    return n, cp, sp, Np, [N for N, _ in shapes], K


def tq2_gemv_fused(mats, x, y=None, ws=None, stream=None):
    """y = concatenation of W_i x over mats = [(codes_i, scales_i), ...]."""
    n, cp, sp, Np, Ns, K = _host_arrays(mats)
    _dev(x, "x")
    if y is None:
        y = torch.empty(sum(Ns), dtype=torch.float32, device=x.device)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check("tq2_gemv_fused", _lib.tq2_gemv_fused(n, cp, sp, Np, K, _ptr(x), _ptr(y), _ptr(ws), wsb,
                                                 _stream(stream)))
    return y


def tq2_gemv_i8_fused(mats, x, s, y=None, ws=None, stream=None):
    n, cp, sp, Np, Ns, K = _host_arrays(mats)
    _dev(x, "x")
    if y is None:
        y = torch.empty(sum(Ns), dtype=torch.float32, device=x.device)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check("tq2_gemv_i8_fused", _lib.tq2_gemv_i8_fused(n, cp, sp, Np, K, _ptr(x), float(s), _ptr(y),
                                                       _ptr(ws), wsb, _stream(stream)))
    return y


def tq2_gemv_gate_up_silu(codes_g, scales_g, codes_u, scales_u, x, h=None, ws=None, stream=None):
    N, K = _shape(codes_g, scales_g)
    if _shape(codes_u, scales_u) != (N, K):
        raise ValueError("gate and up must have the same shape")
    _dev(x, "x")
    if h is None:
        h = torch.empty(N, dtype=torch.float32, device=codes_g.device)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check("tq2_gemv_gate_up_silu", _lib.tq2_gemv_gate_up_silu(
        _ptr(codes_g), _ptr(scales_g), _ptr(codes_u), _ptr(scales_u), N, K, _ptr(x), _ptr(h),
        _ptr(ws), wsb, _stream(stream)))
    return h


def tq2_gemv_i8_requant(codes, scales, x, s_in, s_out, y_q=None, y_deq=None, want_deq=True,
                        ws=None, stream=None):
    N, K = _shape(codes, scales)
    _dev(x, "x")
    if y_q is None:
        y_q = torch.empty(N, dtype=torch.int8, device=codes.device)
    if y_deq is None and want_deq:
        y_deq = torch.empty(N, dtype=torch.float32, device=codes.device)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check("tq2_gemv_i8_requant", _lib.tq2_gemv_i8_requant(
        _ptr(codes), _ptr(scales), N, K, _ptr(x), float(s_in), float(s_out), _ptr(y_q), _ptr(y_deq),
        _ptr(ws), wsb, _stream(stream)))
    return y_q, y_deq


def tq2_gemm_workspace_bytes(N, K, M):
    return int(_lib.tq2_gemm_workspace_bytes(N, K, M))


def tq2_gemm(codes, scales, x, y=None, ws=None, stream=None):
    """Y[M][N] = X[M][K] W^T for x of shape [M, K] (fp16); allocates the
    workspace when none is given."""
    N, K = _shape(codes, scales)
    _dev(x, "x")
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be [M, {K}]")
    M = x.shape[0]
    if y is None:
        y = torch.empty(M, N, dtype=torch.float32, device=codes.device)
    need = tq2_gemm_workspace_bytes(N, K, M)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=codes.device)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check("tq2_gemm", _lib.tq2_gemm(_ptr(codes), _ptr(scales), N, K, _ptr(x), M, _ptr(y), _ptr(ws), wsb,
                                      _stream(stream)))
    return y
