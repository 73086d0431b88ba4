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
_lib.tq2_gemm_noalloc.argtypes = [_P, _P, _I64, _I64, _P, _I64, _P, _P]
_lib.tq2_gemm_noalloc.restype = _I32
_lib.tq2_gemm_i8q_workspace_bytes.argtypes = [_I64, _I64, _I64]
_lib.tq2_gemm_i8q_workspace_bytes.restype = _SZ
_lib.tq2_gemm_i8q.argtypes = [_P, _P, _I64, _I64, _P, _I64, _F, _P, _P, _SZ, _P]
_lib.tq2_gemm_i8q.restype = _I32

TQ2_OK = 0
TQ2_OP_GEMV, TQ2_OP_GATE_UP, TQ2_OP_GEMV_I8, TQ2_OP_GEMV_I8Q = 0, 1, 2, 3
EXPORTED = ("tq2_abi_version", "tq2_status_string", "tq2_codes_bytes", "tq2_scales_bytes",
            "tq2_workspace_bytes", "tq2_pack", "tq2_dequant", "tq2_gemv", "tq2_gemv_gate_up",
            "tq2_quantize_i8", "tq2_gemv_i8q", "tq2_gemv_i8", "tq2_gemv_fused", "tq2_gemv_i8_fused",
            "tq2_gemv_gate_up_silu", "tq2_gemv_i8_requant", "tq2_gemm_workspace_bytes", "tq2_gemm",
            "tq2_gemm_i8q_workspace_bytes", "tq2_gemm_i8q", "tq2_gemm_noalloc")
TQ2_ERR_SCRATCH = 7
TQ2_GEMM_SCRATCH_BYTES = 4194304


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


_F16_BITS = (torch.float16, torch.int16) + ((torch.uint16,) if hasattr(torch, "uint16") else ())
_DTYPE_NAMES = {torch.uint8: "uint8", torch.int8: "int8", torch.int32: "int32", torch.float32: "float32"}


def _dev(t, name, dtypes=None, numel=None, at_least=False):
    """Check a tensor argument's layout before anything reaches the library:
    dtype (binary16 data may be float16 or 16-bit integer bit patterns),
    element count (exact, or a minimum for workspaces) and contiguity.  The
    C ABI sees pointers only, so a short or mistyped buffer would otherwise
    be read or written past its end.  Where the tensors live is checked last,
    for all of a call's tensors at once (_placed)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if dtypes is not None and t.dtype not in dtypes:
        want = "/".join(_DTYPE_NAMES.get(d, str(d).replace("torch.", "")) for d in dtypes)
        raise ValueError(f"{name} must have dtype {want}, got {t.dtype}")
    if numel is not None:
        n = t.numel()
        if (n < numel) if at_least else (n != numel):
            rel = "at least " if at_least else ""
            raise ValueError(f"{name} must hold {rel}{numel} elements, got {n}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _placed(**named):
    """Every tensor of the call is on the GPU, and all on one device."""
    devs = set()
    for name, t in named.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        devs.add(t.device)
    if len(devs) > 1:
        raise ValueError(f"all tensors of a call must be on one device, got {sorted(map(str, devs))}")


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
    """(N, K) of a packed weight: codes uint8 [N][K/4], scales binary16 with
    N*K/256 elements."""
    if not isinstance(codes, torch.Tensor) or codes.dim() != 2:
        raise ValueError("codes must be a 2-D [N][K/4] uint8 tensor")
    N, K = codes.shape[0], codes.shape[1] * 4
    _dev(codes, "codes", (torch.uint8,))
    if K % 256:
        raise ValueError(f"codes must be [N][K/4] with K a multiple of 256, got K = {K}")
    _dev(scales, "scales", _F16_BITS, N * (K // 256))
    return N, K


def _ws(ws):
    if ws is not None:
        _dev(ws, "ws")
    return ws


def _mat_tensors(mats):
    out = {}
    for i, (c, s) in enumerate(mats):
        out[f"codes[{i}]"], out[f"scales[{i}]"] = c, s
    return out


def _wsb(ws):
    if ws is None:
        return 0
    return ws.numel() * ws.element_size()


def tq2_pack(W, codes=None, scales=None, bad_blocks=None, stream=None):
    if not isinstance(W, torch.Tensor) or W.dim() != 2:
        raise ValueError("W must be a 2-D [N][K] float32 tensor")
    N, K = W.shape
    _dev(W, "W", (torch.float32,))
    if K % 256:
        raise ValueError(f"K must be a multiple of 256, got {K}")
    if codes is None:
        codes = torch.empty((N, K // 4), dtype=torch.uint8, device=W.device)
    if scales is None:
        scales = torch.empty((N, K // 256), dtype=torch.float16, device=W.device)
    if bad_blocks is None:
        bad_blocks = torch.empty(1, dtype=torch.int32, device=W.device)
    _dev(codes, "codes", (torch.uint8,), N * (K // 4))
    _dev(scales, "scales", _F16_BITS, N * (K // 256))
    _dev(bad_blocks, "bad_blocks", (torch.int32,), 1, at_least=True)
    _placed(W=W, codes=codes, scales=scales, bad_blocks=bad_blocks)
    _check("tq2_pack", _lib.tq2_pack(_ptr(W), N, K, _ptr(codes), _ptr(scales), _ptr(bad_blocks),
                                     _stream(stream)))
    return codes, scales, bad_blocks


def tq2_dequant(codes, scales, W=None, stream=None):
    N, K = _shape(codes, scales)
    if W is None:
        W = torch.empty((N, K), dtype=torch.float32, device=codes.device)
    _dev(W, "W", (torch.float32,), N * K)
    _placed(codes=codes, scales=scales, W=W)
    _check("tq2_dequant", _lib.tq2_dequant(_ptr(codes), _ptr(scales), N, K, _ptr(W), _stream(stream)))
    return W


def _out(t, name, numel, dtype, device):
    """An output buffer: allocated when not given, else checked."""
    if t is None:
        return torch.empty(numel, dtype=dtype, device=device)
    return _dev(t, name, (dtype,), numel)


def tq2_gemv(codes, scales, x, y=None, ws=None, stream=None):
    N, K = _shape(codes, scales)
    _dev(x, "x", _F16_BITS, K)
    y = _out(y, "y", N, torch.float32, codes.device)
    _placed(codes=codes, scales=scales, x=x, y=y, ws=_ws(ws))
    _check("tq2_gemv", _lib.tq2_gemv(_ptr(codes), _ptr(scales), N, K, _ptr(x), _ptr(y), _ptr(ws),
                                     _wsb(ws), _stream(stream)))
    return y


def tq2_gemv_gate_up(codes_g, scales_g, codes_u, scales_u, x, y=None, ws=None, stream=None):
    N, K = _shape(codes_g, scales_g)
    if _shape(codes_u, scales_u) != (N, K):
        raise ValueError("gate and up must have the same shape")
    _dev(x, "x", _F16_BITS, K)
    y = _out(y, "y", 2 * N, torch.float32, codes_g.device)
    _placed(codes_g=codes_g, scales_g=scales_g, codes_u=codes_u, scales_u=scales_u, x=x, y=y, ws=_ws(ws))
    _check("tq2_gemv_gate_up", _lib.tq2_gemv_gate_up(
        _ptr(codes_g), _ptr(scales_g), _ptr(codes_u), _ptr(scales_u), N, K, _ptr(x), _ptr(y),
        _ptr(ws), _wsb(ws), _stream(stream)))
    return y.view(2, N)


def tq2_quantize_i8(x, s, x_q=None, stream=None):
    _dev(x, "x", _F16_BITS)
    K = x.numel()
    x_q = _out(x_q, "x_q", K, torch.int8, x.device)
    _placed(x=x, x_q=x_q)
    _check("tq2_quantize_i8", _lib.tq2_quantize_i8(_ptr(x), K, float(s), _ptr(x_q), _stream(stream)))
    return x_q.view(x.shape)


def _workspace(op, N, K, ws, device):
    need = tq2_workspace_bytes(op, N, K)
    if ws is None and need not in (0, 2 ** 64 - 1):
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    return ws, _wsb(ws)


def tq2_gemv_i8q(codes, scales, x_q, s, y=None, partials=None, ws=None, stream=None):
    N, K = _shape(codes, scales)
    _dev(x_q, "x_q", (torch.int8,), K)
    y = _out(y, "y", N, torch.float32, codes.device)
    if partials is not None:
        _dev(partials, "partials", (torch.int32,), N * (K // 256))
    ws, wsb = _workspace(TQ2_OP_GEMV_I8Q, N, K, ws, codes.device)
    _placed(codes=codes, scales=scales, x_q=x_q, y=y, partials=partials, ws=_ws(ws))
    _check("tq2_gemv_i8q", _lib.tq2_gemv_i8q(_ptr(codes), _ptr(scales), N, K, _ptr(x_q), float(s),
                                             _ptr(y), _ptr(partials), _ptr(ws), wsb, _stream(stream)))
    return y


def tq2_gemv_i8(codes, scales, x, s, y=None, ws=None, stream=None):
    N, K = _shape(codes, scales)
    _dev(x, "x", _F16_BITS, K)
    y = _out(y, "y", N, torch.float32, codes.device)
    ws, wsb = _workspace(TQ2_OP_GEMV_I8, N, K, ws, codes.device)
    _placed(codes=codes, scales=scales, x=x, y=y, ws=_ws(ws))
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
    _dev(x, "x", _F16_BITS, K)
    y = _out(y, "y", sum(Ns), torch.float32, x.device)
    _placed(x=x, y=y, ws=_ws(ws), **_mat_tensors(mats))
    _check("tq2_gemv_fused", _lib.tq2_gemv_fused(n, cp, sp, Np, K, _ptr(x), _ptr(y), _ptr(ws), _wsb(ws),
                                                 _stream(stream)))
    return y


def tq2_gemv_i8_fused(mats, x, s, y=None, ws=None, stream=None):
    n, cp, sp, Np, Ns, K = _host_arrays(mats)
    _dev(x, "x", _F16_BITS, K)
    y = _out(y, "y", sum(Ns), torch.float32, x.device)
    _placed(x=x, y=y, ws=_ws(ws), **_mat_tensors(mats))
    _check("tq2_gemv_i8_fused", _lib.tq2_gemv_i8_fused(n, cp, sp, Np, K, _ptr(x), float(s), _ptr(y),
                                                       _ptr(ws), _wsb(ws), _stream(stream)))
    return y


def tq2_gemv_gate_up_silu(codes_g, scales_g, codes_u, scales_u, x, h=None, ws=None, stream=None):
    N, K = _shape(codes_g, scales_g)
    if _shape(codes_u, scales_u) != (N, K):
        raise ValueError("gate and up must have the same shape")
    _dev(x, "x", _F16_BITS, K)
    h = _out(h, "h", N, torch.float32, codes_g.device)
    _placed(codes_g=codes_g, scales_g=scales_g, codes_u=codes_u, scales_u=scales_u, x=x, h=h, ws=_ws(ws))
    _check("tq2_gemv_gate_up_silu", _lib.tq2_gemv_gate_up_silu(
        _ptr(codes_g), _ptr(scales_g), _ptr(codes_u), _ptr(scales_u), N, K, _ptr(x), _ptr(h),
        _ptr(ws), _wsb(ws), _stream(stream)))
    return h


def tq2_gemv_i8_requant(codes, scales, x, s_in, s_out, y_q=None, y_deq=None, want_deq=True,
                        ws=None, stream=None):
    N, K = _shape(codes, scales)
    _dev(x, "x", _F16_BITS, K)
    y_q = _out(y_q, "y_q", N, torch.int8, codes.device)
    if y_deq is not None or want_deq:
        y_deq = _out(y_deq, "y_deq", N, torch.float32, codes.device)
    _placed(codes=codes, scales=scales, x=x, y_q=y_q, y_deq=y_deq, ws=_ws(ws))
    _check("tq2_gemv_i8_requant", _lib.tq2_gemv_i8_requant(
        _ptr(codes), _ptr(scales), N, K, _ptr(x), float(s_in), float(s_out), _ptr(y_q), _ptr(y_deq),
        _ptr(ws), _wsb(ws), _stream(stream)))
    return y_q, y_deq


def tq2_gemm_workspace_bytes(N, K, M):
    return int(_lib.tq2_gemm_workspace_bytes(N, K, M))


def tq2_gemm(codes, scales, x, y=None, ws=None, stream=None):
    """Y[M][N] = X[M][K] W^T for x of shape [M, K] (fp16); allocates the
    workspace when none is given."""
    N, K = _shape(codes, scales)
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be a [M, {K}] tensor")
    M = x.shape[0]
    _dev(x, "x", _F16_BITS, M * K)
    y = _out(y, "y", M * N, torch.float32, codes.device)
    need = tq2_gemm_workspace_bytes(N, K, M)
    if ws is None and need and need != 2 ** 64 - 1:
        ws = torch.empty(need, dtype=torch.uint8, device=codes.device)
    if ws is not None and need and need != 2 ** 64 - 1:
        _dev(ws, "ws", None, need // ws.element_size(), at_least=True)
    _placed(codes=codes, scales=scales, x=x, y=y, ws=ws)
    _check("tq2_gemm", _lib.tq2_gemm(_ptr(codes), _ptr(scales), N, K, _ptr(x), M, _ptr(y), _ptr(ws), _wsb(ws),
                                      _stream(stream)))
    return y.view(M, N)


def tq2_gemm_i8q_workspace_bytes(N, K, M):
    return int(_lib.tq2_gemm_i8q_workspace_bytes(N, K, M))


def tq2_gemm_i8q(codes, scales, x_q, s, y=None, ws=None, stream=None):
    """Y[M][N]: the int8 matvec of every row of x_q (shape [M, K], int8,
    quantized with s); allocates the workspace when none is given."""
    N, K = _shape(codes, scales)
    if not isinstance(x_q, torch.Tensor) or x_q.dim() != 2 or x_q.shape[1] != K:
        raise ValueError(f"x_q must be a [M, {K}] tensor")
    M = x_q.shape[0]
    _dev(x_q, "x_q", (torch.int8,), M * K)
    y = _out(y, "y", M * N, torch.float32, codes.device)
    need = tq2_gemm_i8q_workspace_bytes(N, K, M)
    if ws is None and need and need != 2 ** 64 - 1:
        ws = torch.empty(need, dtype=torch.uint8, device=codes.device)
    if ws is not None and need and need != 2 ** 64 - 1:
        _dev(ws, "ws", None, need // ws.element_size(), at_least=True)
    _placed(codes=codes, scales=scales, x_q=x_q, y=y, ws=ws)
    _check("tq2_gemm_i8q", _lib.tq2_gemm_i8q(_ptr(codes), _ptr(scales), N, K, _ptr(x_q), M, float(s), _ptr(y),
                                              _ptr(ws), _wsb(ws), _stream(stream)))
    return y.view(M, N)


def tq2_gemm_noalloc(codes, scales, x, y=None, stream=None):
    """tq2_gemm with the split partials in the library's static scratch (no
    workspace argument, nothing allocated by the library; y is allocated
    here only when not given)."""
    N, K = _shape(codes, scales)
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be a [M, {K}] tensor")
    M = x.shape[0]
    _dev(x, "x", _F16_BITS, M * K)
    y = _out(y, "y", M * N, torch.float32, codes.device)
    _placed(codes=codes, scales=scales, x=x, y=y)
    _check("tq2_gemm_noalloc", _lib.tq2_gemm_noalloc(_ptr(codes), _ptr(scales), N, K, _ptr(x), M, _ptr(y),
                                                      _stream(stream)))
    return y.view(M, N)
