"""Host-side checks of libtq2: it loads, exports every function include/tq2.h
declares, and rejects invalid arguments with the documented status before
any launch.  Fake (never dereferenced) device addresses are used, so these
tests only run where no GPU is visible."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tq2.h")


def _lib_path():
    from ternary_packed_weight_amd import build
    if not os.path.exists(build.LIB):
        build.build()
    return build.LIB


@pytest.fixture(scope="module")
def tq2():
    _lib_path()
    from ternary_packed_weight_amd import tq2 as mod
    return mod


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tq2_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("tq2_pack", "tq2_gemv", "tq2_gemv_gate_up", "tq2_gemv_i8", "tq2_gemv_i8q",
                     "tq2_quantize_i8", "tq2_dequant", "tq2_workspace_bytes", "tq2_gemv_fused",
                     "tq2_gemv_i8_fused", "tq2_gemv_gate_up_silu", "tq2_gemv_i8_requant"):
        assert required in names


def test_library_exports_every_declared_symbol(tq2):
    lib = ctypes.CDLL(_lib_path())
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in tq2.EXPORTED, name
    assert tq2.tq2_abi_version() == 1


def test_sizes(tq2):
    assert tq2.tq2_codes_bytes(4096, 4096) == 4096 * 1024
    assert tq2.tq2_scales_bytes(4096, 4096) == 4096 * 16 * 2
    assert tq2.tq2_codes_bytes(1, 100) == 0
    assert tq2.tq2_workspace_bytes(tq2.TQ2_OP_GEMV, 4096, 4096) == 0
    assert tq2.tq2_workspace_bytes(tq2.TQ2_OP_GATE_UP, 16384, 4096) == 0
    assert tq2.tq2_workspace_bytes(tq2.TQ2_OP_GEMV_I8, 4096, 16384) == 0
    assert tq2.tq2_workspace_bytes(tq2.TQ2_OP_GEMV_I8Q, 4096, 65280) == 0
    assert tq2.tq2_workspace_bytes(tq2.TQ2_OP_GEMV_I8, 4096, 65536) == 2 ** 64 - 1
    assert tq2.tq2_workspace_bytes(99, 1, 256) == 2 ** 64 - 1
    for s in range(7):
        assert isinstance(tq2.tq2_status_string(s), str)


no_gpu = pytest.mark.skipif(
    __import__("torch").cuda.is_available(),
    reason="fake device addresses are only safe to pass where no GPU exists")

A = 1 << 30  # fake, 256-aligned, never dereferenced


def P(addr):
    return ctypes.c_void_p(addr)


@no_gpu
def test_error_paths_gemv(tq2):
    lib = tq2.lib()
    g = lambda c=A, s=A + 2 ** 24, N=16, K=256, x=A + 2 ** 25, y=A + 2 ** 26: lib.tq2_gemv(
        P(c), P(s), N, K, P(x), P(y), None, 0, None)
    assert g(N=0) == 1 and g(N=-3) == 1
    assert g(K=0) == 2 and g(K=100) == 2 and g(K=384) == 2 and g(K=65536 + 256) == 2
    assert g(N=2 ** 31, K=65536) == 2
    assert g(c=0) == 1 and g(x=0) == 1 and g(y=0) == 1
    assert g(c=A + 8) == 3 and g(s=A + 2 ** 24 + 1) == 3 and g(x=A + 2 ** 25 + 4) == 3
    assert g(y=A + 2 ** 26 + 2) == 3
    assert g(y=A + 8) == 1                     # y inside codes
    assert g(y=A + 2 ** 25 - 16) == 1          # y overlapping x
    gu = lib.tq2_gemv_gate_up(P(A), P(A + 4096), P(0), P(A + 8192), 16, 256, P(A + 2 ** 25),
                              P(A + 2 ** 26), None, 0, None)
    assert gu == 1


@no_gpu
def test_error_paths_int8(tq2):
    lib = tq2.lib()

    def g(N=16, K=256, s=0.5, x=A + 2 ** 25, y=A + 2 ** 26):
        return lib.tq2_gemv_i8(P(A), P(A + 2 ** 24), N, K, P(x), ctypes.c_float(s), P(y), None, 0, None)

    assert g(K=65280 + 256) == 2 and g(K=100) == 2 and g(N=0) == 1
    assert g(s=0.0) == 5 and g(s=-1.0) == 5 and g(s=float("inf")) == 5 and g(s=float("nan")) == 5
    assert g(x=0) == 1 and g(y=0) == 1
    assert g(x=A + 2 ** 25 + 8) == 3 and g(y=A + 2 ** 26 + 1) == 3
    assert g(y=A + 64) == 1                    # y inside the code plane
    assert g(y=A + 2 ** 25 + 256) == 1         # y overlapping x
    q = lib.tq2_gemv_i8q(P(A), P(A + 2 ** 24), 16, 256, P(0), ctypes.c_float(1.0), P(A + 2 ** 26),
                         None, None, 0, None)
    assert q == 1
    q = lib.tq2_gemv_i8q(P(A), P(A + 2 ** 24), 16, 256, P(A + 2 ** 25), ctypes.c_float(1.0),
                         P(A + 2 ** 26), P(A + 2 ** 26 + 2), None, 0, None)
    assert q == 3                              # partials misaligned
    q = lib.tq2_gemv_i8q(P(A), P(A + 2 ** 24), 16, 256, P(A + 2 ** 25), ctypes.c_float(1.0),
                         P(A + 2 ** 26), P(A + 2 ** 26), None, 0, None)
    assert q == 1                              # partials alias y
    assert lib.tq2_quantize_i8(P(A), 256, ctypes.c_float(0.0), P(A + 4096), None) == 5
    assert lib.tq2_quantize_i8(P(A), 255, ctypes.c_float(1.0), P(A + 4096), None) == 2
    assert lib.tq2_quantize_i8(P(A), (65536 * 65536) + 256, ctypes.c_float(1.0), P(A + 4096), None) == 2
    assert lib.tq2_quantize_i8(P(A), 256, ctypes.c_float(1.0), P(A + 96), None) == 1
    assert lib.tq2_quantize_i8(P(A), 256, ctypes.c_float(1.0), P(A + 4097), None) == 3


@no_gpu
def test_error_paths_pack(tq2):
    lib = tq2.lib()
    W, C, S, B = A, A + 2 ** 28, A + 2 ** 29, A + 2 ** 29 + 2 ** 20
    assert lib.tq2_pack(P(W), 0, 256, P(C), P(S), P(B), None) == 1
    assert lib.tq2_pack(P(W), 4, 200, P(C), P(S), P(B), None) == 2
    assert lib.tq2_pack(P(W + 4), 4, 256, P(C), P(S), P(B), None) == 3
    assert lib.tq2_pack(P(W), 4, 256, P(C), P(S), P(B + 2), None) == 3
    assert lib.tq2_pack(P(W), 4, 256, P(W + 64), P(S), P(B), None) == 1
    assert lib.tq2_pack(P(0), 4, 256, P(C), P(S), P(B), None) == 1
    assert lib.tq2_dequant(P(C), P(S), 4, 256, P(0), None) == 1
    assert lib.tq2_dequant(P(C), P(S), 4, 256, P(C), None) == 1


@no_gpu
def test_error_paths_fused_and_epilogues(tq2):
    lib = tq2.lib()
    C = (ctypes.c_void_p * 3)(A, A + 2 ** 20, A + 2 ** 21)
    S = (ctypes.c_void_p * 3)(A + 2 ** 22, A + 2 ** 22 + 2 ** 16, A + 2 ** 22 + 2 ** 17)
    N = (ctypes.c_int64 * 3)(4096, 256, 256)
    x, y = A + 2 ** 25, A + 2 ** 26

    def f(nmat=3, n=N, K=4096, xx=x, yy=y):
        return lib.tq2_gemv_fused(nmat, C, S, n, K, P(xx), P(yy), None, 0, None)

    assert f(nmat=0) == 1 and f(nmat=4) == 1
    assert f(n=(ctypes.c_int64 * 3)(4096, 0, 256)) == 1
    assert f(n=(ctypes.c_int64 * 3)(2 ** 29, 2 ** 29, 2 ** 29), K=256) == 2   # rows >= 2^31
    assert f(K=1000) == 2 and f(xx=x + 4) == 3 and f(yy=A + 2 ** 20 + 16) == 1
    assert lib.tq2_gemv_fused(2, None, S, N, 4096, P(x), P(y), None, 0, None) == 1
    assert lib.tq2_gemv_i8_fused(3, C, S, N, 4096, P(x), ctypes.c_float(0.0), P(y), None, 0, None) == 5
    assert lib.tq2_gemv_i8_fused(3, C, S, N, 65536, P(x), ctypes.c_float(1.0), P(y), None, 0, None) == 2
    assert lib.tq2_gemv_gate_up_silu(P(A), P(A + 4096), P(A + 2 ** 20), P(A + 2 ** 20 + 4096), 16, 256,
                                     P(x), P(0), None, 0, None) == 1
    assert lib.tq2_gemv_gate_up_silu(P(A), P(A + 4096), P(A + 2 ** 20), P(A + 2 ** 20 + 4096), 16, 256,
                                     P(x), P(A + 64), None, 0, None) == 1
    rq = lambda s_in=0.1, s_out=0.1, yq=y, yd=A + 2 ** 27: lib.tq2_gemv_i8_requant(
        P(A), P(A + 2 ** 24), 16, 256, P(x), ctypes.c_float(s_in), ctypes.c_float(s_out), P(yq), P(yd),
        None, 0, None)
    assert rq(s_out=0.0) == 5 and rq(s_out=float("nan")) == 5 and rq(s_in=-1.0) == 5
    assert rq(yq=0) == 1 and rq(yd=A + 2 ** 27 + 2) == 3 and rq(yd=y) == 1


@no_gpu
def test_error_paths_gemm(tq2):
    lib = tq2.lib()
    N, K, M = 256, 4096, 16  # K split: a workspace is needed
    need = lib.tq2_gemm_workspace_bytes(N, K, M)
    assert 0 < need < 2 ** 40
    assert lib.tq2_gemm_workspace_bytes(N, 1000, M) == ctypes.c_size_t(-1).value
    assert lib.tq2_gemm_workspace_bytes(N, K, 0) == ctypes.c_size_t(-1).value
    c, s = A, A + 2 ** 24
    x, y, ws = A + 2 ** 26, A + 2 ** 27, A + 2 ** 28

    def g(xx=x, MM=M, yy=y, w=ws, wb=need, KK=K):
        return lib.tq2_gemm(P(c), P(s), N, KK, P(xx), MM, P(yy), P(w), wb, None)

    assert g(MM=0) == 1 and g(MM=65537) == 1 and g(KK=1000) == 2
    assert g(xx=x + 2) == 3 and g(yy=y + 2) == 3
    assert g(w=0) == 4 and g(wb=need - 1) == 4 and g(w=ws + 16) == 4
    assert g(yy=x) == 1                      # y overlapping x
    assert g(w=y) == 4                       # workspace overlapping y


@no_gpu
def test_error_paths_gemm_i8q(tq2):
    lib = tq2.lib()
    N, K, M = 256, 4096, 16  # K split in 4: int64 partials
    need = lib.tq2_gemm_i8q_workspace_bytes(N, K, M)
    assert need == 4 * M * N * 8
    assert lib.tq2_gemm_i8q_workspace_bytes(N, K, 1) == 0       # the one-token kernel
    assert lib.tq2_gemm_i8q_workspace_bytes(4096, 4096, 16) == 0  # 256 row sets: no split
    for m in (2, 3, 4):  # the one-pass few-token int8 matvec
        assert lib.tq2_gemm_i8q_workspace_bytes(256, 4096, m) == 0
        assert lib.tq2_gemm_i8q_workspace_bytes(256, 16384, m) == 0
    assert lib.tq2_gemm_i8q_workspace_bytes(256, 12288, 2) > 0  # 3 chunks: matrix cores, K split
    bad = ctypes.c_size_t(-1).value
    assert lib.tq2_gemm_i8q_workspace_bytes(N, 1000, M) == bad
    assert lib.tq2_gemm_i8q_workspace_bytes(N, 65536, M) == bad  # above the int8 limit
    assert lib.tq2_gemm_i8q_workspace_bytes(N, K, 0) == bad
    c, s = A, A + 2 ** 24
    xq, y, ws = A + 2 ** 26, A + 2 ** 27, A + 2 ** 28

    def g(xx=xq, MM=M, yy=y, w=ws, wb=need, KK=K, sc=0.5):
        return lib.tq2_gemm_i8q(P(c), P(s), N, KK, P(xx), MM, sc, P(yy), P(w), wb, None)

    assert g(MM=0) == 1 and g(MM=65537) == 1 and g(KK=1000) == 2 and g(KK=65536) == 2
    assert g(xx=xq + 2) == 3 and g(yy=y + 2) == 3
    assert g(sc=0.0) == 5 and g(sc=float("nan")) == 5 and g(sc=float("inf")) == 5
    assert g(w=0) == 4 and g(wb=need - 1) == 4 and g(w=ws + 16) == 4
    assert g(yy=xq) == 1                     # y overlapping x_q
    assert g(w=y) == 4                       # workspace overlapping y


@no_gpu
def test_gemm_workspace_only_for_split_k(tq2):
    """The 16384-row shapes run without a K split (no workspace), and so do
    4096 rows below K = 16384 (one row group per wave); 256 rows, and 4096
    rows at K = 16384, split K and need the partials."""
    lib = tq2.lib()
    assert lib.tq2_gemm_workspace_bytes(16384, 4096, 16) == 0
    assert lib.tq2_gemm_workspace_bytes(4096, 4096, 16) == 0
    assert lib.tq2_gemm_workspace_bytes(4096, 12288, 8) == 0
    assert lib.tq2_gemm_workspace_bytes(4096, 16384, 16) == 4 * 16 * 4096 * 4
    assert lib.tq2_gemm_workspace_bytes(256, 4096, 16) % (4 * 16 * 256) == 0
    assert lib.tq2_gemm_workspace_bytes(256, 4096, 16) > 0


@no_gpu
def test_gemm_few_tokens_need_no_workspace(tq2):
    """2 to 4 tokens with K of 1, 2 or 4 chunks of 4096 run the VALU matvec
    (no workspace); other K, and more tokens, take the matrix-core plan."""
    ws = tq2.lib().tq2_gemm_workspace_bytes
    for K in (256, 4096, 4352, 8192, 16384):
        for M in (2, 3, 4):
            assert ws(256, K, M) == 0, (K, M)
    assert ws(256, 4096, 5) > 0        # five tokens: matrix cores, K split for 256 rows
    assert ws(256, 12288, 2) > 0       # three chunks: matrix cores


@no_gpu
def test_gemm_split_rule(tq2):
    """K is split only while the workgroups still fit one per CU (256 CUs):
    the workspace is splits x M x N fp32 partials, or 0 without a split.
    Below K = 16384 a wave takes 4, 2 or 1 row groups, the most that leave
    more workgroups than half the CUs, so medium N runs unsplit."""
    lib = tq2.lib()
    ws = lib.tq2_gemm_workspace_bytes
    assert ws(16384, 4096, 32) == 0                 # 256 row sets, two tiles per wave
    assert ws(16384, 4096, 64) == 0                 # 512 workgroups already
    assert ws(4096, 4096, 48) == 0                  # 192 workgroups: a split would make 384
    assert ws(4096, 16384, 16) == 4 * 16 * 4096 * 4  # 64 row sets -> 4 splits
    assert ws(4096, 16384, 32) == 4 * 32 * 4096 * 4
    assert ws(4096, 16384, 48) == 2 * 48 * 4096 * 4  # 128 workgroups -> 2 splits
    assert ws(4096, 4096, 16) == 0                   # 1 row group per wave: 256 row sets
    assert ws(4096, 4096, 32) == 0                   # 2 per wave: 128 row sets x 2 tiles
    assert ws(4608, 4096, 8) == 0                    # 2 per wave: 144 row sets
    assert ws(1024, 4096, 16) == 4 * 16 * 1024 * 4   # 1 per wave: 64 row sets -> 4 splits
    assert ws(256, 4096, 16) == 4 * 16 * 256 * 4     # 16 row sets -> 4 (every wave keeps its step)


def test_noalloc_scratch_covers_every_split(tq2):
    """tq2_gemm_noalloc's static scratch (TQ2_GEMM_SCRATCH_BYTES) holds the
    split partials of every shape: the plan splits K only while row sets x
    token groups x splits fit the 256 CUs, which bounds the partials by
    2 MiB.  Checked over a grid of shapes and token counts."""
    worst = 0
    for N in (1, 16, 64, 100, 256, 300, 1000, 1024, 2048, 4096, 8192, 16384):
        for K in (256, 1024, 4096, 4352, 16384, 65536):
            for M in (1, 2, 3, 5, 8, 16, 17, 32, 33, 48, 64, 100, 128, 256, 1024):
                worst = max(worst, tq2.tq2_gemm_workspace_bytes(N, K, M))
    assert 0 < worst <= 2 << 20 <= tq2.TQ2_GEMM_SCRATCH_BYTES
    assert "tq2_gemm_noalloc" in declared_functions()
