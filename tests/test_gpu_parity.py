"""GPU parity: every entry point of libtq2 against the CPU oracle on the
same seeded inputs.  Bit-exact for pack, dequant, the quantizer and the int8
path; per-output tolerance 2e-3 * sum_k |d_b(k) x_k| + 1e-6 for the fp16
path.  Inputs of every matvec are packed by the oracle (never by the GPU).
"""
import numpy as np
import pytest

import oracle
from ternary_packed_weight_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def tq2():
    assert torch.cuda.is_available(), "GPU parity tests need the MI355X"
    from ternary_packed_weight_amd import tq2 as mod
    return mod


def _ternary_W(q, d):
    dd = np.repeat(d.astype(np.float32), 256, axis=1)
    return (dd * (q.astype(np.float32) - 1.0)).astype(np.float32)


def _packed(seed, N, K, outliers=False):
    q, d, x = synth.problem(seed, N, K, outliers=outliers)
    codes, scales, bad = oracle.pack(_ternary_W(q, d))
    assert bad == 0
    return q, codes, scales, x


def _to_dev(codes, scales, x=None):
    c = torch.from_numpy(codes).to(DEV)
    s = torch.from_numpy(scales.view(np.float16)).to(DEV)
    if x is None:
        return c, s
    return c, s, torch.from_numpy(np.ascontiguousarray(x, np.float16)).to(DEV)


def _l1(scales, x, N, K):
    """sum_k |d_b(k) x_k| per output (fp64)."""
    d = np.abs(scales.view(np.float16).astype(np.float64)).reshape(N, K // 256)
    ax = np.abs(x.astype(np.float64)).reshape(K // 256, 256).sum(axis=1)
    return (d * ax[None, :]).sum(axis=1)


def _tol(scales, x, N, K):
    """The fp16 path's bound: 2e-3 * sum_k |d_b(k) x_k| + 1e-6 per output."""
    return 2e-3 * _l1(scales, x, N, K) + 1e-6


# Regression bound of the fp16 matvec kernels, from their arithmetic: every
# product of a masked code (a binary16 subnormal q 4^j 2^-24) and an fp16 x
# is exact in fp32; an output then passes through at most 64 sequential fp32
# roundings (a lane's dot2 chain of 16 instructions at up to two roundings
# each, the Horner combine, the scale by d, six cross-lane levels, up to 15
# chunk sums), each within one ulp (2^-23, so no round-to-nearest is
# assumed) of partial sums no larger than 3 sum|d x| (codes q in {0,1,2}
# plus the subtracted x sum).  So |y - y_exact| <= 64 * 2^-23 * 3 sum|d x|
# < 2^-15 sum|d x|, 1/65 of the 2e-3 tolerance: a change that made the
# error 100x worse fails here while the tolerance would still pass it.
# (Measured worst: 2^-16 sum|d x|, on blocks holding activations of 3000.)
KERNEL_REL = 2.0 ** -15
WORST = {}  # test id -> worst err / tol, reported at the end of the session


def _check_f16(y_gpu, y_ref, tol, l1=None, key=None):
    err = np.abs(y_gpu.astype(np.float64) - y_ref.astype(np.float64))
    bad = np.nonzero(err > tol)[0]
    assert bad.size == 0, f"{bad.size} rows out of tolerance, first {bad[:5]}, err {err[bad[:5]]}, tol {tol[bad[:5]]}"
    if l1 is not None:
        kb = KERNEL_REL * l1 + 2.0 ** -40
        over = np.nonzero(err > kb)[0]
        assert over.size == 0, (f"{over.size} rows above the kernel's arithmetic bound 2^-15 sum|d x|, "
                                f"first {over[:5]}: err {err[over[:5]]}, bound {kb[over[:5]]}")
    ratio = float((err / tol).max())
    if key is not None:
        WORST[key] = max(WORST.get(key, 0.0), ratio)
    return ratio


def _check_gemv(y_gpu, y_ref, scales, x, N, K, key):
    """The matvec family's check: the spec tolerance and the kernel bound."""
    return _check_f16(y_gpu, y_ref, _tol(scales, x, N, K), _l1(scales, x, N, K), key)


# ------------------------------------------------------------------ pack

PACK_SHAPES = [(1, 256), (3, 768), (33, 4096), (256, 4096), (5, 16384), (7, 4352)]


@pytest.mark.parametrize("N,K", PACK_SHAPES)
def test_pack_ternary_bit_exact(tq2, N, K):
    q, d, _ = synth.problem(100 + N, N, K)
    W = _ternary_W(q, d)
    c_ref, s_ref, bad_ref = oracle.pack(W)
    c, s, bad = tq2.tq2_pack(torch.from_numpy(W).to(DEV))
    torch.cuda.synchronize()
    assert int(bad.item()) == bad_ref == 0
    assert np.array_equal(c.cpu().numpy(), c_ref)
    assert np.array_equal(s.cpu().numpy().view(np.uint16), s_ref)


@pytest.mark.parametrize("N,K", [(9, 1024), (64, 4096)])
def test_pack_generic_bit_exact(tq2, N, K):
    g = synth.rng(200 + N)
    W = synth.dense_weight(g, N, K)
    # ties: an element at exactly half the block scale, and tiny blocks whose
    # scale is a binary16 subnormal or rounds to zero
    W[0, 1] = np.float32(np.float16(np.abs(W[0, :256]).max())) / 2
    W[1, :256] *= np.float32(1e-6)
    W[2, 256:512] *= np.float32(1e-9)
    W[3, :256] = 0.0
    c_ref, s_ref, bad_ref = oracle.pack(W)
    c, s, bad = tq2.tq2_pack(torch.from_numpy(W).to(DEV))
    torch.cuda.synchronize()
    assert int(bad.item()) == bad_ref == 0
    assert np.array_equal(s.cpu().numpy().view(np.uint16), s_ref)
    assert np.array_equal(c.cpu().numpy(), c_ref)


def test_pack_bad_block_count(tq2):
    W = synth.dense_weight(synth.rng(300), 4, 1024)
    W[0, 5] = np.inf
    W[1, 600] = np.nan
    W[2, 300:310] = 1e6
    _, _, bad_ref = oracle.pack(W)
    _, _, bad = tq2.tq2_pack(torch.from_numpy(W).to(DEV))
    torch.cuda.synchronize()
    assert bad_ref == 3 and int(bad.item()) == 3


def test_dequant_exact(tq2):
    q, codes, scales, _ = _packed(310, 37, 768)
    c, s = _to_dev(codes, scales)
    W = tq2.tq2_dequant(c, s)
    torch.cuda.synchronize()
    assert np.array_equal(W.cpu().numpy(), oracle.dequant(codes, scales, 37, 768))


# ------------------------------------------------------------ fp16 matvec

# K = 12288 .. 36864 take the run-time chunk count (3, 5, 6, 7, 8, 9 chunk-waves
# per row group; 384- to 576-thread workgroups); 12000 x 12288 and
# 8192 x 12288 reach 8 and 4 rows per wave there.
GEMV_SHAPES = [(1, 256), (3, 256), (33, 768), (257, 4096), (256, 4096), (4096, 4096),
               (5, 16384), (130, 4352), (64, 8192), (1000, 16384), (17, 65536),
               (300, 12288), (70, 20480), (33, 24576), (21, 28672), (40, 32768), (9, 36864),
               (8192, 12288), (12000, 12288)]


@pytest.mark.parametrize("N,K", GEMV_SHAPES)
def test_gemv_f16_parity(tq2, N, K):
    _, codes, scales, x = _packed(400 + N + K, N, K)
    c, s, xd = _to_dev(codes, scales, x)
    y = tq2.tq2_gemv(c, s, xd)
    torch.cuda.synchronize()
    y_ref = oracle.gemv(codes, scales, N, K, synth.bits(x))
    _check_gemv(y.cpu().numpy(), y_ref, scales, x, N, K, f"gemv {N}x{K}")


@pytest.mark.parametrize("N,K", [(16384, 4096), (4096, 16384)])
def test_gemv_f16_full_size_every_output(tq2, N, K):
    """The gate/up and down shapes of the decode step in the launch
    configuration the step uses (8 rows per wave with the raised start
    priority; 4 rows per wave over four chunk-waves): every output against
    the oracle."""
    _, codes, scales, x = _packed(2500 + N, N, K)
    c, s, xd = _to_dev(codes, scales, x)
    y = tq2.tq2_gemv(c, s, xd)
    torch.cuda.synchronize()
    _check_gemv(y.cpu().numpy(), oracle.gemv(codes, scales, N, K, synth.bits(x)), scales, x, N, K,
                f"gemv full {N}x{K}")


def test_gemv_f16_outliers(tq2):
    N, K = 4096, 4096
    _, codes, scales, x = _packed(1002, N, K, outliers=True)
    assert np.abs(x.astype(np.float32)).max() > 20
    c, s, xd = _to_dev(codes, scales, x)
    y = tq2.tq2_gemv(c, s, xd)
    torch.cuda.synchronize()
    _check_gemv(y.cpu().numpy(), oracle.gemv(codes, scales, N, K, synth.bits(x)), scales, x, N, K, "gemv outliers")


def test_gemv_f16_one_hot_exact(tq2):
    """x = e_k for every k of two blocks: y = d(q-1) exactly.  Pins the field
    order of the decode, and that binary16 subnormal operands are honoured."""
    N, K = 33, 512
    q, codes, scales, _ = _packed(500, N, K)
    c, s = _to_dev(codes, scales)
    d = scales.view(np.float16).astype(np.float32)
    X = torch.zeros((K, K), dtype=torch.float16, device=DEV)
    X.fill_diagonal_(1.0)
    ys = [tq2.tq2_gemv(c, s, X[k].contiguous()) for k in range(K)]
    torch.cuda.synchronize()
    for k in range(K):
        expect = d[:, k // 256] * (q[:, k].astype(np.float32) - 1)
        assert np.array_equal(ys[k].cpu().numpy(), expect), k


def _range_activations(kind, K, g):
    """Activations that stress how the fp16 paths scale x before the products:
    a constant tiny value (2^-14 + 2^-19 - 2^-24) whose low bits a 4^-3
    down-scale would round away, every one in the same direction; tiny
    random values; blocks holding values >= 256; values near the binary16
    maximum."""
    if kind == "const_tiny":
        return np.full(K, 2.0**-14 + 2.0**-19 - 2.0**-24, np.float16)
    if kind == "tiny":
        return (g.standard_normal(K) * 2.0**-12).astype(np.float16)
    if kind == "big_blocks":
        x = synth.activations(g, K).copy()
        x[g.integers(0, K, 8)] = np.float16(3000.0)
        return x
    assert kind == "near_max"
    return (g.uniform(-1.0, 1.0, K) * 60000.0).astype(np.float16)


RANGE_KINDS = ["const_tiny", "tiny", "big_blocks", "near_max"]


@pytest.mark.parametrize("kind", RANGE_KINDS)
def test_gemv_f16_activation_ranges(tq2, kind):
    N, K = 300, 4352
    _, c, s, _ = _packed(2100, N, K)
    x = _range_activations(kind, K, synth.rng(2101))
    dc, ds, xd = _to_dev(c, s, x)
    y = tq2.tq2_gemv(dc, ds, xd)
    torch.cuda.synchronize()
    _check_gemv(y.cpu().numpy(), oracle.gemv(c, s, N, K, synth.bits(x)), s, x, N, K, f"gemv range {kind}")


def test_gemv_f16_special_values(tq2):
    N, K = 8, 1024
    q, codes, scales, x = _packed(510, N, K)
    # subnormal and large activations, and a subnormal block scale
    x = x.copy()
    x[:8] = np.array([6e-8, -6e-8, 1e-5, -3e-5, 60000, -60000, 0.0, -0.0], np.float16)
    scales = scales.copy()
    scales[0, 0] = 0x0001
    scales[1, 1] = 0x7BFF
    c, s, xd = _to_dev(codes, scales, x)
    y = tq2.tq2_gemv(c, s, xd)
    torch.cuda.synchronize()
    _check_gemv(y.cpu().numpy(), oracle.gemv(codes, scales, N, K, synth.bits(x)), scales, x, N, K,
                "gemv special values")
    # all codes 1 -> zero up to rounding: the zero point is factored out as
    # the block sum of x, so the fp16 path cancels two fp32 sums (the int8
    # path is exact)
    ones = np.full((N, K // 4), 0x55, np.uint8)
    c1, s1 = _to_dev(ones, scales)
    y = tq2.tq2_gemv(c1, s1, xd)
    torch.cuda.synchronize()
    l1 = (_tol(scales, x, N, K) - 1e-6) / 2e-3
    assert np.all(np.abs(y.cpu().numpy()) <= 1e-5 * l1)


def test_gemv_f16_negation_and_determinism(tq2):
    N, K = 300, 4096
    q, codes, scales, x = _packed(520, N, K)
    neg, _, _ = oracle.pack(_ternary_W((2 - q).astype(np.uint8), scales.view(np.float16)))
    c, s, xd = _to_dev(codes, scales, x)
    cn = torch.from_numpy(neg).to(DEV)
    y1 = tq2.tq2_gemv(c, s, xd)
    y2 = tq2.tq2_gemv(c, s, xd)
    yn = tq2.tq2_gemv(cn, s, xd)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    tol = _tol(scales, x, N, K)
    _check_gemv(yn.cpu().numpy(), -oracle.gemv(codes, scales, N, K, synth.bits(x)), scales, x, N, K, "gemv negated")
    assert np.all(np.abs((yn + y1).cpu().numpy()) <= 1e-5 * (tol - 1e-6) / 2e-3)


@pytest.mark.parametrize("N,K", [(3, 256), (100, 768), (2048, 4096), (70, 20480), (2000, 12288)])
def test_gate_up_parity(tq2, N, K):
    _, cg, sg, x = _packed(600 + N, N, K)
    _, cu, su, _ = _packed(700 + N, N, K)
    dcg, dsg, xd = _to_dev(cg, sg, x)
    dcu, dsu = _to_dev(cu, su)
    y = tq2.tq2_gemv_gate_up(dcg, dsg, dcu, dsu, xd)
    yg = tq2.tq2_gemv(dcg, dsg, xd)
    yu = tq2.tq2_gemv(dcu, dsu, xd)
    torch.cuda.synchronize()
    yc = y.cpu().numpy()
    assert yc.shape == (2, N)
    _check_gemv(yc[0], oracle.gemv(cg, sg, N, K, synth.bits(x)), sg, x, N, K, f"gate_up {N}x{K}")
    _check_gemv(yc[1], oracle.gemv(cu, su, N, K, synth.bits(x)), su, x, N, K, f"gate_up {N}x{K}")
    # same per-row arithmetic as the single matvec
    assert torch.equal(y[0], yg) and torch.equal(y[1], yu)


def test_gate_up_full_size_every_output(tq2):
    """Fused gate+up at 2 x 16384 x 4096 in the launch configuration the
    bench times (1024 workgroups): all 32768 outputs against the oracle."""
    N, K = 16384, 4096
    _, cg, sg, x = _packed(1003, N, K)
    g2 = synth.rng(1103)
    qu = synth.codes(g2, N, K)
    du = synth.scales(g2, N, K)
    cu, su, _ = oracle.pack(_ternary_W(qu, du))
    dcg, dsg, xd = _to_dev(cg, sg, x)
    dcu, dsu = _to_dev(cu, su)
    y = tq2.tq2_gemv_gate_up(dcg, dsg, dcu, dsu, xd)
    torch.cuda.synchronize()
    yc = y.cpu().numpy()
    for m, (cc, ss) in enumerate([(cg, sg), (cu, su)]):
        _check_gemv(yc[m], oracle.gemv(cc, ss, N, K, synth.bits(x)), ss, x, N, K, "gate_up full 2x16384x4096")


def test_decode_step_sampled(tq2):
    """The 224-linear decode step exactly as bench.py builds and times it
    (weights packed by tq2_pack, one HIP graph, replayed): ten sampled rows of
    every linear, re-drawn from the same seeds and packed by the oracle."""
    import bench
    stack, _ = bench.build_stack(tq2, synth, torch)
    g = bench.capture(torch, [(lambda e=e: tq2.tq2_gemv(e["codes"], e["scales"], e["x"], y=e["y"]))
                              for e in stack])
    for e in stack:
        e["y"].fill_(float("nan"))
    g.replay()
    g.replay()
    torch.cuda.synchronize()
    sel = synth.rng(6)
    worst = 0.0
    for i, e in enumerate(stack):
        l, p = divmod(i, len(bench.PROJ))
        N, K = e["N"], e["K"]
        q, d, _ = synth.torch_problem(10000 + 7 * l + p, N, K)
        rows = np.unique(np.concatenate([sel.choice(N, 8, replace=False), [0, N - 1]]))
        ri = torch.from_numpy(rows).to(DEV)
        qh, dh = q[ri].cpu().numpy(), d[ri].cpu().numpy()
        del q, d
        x = e["x"].cpu().numpy()
        codes, scales, bad = oracle.pack(_ternary_W(qh, dh))
        assert bad == 0
        ref = oracle.gemv(codes, scales, rows.size, K, synth.bits(x))
        got = e["y"].cpu().numpy()[rows]
        worst = max(worst, _check_gemv(got, ref, scales, x, rows.size, K, "decode step sampled"))
    assert worst <= 1.0


# ------------------------------------------------------------ int8 path

def test_quantize_bit_exact(tq2):
    K = 16384
    x = synth.activations(synth.rng(800), K)
    x = synth.add_outliers(synth.rng(801), x)
    for div in (100, 200, 7):
        s = np.float32(np.float32(np.abs(x.astype(np.float32)).max()) / np.float32(div))
        xq = tq2.tq2_quantize_i8(torch.from_numpy(x).to(DEV), s)
        torch.cuda.synchronize()
        assert np.array_equal(xq.cpu().numpy(), oracle.quantize_i8(synth.bits(x), s)), div


def test_quantize_ties_and_clamps(tq2):
    vals = np.array([1.25, 1.75, -1.25, -1.75, 0.25, 0.75, 63.5, 63.75, 64.0, -64.0, -64.5,
                     -63.75, 0.0, -0.0] + [0.0] * 242, np.float16)
    for s in (0.5, 3.0, 0.1, 1.0 / 3.0):
        xq = tq2.tq2_quantize_i8(torch.from_numpy(vals).to(DEV), np.float32(s))
        torch.cuda.synchronize()
        assert np.array_equal(xq.cpu().numpy(), oracle.quantize_i8(synth.bits(vals), np.float32(s))), s
    # every finite binary16 value against the oracle, for scales that put
    # many quotients exactly on or next to half-integers (powers of two,
    # thirds, tenths) and for arbitrary ones
    allh = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    allh = np.where(np.isfinite(allh), allh, np.float16(0)).astype(np.float16)
    xd = torch.from_numpy(allh).to(DEV)
    scales = [0.0371, 0.5, 1.0 / 3.0, 0.1, 2.0 ** -10, 3.0, 100.0, 1e-3, 7.0 / 1024.0, 65504.0 / 127]
    scales += list(synth.rng(8).uniform(1e-4, 1.0, 6))
    for s in scales:
        s = np.float32(s)
        xq = tq2.tq2_quantize_i8(xd, s)
        torch.cuda.synchronize()
        assert np.array_equal(xq.cpu().numpy(), oracle.quantize_i8(synth.bits(allh), s)), float(s)


def test_gemv_i8_fused_quantizer_all_fp16(tq2):
    """The quantizer inside the fused int8 matvec agrees with the oracle on
    every finite binary16 activation (K = 65280 covers 63488 of them), for
    scales with many exact ties (powers of two, 1/127), ordinary ones, one so
    small that most values clamp and one so large that most round to 0."""
    allh = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    allh = allh[np.isfinite(allh)][:65280].astype(np.float16)
    K = allh.size
    N = 8
    q, codes, scales, _ = _packed(970, N, K)
    for s in (np.float32(0.5), np.float32(0.25), np.float32(1.0 / 3.0), np.float32(0.0371),
              np.float32(0.1), np.float32(1.0 / 127.0), np.float32(2.0**-9), np.float32(1000.0)):
        c, sc, xd = _to_dev(codes, scales, allh)
        P = torch.empty((N, K // 256), dtype=torch.int32, device=DEV)
        y = tq2.tq2_gemv_i8(c, sc, xd, s)
        xq = tq2.tq2_quantize_i8(xd, s)
        y2 = tq2.tq2_gemv_i8q(c, sc, xq, s, partials=P)
        torch.cuda.synchronize()
        xq_ref = oracle.quantize_i8(synth.bits(allh), s)
        y_ref, P_ref = oracle.gemv_i8q(codes, scales, N, K, xq_ref, s)
        assert np.array_equal(P.cpu().numpy(), P_ref)
        assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.view(np.uint32)), float(s)
        assert np.array_equal(y2.cpu().numpy().view(np.uint32), y_ref.view(np.uint32)), float(s)


I8_SHAPES = [(1, 256, 100), (3, 768, 100), (33, 4096, 200), (257, 4352, 100), (4096, 16384, 100),
             (4096, 16384, 200), (11, 65280, 100),
             # run-time chunk counts 3, 5, 6, 7, 8 (384- to 512-thread workgroups)
             (300, 12288, 100), (70, 20480, 200), (33, 24576, 100), (21, 28672, 100), (40, 32768, 200),
             (8192, 12288, 100)]


@pytest.mark.parametrize("N,K,div", I8_SHAPES)
def test_gemv_i8_bit_exact(tq2, N, K, div):
    q, codes, scales, x = _packed(900 + N + div, N, K, outliers=(div == 200))
    s = np.float32(np.float32(np.abs(x.astype(np.float32)).max()) / np.float32(div))
    c, sc, xd = _to_dev(codes, scales, x)
    y = tq2.tq2_gemv_i8(c, sc, xd, s)
    xq = tq2.tq2_quantize_i8(xd, s)
    P = torch.empty((N, K // 256), dtype=torch.int32, device=DEV)
    y2 = tq2.tq2_gemv_i8q(c, sc, xq, s, partials=P)
    torch.cuda.synchronize()
    xq_ref = oracle.quantize_i8(synth.bits(x), s)
    y_ref, P_ref = oracle.gemv_i8q(codes, scales, N, K, xq_ref, s)
    assert np.array_equal(xq.cpu().numpy(), xq_ref)
    assert np.array_equal(P.cpu().numpy(), P_ref)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.view(np.uint32))
    assert np.array_equal(y2.cpu().numpy().view(np.uint32), y_ref.view(np.uint32))


def _matvec_sweep_cases(seed=11):
    """Seeded one-token shapes: N in 1..300, 300..6000 or 6000..40000, K a
    multiple of 256 up to 255 blocks (the int8 path's limit), N*K <= 2^27.
    With this seed: 1, 2, 3, 5 and 12 chunks of 4096 (the run-time chunk
    kernels among them), full and partial last chunks, 2, 4 and 8 rows per
    wave, ragged row groups."""
    g = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for nlo, nhi in ((1, 300), (300, 6000), (6000, 40000)):
        for kb in ((1, 16), (17, 64), (65, 255)):
            while True:
                N, K = int(g.integers(nlo, nhi + 1)), 256 * int(g.integers(kb[0], kb[1] + 1))
                if N * K <= 1 << 27:
                    break
            cases.append((N, K))
    return cases


@pytest.mark.parametrize("N,K", _matvec_sweep_cases())
def test_matvec_shape_sweep(tq2, N, K):
    """Seeded shapes through tq2_gemv (the fp16 bound and the kernel's own
    bound) and tq2_gemv_i8 (bit-exact: codes, partial sums, outputs)."""
    q, codes, scales, x = _packed(6000 + N, N, K)
    c, sc, xd = _to_dev(codes, scales, x)
    y = tq2.tq2_gemv(c, sc, xd)
    s = np.float32(np.float32(np.abs(x.astype(np.float32)).max()) / np.float32(100))
    yi = tq2.tq2_gemv_i8(c, sc, xd, s)
    torch.cuda.synchronize()
    _check_gemv(y.cpu().numpy(), oracle.gemv(codes, scales, N, K, synth.bits(x)), scales, x, N, K,
                f"gemv sweep {N}x{K}")
    yi_ref, _ = oracle.gemv_i8q(codes, scales, N, K, oracle.quantize_i8(synth.bits(x), s), s)
    assert np.array_equal(yi.cpu().numpy().view(np.uint32), yi_ref.view(np.uint32))


def test_gemv_i8_extreme_scales_and_one_hot(tq2):
    N, K = 5, 512
    q, codes, scales, _ = _packed(950, N, K)
    scales = scales.copy()
    scales[0, 0], scales[1, 1], scales[2, 0], scales[3, 1] = 0x7BFF, 0x0001, 0x0400, 0x3C00
    c, sc = _to_dev(codes, scales)
    s = np.float32(0.01)
    X = torch.zeros((K, K), dtype=torch.float16, device=DEV)
    X.fill_diagonal_(1.0)
    ys = [tq2.tq2_gemv_i8(c, sc, X[k].contiguous(), s) for k in range(K)]
    torch.cuda.synchronize()
    for k in range(K):
        xq = np.zeros(K, np.int8)
        xq[k] = 100
        y_ref, _ = oracle.gemv_i8q(codes, scales, N, K, xq, s)
        assert np.array_equal(ys[k].cpu().numpy().view(np.uint32), y_ref.view(np.uint32)), k


def test_gemv_i8_determinism_and_negation(tq2):
    N, K = 512, 16384
    q, codes, scales, x = _packed(960, N, K)
    neg, _, _ = oracle.pack(_ternary_W((2 - q).astype(np.uint8), scales.view(np.float16)))
    s = np.float32(np.float32(np.abs(x.astype(np.float32)).max()) / np.float32(100))
    c, sc, xd = _to_dev(codes, scales, x)
    y1 = tq2.tq2_gemv_i8(c, sc, xd, s)
    y2 = tq2.tq2_gemv_i8(c, sc, xd, s)
    yn = tq2.tq2_gemv_i8(torch.from_numpy(neg).to(DEV), sc, xd, s)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.equal(yn, -y1)


# ------------------------------------------------- fused linears, epilogues

@pytest.mark.parametrize("Ns,K", [((4096, 256, 256), 4096), ((33, 7, 130), 768), ((5, 9), 16384),
                                  ((33, 7, 130), 12288), ((5, 9), 20480), ((40, 3, 17), 32768)])
def test_fused_fp16_matches_single_calls(tq2, Ns, K):
    """q/k/v-style fusion: one kernel over up to three matrices sharing x.
    Each output equals the single-matrix call bit for bit (same per-row
    arithmetic) and is within tolerance of the oracle."""
    mats, host = [], []
    x = None
    for i, N in enumerate(Ns):
        _, c, s, xx = _packed(1300 + 7 * i + N, N, K)
        x = xx if x is None else x
        host.append((c, s))
        mats.append(_to_dev(c, s))
    xd = torch.from_numpy(x).to(DEV)
    y = tq2.tq2_gemv_fused(mats, xd)
    singles = [tq2.tq2_gemv(c, s, xd) for (c, s) in mats]
    torch.cuda.synchronize()
    off = 0
    for (c, s), ys, N in zip(host, singles, Ns):
        assert torch.equal(y[off:off + N], ys)
        _check_gemv(y[off:off + N].cpu().numpy(), oracle.gemv(c, s, N, K, synth.bits(x)), s, x, N, K,
                    f"fused {Ns}x{K}")
        off += N


@pytest.mark.parametrize("Ns,K", [((4096, 256, 256), 4096), ((16384, 16384), 4096), ((3, 65), 16384),
                                  ((33, 7, 130), 12288), ((5, 9), 20480), ((40, 3, 17), 32768)])
def test_fused_int8_bit_exact(tq2, Ns, K):
    mats, host = [], []
    x = None
    for i, N in enumerate(Ns):
        _, c, s, xx = _packed(1400 + 7 * i + N, N, K)
        x = xx if x is None else x
        host.append((c, s))
        mats.append(_to_dev(c, s))
    sc = np.float32(np.float32(np.abs(x.astype(np.float32)).max()) / np.float32(100))
    xd = torch.from_numpy(x).to(DEV)
    y = tq2.tq2_gemv_i8_fused(mats, xd, sc)
    torch.cuda.synchronize()
    yc = y.cpu().numpy()
    off = 0
    for (c, s), N in zip(host, Ns):
        ref = oracle.gemv_i8(c, s, N, K, synth.bits(x), sc)
        assert np.array_equal(yc[off:off + N].view(np.uint32), ref.view(np.uint32))
        off += N


@pytest.mark.parametrize("N,K", [(1, 256), (7, 768), (2048, 4096), (16384, 4096), (130, 16384), (9, 32768)])
def test_gate_up_silu(tq2, N, K):
    """h = silu(g)*u against the oracle: g, u each within the fp16 tolerance
    and the fp32 epilogue within a few ulp."""
    _, cg, sg, x = _packed(1500 + N, N, K)
    _, cu, su, _ = _packed(1600 + N, N, K)
    dcg, dsg, xd = _to_dev(cg, sg, x)
    dcu, dsu = _to_dev(cu, su)
    h = tq2.tq2_gemv_gate_up_silu(dcg, dsg, dcu, dsu, xd)
    torch.cuda.synchronize()
    g = oracle.gemv(cg, sg, N, K, synth.bits(x)).astype(np.float64)
    u = oracle.gemv(cu, su, N, K, synth.bits(x)).astype(np.float64)
    tg, tu = _tol(sg, x, N, K), _tol(su, x, N, K)
    href = oracle.silu_mul(g.astype(np.float32), u.astype(np.float32))
    silu = g / (1 + np.exp(-g))
    bound = 1.1 * tg * (np.abs(u) + tu) + (np.abs(silu) + 1.1 * tg) * tu + 1e-5 * np.abs(href) + 1e-6
    err = np.abs(h.cpu().numpy().astype(np.float64) - href)
    assert np.all(err <= bound), (np.argmax(err / bound), float((err / bound).max()))


@pytest.mark.parametrize("N,K,div_in,s_out", [(4096, 16384, 100, 0.05), (33, 768, 200, 0.002), (5, 4352, 100, 0.5)])
def test_int8_requant_bit_exact(tq2, N, K, div_in, s_out):
    _, c, s, x = _packed(1700 + N, N, K, outliers=(div_in == 200))
    s_in = np.float32(np.float32(np.abs(x.astype(np.float32)).max()) / np.float32(div_in))
    dc, ds, xd = _to_dev(c, s, x)
    yq, yd = tq2.tq2_gemv_i8_requant(dc, ds, xd, s_in, np.float32(s_out))
    torch.cuda.synchronize()
    y_ref = oracle.gemv_i8(c, s, N, K, synth.bits(x), s_in)
    yq_ref, yd_ref = oracle.requant_i8(y_ref, np.float32(s_out))
    assert np.array_equal(yq.cpu().numpy(), yq_ref)
    assert np.array_equal(yd.cpu().numpy().view(np.uint32), yd_ref.view(np.uint32))
    if s_out == 0.002:
        assert np.count_nonzero(np.abs(yq_ref.astype(np.int32)) >= 127) > 0   # saturation exercised


# ------------------------------------------------------------ several tokens

GEMM_SHAPES = [(256, 4096, 16), (33, 768, 5), (4096, 4096, 2), (1000, 1280, 17), (64, 256, 1),
               (4096, 16384, 16), (16384, 4096, 8), (7, 65280, 3), (300, 4352, 33),
               (4096, 16384, 20), (16384, 4096, 40),
               (16384, 4096, 4),   # fewest tokens that stage x through LDS on a large shape
               (300, 4352, 100),   # seven token tiles, the last one ragged
               # fewer row groups per wave below 16384 columns: 2 per wave, K unsplit;
               # 1 per wave over 3 and 2 load batches; 1 per wave, K split in 4, ragged N
               (4608, 4096, 8), (4096, 12288, 8), (4096, 8192, 16), (1001, 4096, 7)]


@pytest.mark.parametrize("N,K,M", GEMM_SHAPES)
def test_gemm_parity(tq2, N, K, M):
    """Y = X W^T for M tokens against the oracle (one matvec per token), with
    the fp16-path tolerance per output; tiles of 16 tokens, ragged N and K
    not a multiple of the split all covered."""
    _, c, s, _ = _packed(1800 + N + M, N, K)
    g = synth.rng(1900 + M)
    X = np.stack([synth.activations(g, K) for _ in range(M)])
    dc, ds = _to_dev(c, s)
    Xd = torch.from_numpy(np.ascontiguousarray(X, np.float16)).to(DEV)
    Y = tq2.tq2_gemm(dc, ds, Xd)
    torch.cuda.synchronize()
    ref = oracle.gemm(c, s, N, K, synth.bits(X))
    Yc = Y.cpu().numpy()
    for m in range(M):
        _check_f16(Yc[m], ref[m], _tol(s, X[m], N, K), key=f"gemm {N}x{K} M={M}")


# (N, K, M): the batched int8 matvec's plans (row groups per wave 4, 2, 1;
# 4- and 8-wave workgroups; K split or not; one or two steps per load batch;
# x_q through LDS or per lane), ragged N and token tiles, K up to the int8
# limit, and M = 1 (the one-token kernel)
GEMM_I8_SHAPES = [(16384, 4096, 16), (4096, 16384, 16), (4096, 4096, 8), (4608, 4096, 5), (256, 4096, 16),
                  (33, 768, 3), (1000, 1280, 17), (3, 256, 40), (7, 65280, 3), (4096, 12288, 2),
                  (300, 4352, 33), (16384, 4096, 1), (16384, 4096, 32),
                  # 2 to 4 tokens on the one-pass int8 matvec (1, 2 and 4 chunks,
                  # partial last chunks, ragged rows, 16384x4096 at 3 on its 24 MiB
                  # cap); 16384x4096 at 4 and 4096x16384 at 3 past it
                  (4096, 4096, 2), (4096, 4096, 4), (16384, 4096, 2), (4096, 16384, 2),
                  (257, 4352, 2), (1001, 7936, 4), (16384, 4096, 3), (16384, 4096, 4), (4096, 16384, 3)]


@pytest.mark.parametrize("N,K,M", GEMM_I8_SHAPES)
def test_gemm_i8q_bit_exact(tq2, N, K, M):
    """tq2_gemm_i8q against the oracle and against tq2_gemv_i8q on every
    token, bit for bit, with a workspace exactly as large as asked for."""
    _, c, s_, x = _packed(7000 + N + M, N, K)
    g = synth.rng(7100 + M)
    X = np.stack([synth.activations(g, K) for _ in range(M)])
    s = np.float32(np.float32(np.abs(X.astype(np.float32)).max()) / np.float32(100))
    XQ = np.stack([oracle.quantize_i8(synth.bits(X[m]), s) for m in range(M)])
    dc, ds = _to_dev(c, s_)
    XQd = torch.from_numpy(XQ).to(DEV)
    # all M tokens quantized in one call, bit-equal to the oracle per token
    XQg = tq2.tq2_quantize_i8(torch.from_numpy(np.ascontiguousarray(X, np.float16)).to(DEV), s)
    assert XQg.shape == (M, K) and np.array_equal(XQg.cpu().numpy(), XQ)
    need = tq2.tq2_gemm_i8q_workspace_bytes(N, K, M)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV) if need else None
    Y = tq2.tq2_gemm_i8q(dc, ds, XQd, s, ws=ws)
    Y2 = tq2.tq2_gemm_i8q(dc, ds, XQd, s, ws=ws)
    ys = [tq2.tq2_gemv_i8q(dc, ds, XQd[m].contiguous(), s) for m in range(min(M, 4))]
    torch.cuda.synchronize()
    ref = oracle.gemm_i8q(c, s_, N, K, XQ, s)
    Yc = Y.cpu().numpy()
    assert np.array_equal(Yc.view(np.uint32), ref.view(np.uint32))
    assert torch.equal(Y, Y2)
    for m, y in enumerate(ys):
        assert np.array_equal(y.cpu().numpy().view(np.uint32), Yc[m].view(np.uint32))


def test_gemm_i8q_tokens_independent_and_extreme_scales(tq2):
    """A token's output does not depend on the other tokens (a permutation of
    the tokens permutes the outputs, bit for bit); scales at the top and
    bottom of binary16 and saturated activations stay exact."""
    N, K, M = 4096, 4096, 16
    _, c, s_, _ = _packed(7200, N, K)
    s_ = s_.copy()
    s_[0, 0], s_[1, 1], s_[17, 3], s_[4095, 15] = 0x7BFF, 0x0001, 0x7BFF, 0x0400
    g = synth.rng(7201)
    XQ = g.integers(-128, 128, size=(M, K), dtype=np.int8)
    XQ[3, :] = 127
    XQ[4, :] = -128
    s = np.float32(0.02)
    dc, ds = _to_dev(c, s_)
    Y = tq2.tq2_gemm_i8q(dc, ds, torch.from_numpy(XQ).to(DEV), s)
    perm = np.array([5, 2, 15, 0, 9, 3, 1, 4, 14, 6, 8, 13, 7, 10, 12, 11])
    Yp = tq2.tq2_gemm_i8q(dc, ds, torch.from_numpy(np.ascontiguousarray(XQ[perm])).to(DEV), s)
    torch.cuda.synchronize()
    ref = oracle.gemm_i8q(c, s_, N, K, XQ, s)
    assert np.array_equal(Y.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    assert torch.equal(Yp, Y[torch.from_numpy(perm).to(DEV)])


def _gemm_sweep_cases(seed=7):
    """Seeded shapes for the batched planner, one per (N range, M range):
    N in 1..300, 1000..6000 or 8000..20000; M = 1, 2..4, 5..16 or 17..40;
    K a multiple of 256 up to 64 blocks; N*K <= 2^26 and N*K*M <= 2^30, so
    that the oracle finishes in seconds.  With this seed the plans include
    the one-token kernel, the one-pass few-token matvec, the matrix cores
    with 1, 2 and 4 row groups per wave, K split and unsplit, one and two
    steps per load batch, x through LDS and through registers."""
    g = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for nlo, nhi in ((1, 300), (1000, 6000), (8000, 20000)):
        for mlo, mhi in ((1, 1), (2, 4), (5, 16), (17, 40)):
            while True:
                N, K = int(g.integers(nlo, nhi + 1)), 256 * int(g.integers(1, 65))
                M = int(g.integers(mlo, mhi + 1))
                if N * K <= 1 << 26 and N * K * M <= 1 << 30:
                    break
            cases.append((N, K, M))
    return cases


@pytest.mark.parametrize("N,K,M", _gemm_sweep_cases())
def test_gemm_plan_sweep(tq2, N, K, M):
    """Random shapes and token counts through every route of the batched
    planner (one-token kernel, one-pass few-token matvec, matrix cores with
    1, 2 or 4 row groups per wave, K split or not, one or two token tiles,
    x through LDS or registers) against the oracle, and a repeated call
    bitwise identical."""
    _, c, s, _ = _packed(5000 + N + M, N, K)
    g = synth.rng(5100 + M)
    X = np.stack([synth.activations(g, K) for _ in range(M)])
    dc, ds = _to_dev(c, s)
    Xd = torch.from_numpy(np.ascontiguousarray(X, np.float16)).to(DEV)
    Y = tq2.tq2_gemm(dc, ds, Xd)
    Y2 = tq2.tq2_gemm(dc, ds, Xd)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2)
    ref = oracle.gemm(c, s, N, K, synth.bits(X))
    Yc = Y.cpu().numpy()
    for m in range(M):
        _check_f16(Yc[m], ref[m], _tol(s, X[m], N, K), key=f"gemm sweep {N}x{K} M={M}")


@pytest.mark.parametrize("N,K", [(4096, 16384), (4096, 4096)])
def test_gemm_token_independence_and_determinism(tq2, N, K):
    """A token's output does not depend on the other tokens of the call, and
    repeated calls are bitwise identical (split partials added in order).
    16 tokens (matrix cores) and 5 tokens (matrix cores, x loaded per lane)
    give the same bits for a token; 1 and 2 tokens run the VALU matvec
    kernels, bit-equal to tq2_gemv, and within the fp16 tolerance of the
    matrix-core result.  4096x16384 runs 4 row groups per wave with K split
    in 4; 4096x4096 one row group per wave, K unsplit."""
    _, c, s, _ = _packed(1950, N, K)
    g = synth.rng(1951)
    X = np.stack([synth.activations(g, K) for _ in range(16)])
    dc, ds = _to_dev(c, s)
    Xd = torch.from_numpy(np.ascontiguousarray(X, np.float16)).to(DEV)
    Y1 = tq2.tq2_gemm(dc, ds, Xd)
    Y2 = tq2.tq2_gemm(dc, ds, Xd)
    Y5 = tq2.tq2_gemm(dc, ds, Xd[1:6].contiguous())
    Y3 = tq2.tq2_gemm(dc, ds, Xd[4:6].contiguous())
    Y4 = tq2.tq2_gemm(dc, ds, Xd[5:6].contiguous())
    Yv = tq2.tq2_gemv(dc, ds, Xd[5].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)
    assert torch.equal(Y1[5], Y5[4])
    assert torch.equal(Y3[1], Yv)
    assert torch.equal(Y4[0], Yv)
    assert tq2.tq2_gemm_workspace_bytes(N, K, 1) == 0
    assert tq2.tq2_gemm_workspace_bytes(N, K, 2) == 0
    _check_f16(Y1[5].cpu().numpy(), Yv.cpu().numpy().astype(np.float64), 2 * _tol(s, X[5], N, K))


# (N, K, M, one-pass VALU route): 2 to 4 tokens take it for K of 1, 2 or 4
# chunks while all workgroups together stage at most 32 MiB of activations;
# the others take the matrix cores
FEW_TOKEN_SHAPES = [(16384, 4096, 2, True), (16384, 4096, 3, False), (16384, 4096, 4, False),
                    (4096, 16384, 2, True), (4096, 16384, 4, False), (4096, 4096, 4, True),
                    (1001, 8192, 3, True), (257, 4352, 2, True), (256, 4096, 3, True),
                    (33, 768, 4, True), (3, 256, 2, True), (4096, 12288, 3, False)]


@pytest.mark.parametrize("N,K,M,valu", FEW_TOKEN_SHAPES)
def test_gemm_few_tokens_equal_gemv(tq2, N, K, M, valu):
    """2 to 4 tokens on the one-pass VALU matvec (each code word masked once
    for all tokens): every token's output equals tq2_gemv's on that token bit
    for bit (fewer rows per wave than tq2_gemv, same per-row sums), and no
    workspace is needed.  Every route: the oracle's output within the fp16
    tolerance."""
    _, c, s, _ = _packed(2600 + N + M, N, K)
    g = synth.rng(2700 + M)
    X = np.stack([synth.activations(g, K) for _ in range(M)])
    dc, ds = _to_dev(c, s)
    Xd = torch.from_numpy(np.ascontiguousarray(X, np.float16)).to(DEV)
    need = tq2.tq2_gemm_workspace_bytes(N, K, M)
    ws = torch.empty(max(256, need), dtype=torch.uint8, device=DEV)
    Y = tq2.tq2_gemm(dc, ds, Xd, ws=ws)
    Yv = [tq2.tq2_gemv(dc, ds, Xd[m].contiguous()) for m in range(M)]
    torch.cuda.synchronize()
    ref = oracle.gemm(c, s, N, K, synth.bits(X))
    Yc = Y.cpu().numpy()
    if valu:
        assert need == 0
        for m in range(M):
            assert torch.equal(Y[m], Yv[m]), (N, K, M, m)
    for m in range(M):
        _check_f16(Yc[m], ref[m], _tol(s, X[m], N, K), key=f"gemm few {N}x{K} M={M}")


@pytest.mark.parametrize("M", [3, 17])
@pytest.mark.parametrize("kind", RANGE_KINDS)
def test_gemm_activation_ranges(tq2, kind, M):
    """The batched path scales its B operands per (token, block); tiny
    activations must come through exactly and large ones within tolerance.
    3 tokens: x loaded per lane; 17: x staged through LDS, two tiles."""
    N, K = 300, 4352
    _, c, s, _ = _packed(2200, N, K)
    g = synth.rng(2201)
    X = np.stack([_range_activations(kind, K, g) for _ in range(M)])
    dc, ds = _to_dev(c, s)
    Y = tq2.tq2_gemm(dc, ds, torch.from_numpy(np.ascontiguousarray(X, np.float16)).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.gemm(c, s, N, K, synth.bits(X))
    Yc = Y.cpu().numpy()
    for m in range(M):
        _check_f16(Yc[m], ref[m], _tol(s, X[m], N, K), key=f"gemm range {kind} M={M}")


def test_graph_capture_replay(tq2):
    """The entry points captured in one HIP graph (torch's graph API) and
    replayed three times, with new inputs copied into the captured buffers and
    the same calls run eagerly between the replays: every replay equals the
    eager result on the same inputs bit for bit (all kernels are
    deterministic).  Covers the split-K batched path (workspace plus the
    reduce kernel), the two-tile batched path, the few-token one-pass
    matvec (2 tokens at 4096x16384, whose LDS needs the raised limit) and
    the batched int8 matvec (split K into int64 partials; x_q through LDS)."""
    (_, ca, sa, _), (_, cb, sb, _), (_, cc, scc, _) = (
        _packed(2300, 256, 4096), _packed(2301, 4096, 16384), _packed(2302, 1000, 1280))
    (dca, dsa), (dcb, dsb), (dcc, dsc) = _to_dev(ca, sa), _to_dev(cb, sb), _to_dev(cc, scc)
    f16 = dict(dtype=torch.float16, device=DEV)
    xa, xb = torch.empty(4096, **f16), torch.empty(16384, **f16)
    Xb, Xc, X2 = torch.empty((20, 16384), **f16), torch.empty((5, 1280), **f16), torch.empty((2, 16384), **f16)
    ya, ygu, hh = (torch.empty(256, device=DEV), torch.empty((2, 256), device=DEV),
                   torch.empty(256, device=DEV))
    yi8, Yb, Yc = torch.empty(4096, device=DEV), torch.empty((20, 4096), device=DEV), torch.empty(
        (5, 1000), device=DEV)
    Y2 = torch.empty((2, 4096), device=DEV)
    XQa, XQb = (torch.empty((16, 4096), dtype=torch.int8, device=DEV),
                torch.empty((8, 16384), dtype=torch.int8, device=DEV))
    YQa, YQb = torch.empty((16, 256), device=DEV), torch.empty((8, 4096), device=DEV)
    wsq = torch.empty(max(256, tq2.tq2_gemm_i8q_workspace_bytes(256, 4096, 16)), dtype=torch.uint8, device=DEV)
    assert tq2.tq2_gemm_i8q_workspace_bytes(256, 4096, 16) > 0  # int64 split sums and their reduce
    assert tq2.tq2_gemm_workspace_bytes(4096, 16384, 2) == 0  # the one-pass few-token route
    wsb = torch.empty(max(256, tq2.tq2_gemm_workspace_bytes(4096, 16384, 20)), dtype=torch.uint8, device=DEV)
    wsc = torch.empty(max(256, tq2.tq2_gemm_workspace_bytes(1000, 1280, 5)), dtype=torch.uint8, device=DEV)
    assert tq2.tq2_gemm_workspace_bytes(4096, 16384, 20) > 0  # split K (and two tiles) in the graph
    s_in = np.float32(0.03)

    def run():
        tq2.tq2_gemv(dca, dsa, xa, y=ya)
        tq2.tq2_gemv_gate_up(dca, dsa, dca, dsa, xa, y=ygu)
        tq2.tq2_gemv_gate_up_silu(dca, dsa, dca, dsa, xa, h=hh)
        tq2.tq2_gemv_i8(dcb, dsb, xb, s_in, y=yi8)
        tq2.tq2_gemm(dcb, dsb, Xb, y=Yb, ws=wsb)
        tq2.tq2_gemm(dcc, dsc, Xc, y=Yc, ws=wsc)
        tq2.tq2_gemm(dcb, dsb, X2, y=Y2)
        tq2.tq2_gemm_i8q(dca, dsa, XQa, s_in, y=YQa, ws=wsq)
        tq2.tq2_gemm_i8q(dcb, dsb, XQb, s_in, y=YQb)

    outs = [ya, ygu, hh, yi8, Yb, Yc, Y2, YQa, YQb]

    def fill(seed):
        g = synth.rng(seed)
        for t in (xa, xb, Xb, Xc, X2):
            vals = np.stack([synth.activations(g, t.shape[-1]) for _ in range(t.numel() // t.shape[-1])])
            t.copy_(torch.from_numpy(vals.reshape(t.shape)))
        for t in (XQa, XQb):
            t.copy_(torch.from_numpy(g.integers(-128, 128, size=tuple(t.shape), dtype=np.int8)))

    fill(2310)
    run()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        fill(2320 + rep)
        graph.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        run()
        torch.cuda.synchronize()
        for name, a, b in zip(["gemv", "gate_up", "silu", "i8", "gemm_splitk_2tile", "gemm", "gemm_few",
                               "gemm_i8q_splitk", "gemm_i8q"], got, outs):
            assert torch.equal(a, b), (rep, name)


def test_side_stream(tq2):
    """Calls on a non-default stream (passed explicitly) give the same bits as
    on the default stream (the matvec, the batched fp16 and int8 calls)."""
    N, K, M = 4096, 4096, 3
    _, c, s, x = _packed(2400, N, K)
    dc, ds, xd = _to_dev(c, s, x)
    X = torch.stack([xd, xd.flip(0), xd * 0.5]).contiguous()
    XQ3 = tq2.tq2_quantize_i8(X, 0.05)   # 3 tokens: the one-pass int8 matvec
    XQ16 = tq2.tq2_quantize_i8(torch.cat([X] * 6)[:16].contiguous(), 0.05)  # the int8 matrix cores
    y0 = tq2.tq2_gemv(dc, ds, xd)
    Y0 = tq2.tq2_gemm(dc, ds, X)
    Q0, Q16 = tq2.tq2_gemm_i8q(dc, ds, XQ3, 0.05), tq2.tq2_gemm_i8q(dc, ds, XQ16, 0.05)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    y1 = torch.empty_like(y0)
    Y1 = torch.empty_like(Y0)
    Q1, Q17 = torch.empty_like(Q0), torch.empty_like(Q16)
    ws = torch.empty(max(256, tq2.tq2_gemm_workspace_bytes(N, K, M)), dtype=torch.uint8, device=DEV)
    wsq = torch.empty(max(256, tq2.tq2_gemm_i8q_workspace_bytes(N, K, 16)), dtype=torch.uint8, device=DEV)
    tq2.tq2_gemv(dc, ds, xd, y=y1, stream=st)
    tq2.tq2_gemm(dc, ds, X, y=Y1, ws=ws, stream=st)
    tq2.tq2_gemm_i8q(dc, ds, XQ3, 0.05, y=Q1, stream=st)
    tq2.tq2_gemm_i8q(dc, ds, XQ16, 0.05, y=Q17, ws=wsq, stream=st)
    st.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    assert torch.equal(Y0, Y1)
    assert torch.equal(Q0, Q1) and torch.equal(Q16, Q17)
