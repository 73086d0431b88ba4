"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module draws random numbers and nothing else: it holds none of the
matvec's arithmetic (no packing, no dequantization, no quantization).  The
distributions are those of the MiniCPM4-8B-shaped decode workload: ternary
codes with P(0)=0.3, P(1)=0.4, P(2)=0.3, one fp16 block scale per 256
weights drawn from U[0.005, 0.05], and fp16 activations from N(0, 1),
optionally with 0.1% of the positions scaled by 50.

Two recipes:
  * numpy (PCG64) -- used for every size the CPU oracle checks;
  * torch on the GPU (Philox) -- used by the bench for the 1.96 GB decode
    stack, which numpy would take minutes to draw.  Host copies of any rows
    the oracle checks are taken from the same device tensors.
Draw order within one seed: codes, then scales, then x, then outlier indices.
"""
import numpy as np

BLOCK = 256


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def codes(g: np.random.Generator, N: int, K: int) -> np.ndarray:
    """Ternary codes in {0,1,2}, uint8 [N][K], mix 0.3 / 0.4 / 0.3."""
    u = g.integers(0, 10, size=(N, K), dtype=np.uint8)
    return ((u >= 3).astype(np.uint8) + (u >= 7).astype(np.uint8))


def scales(g: np.random.Generator, N: int, K: int, lo=0.005, hi=0.05) -> np.ndarray:
    """fp16 block scales [N][K/256] as float16 (round to nearest even)."""
    return g.uniform(lo, hi, size=(N, K // BLOCK)).astype(np.float16)


def activations(g: np.random.Generator, K: int) -> np.ndarray:
    """fp16 x ~ N(0, 1), float16 [K]."""
    return g.standard_normal(K).astype(np.float16)


def add_outliers(g: np.random.Generator, x: np.ndarray, frac=0.001, factor=50.0) -> np.ndarray:
    """Scale round(frac*K) distinct positions of x by `factor` (fp32, then fp16)."""
    x = x.copy()
    n_out = int(round(frac * x.size))
    idx = g.choice(x.size, size=n_out, replace=False)
    x[idx] = (x[idx].astype(np.float32) * np.float32(factor)).astype(np.float16)
    return x


def dense_weight(g: np.random.Generator, N: int, K: int, sigma=0.02) -> np.ndarray:
    """A generic real fp32 weight (not of ternary form), for the packer."""
    return (g.standard_normal((N, K)) * sigma).astype(np.float32)


def bits(a: np.ndarray) -> np.ndarray:
    """The uint16 bit patterns of a float16 array."""
    return np.ascontiguousarray(a, dtype=np.float16).view(np.uint16)


def problem(seed: int, N: int, K: int, outliers: bool = False):
    """One seeded (q, d, x) triple in the documented draw order."""
    g = rng(seed)
    q = codes(g, N, K)
    d = scales(g, N, K)
    x = activations(g, K)
    if outliers:
        x = add_outliers(g, x)
    return q, d, x


# ---- device recipe (bench only) ----

def torch_problem(seed: int, N: int, K: int, device="cuda"):
    """(q uint8 [N][K], d float16 [N][K/256], x float16 [K]) drawn on `device`
    with torch's generator seeded by `seed`; same distributions as above."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    u = torch.randint(0, 10, (N, K), dtype=torch.uint8, device=device, generator=g)
    q = (u >= 3).to(torch.uint8) + (u >= 7).to(torch.uint8)
    del u
    d = torch.empty((N, K // BLOCK), dtype=torch.float32, device=device)
    d.uniform_(0.005, 0.05, generator=g)
    d = d.to(torch.float16)
    x = torch.randn(K, dtype=torch.float32, device=device, generator=g).to(torch.float16)
    return q, d, x


def torch_activations(seed: int, K: int, device="cuda"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(K, dtype=torch.float32, device=device, generator=g).to(torch.float16)


def torch_add_outliers(seed: int, x, frac=0.001, factor=50.0):
    """Scale round(frac*K) distinct positions of x (drawn with torch's
    generator seeded by `seed`, on x's device) by `factor` in fp32, then
    round to fp16: the device form of add_outliers."""
    import torch
    g = torch.Generator(device=x.device)
    g.manual_seed(seed)
    n_out = int(round(frac * x.numel()))
    idx = torch.randperm(x.numel(), generator=g, device=x.device)[:n_out]
    x = x.clone()
    x[idx] = (x[idx].float() * factor).to(torch.float16)
    return x
