"""Build libtq2.so in-tree with hipcc for gfx950.

Flags: -O3, no fast-math (IEEE division and rounding are part of the
definition of pack and of the int8 quantizer), packed-fp32 ops disabled,
code object v5.  Output: ternary_packed_weight_amd/libtq2.so.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtq2.so")
PROBE_LIB = os.path.join(HERE, "libtq2probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = [os.path.join(CSRC, "tq2_kernels.hip"), os.path.join(CSRC, "tq2_api.cpp")]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _hipcc(sources, out, verbose, extra=()):
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, *sources, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    errs = [l for l in res.stderr.splitlines() if "error" in l]
    if errs:
        raise RuntimeError("\n".join(errs))
    # a kernel whose host-side stub was dropped links without complaint and
    # only fails at load time: refuse undefined symbols of our own namespace
    und = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    own = [l.split()[-1] for l in und.stdout.splitlines() if "_ZN3tq2" in l]
    if und.returncode != 0 or own:
        raise RuntimeError(f"{out}: undefined library symbols: {own or und.stderr}")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False, extra=()) -> str:
    """Build libtq2.so (the library) and libtq2probe.so (bench calibration)."""
    _hipcc([os.path.join(CSRC, "tq2_probes.hip")], PROBE_LIB, verbose, extra)
    return _hipcc(SOURCES, LIB, verbose, extra)


if __name__ == "__main__":
    print(build(verbose=True))
