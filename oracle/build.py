"""Compile the CPU oracle (test infrastructure) into oracle/liboracle.so.

Plain C, -O2, no fast-math, no FMA contraction, OpenMP over rows only.
build(sanitize=True) writes a second library instrumented with
AddressSanitizer and UndefinedBehaviorSanitizer (host code only; it is
loaded by a test under the sanitizer runtime, never by the default path).
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "tq2_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
SAN_LIB = os.path.join(HERE, "liboracle_san.so")
CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
          "-fPIC", "-shared", "-Wall", "-Wextra"]
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = SAN_LIB if sanitize else LIB
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *(SAN_FLAGS if sanitize else []), SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def asan_runtime() -> str:
    """Path of gcc's AddressSanitizer runtime (to preload into a Python
    process that loads the instrumented library)."""
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()


if __name__ == "__main__":
    print(build(verbose=True))
