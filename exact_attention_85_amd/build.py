"""Compiles the HIP kernels and the C-ABI host code into libfa2.so (gfx950 only)."""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfa2.so")
# race-check build: every LDS slot is filled with NaN before its asynchronous load
POISON_LIB = os.path.join(PKG, "libfa2_poison.so")
SOURCES = [os.path.join(CSRC, n) for n in ("fa2_fwd.hip", "fa2_bwd.hip", "fa2_fp8.hip", "fa2_noalloc.hip", "fa2_probe.hip", "fa2_api.cpp")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep the compiler from emitting packed fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def build(verbose: bool = False, extra_flags=(), poison: bool = False) -> str:
    lib = POISON_LIB if poison else LIB
    extra = list(extra_flags) + (["-DFA2_POISON_LDS"] if poison else [])
    cmd = [HIPCC] + FLAGS + extra + SOURCES + ["-o", lib + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that note is harmless
    noise = "packed-fp32-ops"
    msgs = [ln for ln in (proc.stdout + proc.stderr).splitlines() if noise not in ln]
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    args = sys.argv[1:]
    build(verbose=True, extra_flags=[a for a in args if a.startswith("-") and a != "--poison"],
          poison="--poison" in args)
