"""Builds libfa2.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950.

    python -m attention_forward_fa2_amd.build          # from the repository root
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfa2.so")
# Debug build for the race check: every LDS ring stage is filled with NaN
# before each refill (FA2_POISON_LDS); only the tests load it.
POISON_LIB = os.path.join(PKG, "libfa2_poison.so")
# Variant with 32x32x16 MFMAs for the D = 64 instances without dropout
# (FA2_D64_MF=32): fewer cycles per launch, but measured slower because the
# GPU holds a lower clock under it; kept for that comparison, parity-tested.
MF32_LIB = os.path.join(PKG, "libfa2_mf32.so")
SOURCES = ["fa2_api.hip", "fa2_fwd_kernel.hip"]
# Host-only library over the kernel's index arithmetic (fa2_index.h), for the
# CPU tests that check their emulation against it.
INDEX_PROBE_SRC = os.path.join(ROOT, "tests", "index_probe", "fa2_index_probe.hip")
INDEX_PROBE_LIB = os.path.join(ROOT, "tests", "index_probe", "libfa2_index_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep hipcc from emitting packed fp32 VALU ops (v_pk_*_f32).
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in ordinary VGPRs: the softmax reads them with VALU ops
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # device code only: for finite inputs no NaN ever reaches the kernel's
    # max/min (masked scores are -inf, not NaN), so fmaxf need not canonicalise
    # its MFMA-produced inputs. The host code keeps IEEE semantics, so its
    # checks of the scale and the dropout probability see NaN as NaN.
    "-Xarch_device", "-fno-honor-nans",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def build(out: str = LIB, extra_flags=None, verbose: bool = False) -> str:
    """Compile every source into ``out`` (atomically replaced)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *(extra_flags or []), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless.
    err = "\n".join(line for line in res.stderr.splitlines() if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


def build_poison(out: str = POISON_LIB, verbose: bool = False) -> str:
    """The poisoned-LDS debug library (same sources, FA2_POISON_LDS=1)."""
    return build(out, ["-DFA2_POISON_LDS=1"], verbose)


def build_index_probe(out: str = INDEX_PROBE_LIB, verbose: bool = False) -> str:
    """The host-only index probe (no GPU code)."""
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-fPIC", "-shared", "-Wall", "-I", CSRC,
           INDEX_PROBE_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
    os.replace(tmp, out)
    return out


def build_all(verbose: bool = False) -> list:
    """The library, its two variants and the index probe, compiled concurrently."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(4) as ex:
        futs = [ex.submit(build, LIB, None, verbose), ex.submit(build_poison, POISON_LIB, verbose),
                ex.submit(build, MF32_LIB, ["-DFA2_D64_MF=32"], verbose),
                ex.submit(build_index_probe, INDEX_PROBE_LIB, verbose)]
        return [f.result() for f in futs]


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description="Build libfa2.so and its two variants (poisoned LDS, 32x32x16 MFMAs) "
                                             "for gfx950.")
    ap.add_argument("--out", help="build only the main library, to this path (a variant build for comparisons)")
    ap.add_argument("--define", action="append", default=[], metavar="NAME=VALUE",
                    help="preprocessor definition for a variant build, e.g. FA2_D64_MF=32 (with --out)")
    args = ap.parse_args()
    if args.out:
        print(build(args.out, [f"-D{d}" for d in args.define], verbose=True))
    else:
        for path in build_all(verbose=True):
            print(path)
