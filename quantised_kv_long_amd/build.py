"""Build the HIP library ``libkvq.so`` in-tree for gfx950.

Usage: ``python -m quantised_kv_long_amd.build`` (or ``build()`` from Python).
Every source under ``csrc/`` is compiled by hipcc in one invocation.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkvq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # code object v5: loadable by the HIP runtime that ships with torch as well
    # as by the system one
    "-mcode-object-version=5",
    # never emit packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # binary32 division and square root stay correctly rounded (the quantiser
    # depends on it); this is hipcc's default, stated explicitly
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math",
    # LDS tiles are written and read through different pointer types
    "-fno-strict-aliasing",
    # matrix-core results and accumulators in ordinary VGPRs (the VGPR form of
    # v_mfma): no accumulator-register copies around every use, and the
    # head_dim-128 decode kernels fit in 256 registers (two waves per SIMD)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    # the first kernel-argument dwords (up to the 14 free user SGPRs) arrive in
    # scalar registers instead of being loaded from the argument buffer: the
    # merge kernel takes scalar arguments so that it reads no argument from
    # memory (struct arguments are not preloaded; a launch on a part without
    # preloading runs the compiler's load-and-branch preamble instead)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


PROBE_SRC = os.path.join(PKG, "probe", "stream_read.hip")
PROBE_LIB = os.path.join(PKG, "libkvq_probe.so")
TIMELINE_SRC = os.path.join(PKG, "probe", "timeline.hip")
TIMELINE_LIB = os.path.join(PKG, "libkvq_timeline.so")


def _hipcc(srcs: list[str], out: str, extra: list[str] | None, verbose: bool) -> str:
    cmd = [HIPCC, *HIP_FLAGS, *(extra or []), f"-I{INCLUDE}", f"-I{CSRC}", *srcs, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(out + ".tmp", out)
    return out


def build(out: str = LIB, extra: list[str] | None = None, verbose: bool = False) -> str:
    """The decode-path library: every csrc/*.hip and *.cpp."""
    return _hipcc(sources(), out, extra, verbose)


def build_probe(out: str = PROBE_LIB, verbose: bool = False) -> str:
    """The streaming-read probe the benchmark measures the achievable HBM
    read bandwidth with (not part of the decode path)."""
    return _hipcc([PROBE_SRC], out, None, verbose)


def build_timeline(out: str = TIMELINE_LIB, verbose: bool = False) -> str:
    """The library again, with the attention kernel's per-workgroup timeline
    (probe/timeline.hip compiles csrc/decode_mfma.hip with the timeline points
    defined; not part of the decode path)."""
    srcs = [TIMELINE_SRC if os.path.basename(f) == "decode_mfma.hip" else f for f in sources()]
    return _hipcc(srcs, out, None, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_probe(verbose=True))
    print(build_timeline(verbose=True))
