"""Build libbsa.so (the HIP kernels and the C-ABI) in-tree for gfx950 with hipcc, and beside it
libbsa_peak.so (the benchmark's measured-ceiling probes, not part of the attention path).

    python -m block_sparse_attention_landmark_amd.build
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libbsa.so")
PEAK_LIB = os.path.join(PKG, "libbsa_peak.so")
PEAK_SOURCES = ["peak_probe.hip"]
SOURCES = ["bsa_api.hip", "pool.hip", "select.hip", "attend_prefill.hip", "attend_decode.hip",
           "attend_f32.hip", "attend_backward.hip", "lsa.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-result",
    # keep the compiler from forming packed float32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libbsa.so")


def _run(cmd, verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = [ln for ln in res.stderr.splitlines()
            if "packed-fp32-ops' is not a recognized feature" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    if verbose and errs:
        print("\n".join(errs), file=sys.stderr)


def _jobs() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _compile(sources, out: str, verbose: bool, defines=()) -> None:
    """Compile each source to an object file in parallel (each carries its own gfx950 code
    object), then link them into one shared library."""
    tag = os.path.splitext(os.path.basename(out))[0]
    objdir = os.path.join(PKG, "_build", tag)
    os.makedirs(objdir, exist_ok=True)
    flags = [f for f in HIPCC_FLAGS if f != "-shared"] + [f"-D{d}" for d in defines]
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in sources]
    cmds = [[hipcc(), *flags, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(sources, objs)]
    with ThreadPoolExecutor(max_workers=_jobs()) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = out + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every source into libbsa.so next to this file, and the probes into
    libbsa_peak.so; returns the path of libbsa.so."""
    _compile(SOURCES, LIB, verbose)
    _compile(PEAK_SOURCES, PEAK_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
