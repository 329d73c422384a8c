"""Build libbsa.so (the HIP kernels and the C-ABI) in-tree for gfx950 with hipcc, and beside it
libbsa_peak.so (the benchmark's measured-ceiling probes, not part of the attention path) and
libbsa_sync.so (the race-check build of the same sources: every direct-to-LDS copy fully
synchronised, for the tests that compare its bits with libbsa.so's).

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
SYNC_LIB = os.path.join(PKG, "libbsa_sync.so")
PEAK_SOURCES = ["peak_probe.hip"]
SOURCES = ["bsa_api.hip", "pool.hip", "select.hip", "attend_prefill.hip", "attend_decode.hip",
           "attend_f32.hip", "attend_backward.hip", "lsa.hip"]
# per-source code generation options (none at present)
SOURCE_FLAGS = {}

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


def _plan(sources, out: str, defines=()):
    """Compile commands (one object per source; each carries its own gfx950 code object) and
    the link command of one shared library."""
    tag = os.path.splitext(os.path.basename(out))[0]
    objdir = os.path.join(PKG, "_build", tag)
    os.makedirs(objdir, exist_ok=True)
    flags = [f for f in HIPCC_FLAGS if f != "-shared"] + [f"-D{d}" for d in defines]
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in sources]
    cmds = [[hipcc(), *flags, *SOURCE_FLAGS.get(s, []), "-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(sources, objs)]
    link = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out + ".tmp"]
    return cmds, link, out


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel) into libbsa.so next to this file, the probes into
    libbsa_peak.so and the race-check build into libbsa_sync.so; returns libbsa.so's path."""
    plans = [_plan(SOURCES, LIB), _plan(PEAK_SOURCES, PEAK_LIB),
             _plan(SOURCES, SYNC_LIB, defines=("BSA_SYNC_COPIES",))]
    with ThreadPoolExecutor(max_workers=_jobs()) as ex:
        for f in [ex.submit(_run, c, verbose) for cmds, _, _ in plans for c in cmds]:
            f.result()
    for _, link, out in plans:
        _run(link, verbose)
        os.replace(out + ".tmp", out)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
