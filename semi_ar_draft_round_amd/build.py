"""Build libdspark.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m semi_ar_draft_round_amd.build

Compiles every csrc/*.hip with hipcc (one object per source, in parallel)
and links them into one shared library next to this file.  No GPU is
needed: hipcc cross-compiles for gfx950.
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libdspark.so")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    f"--offload-arch={ARCH}",
    # never let the compiler form packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the gfx feature flag; that warning is noise
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def build(verbose: bool = False, csrc: str = CSRC, out: str = LIB) -> str:
    """Compile every source of `csrc` to an object (in parallel), then link
    the shared library `out`."""
    import concurrent.futures
    import tempfile
    sources = sorted(glob.glob(os.path.join(csrc, "*.hip")))
    compile_flags = [f for f in FLAGS if f != "-shared"]
    with tempfile.TemporaryDirectory(prefix="dspark_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in sources]
        jobs = min(len(sources), max(1, min(16, os.cpu_count() or 1)))
        with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
            futs = [ex.submit(_run, [hipcc(), *compile_flags, f"-I{INCLUDE}", "-c", "-o", obj, src], verbose)
                    for src, obj in zip(sources, objs)]
            for f in futs:
                f.result()
        tmp = out + ".tmp"
        _run([hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs], verbose)
        os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
