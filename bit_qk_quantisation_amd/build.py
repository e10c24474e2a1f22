"""Build libbinattn.so (the HIP kernels and the C ABI) for gfx950, in tree.

    python -m bit_qk_quantisation_amd.build

hipcc compiles every csrc/*.hip file (in parallel, one object each) and
links them into one shared library next to this file.  Packed fp32 VALU
forms are disabled for all device code.
"""

from __future__ import annotations

import os
import pathlib
import shutil
import subprocess
import sys

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIB = PKG / "libbinattn.so"
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libbinattn.so)")


def sources():
    return sorted(str(p) for p in CSRC.glob("*.hip"))


OBJ = PKG / "_build"
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False, extra=()) -> pathlib.Path:
    """Compile every kernel and the host layer into LIB; returns its path.
    Each source compiles to its own object, in parallel (no device code
    crosses files), and one link makes the library."""
    from concurrent.futures import ThreadPoolExecutor

    OBJ.mkdir(exist_ok=True)
    tag = os.getpid()
    jobs = []
    for src in sources():
        obj = OBJ / (pathlib.Path(src).stem + f".{tag}.o")
        jobs.append((obj, [hipcc(), f"--offload-arch={ARCH}", *FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", *extra,
                           "-c", src, "-o", str(obj)]))
    workers = max(1, min(len(jobs), os.cpu_count() or 1))
    with ThreadPoolExecutor(workers) as ex:
        for f in [ex.submit(_run, cmd, verbose) for _, cmd in jobs]:
            f.result()
    tmp = LIB.with_name(LIB.name + f".tmp{tag}")
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *[str(o) for o, _ in jobs], "-o", str(tmp)],
         verbose)
    for o, _ in jobs:
        o.unlink()
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
