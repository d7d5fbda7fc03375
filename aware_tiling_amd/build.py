"""Build the gfx950 HIP library ``libaware_tiling.so`` in-tree.

Every translation unit under ``csrc/`` is compiled by hipcc for gfx950 only
(one ``-c`` per file, in parallel), then linked into one shared object next
to this file.  Packed fp32 instruction selection is disabled for device
code (``-packed-fp32-ops``); the host pass warns that it does not know the
feature, which is harmless.

Usage: ``python -m aware_tiling_amd.build`` or ``build()`` from Python.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libaware_tiling.so")
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}",
          "-Wall", "-Wno-unused-function"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def _compile(src: str, obj: str, extra: list[str]) -> tuple[str, str]:
    is_hip = src.endswith(".hip")
    cmd = [HIPCC] + COMMON + (DEVICE + ["-x", "hip"] if is_hip else []) + extra + ["-c", src,
                                                                                   "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return src, r.stderr


def build(out: str = OUT, extra: list[str] | None = None, jobs: int = 8,
          verbose: bool = False) -> str:
    """Compile all sources and link ``out``; returns its path."""
    extra = list(extra or [])
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    objs = [os.path.join(BUILD_DIR, os.path.basename(s) + ".o") for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        for src, err in ex.map(lambda so: _compile(so[0], so[1], extra), zip(srcs, objs)):
            if verbose and err.strip():
                print(f"[{os.path.basename(src)}]\n{err}", file=sys.stderr)
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
