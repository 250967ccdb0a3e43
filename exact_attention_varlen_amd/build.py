"""Ahead-of-time build of the gfx950 attention library ``libattn_varlen.so``.

Compiles every source under ``csrc/`` with hipcc for gfx950 in parallel and
links one shared library next to this file. Usage::

    python -m exact_attention_varlen_amd.build [--jobs N] [--verbose]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libattn_varlen.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["av_api.cpp", "av_prof.cpp", "av_fwd.hip", "av_fwd_split.hip", "av_fwd_persist.hip", "av_validate.hip",
           "av_bwd.hip", "av_bwd_d256.hip", "av_noalloc.hip"]

# -Xclang -target-feature -Xclang -packed-fp32-ops keeps the device compiler from
# forming packed fp32 instructions; the host pass warns that it does not know the
# feature, which is harmless and filtered from the log below.
HIP_FLAGS = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the gfx950 library cannot be built")


def _filter(log: str) -> str:
    keep = [ln for ln in log.splitlines() if "packed-fp32-ops" not in ln or "error" in ln.lower()]
    return "\n".join(keep)


def _compile(src: str, extra, verbose: bool, build_dir: str = BUILD_DIR) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIP_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    t0 = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    log = _filter(r.stdout + r.stderr)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{log}")
    if verbose and log.strip():
        print(log, flush=True)
    if verbose:
        print(f"  {src}: {time.time() - t0:.1f}s", flush=True)
    return obj


def build(jobs: int = 0, verbose: bool = False, extra_flags=(), out: str = LIB_NAME) -> str:
    """Compile all sources for gfx950 and link ``libattn_varlen.so`` (or a variant
    named ``out`` in the same directory, built with ``extra_flags``). Returns its path."""
    if os.path.basename(out) != out or not out.endswith(".so"):
        raise ValueError("out must be a .so file name in the package directory")
    lib_path = os.path.join(HERE, out)
    build_dir = BUILD_DIR if out == LIB_NAME else os.path.join(BUILD_DIR, os.path.splitext(out)[0])
    os.makedirs(build_dir, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra_flags), verbose, build_dir), SOURCES))
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {LIB_NAME} failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path}", flush=True)
    return lib_path


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--extra", action="append", default=[], help="extra hipcc flag (repeatable)")
    ap.add_argument("--out", default=LIB_NAME, help="library file name (a variant build; default the library)")
    a = ap.parse_args(argv)
    build(a.jobs, a.verbose, a.extra, a.out)
    return 0


if __name__ == "__main__":
    sys.exit(main())
