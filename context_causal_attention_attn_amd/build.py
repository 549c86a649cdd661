"""Build the HIP library ``libcpattn.so`` in-tree for gfx950.

Every HIP source under ``csrc/`` and the C ABI source are compiled by hipcc
for gfx950 only, with packed-FP32 instruction selection switched off, and
linked into one shared library next to this file. Objects go to
``_build/`` (not part of the repository). Next to the library,
``libcpattn.so.sha256`` records a digest of the sources and flags it was
built from; ``is_current()`` compares it with the sources on disk.

Usage: ``python -m context_causal_attention_attn_amd.build`` or ``build()``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_NAME = "libcpattn.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

ARCH = "gfx950"
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


STAMP_SUFFIX = ".sha256"


def sources_digest(extra_flags=()) -> str:
    """SHA-256 over every source the library is built from (kernels, C ABI,
    the public header) and the compile flags: a library whose stamp differs
    was built from other code."""
    import hashlib
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h"))
                   + glob.glob(os.path.join(CSRC, "*.cpp")) + [os.path.join(INCLUDE, "cp_attn.h")])
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    flags = [f for f in COMMON_FLAGS if f not in ("-I", INCLUDE, CSRC)]   # include paths differ per checkout
    h.update(" ".join(flags + list(extra_flags)).encode())
    return h.hexdigest()


def is_current(lib_path: str = None) -> bool:
    """True when the library exists and its stamp matches the sources."""
    lib_path = lib_path or LIB_PATH
    try:
        with open(lib_path + STAMP_SUFFIX) as fh:
            return os.path.exists(lib_path) and fh.read().strip() == sources_digest()
    except OSError:
        return False


def _hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand):
        raise RuntimeError(f"hipcc not found (looked for {cand})")
    return cand


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(hipcc: str, src: str, extra):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc, *COMMON_FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra_flags=(), out_path: str = None, build_dir: str = None) -> str:
    """Compile and link the library; returns its path. Always recompiles.
    ``extra_flags``/``out_path``/``build_dir`` build a variant elsewhere."""
    hipcc = _hipcc()
    global BUILD_DIR
    lib_path = out_path or LIB_PATH
    if build_dir:
        BUILD_DIR = build_dir
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")), 16)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(hipcc, s, list(extra_flags)), srcs))
    tmp = lib_path + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib_path)
    with open(lib_path + STAMP_SUFFIX, "w") as fh:
        fh.write(sources_digest(extra_flags) + "\n")
    if verbose:
        print(f"built {lib_path} from {len(srcs)} sources", file=sys.stderr)
    return lib_path


if __name__ == "__main__":
    print(build(verbose=True))
