"""Build libpkv.so (gfx950) in-tree with hipcc: one object per source, compiled in parallel, then linked.

Usage: python -m paged_kv_cache_164_amd.build   (or call build()).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpkv.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# "-packed-fp32-ops" keeps packed-fp32 VALU instructions out of the generated code: every fp32
# operation is issued as its scalar-per-lane form.
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-mcode-object-version=5", "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# Per-file flags.  The multi-query kernel's maxima see no NaN (masked keys are -inf; values past
# a range are zeroed before any product), so fmaxf need not quiet its inputs first: without
# -fno-honor-nans every operand of a max costs an extra canonicalising v_max.
FILE_FLAGS = {"attention_prefill.hip": ["-fno-honor-nans"]}


def _compile(src: str, out_dir: str = OUT_DIR, extra=()) -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = ([HIPCC] + COMMON + FILE_FLAGS.get(os.path.basename(src), []) + [f"-I{INCLUDE}"]
           + list(extra) + lang + ["-c", src, "-o", obj])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra_flags=(), lib_path: str = LIB) -> str:
    """Compile every source in csrc/ and link ``lib_path`` (extra_flags: e.g. -D tuning knobs)."""
    out_dir = OUT_DIR if lib_path == LIB else os.path.join(os.path.dirname(lib_path), "_build")
    os.makedirs(out_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, out_dir, extra_flags), srcs))
    tmp = lib_path + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path}")
    return lib_path


# Host-only test helper: runs the kernels' address functions (csrc/pkv_tile_addr.h) on the CPU.
TILECHECK_SRC = os.path.join(os.path.dirname(HERE), "tests", "native", "tile_check.hip")
TILECHECK_LIB = os.path.join(os.path.dirname(HERE), "tests", "native", "libpkv_tilecheck.so")


def build_tilecheck(verbose: bool = False) -> str:
    cmd = [HIPCC, "--offload-host-only", "-x", "hip", "-O2", "-std=c++17", "-shared", "-fPIC",
           "-Wall", "-Wno-unused-function", f"-I{CSRC}", f"-I{INCLUDE}", TILECHECK_SRC, "-o",
           TILECHECK_LIB + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {TILECHECK_SRC}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(TILECHECK_LIB + ".tmp", TILECHECK_LIB)
    if verbose:
        print(f"built {TILECHECK_LIB}")
    return TILECHECK_LIB


if __name__ == "__main__":
    build(verbose=True)
    build_tilecheck(verbose=True)
    sys.exit(0)
