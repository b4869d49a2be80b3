"""Builds libtokengate.so (the C-ABI library) in-tree with hipcc for gfx950.

    python -m learned_token_pruning_scorer_amd.build

Every HIP source is compiled to an object and linked into one shared library next
to this file.  Packed-FP32 instructions are disabled for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB_NAME = "libtokengate.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["tg_api.hip", "tg_score.hip", "tg_select.hip", "tg_gather.hip", "tg_attention.hip",
           "tg_attention_bwd.hip", "tg_qkv.hip", "tg_check.hip"]
# The debug library: the same sources with TG_DEBUG, whose attention entry points also
# check that pos is strictly increasing (synchronising the stream) before launching.
DEBUG_LIB_NAME = "libtokengate_debug.so"
DEBUG_LIB_PATH = os.path.join(HERE, DEBUG_LIB_NAME)
ARCH = "gfx950"
# Per-source extra flags.  The attention kernel's inputs are finite by contract; without
# NaN semantics the compiler does not re-canonicalise every MFMA result before taking a
# max, which halves the vector instructions of the row max.
EXTRA_FLAGS = {"tg_attention.hip": ["-fno-honor-nans"]}


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def common_flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        "-Wno-unused-command-line-argument",
    ]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def _build_lib(cc, obj_dir, lib_path, defines):
    os.makedirs(obj_dir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(obj_dir, src.replace(".hip", ".o"))
        _run([cc, *common_flags(), *defines, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    workers = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8"))))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = lib_path + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, lib_path)


def build(verbose: bool = False, debug: bool = True) -> str:
    """Builds libtokengate.so and (debug=True) libtokengate_debug.so; returns the first's path."""
    cc = hipcc()
    _build_lib(cc, os.path.join(HERE, "_build"), LIB_PATH, [])
    if verbose:
        print(f"built {LIB_PATH}")
    if debug:
        _build_lib(cc, os.path.join(HERE, "_build", "debug"), DEBUG_LIB_PATH, ["-DTG_DEBUG"])
        if verbose:
            print(f"built {DEBUG_LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
