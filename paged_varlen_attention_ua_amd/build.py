"""Build libua.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Usage: python -m paged_varlen_attention_ua_amd.build  (or build() from Python).
Every kernel is compiled with packed fp32 instructions disabled.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libua.so")
BUILD_DIR = os.path.join(HERE, "_build")
# (source, object, extra flags): the two kernel files are compiled once per
# query dtype (UA_QT) so their instantiations build in parallel.
SOURCES = [
    ("ua_api.cpp", "ua_api.o", []),
    ("ua_small.hip", "ua_small_f16.o", ["-DUA_QT=0"]),
    ("ua_small.hip", "ua_small_bf16.o", ["-DUA_QT=1"]),
    ("ua_large.hip", "ua_large_f16.o", ["-DUA_QT=0"]),
    ("ua_large.hip", "ua_large_bf16.o", ["-DUA_QT=1"]),
    ("ua_reduce.hip", "ua_reduce.o", []),
    ("ua_check.hip", "ua_check.o", []),
    ("ua_noalloc.hip", "ua_noalloc.o", []),
]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument", "-Wno-pass-failed",
    f"-I{os.path.join(HERE, '..', 'include')}",
]


def _compile(entry):
    src, obj_name, extra = entry
    obj = os.path.join(BUILD_DIR, obj_name)
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *COMMON, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose=False):
    """Compile every source and link libua.so; always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
