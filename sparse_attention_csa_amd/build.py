"""Build libcsa.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Usage: python -m sparse_attention_csa_amd.build [-v]
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcsa.so")

SOURCES = ["api.cpp", "profile.cpp", "compress.hip", "indexer.hip", "attend.hip", "attend_mfma.hip", "attend_rows.hip",
           "indexer_mfma.hip", "topk.hip", "noalloc.hip"]

ARCH = os.environ.get("CSA_OFFLOAD_ARCH", "gfx950")

# packed-fp32 instructions are disabled for all device code
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", INCLUDE, "-I", CSRC,
]


# per-source extra flags.  The indexer scan keeps its MFMA results in VGPRs
# (its in-lane epilogue reads every result; accumulation registers would
# need a copy per value).
EXTRA = {"indexer_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         # LDS reads clustered ahead of the products that consume them
         "attend_rows.hip": ["-mllvm", "-amdgpu-sched-strategy=max-memory-clause"]}


def hipcc():
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found")
    return p


def _compile(src, verbose):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc(), *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).strip()
    # the host pass does not know the packed-fp32 feature; that note is harmless
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n" + "\n".join(lines))
    return obj, "\n".join(lines)


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    for obj, log in results:
        if log and verbose:
            print(log)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
