"""Build libhils.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m long_context_sparse_hils_amd.build [--debug-sync]

--debug-sync builds libhils_debug_sync.so instead: the same sources with
HILS_DEBUG_SYNC defined, which serialises every LDS hand-off the kernels
otherwise leave to ordering (extra workgroup barriers, each LDS DMA waiting
for itself).  Its results must be bit-identical to libhils.so's.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libhils.so")
OBJ = os.path.join(HERE, "_build")
OUT_DEBUG_SYNC = os.path.join(HERE, "libhils_debug_sync.so")
OBJ_DEBUG_SYNC = os.path.join(HERE, "_build_debug_sync")
# the streaming-read reference the benchmark sets HBM-bound kernels against
OUT_HBM_REF = os.path.join(HERE, "libhils_hbm_ref.so")
ARCH = os.environ.get("HILS_OFFLOAD_ARCH", "gfx950")

SOURCES = ["summary.hip", "prefill_valu.hip", "prefill_mfma.hip", "prefill_chunks.hip", "prefill_long.hip", "score_mfma.hip", "decode.hip", "backward.hip", "backward_mfma.hip",
           "api.cpp"]

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from forming packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found")
    return p


def _compile(src: str, obj_dir: str = OBJ, extra=()) -> str:
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True, debug_sync: bool = False) -> str:
    out, obj_dir = (OUT_DEBUG_SYNC, OBJ_DEBUG_SYNC) if debug_sync else (OUT, OBJ)
    extra = ("-DHILS_DEBUG_SYNC",) if debug_sync else ()
    os.makedirs(obj_dir, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir, extra), srcs))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


def build_hbm_ref(verbose: bool = True) -> str:
    tmp = OUT_HBM_REF + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *FLAGS, "-shared", os.path.join(CSRC, "hbm_ref.hip"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT_HBM_REF)
    if verbose:
        print(f"built {OUT_HBM_REF}")
    return OUT_HBM_REF


if __name__ == "__main__":
    build(debug_sync="--debug-sync" in sys.argv[1:])
    sys.exit(0)
