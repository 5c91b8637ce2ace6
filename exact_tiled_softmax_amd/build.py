"""Build libattn.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python exact_tiled_softmax_amd/build.py [-v]   (runs without importing the package)

Each source is compiled to an object under <repo>/_build/ (in parallel), then
linked into exact_tiled_softmax_amd/libattn.so next to this file.  The dense
MFMA kernels (dense_fwd.hip, dense_dkdv.hip, dense_dq.hip) are compiled once
per (dtype, head width) with -DETS_DT / -DETS_D, so that their instantiations
build in parallel.  Packed fp32 vector instructions are disabled for all device
code.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libattn.so")
BUILD = os.path.join(ROOT, "_build")

_PER_COMBO = ["dense_fwd.hip", "dense_dkdv.hip", "dense_dq.hip"]
_COMBOS = [(2, 128), (2, 64), (1, 128), (1, 64)]  # (dtype code: 2 = bf16, 1 = fp16; head width)
# (source, extra defines, object name), slowest first
UNITS = ([(src, [f"-DETS_DT={dt}", f"-DETS_D={d}"], f"{src[:-4]}_{dt}_{d}.o")
          for src in _PER_COMBO for dt, d in _COMBOS] +
         [(src, [], src.rsplit(".", 1)[0] + ".o")
          for src in ("sparse.hip", "dense_bwd.hip", "dense_f32.hip", "abi.cpp", "dropout.hip", "probe.hip",
                     "debug.hip")])

ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
    "-Wall", "-Wno-unused-function",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP kernels)")


def _compile(unit, verbose):
    src, defines, objname = unit
    obj = os.path.join(BUILD, objname)
    cmd = [hipcc()] + FLAGS + defines + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-x")
        cmd.insert(2, "hip")
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if verbose and msg.strip():
        print(msg)
    return obj


def build(verbose=False):
    """Compile every source and link libattn.so.  Always recompiles."""
    os.makedirs(BUILD, exist_ok=True)
    workers = max(1, min(len(UNITS), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(lambda u: _compile(u, verbose), UNITS))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
