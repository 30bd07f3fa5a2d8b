"""Build libhils.so (the HiLS HIP library) for gfx950 with hipcc, in-tree.

python -m chunk_wise_sparse_amd.csrc.build   (or build() from Python)
Objects go to csrc/_build/, the library to chunk_wise_sparse_amd/libhils.so.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
SOURCES = ["hils_api.hip", "qcal.hip", "select.hip", "select_fast.hip", "attention.hip", "decode.hip",
           "dense.hip", "backward.hip", "pad.hip", "local.hip", "hope.hip", "gchunk.hip", "landmark.hip"]
LIB = os.path.join(PKG, "libhils.so")
# Per-file flags.  Selection and attention take finite scores only, so NaN handling is dropped
# there (max/min then need no NaN quieting of their operands).
FILE_FLAGS = {
    # MFMA results in ordinary VGPRs (no accumulation-register copies before the VALU work)
    "select_fast.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"],
    "attention.hip": ["-fno-honor-nans"],
    "dense.hip": ["-fno-honor-nans"],
    "backward.hip": ["-fno-honor-nans"],
}
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    # keep packed fp32 instructions out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return path


def _compile(src: str, obj: str, extra) -> str:
    cmd = [hipcc(), *CFLAGS, *extra, "-c", os.path.join(HERE, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, extra=()) -> str:
    out_dir = os.path.join(HERE, "_build")
    os.makedirs(out_dir, exist_ok=True)
    objs = [os.path.join(out_dir, s.replace(".hip", ".o")) for s in SOURCES]
    jobs = min(len(SOURCES), os.cpu_count() or 1, 8)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda so: _compile(so[0], so[1], FILE_FLAGS.get(so[0], []) + list(extra)),
                    zip(SOURCES, objs)))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
