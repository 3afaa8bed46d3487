"""Build libpagedkv.so for gfx950 in-tree with hipcc.

    python -m paged_kv_cache_435_amd.build

Every HIP source under csrc/ is compiled to an object (in parallel), then linked
into ``paged_kv_cache_435_amd/libpagedkv.so``.  No fast-math: the INT8/FP8
quantizers rely on IEEE division and round-half-even.  Packed-FP32 instruction
selection is turned off for all device code.

Denormals are kept, explicitly, for every floating-point type
(``-fdenormal-fp-math=ieee``, ``-fno-gpu-flush-denormals-to-zero``): with f16
queries, INT8 and INT4 codes enter the matrix instructions as f16 subnormals
(code + offset) * 2^-24, so a mode that flushed f16 denormals would turn every
code into zero.  The kernels' descriptors then carry denormal mode 3 (in and out
kept) for f32 and for f16/f64.
"""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpagedkv.so")
OBJ_DIR = os.path.join(PKG, "_build")

ARCH = os.environ.get("PKV_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fdenormal-fp-math=ieee", "-fno-gpu-flush-denormals-to-zero",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def build(verbose=False, out=None, defines=()):
    """Compile every csrc/*.hip and link libpagedkv.so (or ``out``).  ``defines``
    are extra -D flags (compile-time tuning knobs).  Returns the library path."""
    lib = out or LIB
    obj_dir = OBJ_DIR if out is None else out + ".objs"
    os.makedirs(obj_dir, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(obj_dir, os.path.basename(s)[:-4] + ".o") for s in sources]
    extra = [f"-D{d}" for d in defines]

    def compile_one(pair):
        src, obj = pair
        return _run([HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj])

    with ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        logs = list(ex.map(compile_one, zip(sources, objs)))
    tmp = lib + ".tmp"
    logs.append(_run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]))
    os.replace(tmp, lib)
    if verbose:
        for log in logs:
            if log.strip():
                print(log)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
