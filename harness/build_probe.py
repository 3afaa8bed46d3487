"""Build the streaming yardstick kernels (``harness/libpkvprobe.so``) for gfx950,
with the library's compile flags.  Not part of the attention path.

    python -m harness.build_probe
"""
import os
import sys

from paged_kv_cache_435_amd import build as _lib_build

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc", "pkv_probe.hip")
LIB = os.path.join(HERE, "libpkvprobe.so")


def build(verbose=False):
    tmp = LIB + ".tmp"
    log = _lib_build._run([_lib_build.HIPCC, *_lib_build.CFLAGS, "-shared", SRC, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose and log.strip():
        print(log)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
