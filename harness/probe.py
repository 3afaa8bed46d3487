"""Streaming HBM yardsticks (``libpkvprobe.so``): a plain read of a buffer and a
plain copy, timed with events on the current stream.  Used by the benchmark to
report the decode kernel's bandwidth against what a trivial kernel reaches on
the same device, and to calibrate hardware byte counters.  Not part of the
attention path."""
import ctypes
import os

import torch

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkvprobe.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build with `python -m harness.build_probe`")
        lib = ctypes.CDLL(path)
        lib.pkv_probe_grid.restype = ctypes.c_int32
        lib.pkv_probe_read.restype = ctypes.c_int32
        lib.pkv_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                       ctypes.c_void_p]
        lib.pkv_probe_read_slabs.restype = ctypes.c_int32
        lib.pkv_probe_read_slabs.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                             ctypes.c_int32, ctypes.c_void_p]
        lib.pkv_probe_copy.restype = ctypes.c_int32
        lib.pkv_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                       ctypes.c_void_p]
        _LIB = lib
    return _LIB


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def read_gbps(nbytes=4 << 30, reps=10, device="cuda", slabs=0):
    """Median GB/s of a plain read of a fresh ``nbytes`` buffer: grid-stride
    16-byte loads, or (``slabs`` > 0) contiguous 16 KB slabs per workgroup over
    ``slabs`` workgroups of 4 waves."""
    lib = _lib()
    if slabs:
        fn = lambda x, n, s, st: lib.pkv_probe_read_slabs(x, n, s, slabs, st)
    else:
        fn = lib.pkv_probe_read
    x = torch.empty(nbytes, dtype=torch.uint8, device=device)
    x.fill_(1)
    sink = torch.empty(lib.pkv_probe_grid(), dtype=torch.int32, device=device)
    times = []
    for _ in range(reps + 2):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        if fn(ctypes.c_void_p(x.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()), _stream()):
            raise RuntimeError("pkv_probe_read failed")
        e1.record()
        times.append((e0, e1))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in times[2:])
    del x, sink
    return nbytes / (ms[len(ms) // 2] * 1e-3) / 1e9


def copy(dst, src):
    """One launch of the plain copy kernel (dst, src: same byte size, multiple of 16)."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("dst and src sizes differ")
    if _lib().pkv_probe_copy(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()),
                             n, _stream()):
        raise RuntimeError("pkv_probe_copy failed")
