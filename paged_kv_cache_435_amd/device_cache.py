"""Device-resident caches for a workload: pools filled, quantized, poisoned.

Setup for tests and the benchmark.  It draws the seeded inputs of
``workloads``, stores them in the cache format through the library's own
``kv_quantize`` (INT8 per row / FP8 per tensor) and fills every slot no live
token occupies with poison — NaN for float caches, a NaN scale for INT8, the
NaN code 0x7F for FP8 — so any read of a free block, a block tail or a slot
whose append has not happened yet shows up in the output.  The slot of each
sequence's newest token is poisoned too when the workload appends it, so a
missing append is visible.

With ``keep_sources=True`` the seeded source pools (before quantization and
poisoning) are also kept as host tensors, so a checker can build its own stored
cache from the same draws instead of reading the library's output.
``to_host`` copies the stored bytes back (used to time a CPU reference on them).
"""
import numpy as np
import torch

from . import kv_quantize
from . import workloads as W

_CACHE_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
                "i8": torch.int8, "fp8": torch.uint8}


def poison_mask(w):
    """bool [NB][bs]: slots to poison before any append."""
    mask = W.unused_slot_mask(w)
    if w.appends:
        slots = w.append_slots()
        mask[slots // w.block_size, slots % w.block_size] = True
    return mask


class DeviceCase:
    """Device tensors of one layer of a workload."""

    def __init__(self, w, device="cuda", layer=0, mask=None, keep_sources=False):
        self.w = w
        self.layer = layer
        self.device = device
        if mask is None:
            mask = poison_mask(w)
        mask_t = torch.from_numpy(mask).to(device)                      # [NB][bs]
        self.block_tables = torch.from_numpy(w.block_tables).to(device)
        self.context_lens = torch.from_numpy(w.context_lens).to(device)
        self.q = W.query(w, device, layer)
        self.out = torch.empty_like(self.q)
        self.k_scale = self.v_scale = None
        caches, scales = [], []
        self.sources = {}
        for which in ("k", "v"):
            src = W.pool_source(w, which, device, layer)
            if keep_sources:
                self.sources[which] = src.cpu()
            if w.kv_format in ("f32", "f16", "bf16"):
                src.permute(0, 2, 1, 3)[mask_t] = float("nan")
                caches.append(src)
                scales.append(None)
            elif w.kv_format == "i8":
                codes = torch.empty(src.shape, dtype=torch.int8, device=device)
                sc = torch.empty(src.shape[:-1], dtype=torch.float32, device=device)
                kv_quantize(src, codes, sc)
                sc.permute(0, 2, 1)[mask_t] = float("nan")
                caches.append(codes)
                scales.append(sc)
            else:
                codes = torch.empty(src.shape, dtype=torch.uint8, device=device)
                sc = torch.empty(1, dtype=torch.float32, device=device)
                kv_quantize(src, codes, sc, out_dtype="fp8")
                codes.permute(0, 2, 1, 3)[mask_t] = 0x7F
                caches.append(codes)
                scales.append(sc)
            del src
        self.k_cache, self.v_cache = caches
        self.k_scale, self.v_scale = scales
        if w.appends:
            self.new_k, self.new_v = W.new_rows(w, device, layer)
            self.slots = torch.from_numpy(w.append_slots()).to(device)
        else:
            self.new_k = self.new_v = self.slots = None

    @property
    def kv_dtype(self):
        return {"i8": "i8", "fp8": "fp8"}.get(self.w.kv_format)


def q_to_host(q):
    return q.float().cpu().numpy().astype(np.float64)


def cache_to_host(t, fmt):
    if fmt == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def to_host(case):
    """Stored bytes of one layer, as the CPU reference takes them."""
    w = case.w
    h = dict(q=q_to_host(case.q), k_cache=cache_to_host(case.k_cache, w.kv_format),
             v_cache=cache_to_host(case.v_cache, w.kv_format),
             block_tables=w.block_tables, context_lens=w.context_lens,
             scale=w.scale, block_size=w.block_size, kv_format=w.kv_format)
    if w.kv_format == "i8":
        h["k_scale"] = case.k_scale.cpu().numpy()
        h["v_scale"] = case.v_scale.cpu().numpy()
    elif w.kv_format == "fp8":
        h["k_scale"] = np.float32(case.k_scale.item())
        h["v_scale"] = np.float32(case.v_scale.item())
    else:
        h["k_scale"] = h["v_scale"] = None
    return h
