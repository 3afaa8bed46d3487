"""Seeded synthetic inputs for the paged decode path.

This module only draws inputs; it holds none of the method's arithmetic (no
attention, no quantization).  Both the GPU path's callers (tests, benchmark)
and the CPU oracle's callers take their inputs from here.  It plays the role
of the block manager the pages describe ([P1] «LLM推理显存优化：KV
Cache管理3大策略实测，节省60%显存开销» §2; [P3] «大模型推理加速实战：KV
Cache内存优化与PagedAttention分页管理方案», PagedAttention section): it hands
out physical blocks from a shuffled pool and writes the block tables and the
slots of appended tokens.

The five workloads (shapes of the Llama-2 family the pages discuss):

  tiny_fp32     fp32, MHA 4/4 heads, d 64, bs 16, contexts 37 and 64, pool of 16
  llama7b_bf16  bf16, MHA 32/32, d 128, bs 16, batch 8, every context 4096
  llama70b_gqa8 fp16, GQA 64/8, d 128, bs 16, batch 32, contexts U[512, 32768]
  llama13b_int8 fp16 q, INT8 KV (per-row scale), MHA 40/40, d 128, bs 16, batch 32,
                2048 cached tokens + 1 appended (decode over 2049);
                K/V ~ N(0,1) with 1% of elements scaled by 8
  llama70b_fp8  fp16 q, FP8 E4M3FN KV (per-tensor scale), GQA 64/8, d 128,
                batch 64, log-normal contexts (median 4096, sigma 1) clipped to
                [128, 32768], 80 layers, bs 16 or 256
  llama13b_int4 the llama13b_int8 case with an INT4 cache (per-row scale,
                packed nibbles)
  llama70b_int4 the llama70b_gqa8 case with an INT4 cache
  llama70b_gqa8_32k  the llama70b_gqa8 layer with every context at 32768 tokens:
                4 GiB of K+V per decode step, pools of 2.7 GB per cache (past
                2**31 bytes)

Pools hold 1.25x the blocks the sequences need (16 for the tiny case).  Blocks
are dealt from ``default_rng(1).permutation(pool)`` to sequence 0's logical
blocks in order, then sequence 1's, and so on.  Unused blocks and the tail
slots of each sequence's last block are "poisoned" (NaN for float caches) by
the callers, using ``unused_slot_mask``.
"""
import math
from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass
class Workload:
    name: str
    q_dtype: torch.dtype
    kv_format: str            # "f32" | "f16" | "bf16" | "i8" | "fp8" | "i4"
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    layers: int
    context_lens: np.ndarray  # int32 [B]: tokens decode attends over (after any append)
    num_blocks: int
    block_tables: np.ndarray  # int32 [B][MB], -1 past each sequence's blocks
    appends: bool             # one new token per sequence is appended before decode
    outliers: bool = False    # 1% of K/V source elements scaled by 8
    seeds: dict = field(default_factory=dict)

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def max_context_len(self):
        return int(self.context_lens.max()) if len(self.context_lens) else 0

    @property
    def group(self):
        return self.num_q_heads // self.num_kv_heads

    def kv_bytes_per_layer(self):
        """Algorithmic KV bytes one decode step reads per layer: K and V rows of
        every context token of every KV head, plus INT8 / INT4 row scales."""
        bits = {"f32": 32, "f16": 16, "bf16": 16, "i8": 8, "fp8": 8, "i4": 4}[self.kv_format]
        tokens = int(self.context_lens.astype(np.int64).sum())
        b = 2 * tokens * self.num_kv_heads * self.head_dim * bits // 8
        if self.kv_format in ("i8", "i4"):
            b += 2 * tokens * self.num_kv_heads * 4
        return b

    def append_slots(self):
        """int64 [B]: pool slot of each sequence's newest token (position ctx - 1),
        = physical block * block_size + offset; -1 for an empty sequence."""
        pos = self.context_lens.astype(np.int64) - 1
        phys = self.block_tables[np.arange(self.batch), np.maximum(pos, 0) // self.block_size]
        slots = phys.astype(np.int64) * self.block_size + np.maximum(pos, 0) % self.block_size
        return np.where(pos >= 0, slots, -1)   # (an empty sequence appends nothing)


def deal_blocks(context_lens, block_size, num_blocks, seed=1):
    """Block tables from a seeded shuffle of the pool.  Raises if the pool is too small."""
    need = [-(-int(c) // block_size) for c in context_lens]
    if sum(need) > num_blocks:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {sum(need)}")
    perm = np.random.default_rng(seed).permutation(num_blocks)
    mb = max(max(need) if need else 1, 1)
    tables = np.full((len(need), mb), -1, dtype=np.int32)
    k = 0
    for b, n in enumerate(need):
        tables[b, :n] = perm[k:k + n]
        k += n
    return tables


def pool_for(context_lens, block_size, factor=1.25):
    need = sum(-(-int(c) // block_size) for c in context_lens)
    return max(int(math.ceil(need * factor)), 1)


def unused_slot_mask(w):
    """bool [NB][bs]: True where no live token lives (free blocks, tails)."""
    mask = np.ones((w.num_blocks, w.block_size), dtype=bool)
    for b in range(w.batch):
        c = int(w.context_lens[b])
        for j in range(-(-c // w.block_size)):
            n = min(w.block_size, c - j * w.block_size)
            mask[w.block_tables[b, j], :n] = False
    return mask


def make(name, block_size=None, layers=None):
    """The named workload.  ``block_size``/``layers`` override the FP8 case's."""
    if name == "tiny_fp32":
        ctx = np.array([37, 64], dtype=np.int32)
        bs = 16
        nb = 16
        return Workload(name, torch.float32, "f32", 2, 4, 4, 64, bs, 1, ctx, nb,
                        deal_blocks(ctx, bs, nb), appends=False,
                        seeds=dict(context=None, permutation=1, q=2, k=3, v=4))
    if name == "llama7b_bf16":
        ctx = np.full(8, 4096, dtype=np.int32)
        bs = 16
        nb = pool_for(ctx, bs)
        return Workload(name, torch.bfloat16, "bf16", 8, 32, 32, 128, bs, 1, ctx, nb,
                        deal_blocks(ctx, bs, nb), appends=True,
                        seeds=dict(context=None, permutation=1, q=2, k=3, v=4, new=6))
    if name in ("llama70b_gqa8", "llama70b_int4"):
        ctx = np.random.default_rng(0).integers(512, 32768, 32, endpoint=True).astype(np.int32)
        bs = 16
        nb = pool_for(ctx, bs)
        fmt = "f16" if name == "llama70b_gqa8" else "i4"
        return Workload(name, torch.float16, fmt, 32, 64, 8, 128, bs, 1, ctx, nb,
                        deal_blocks(ctx, bs, nb), appends=True,
                        seeds=dict(context=0, permutation=1, q=2, k=3, v=4, new=6))
    if name == "llama70b_gqa8_32k":
        ctx = np.full(32, 32768, dtype=np.int32)
        bs = 16
        nb = pool_for(ctx, bs)
        return Workload(name, torch.float16, "f16", 32, 64, 8, 128, bs, 1, ctx, nb,
                        deal_blocks(ctx, bs, nb), appends=True,
                        seeds=dict(context=None, permutation=1, q=2, k=3, v=4, new=6))
    if name in ("llama13b_int8", "llama13b_int4"):
        ctx = np.full(32, 2049, dtype=np.int32)
        bs = 16
        nb = pool_for(ctx, bs)
        fmt = "i8" if name == "llama13b_int8" else "i4"
        return Workload(name, torch.float16, fmt, 32, 40, 40, 128, bs, 1, ctx, nb,
                        deal_blocks(ctx, bs, nb), appends=True, outliers=True,
                        seeds=dict(context=None, permutation=1, q=2, k=3, v=4, outliers=5, new=6))
    if name == "llama70b_fp8":
        bs = block_size or 16
        z = np.random.default_rng(0).standard_normal(64)
        ctx = np.clip(np.rint(np.exp(math.log(4096.0) + 1.0 * z)), 128, 32768).astype(np.int32)
        nb = pool_for(ctx, bs)
        return Workload(name, torch.float16, "fp8", 64, 64, 8, 128, bs, layers or 80, ctx, nb,
                        deal_blocks(ctx, bs, nb), appends=True,
                        seeds=dict(context=0, permutation=1, q=2, k=3, v=4, new=6))
    raise KeyError(name)


NAMES = ("tiny_fp32", "llama7b_bf16", "llama70b_gqa8", "llama13b_int8", "llama70b_fp8",
         "llama13b_int4", "llama70b_int4", "llama70b_gqa8_32k")


# Several new query tokens per sequence (paged_attention_multi_query): each
# returns the workload (contexts count the new tokens) and the new tokens per
# sequence.
#   llama70b_verify4    the llama70b_gqa8 batch with 4 draft tokens per sequence
#                       to verify
#   llama70b_prefill512 8 sequences of the 70B GQA-8 shape, cached prefixes
#                       U[0, 4096] (seed 0) and a 512-token prompt chunk each
MULTI_NAMES = ("llama70b_verify4", "llama70b_prefill512", "llama70b_prefill512_fp8",
               "llama70b_prefill512_i8", "llama70b_prefill512_i4")


def make_multi(name):
    if name == "llama70b_verify4":
        w = make("llama70b_gqa8")
        w.name, w.appends = name, False
        return w, np.full(w.batch, 4, dtype=np.int64)
    if name in ("llama70b_prefill512", "llama70b_prefill512_fp8", "llama70b_prefill512_i8",
                "llama70b_prefill512_i4"):
        # 512-token prompt chunks of 8 sequences with prefixes U[0, 4096]; f16
        # queries over an f16, FP8 E4M3FN, INT8 or INT4 cache
        prefix = np.random.default_rng(0).integers(0, 4096, 8, endpoint=True)
        ctx = (prefix + 512).astype(np.int32)
        bs = 16
        nb = pool_for(ctx, bs)
        fmt = {"fp8": "fp8", "i8": "i8", "i4": "i4"}.get(name.rsplit("_", 1)[-1], "f16")
        w = Workload(name, torch.float16, fmt, 8, 64, 8, 128, bs, 1, ctx, nb,
                     deal_blocks(ctx, bs, nb), appends=False,
                     seeds=dict(context=0, permutation=1, q=2, k=3, v=4, new=6))
        return w, np.full(8, 512, dtype=np.int64)
    raise KeyError(name)


def custom(q_dtype, kv_format, context_lens, num_q_heads, num_kv_heads, head_dim, block_size,
           pool_factor=1.25, extra_blocks=0, perm_seed=1, appends=False, name="custom"):
    """A workload of any shape, dealt the same way (for edge-case tests)."""
    ctx = np.asarray(context_lens, dtype=np.int32)
    nb = pool_for(ctx, block_size, pool_factor) + extra_blocks
    return Workload(name, q_dtype, kv_format, len(ctx), num_q_heads, num_kv_heads, head_dim,
                    block_size, 1, ctx, nb, deal_blocks(ctx, block_size, nb, perm_seed),
                    appends=appends, seeds=dict(permutation=perm_seed, q=2, k=3, v=4, new=6))


# ---------------------------------------------------------------------------
# Tensors.  Everything is drawn in float32 from a seeded torch.Generator on the
# given device, then cast to the storage dtype.
# ---------------------------------------------------------------------------
def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def randn(shape, seed, device, dtype=torch.float32, layer=0):
    g = _gen(device, seed * 1000003 + layer)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(dtype)


def query(w, device, layer=0):
    return randn((w.batch, w.num_q_heads, w.head_dim), w.seeds["q"], device, w.q_dtype, layer)


def new_rows(w, device, layer=0):
    """Source K and V rows [B][Hkv][d] of the token appended to each sequence."""
    src = w.q_dtype
    k = randn((w.batch, w.num_kv_heads, w.head_dim), w.seeds["new"], device, src, layer)
    v = randn((w.batch, w.num_kv_heads, w.head_dim), w.seeds["new"] + 1, device, src, layer)
    return k, v


def pool_source(w, which, device, layer=0, dtype=None):
    """Source values of the whole K ("k") or V ("v") pool [NB][Hkv][bs][d] in
    ``dtype`` (default: the query dtype for quantized caches, else the cache
    dtype), with the 1% x8 outliers where the workload asks for them."""
    seed = w.seeds[which]
    shape = (w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
    x = randn(shape, seed, device, torch.float32, layer)
    if w.outliers:
        g = _gen(device, w.seeds["outliers"] * 1000003 + layer * 2 + (which == "v"))
        mask = torch.rand(shape, generator=g, device=device) < 0.01
        x = torch.where(mask, x * 8.0, x)
    if dtype is None:
        dtype = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}.get(
            w.kv_format, w.q_dtype)
    return x.to(dtype)
