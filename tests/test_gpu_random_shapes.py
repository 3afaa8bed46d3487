"""Seeded random shapes, decode and multi-token calls, against the CPU oracle.

The fixed-shape tests pick the cases the pages and the design name; this sweep
draws the rest from a fixed seed, so it is the same on every run: every cache
format with the query types it takes, head_dim 64 / 128, block sizes 16 / 256,
1-8 KV heads with groups from MQA to wider than one 16-head tile, 1-12
sequences whose contexts include 0, 1, block-size multiples and their
neighbours, pools 1-2x the demand.  Multi-token calls draw 1-40 new tokens per
sequence (never more than its context).  Every output row is compared with the
oracle elementwise and by relative L2 (tests.gpu_util.compare)."""
import numpy as np
import pytest
import torch

from harness import workloads as W
from tests.gpu_util import run_and_check

pytestmark = pytest.mark.gpu

_Q_FOR = {"f32": [torch.float32], "f16": [torch.float16], "bf16": [torch.bfloat16],
          "i8": [torch.float16, torch.bfloat16], "fp8": [torch.float16, torch.bfloat16],
          "i4": [torch.float16, torch.bfloat16, torch.float32]}


def _draw(seed):
    rng = np.random.default_rng(seed)
    fmt = ["f32", "f16", "bf16", "i8", "fp8", "i4"][seed % 6]
    q_dtype = _Q_FOR[fmt][rng.integers(len(_Q_FOR[fmt]))]
    d = 128 if fmt == "i4" else int(rng.choice([64, 128]))
    bs = int(rng.choice([16, 256]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 3, 5, 8, 16, 20]))
    b = int(rng.integers(1, 13))
    special = [0, 1, bs - 1, bs, bs + 1, 2 * bs, 3 * bs - 1]
    ctx = [int(rng.choice(special)) if rng.random() < 0.4 else int(rng.integers(1, 3001))
           for _ in range(b)]
    if max(ctx) == 0:
        ctx[0] = 1
    pool = float(rng.uniform(1.0, 2.0))
    return fmt, q_dtype, d, bs, hkv, g, ctx, pool


@pytest.mark.parametrize("seed", range(24))
def test_random_decode(seed):
    fmt, q_dtype, d, bs, hkv, g, ctx, pool = _draw(seed)
    w = W.custom(q_dtype, fmt, ctx, g * hkv, hkv, d, bs, pool_factor=pool, perm_seed=seed + 7,
                 name=f"rand{seed}-{fmt}-d{d}-bs{bs}-{g * hkv}x{hkv}")
    run_and_check(w)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("seed", range(100, 112))
def test_random_multi_query(seed):
    from tests.test_gpu_multi import run_multi
    fmt, q_dtype, d, bs, hkv, g, ctx, pool = _draw(seed)
    rng = np.random.default_rng(seed + 1)
    ctx = [max(c, 1) for c in ctx]
    lens = [int(min(c, rng.integers(1, 41))) for c in ctx]
    w = W.custom(q_dtype, fmt, ctx, g * hkv, hkv, d, bs, pool_factor=pool, perm_seed=seed + 7,
                 name=f"rand{seed}-{fmt}-d{d}-bs{bs}-{g * hkv}x{hkv}")
    run_multi(w, lens)
    torch.cuda.empty_cache()
