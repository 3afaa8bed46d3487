"""Pins for oracle.multi (CPU only): several new query tokens per sequence,
causal over the paged cache.

* A whole prompt in one step (L = context) equals torch's scaled-dot-product
  attention with ``is_causal=True`` in float64 on the contiguous K/V, repeated
  to the query heads (a library routine independent of the oracle).
* One new token per sequence equals the (separately pinned) decode oracle.
* Brute force with an explicit mask matrix on tiny inputs.
* A prompt fed in chunks (the cache growing chunk by chunk) gives the rows a
  single full step gives: only positions, not chunking, decide a row.
* Rows past the cached tokens (L > context) are zeros.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention, multi, quant
from tests.test_oracle_attention import scatter_to_pool


def _case(rng, ctx_lens, Hkv, d, bs, pool_factor=1.4):
    # values exact in float32, the storage format the cases use
    K = [rng.standard_normal((Hkv, c, d)).astype(np.float32).astype(np.float64) for c in ctx_lens]
    V = [rng.standard_normal((Hkv, c, d)).astype(np.float32).astype(np.float64) for c in ctx_lens]
    need = sum(-(-c // bs) for c in ctx_lens)
    nb = max(int(need * pool_factor) + 1, 2)
    seed = int(rng.integers(1 << 30))
    kpool, tables = scatter_to_pool(K, ctx_lens, bs, nb, np.random.default_rng(seed))
    vpool, _ = scatter_to_pool(V, ctx_lens, bs, nb, np.random.default_rng(seed))
    return K, V, kpool.astype(np.float32), vpool.astype(np.float32), tables


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (6, 1)])
def test_whole_prompt_is_causal_sdpa(Hq, Hkv):
    rng = np.random.default_rng(Hq * 10 + Hkv)
    ctx = [37, 70, 16]
    d, bs, scale = 32, 16, 0.17
    K, V, kpool, vpool, tables = _case(rng, ctx, Hkv, d, bs)
    q = rng.standard_normal((sum(ctx), Hq, d))
    got = multi.multi_query_attention(q, ctx, kpool, vpool, tables, ctx, scale, bs, "f32")
    G = Hq // Hkv
    start = 0
    for b, c in enumerate(ctx):
        qq = torch.from_numpy(q[start:start + c]).permute(1, 0, 2)                 # [Hq][c][d]
        kk = torch.from_numpy(K[b]).repeat_interleave(G, dim=0)                       # [Hq][c][d]
        vv = torch.from_numpy(V[b]).repeat_interleave(G, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq[None], kk[None], vv[None], is_causal=True, scale=scale)[0].permute(1, 0, 2)
        assert np.allclose(got[start:start + c], ref.numpy(), rtol=1e-12, atol=1e-12)
        start += c


def test_one_new_token_is_decode():
    rng = np.random.default_rng(3)
    ctx = [1, 40, 129]
    Hq, Hkv, d, bs = 8, 2, 16, 16
    _, _, kpool, vpool, tables = _case(rng, ctx, Hkv, d, bs)
    q = rng.standard_normal((len(ctx), Hq, d))
    got = multi.multi_query_attention(q, [1, 1, 1], kpool, vpool, tables, ctx, 0.3, bs, "f32")
    ref = attention.decode_attention(q, kpool, vpool, tables, ctx, 0.3, bs, "f32")
    assert np.array_equal(got, ref)


def test_brute_force_mask_matrix():
    rng = np.random.default_rng(4)
    ctx, L = [9], [5]
    Hq, Hkv, d, bs = 2, 1, 3, 4
    K, V, kpool, vpool, tables = _case(rng, ctx, Hkv, d, bs)
    q = rng.standard_normal((5, Hq, d))
    got = multi.multi_query_attention(q, L, kpool, vpool, tables, ctx, 0.5, bs, "f32")
    # query j sits at position 4 + j; mask[j][t] = t <= 4 + j
    for j in range(5):
        for h in range(Hq):
            z = [0.5 * sum(q[j, h, e] * K[0][0, t, e] for e in range(d)) if t <= 4 + j else None
                 for t in range(9)]
            m = max(x for x in z if x is not None)
            w = [math.exp(x - m) if x is not None else 0.0 for x in z]
            s = sum(w)
            o = [sum(w[t] * V[0][0, t, e] for t in range(9)) / s for e in range(d)]
            assert np.allclose(got[j, h], o, rtol=1e-12, atol=1e-13)


def test_chunks_give_the_rows_of_one_full_step():
    rng = np.random.default_rng(5)
    n, Hq, Hkv, d, bs = 50, 4, 2, 16, 16
    K, V, kpool, vpool, tables = _case(rng, [n], Hkv, d, bs)
    q = rng.standard_normal((n, Hq, d))
    full = multi.multi_query_attention(q, [n], kpool, vpool, tables, [n], 0.25, bs, "f32")
    done = 0
    for L in (7, 16, 1, 26):
        part = multi.multi_query_attention(q[done:done + L], [L], kpool, vpool, tables,
                                           [done + L], 0.25, bs, "f32", check_tables=False)
        assert np.allclose(part, full[done:done + L], rtol=1e-13, atol=1e-14)
        done += L
    assert done == n


def test_rows_before_the_cache_are_zero_and_int8_reads_its_scales():
    rng = np.random.default_rng(6)
    Hq, Hkv, d, bs = 4, 4, 16, 16
    _, _, kpool, vpool, tables = _case(rng, [3], Hkv, d, bs)
    q = rng.standard_normal((5, Hq, d))
    got = multi.multi_query_attention(q, [5], kpool, vpool, tables, [3], 0.25, bs, "f32")
    assert np.all(got[:2] == 0) and np.all(np.isfinite(got[2:]))
    kq, ks = quant.quantize_int8_rows(np.nan_to_num(kpool).astype(np.float32))
    vq, vs = quant.quantize_int8_rows(np.nan_to_num(vpool).astype(np.float32))
    i8 = multi.multi_query_attention(q[2:], [3], kq, vq, tables, [3], 0.25, bs, "i8", ks, vs)
    f = multi.multi_query_attention(q[2:], [3], kpool, vpool, tables, [3], 0.25, bs, "f32")
    assert 0 < np.abs(i8 - f).max() < 0.05


def test_sampled_rows_match_the_full_computation():
    rng = np.random.default_rng(7)
    ctx, L = [30, 45], [4, 9]
    Hq, Hkv, d, bs = 8, 2, 16, 16
    _, _, kpool, vpool, tables = _case(rng, ctx, Hkv, d, bs)
    q = rng.standard_normal((13, Hq, d))
    full = multi.multi_query_attention(q, L, kpool, vpool, tables, ctx, 0.2, bs, "f32")
    rows = [(0, 1), (5, 7), (12, 0)]
    part = multi.multi_query_attention(q, L, kpool, vpool, tables, ctx, 0.2, bs, "f32", rows=rows)
    for r, h in rows:
        assert np.array_equal(part[r, h], full[r, h])
    assert np.isnan(part[1, 1]).all()
