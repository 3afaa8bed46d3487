"""Pins for oracle.attention (CPU only).

The oracle is checked against things other than itself:
* brute force with scalar loops on tiny inputs;
* torch's scaled_dot_product_attention in float64 on contiguous K/V expanded to
  every query head (MHA, GQA and MQA reduce to textbook attention there);
* invariants: softmax weights sum to one, permuting physical blocks changes
  nothing, the identity table equals the contiguous layout, 16- and 256-token
  blocks agree;
* special cases with known answers: one token, a zero query, needles;
* dequantized INT8/FP8 caches land within the quantizers' error bounds of the
  float answer (this catches a dequant that multiplies instead of divides).
The contiguous K/V are scattered into the pool here with numpy fancy indexing,
not with oracle.paging, so a gather bug cannot cancel out.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention, quant, widen


def scatter_to_pool(K, ctx_lens, bs, num_blocks, rng, fill=np.nan):
    """K: list over sequences of [Hkv][ctx_b][d] float arrays.  Returns pool
    [NB][Hkv][bs][d] and block tables [B][MB] drawn from a random permutation."""
    B = len(K)
    Hkv, _, d = K[0].shape
    need = [-(-c // bs) for c in ctx_lens]
    MB = max(max(need), 1)
    assert sum(need) <= num_blocks
    perm = rng.permutation(num_blocks)
    tables = np.full((B, MB), -1, dtype=np.int32)
    pool = np.full((num_blocks, Hkv, bs, d), fill, dtype=np.float64)
    k = 0
    for b in range(B):
        for j in range(need[b]):
            tables[b, j] = perm[k]
            k += 1
        pos = np.arange(ctx_lens[b])
        phys = tables[b, pos // bs]
        pool[phys, :, pos % bs, :] = np.transpose(K[b], (1, 0, 2))
    return pool, tables


def sdpa_reference(q, K, V, scale):
    """torch SDPA (fp64) per sequence on K/V repeated to every query head."""
    B, Hq, d = q.shape
    out = np.zeros((B, Hq, d))
    for b in range(B):
        Hkv = K[b].shape[0]
        G = Hq // Hkv
        qt = torch.tensor(q[b], dtype=torch.float64)[None, :, None, :]
        kt = torch.tensor(K[b], dtype=torch.float64).repeat_interleave(G, dim=0)[None]
        vt = torch.tensor(V[b], dtype=torch.float64).repeat_interleave(G, dim=0)[None]
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
        out[b] = o[0, :, 0, :].numpy()
    return out


def random_case(rng, B, Hq, Hkv, d, bs, ctx_lens, pool_factor=1.5):
    q = rng.standard_normal((B, Hq, d))
    K = [rng.standard_normal((Hkv, c, d)) for c in ctx_lens]
    V = [rng.standard_normal((Hkv, c, d)) for c in ctx_lens]
    need = sum(-(-c // bs) for c in ctx_lens)
    nb = max(int(need * pool_factor) + 1, 2)
    kpool, tables = scatter_to_pool(K, ctx_lens, bs, nb, np.random.default_rng(rng.integers(1 << 30)))
    vpool = np.full_like(kpool, np.nan)
    for b, c in enumerate(ctx_lens):
        pos = np.arange(c)
        phys = tables[b, pos // bs]
        vpool[phys, :, pos % bs, :] = np.transpose(V[b], (1, 0, 2))
    return q, K, V, kpool, vpool, tables


def brute_force(q, K, V, scale):
    """Scalar loops, math.exp, no numpy reductions."""
    B, Hq, d = len(q), len(q[0]), len(q[0][0])
    out = [[[0.0] * d for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        Hkv = len(K[b])
        G = Hq // Hkv
        for h in range(Hq):
            g = h // G
            T = len(K[b][g])
            z = []
            for t in range(T):
                s = 0.0
                for i in range(d):
                    s += q[b][h][i] * K[b][g][t][i]
                z.append(scale * s)
            m = max(z)
            e = [math.exp(x - m) for x in z]
            tot = sum(e)
            for i in range(d):
                acc = 0.0
                for t in range(T):
                    acc += e[t] / tot * V[b][g][t][i]
                out[b][h][i] = acc
    return np.array(out)


@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (2, 1), (4, 2)])
def test_brute_force_tiny(Hq, Hkv):
    rng = np.random.default_rng(7)
    d, bs = 8, 2
    ctx = [1, 3, 2]
    q, K, V, kpool, vpool, tables = random_case(rng, 3, Hq, Hkv, d, bs, ctx)
    got = attention.decode_attention(q, kpool.astype(np.float32), vpool.astype(np.float32), tables,
                                     ctx, 0.35, bs, "f32")
    Kf = [k.astype(np.float32).astype(np.float64).tolist() for k in K]
    Vf = [v.astype(np.float32).astype(np.float64).tolist() for v in V]
    want = brute_force(q.tolist(), Kf, Vf, 0.35)
    assert np.allclose(got, want, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("Hq,Hkv,bs", [(4, 4, 16), (8, 2, 16), (8, 1, 16), (6, 3, 256), (64, 8, 16)])
def test_matches_torch_sdpa(Hq, Hkv, bs):
    rng = np.random.default_rng(Hq * 100 + Hkv + bs)
    d = 64 if Hq != 64 else 128
    ctx = [37, 64, 1, 300] if bs == 16 else [37, 600]
    q, K, V, kpool, vpool, tables = random_case(rng, len(ctx), Hq, Hkv, d, bs, ctx)
    scale = 1.0 / math.sqrt(d)
    got = attention.decode_attention(q, kpool.astype(np.float32), vpool.astype(np.float32), tables,
                                     ctx, scale, bs, "f32")
    K32 = [k.astype(np.float32).astype(np.float64) for k in K]
    V32 = [v.astype(np.float32).astype(np.float64) for v in V]
    want = sdpa_reference(q, K32, V32, scale)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_weights_sum_to_one():
    rng = np.random.default_rng(3)
    ctx = [5, 77, 200]
    q, K, V, kpool, vpool, tables = random_case(rng, 3, 4, 2, 32, 16, ctx)
    _, w = attention.decode_attention(q, kpool, vpool, tables, ctx, 0.2, 16, "f32", return_weights=True)
    for (b, h), ww in w.items():
        assert ww.shape == (ctx[b],)
        assert abs(ww.sum() - 1.0) < 1e-12
        assert np.all(ww >= 0)


def test_permuting_physical_blocks_changes_nothing():
    rng = np.random.default_rng(11)
    ctx = [40, 17, 64]
    q, K, V, kpool, vpool, tables = random_case(rng, 3, 4, 4, 16, 16, ctx, pool_factor=3)
    a = attention.decode_attention(q, kpool, vpool, tables, ctx, 0.25, 16, "f32")
    NB = kpool.shape[0]
    pi = np.random.default_rng(12).permutation(NB)   # block p moves to pi[p]
    kp = np.empty_like(kpool)
    vp = np.empty_like(vpool)
    kp[pi] = kpool
    vp[pi] = vpool
    t2 = np.where(tables >= 0, pi[np.maximum(tables, 0)], -1).astype(np.int32)
    b = attention.decode_attention(q, kp, vp, t2, ctx, 0.25, 16, "f32")
    assert np.array_equal(a, b)


def test_identity_table_equals_contiguous_layout():
    rng = np.random.default_rng(5)
    B, Hq, Hkv, d, bs, T = 2, 4, 2, 16, 16, 48
    q = rng.standard_normal((B, Hq, d))
    K = rng.standard_normal((B, Hkv, T, d)).astype(np.float32)
    V = rng.standard_normal((B, Hkv, T, d)).astype(np.float32)
    nblk = T // bs
    # Identity table: sequence b's logical block j lives at physical b * nblk + j.
    kpool = K.reshape(B, Hkv, nblk, bs, d).transpose(0, 2, 1, 3, 4).reshape(B * nblk, Hkv, bs, d)
    vpool = V.reshape(B, Hkv, nblk, bs, d).transpose(0, 2, 1, 3, 4).reshape(B * nblk, Hkv, bs, d)
    tables = np.arange(B * nblk, dtype=np.int32).reshape(B, nblk)
    a = attention.decode_attention(q, kpool, vpool, tables, [T] * B, 0.3, bs, "f32")
    c = attention.contiguous_attention(q, K.astype(np.float64), V.astype(np.float64), 0.3)
    assert np.allclose(a, c, rtol=1e-14, atol=1e-14)


def test_block_sizes_16_and_256_agree():
    rng = np.random.default_rng(9)
    ctx = [300, 513]
    q = rng.standard_normal((2, 4, 32))
    K = [rng.standard_normal((2, c, 32)) for c in ctx]
    V = [rng.standard_normal((2, c, 32)) for c in ctx]
    outs = []
    for bs in (16, 256):
        need = sum(-(-c // bs) for c in ctx)
        kpool, tables = scatter_to_pool(K, ctx, bs, need + 3, np.random.default_rng(bs))
        vpool, _ = scatter_to_pool(V, ctx, bs, need + 3, np.random.default_rng(bs))
        outs.append(attention.decode_attention(q, kpool, vpool, tables, ctx, 0.17, bs, "f32"))
    assert np.allclose(outs[0], outs[1], rtol=1e-13, atol=1e-13)


def test_single_token_returns_its_value_row():
    rng = np.random.default_rng(1)
    q, K, V, kpool, vpool, tables = random_case(rng, 2, 4, 2, 16, 16, [1, 1])
    out = attention.decode_attention(q, kpool, vpool, tables, [1, 1], 0.5, 16, "f32")
    for b in range(2):
        for h in range(4):
            assert np.array_equal(out[b, h], V[b][h // 2][0].astype(np.float32).astype(np.float64))


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(2)
    ctx = [33, 70]
    q, K, V, kpool, vpool, tables = random_case(rng, 2, 2, 1, 16, 16, ctx)
    q[:] = 0
    out = attention.decode_attention(q, kpool, vpool, tables, ctx, 0.5, 16, "f32")
    for b in range(2):
        want = V[b][0].astype(np.float32).astype(np.float64).mean(axis=0)
        assert np.allclose(out[b, 0], want, rtol=1e-13, atol=1e-13)


def test_needles_pick_out_their_rows():
    """One key parallel to the query and large: its weight is ~1, so the output is
    that token's value row — which pins where every logical position is read from."""
    rng = np.random.default_rng(4)
    ctx = [50]
    d = 16
    for t in [0, 15, 16, 31, 32, 49]:
        q, K, V, kpool, vpool, tables = random_case(rng, 1, 2, 1, d, 16, ctx)
        K[0][0] *= 0.01
        K[0][0][t] = 40.0 * q[0, 0] / np.linalg.norm(q[0, 0])
        kpool2, tables2 = scatter_to_pool(K, ctx, 16, 8, np.random.default_rng(t))
        vpool2, _ = scatter_to_pool(V, ctx, 16, 8, np.random.default_rng(t))
        out = attention.decode_attention(q, kpool2, vpool2, tables2, ctx, 1.0, 16, "f32")
        assert np.allclose(out[0, 0], V[0][0][t].astype(np.float32), atol=1e-6)


def test_empty_context_gives_zeros():
    rng = np.random.default_rng(6)
    q, K, V, kpool, vpool, tables = random_case(rng, 2, 2, 2, 8, 16, [5, 9])
    out = attention.decode_attention(q, kpool, vpool, tables, [0, 9], 0.5, 16, "f32")
    assert np.all(out[0] == 0)
    assert np.all(np.isfinite(out[1]))


def test_unused_slots_are_never_read():
    """Pools are filled with NaN outside the live rows (scatter_to_pool); any read
    of a tail slot or a free block would make the output NaN."""
    rng = np.random.default_rng(8)
    ctx = [17, 1, 31]
    q, K, V, kpool, vpool, tables = random_case(rng, 3, 4, 2, 8, 16, ctx)
    assert np.isnan(kpool).any()
    out = attention.decode_attention(q, kpool, vpool, tables, ctx, 0.5, 16, "f32")
    assert np.all(np.isfinite(out))


def test_table_validation():
    with pytest.raises(ValueError):
        attention.validate_tables([[0, 1], [1, 2]], [32, 20], 4, 16)     # block 1 aliased
    with pytest.raises(ValueError):
        attention.validate_tables([[0, 5]], [20], 4, 16)                 # out of the pool
    with pytest.raises(ValueError):
        attention.validate_tables([[0, 1]], [33], 4, 16)                 # longer than the table
    with pytest.raises(ValueError):
        attention.validate_tables([[0, -1]], [20], 4, 16)                # padding reached
    attention.validate_tables([[0, -1], [1, 2]], [16, 20], 4, 16)        # padding beyond ctx is fine


def test_int8_cache_stays_within_quantization_error():
    """Attention over an INT8 cache (q / s dequant) vs over the float rows it came
    from: the difference is bounded by the row quantization error."""
    rng = np.random.default_rng(21)
    ctx = [64, 100]
    q, K, V, _, _, _ = random_case(rng, 2, 4, 2, 32, 16, ctx)
    bs = 16
    need = sum(-(-c // bs) for c in ctx)
    kpool, tables = scatter_to_pool(K, ctx, bs, need + 2, np.random.default_rng(1), fill=0.0)
    vpool, _ = scatter_to_pool(V, ctx, bs, need + 2, np.random.default_rng(1), fill=0.0)
    kq, ks = quant.quantize_int8_rows(kpool.astype(np.float32))
    vq, vs = quant.quantize_int8_rows(vpool.astype(np.float32))
    f = attention.decode_attention(q, kpool, vpool, tables, ctx, 0.2, bs, "f32")
    i8 = attention.decode_attention(q, kq, vq, tables, ctx, 0.2, bs, "i8", ks, vs)
    err = np.max(np.abs(f - i8))
    assert err < 0.05
    assert err > 0   # it is a lossy format


def test_fp8_cache_stays_within_quantization_error():
    rng = np.random.default_rng(22)
    ctx = [64, 100]
    q, K, V, _, _, _ = random_case(rng, 2, 4, 2, 32, 16, ctx)
    bs = 16
    need = sum(-(-c // bs) for c in ctx)
    kpool, tables = scatter_to_pool(K, ctx, bs, need + 2, np.random.default_rng(1), fill=0.0)
    vpool, _ = scatter_to_pool(V, ctx, bs, need + 2, np.random.default_rng(1), fill=0.0)
    kc, ksc = quant.quantize_fp8(kpool.astype(np.float32))
    vc, vsc = quant.quantize_fp8(vpool.astype(np.float32))
    f = attention.decode_attention(q, kpool, vpool, tables, ctx, 0.2, bs, "f32")
    f8 = attention.decode_attention(q, kc, vc, tables, ctx, 0.2, bs, "fp8", ksc, vsc)
    err = np.max(np.abs(f - f8))
    assert err < 0.1
    assert err > 0


def test_bf16_widening_is_exact():
    x = torch.randn(1000, dtype=torch.float32).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(widen.widen_kv(bits, "bf16"), x.to(torch.float64).numpy())


def test_int4_cache_stays_within_quantization_error():
    """INT4 (7 / absmax per row, packed nibbles) vs the float rows it came from:
    lossy, and further from the float result than INT8 over the same rows."""
    rng = np.random.default_rng(21)
    ctx = [64, 100]
    q, K, V, _, _, _ = random_case(rng, 2, 4, 2, 32, 16, ctx)
    bs = 16
    need = sum(-(-c // bs) for c in ctx)
    kpool, tables = scatter_to_pool(K, ctx, bs, need + 2, np.random.default_rng(1), fill=0.0)
    vpool, _ = scatter_to_pool(V, ctx, bs, need + 2, np.random.default_rng(1), fill=0.0)
    k4, ks = quant.quantize_int4_rows(kpool.astype(np.float32))
    v4, vs = quant.quantize_int4_rows(vpool.astype(np.float32))
    k8, ks8 = quant.quantize_int8_rows(kpool.astype(np.float32))
    v8, vs8 = quant.quantize_int8_rows(vpool.astype(np.float32))
    f = attention.decode_attention(q, kpool, vpool, tables, ctx, 0.2, bs, "f32")
    i4 = attention.decode_attention(q, quant.pack_int4(k4), quant.pack_int4(v4), tables, ctx,
                                    0.2, bs, "i4", ks, vs)
    i8 = attention.decode_attention(q, k8, v8, tables, ctx, 0.2, bs, "i8", ks8, vs8)
    e4, e8 = np.max(np.abs(f - i4)), np.max(np.abs(f - i8))
    assert 0 < e8 < e4 < 0.5
    # the same codes fed as unpacked INT8 codes with the INT4 scales give the
    # same attention: packing is lossless
    same = attention.decode_attention(q, k4, v4, tables, ctx, 0.2, bs, "i8", ks, vs)
    assert np.array_equal(same, i4)
