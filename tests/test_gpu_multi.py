"""paged_attention_multi_query on the GPU vs the CPU oracle (oracle.multi):
several new query tokens per sequence, causal over the paged cache.

The cache is filled by the library's append from seeded sources (every
context token, new ones included), unused slots poisoned; the oracle builds
its own stored cache from host copies of the same draws (tests.gpu_util
OracleSide) and its own causal attention over it.  Shapes: every KV format,
ragged contexts and query counts, whole prompts, draft-verification shapes
(a few tokens on long contexts, split over many items), MHA / GQA / MQA and
groups wider than a 16-row tile, both block sizes, rows before the cache."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_435_amd as pkv
from harness import workloads as W
from harness.device_cache import DeviceCase
from tests.gpu_util import OracleSide, compare, say, widen32

pytestmark = pytest.mark.gpu


def _queries(w, q_lens, seed=41):
    T = int(sum(q_lens))
    g = torch.Generator().manual_seed(seed)
    return torch.randn(T, w.num_q_heads, w.head_dim, generator=g).to(w.q_dtype)


def run_multi(w, q_lens, seqs_check=None, what="", rows_of=None, want_ref=False):
    q_lens = np.asarray(q_lens, dtype=np.int64)
    say(f"[multi] {what or w.name} fmt={w.kv_format} q={w.q_dtype} B={w.batch} "
        f"Hq={w.num_q_heads} Hkv={w.num_kv_heads} d={w.head_dim} bs={w.block_size} "
        f"ctx={w.context_lens.tolist()[:8]} L={q_lens.tolist()[:8]}")
    case = DeviceCase(w, keep_sources=True)
    q = _queries(w, q_lens)
    starts = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    out = torch.empty_like(q, device="cuda")
    pkv.paged_attention_multi_query(out, q.cuda(), torch.from_numpy(starts).cuda(), case.k_cache,
                                    case.v_cache, case.block_tables, case.context_lens, w.scale,
                                    w.max_context_len, k_scale=case.k_scale, v_scale=case.v_scale,
                                    kv_dtype=case.kv_dtype)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    side = OracleSide(w, case, seqs_check)   # the checked sequences (all by default), compact pool
    if seqs_check is not None:
        pick = rows_of or (lambda b: range(starts[b], starts[b + 1]))
        rows = [(r, h) for b in seqs_check for r in pick(b) for h in range(w.num_q_heads)]
        keep = sorted(int(b) for b in seqs_check)
        q_lens_o = q_lens[keep]
        starts_o = np.concatenate([[0], np.cumsum(q_lens_o)])
        q_o = np.concatenate([widen32(q[starts[b]:starts[b + 1]]) for b in keep]).astype(np.float64)
        remap = {}
        for i, b in enumerate(keep):
            for j in range(int(q_lens[b])):
                remap[int(starts[b]) + j] = int(starts_o[i]) + j
        rows_o = [(remap[r], h) for r, h in rows]
        ref_o = oracle.multi_query_attention(q_o, q_lens_o, side.k_cache, side.v_cache, side.tables,
                                             side.context_lens, w.scale, w.block_size,
                                             w.kv_format, side.k_scale, side.v_scale, rows=rows_o)
        idx = sorted({r for r, _ in rows})
        ref = np.full_like(got, np.nan)
        for r in idx:
            ref[r] = ref_o[remap[r]]
        compare(got[idx], ref[idx], w.kv_format, what or w.name)
        return got, case, q, starts
    ref = oracle.multi_query_attention(widen32(q).astype(np.float64), q_lens, side.k_cache,
                                       side.v_cache, side.tables, side.context_lens, w.scale,
                                       w.block_size, w.kv_format, side.k_scale, side.v_scale)
    compare(got, ref, w.kv_format, what or w.name)
    if want_ref:
        return got, case, q, starts, ref
    return got, case, q, starts


@pytest.mark.parametrize("q_dtype,kv", [
    (torch.float16, "f16"), (torch.bfloat16, "bf16"), (torch.float32, "f32"),
    (torch.float16, "i8"), (torch.bfloat16, "fp8"), (torch.float16, "i4"), (torch.bfloat16, "i4"),
    (torch.float32, "i4"),
])
def test_dtype_pairs_ragged(q_dtype, kv):
    w = W.custom(q_dtype, kv, [1, 17, 300, 1025, 2600], 8, 2, 128, 16, name=f"multi-{kv}")
    run_multi(w, [1, 5, 16, 33, 100])


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2), (16, 1), (40, 1)])
def test_whole_prompts(hq, hkv):
    w = W.custom(torch.float16, "f16", [37, 64, 100], hq, hkv, 128, 16, name=f"prompt-{hq}-{hkv}")
    run_multi(w, [37, 64, 100])


def test_draft_verification_long_contexts():
    """Four draft tokens per sequence on the 70B GQA-8 shape: few rows, long
    contexts, so each row tile is split over many items and merged."""
    ctx = np.random.default_rng(0).integers(512, 16384, 12, endpoint=True)
    w = W.custom(torch.float16, "f16", ctx, 64, 8, 128, 16, name="verify")
    run_multi(w, [4] * 12, seqs_check=[int(np.argmax(ctx)), int(np.argmin(ctx)), 5])


@pytest.mark.parametrize("bs", [16, 256])
def test_chunked_prefill_and_block_sizes(bs):
    w = W.custom(torch.bfloat16, "bf16", [700, 1300, 260], 32, 8, 64, bs, name=f"chunk-bs{bs}")
    run_multi(w, [256, 100, 260])


@pytest.mark.parametrize("hq,hkv", [(16, 2), (128, 1)])
def test_one_token_each_equals_decode(hq, hkv):
    """(128 query heads over one KV head: 128 rows per sequence, which would
    reach the prompt-chunk kernel's threshold; one token per sequence stays on
    the decode-shaped kernel, bit for bit equal to decode.)"""
    w = W.custom(torch.float16, "f16", [5, 900, 3000, 17], hq, hkv, 128, 16, name=f"L1-{hq}x{hkv}")
    got, case, q, starts = run_multi(w, [1, 1, 1, 1])
    dec = torch.empty_like(case.q)
    pkv.paged_attention_decode(dec, q.cuda(), case.k_cache, case.v_cache, case.block_tables,
                               case.context_lens, w.scale, w.max_context_len)
    torch.cuda.synchronize()
    assert np.array_equal(got, dec.float().cpu().numpy().astype(np.float64))


def test_rows_before_the_cache_are_zeros():
    w = W.custom(torch.float16, "f16", [3, 40], 4, 2, 128, 16, name="short")
    got, _, _, _ = run_multi(w, [5, 2])
    assert np.all(got[:2] == 0)


def test_workspace_too_small_raises():
    w = W.custom(torch.float16, "f16", [300], 4, 2, 128, 16, name="ws")
    case = DeviceCase(w)
    q = _queries(w, [8]).cuda()
    starts = torch.tensor([0, 8], dtype=torch.int32, device="cuda")
    tiny = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(RuntimeError, match="workspace"):
        pkv.paged_attention_multi_query(torch.empty_like(q), q, starts, case.k_cache, case.v_cache,
                                        case.block_tables, case.context_lens, w.scale,
                                        w.max_context_len, workspace=tiny)


@pytest.mark.parametrize("name", W.MULTI_NAMES)
def test_benchmark_workloads_sampled(name):
    """The benchmark's multi-token workloads at full size, in the configuration
    it times: the shortest and longest sequence plus one more, every query
    token of a verification step, and the first, middle and last rows of each
    512-token chunk, every query head."""
    w, q_lens = W.make_multi(name)
    ctx = w.context_lens
    seqs = sorted({int(np.argmin(ctx)), int(np.argmax(ctx)), 3})
    if name.startswith("llama70b_prefill512"):
        starts = np.concatenate([[0], np.cumsum(q_lens)])
        pick = lambda b: [int(starts[b]), int(starts[b]) + 255, int(starts[b + 1]) - 1]
        run_multi(w, q_lens, seqs_check=seqs, rows_of=pick)
    else:
        run_multi(w, q_lens, seqs_check=seqs)


def test_sequences_without_new_tokens_are_skipped():
    """Zero new tokens for some sequences (they contribute no rows), the others
    ragged, on an INT8 cache."""
    w = W.custom(torch.float16, "i8", [500, 90, 1200, 33, 700], 16, 4, 128, 16, name="L0")
    run_multi(w, [0, 7, 0, 33, 1])


# Prompt chunks: a mean of several hundred (query token, head) rows per
# sequence, f16/bf16 queries over a cache of their type, FP8, INT8 or INT4, so
# the calls take the LDS-sharing prefill kernel.  Cases: ragged chunk lengths, a sequence with no
# new tokens, one with more new tokens than cached ones (rows before the
# cache), a whole prompt (L = context), both block sizes, d 64 and 128, GQA,
# MHA and MQA, KV head counts that are not powers of two.
@pytest.mark.parametrize("q_dtype,d,bs,hq,hkv,ctx,lens,kv", [
    (torch.float16, 128, 16, 8, 2, [700, 64, 1500, 300, 90], [300, 100, 200, 0, 90], None),
    (torch.bfloat16, 128, 256, 8, 2, [700, 64, 1500, 300, 90], [300, 100, 200, 0, 90], None),
    (torch.float16, 64, 256, 4, 4, [600, 1000], [600, 400], None),
    (torch.bfloat16, 64, 16, 16, 1, [300, 129], [64, 129], None),
    (torch.float16, 128, 16, 8, 2, [700, 64, 1500, 300, 90], [300, 100, 200, 0, 90], "fp8"),
    (torch.bfloat16, 128, 256, 16, 1, [300, 129], [64, 129], "fp8"),
    (torch.bfloat16, 64, 16, 4, 4, [600, 1000], [600, 400], "fp8"),
    (torch.float16, 128, 16, 8, 2, [700, 64, 1500, 300, 90], [300, 100, 200, 0, 90], "i8"),
    (torch.bfloat16, 128, 256, 16, 1, [300, 129], [64, 129], "i8"),
    (torch.float16, 64, 256, 4, 4, [600, 1000], [600, 400], "i8"),
    (torch.float16, 128, 16, 8, 2, [700, 64, 1500, 300, 90], [300, 100, 200, 0, 90], "i4"),
    (torch.bfloat16, 128, 256, 16, 1, [300, 129], [64, 129], "i4"),
    (torch.float16, 128, 256, 4, 4, [600, 1000], [600, 400], "i4"),
    # three KV heads (not a power of two: the planning pass divides, and a row
    # group's heads are numbered 3 apart), at G = 4 and G = 3
    (torch.float16, 128, 16, 12, 3, [700, 64, 1500, 300, 90], [300, 100, 200, 0, 90], None),
    (torch.bfloat16, 128, 16, 9, 3, [900, 500, 40], [300, 200, 40], "i8"),
])
def test_prompt_chunks(q_dtype, d, bs, hq, hkv, ctx, lens, kv):
    """(FP8 rows: the same kernel over an FP8 E4M3FN cache, codes converted
    after the LDS read.  INT8 and INT4 rows: row-scaled codes, offset f16
    subnormals with f16 queries, exact bf16 with bf16 queries; unused slots'
    scales are NaN.)"""
    kv = kv or ("f16" if q_dtype == torch.float16 else "bf16")
    w = W.custom(q_dtype, kv, ctx, hq, hkv, d, bs, name=f"prompt-{kv}-d{d}-bs{bs}-{hq}x{hkv}")
    got, _, _, starts = run_multi(w, lens)
    if ctx[1] < lens[1] and len(lens) > 2:
        assert np.all(got[starts[1]:starts[1] + lens[1] - ctx[1]] == 0)


def test_prompt_chunk_on_a_long_context_is_split_and_merged():
    """One 64-token chunk (512 rows at G = 8) on a 12,000-token context: few
    virtual sequences, many tiles, so each one's context is cut into several
    items and merged.  Every row of the chunk is checked."""
    w = W.custom(torch.float16, "f16", [12000], 8, 1, 128, 16, name="prompt-split")
    run_multi(w, [64])


def test_prompt_chunks_of_mixed_lengths():
    """512-token chunks at GQA-8 over contexts of 9,000, 5,000, 300 and 4,500
    tokens: 1,024 virtual sequences, enough to fill the GPU, so items take whole
    contexts up to 512 tiles (the 5,000- and 4,500-token rows: items of more
    than 256 tiles) and the longest rows' contexts are cut into 2 items.  The workgroups take the groups longest first, which interleaves
    sequences, row groups and chunks of every size."""
    w = W.custom(torch.float16, "f16", [9000, 5000, 300, 4500], 64, 8, 128, 16,
                 name="prompt-mixed")
    lens = [512] * 4
    starts = np.concatenate([[0], np.cumsum(lens)])
    # (the first and last 24 tokens of each checked chunk: several row groups each)
    ends = lambda b: list(range(starts[b], starts[b] + 24)) + list(range(starts[b + 1] - 24, starts[b + 1]))
    run_multi(w, lens, seqs_check=[0, 2, 3], rows_of=ends)


@pytest.mark.parametrize("lens", [[1, 1, 1, 1, 1], [3, 2, 4, 1, 1]])
def test_merge_one_round_limit(lens):
    """Items of the minimum 8 tiles: a row over a context of n tiles is merged
    from ceil(n / 8) partials, and this merge loads up to 4 x 64 / 32 = 8 of
    them in one round at d 128.  Contexts of 1023-1040 tokens give a row
    group 8 or 9 partials, on both sides of that switch."""
    w = W.custom(torch.bfloat16, "bf16", [1024, 1025, 1023, 1040, 1], 16, 2, 128, 16,
                 name="multi-merge-limit")
    run_multi(w, lens)


@pytest.mark.parametrize("hq,hkv,qlen", [(64, 8, None), (16, 2, 16)])
def test_more_than_1024_sequences(hq, hkv, qlen):
    """1100 sequences: the planning pass takes them in two rounds of 1024 and
    its virtual sequences pass the 4096 whose contexts it keeps in LDS.  One
    or two draft tokens each at GQA-8 (the multi-token decode kernel), or
    16-token chunks at G = 8 (the prompt-chunk kernel).  Sampled sequences
    from both rounds are checked."""
    rng = np.random.default_rng(7)
    B = 1100
    lens = rng.integers(1, 3, B) if qlen is None else np.full(B, qlen)
    ctx = np.maximum(rng.integers(16, 100, B), lens)
    w = W.custom(torch.float16, "f16", ctx, hq, hkv, 128, 16, name=f"B{B}-{hq}x{hkv}")
    run_multi(w, lens, seqs_check=[0, 511, 1023, 1024, 1099])


def test_prompt_chunks_past_4096_row_groups():
    """4200 sequences of 16-token chunks at G = 8: one 128-row group each, so
    the planning pass takes its row groups in five rounds of 1024 and the
    contexts of those past the 4096 it keeps in LDS come from the workspace.
    Sampled sequences on both sides of each limit are checked."""
    rng = np.random.default_rng(11)
    B = 4200
    lens = np.full(B, 16)
    ctx = rng.integers(16, 80, B)
    w = W.custom(torch.float16, "f16", ctx, 16, 2, 128, 16, name=f"B{B}-rowgroups")
    run_multi(w, lens, seqs_check=[0, 1023, 1024, 4095, 4096, 4199])


@pytest.mark.parametrize("q_len", [4, 512])
def test_pool_past_2_31_bytes(q_len):
    """A 2.8 GB fp16 pool per cache read only from its blocks past the 2**31-byte
    mark: 4 draft tokens per sequence (the decode-shaped kernel) and 512-token
    prompt chunks (the prompt-chunk kernel).  Every (row, head) output must
    match the oracle's (relative L2)."""
    from tests.gpu_util import per_head_rel_l2
    from tests.test_gpu_decode import _high_block_workload
    w = _high_block_workload("multi_pool_past_2_31", torch.float16, "f16", 16, 85197, True,
                             nseq=4, ctx=2048)
    got, case, _, _, ref = run_multi(w, [q_len] * 4, want_ref=True)
    e = per_head_rel_l2(got, ref)
    say(f"  per-row relative L2 error: max {e.max():.3e}")
    assert e.max() < 1e-2
    del case
    torch.cuda.empty_cache()
