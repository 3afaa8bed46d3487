"""The named workloads at full size, in the launch configuration the
benchmark times (append of one token per sequence, then decode), against the
CPU oracle: every sequence for the small ones; for the large ones the shortest
and the longest sequence plus seeded random ones, each with all its query
heads, and the first and last layer of the 80-layer FP8 case.  The stored
bytes at every live slot of the checked sequences are compared bit for bit
with the oracle's own quantized and appended cache."""
import numpy as np
import pytest
import torch

from harness import workloads as W
from tests.gpu_util import OracleSide, per_head_rel_l2, run_and_check

pytestmark = pytest.mark.gpu


def _sample_seqs(w, n_seq, seed=0):
    ctx = w.context_lens
    picks = {int(np.argmin(ctx)), int(np.argmax(ctx))}
    rng = np.random.default_rng(seed)
    for b in rng.permutation(w.batch):
        if len(picks) >= n_seq:
            break
        picks.add(int(b))
    return sorted(picks)


def test_tiny_fp32_whole():
    err, _, _ = run_and_check(W.make("tiny_fp32"))
    assert err < 1e-5


def test_llama7b_bf16_whole():
    run_and_check(W.make("llama7b_bf16"))


def test_llama70b_gqa8_sampled():
    w = W.make("llama70b_gqa8")
    run_and_check(w, seqs=_sample_seqs(w, 6))


def test_llama13b_int8_whole():
    run_and_check(W.make("llama13b_int8"))


@pytest.mark.parametrize("bs", [16, 256])
def test_llama70b_fp8_sampled_layers(bs):
    w = W.make("llama70b_fp8", block_size=bs)
    for layer in (0, w.layers - 1):
        run_and_check(w, seqs=_sample_seqs(w, 5, seed=layer), layer=layer)
        torch.cuda.empty_cache()


def test_llama13b_int4_whole():
    run_and_check(W.make("llama13b_int4"))


def test_llama70b_int4_sampled():
    w = W.make("llama70b_int4")
    run_and_check(w, seqs=_sample_seqs(w, 6))


def test_llama70b_gqa8_32k_sampled():
    # every context at 32K: pools of 2.7 GB per cache, so tile offsets pass 2**31
    # bytes; outputs are ~4e-2 at most, so each head's row is also held to a
    # relative L2 error (fp16 rounding gives ~3e-4)
    w = W.make("llama70b_gqa8_32k")
    seqs = [0, 17, w.batch - 1]
    _, case, got = run_and_check(w, seqs=seqs)
    ref = OracleSide(w, case, seqs).attention()
    e = per_head_rel_l2(got[seqs], ref)
    assert e.max() < 1e-2, f"per-head relative L2 error {e.max():.3e}"
    del case
    torch.cuda.empty_cache()


def test_two_round_plan_int4_32k_sampled():
    # The 70B GQA-8 layer at every context 32K over an INT4 cache: INT4 items stop
    # at 256 tiles, so 524,288 tiles over 2,048 slots need two rounds of items.
    ctx = [32768] * 32
    w = W.custom(torch.float16, "i4", ctx, 64, 8, 128, 16, name="int4-32k-two-rounds")
    run_and_check(w, seqs=[0, 13, 31])
    torch.cuda.empty_cache()
