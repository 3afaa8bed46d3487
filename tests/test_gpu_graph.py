"""The decode step (append + paged_attention_decode) and a multi-token call
captured into a HIP graph and replayed: the library enqueues only kernels (no
allocation, no memset), so a captured step must give the eager step's output
bit for bit on every replay, with other eager work and synchronisations
between replays."""
import numpy as np
import pytest
import torch

import paged_kv_cache_435_amd as pkv
from harness import workloads as W
from harness.device_cache import DeviceCase
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kv", ["f16", "i4"])
def test_captured_decode_step_replays_bit_exact(kv):
    w = W.custom(torch.float16, kv, [300, 2049, 5000, 17], 16, 2, 128, 16, appends=True,
                 name=f"graph-{kv}")
    say(f"[graph] {w.name}")
    case = DeviceCase(w)
    ws = torch.empty(max(pkv.paged_attention_workspace_size(w.batch, w.num_q_heads,
                                                            w.num_kv_heads, w.head_dim,
                                                            w.max_context_len), 1),
                     dtype=torch.uint8, device="cuda")

    def step():
        pkv.kv_cache_append(case.new_k, case.new_v, case.slots, case.k_cache, case.v_cache,
                            case.k_scale, case.v_scale, kv_dtype=case.kv_dtype)
        pkv.paged_attention_decode(case.out, case.q, case.k_cache, case.v_cache,
                                   case.block_tables, case.context_lens, w.scale,
                                   w.max_context_len, k_scale=case.k_scale, v_scale=case.v_scale,
                                   kv_dtype=case.kv_dtype, workspace=ws)

    step()                                   # eager (also settles one-time host queries)
    torch.cuda.synchronize()
    eager = case.out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for i in range(4):
        case.out.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()   # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(case.out, eager), f"replay {i} differs from the eager step"


@pytest.mark.parametrize("q_lens", [[64, 100, 1], [4, 4, 4]])
def test_captured_multi_query_replays_bit_exact(q_lens):
    """[64, 100, 1]: 220 rows per sequence on average, the prompt-chunk kernel;
    [4, 4, 4]: draft tokens, the multi-token decode kernel."""
    w = W.custom(torch.float16, "f16", [700, 1300, 260], 32, 8, 128, 16, name="graph-multi")
    q_lens = np.array(q_lens)
    say(f"[graph] {w.name} L={q_lens.tolist()}")
    case = DeviceCase(w)
    g0 = torch.Generator(device="cuda")
    g0.manual_seed(3)
    q = torch.randn(int(q_lens.sum()), w.num_q_heads, w.head_dim, generator=g0,
                    device="cuda").half()
    out = torch.empty_like(q)
    starts = torch.tensor(np.concatenate([[0], np.cumsum(q_lens)]), dtype=torch.int32,
                          device="cuda")
    ws = torch.empty(pkv.paged_attention_multi_workspace_size(w.batch, q.shape[0], w.num_q_heads,
                                                              w.num_kv_heads, w.head_dim,
                                                              w.max_context_len),
                     dtype=torch.uint8, device="cuda")

    def call():
        pkv.paged_attention_multi_query(out, q, starts, case.k_cache, case.v_cache,
                                        case.block_tables, case.context_lens, w.scale,
                                        w.max_context_len, workspace=ws)

    call()
    torch.cuda.synchronize()
    eager = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    torch.cuda.synchronize()
    for i in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs from the eager call"
