"""CPU oracle for decode attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plainly correct
reference that the HIP library is checked against.  Only the test suite, the
smoke check and the CPU-baseline leg of the benchmark may import it; the
product path never does.  It imports nothing from the product package and
shares no code with it (the only thing both sides consume is the seeded input
generator, which holds none of the method's arithmetic).

Pages this follows (titles as published; cited below by the short tag):

  [P1] «LLM推理显存优化：KV Cache管理3大策略实测，节省60%显存开销» (mlqm.cn)
  [P2] «生产级 LLM 推理的 KV 缓存优化» — "The Ultimate Guide to KV Cache
       Optimization for LLM Inference"
  [P3] «大模型推理加速实战：KV Cache内存优化与PagedAttention分页管理方案»

Arithmetic is float64 except where a page fixes the precision of a step that
decides an integer: the INT8 quantizer ([P1] §4, quantize_tensor) and the FP8
encoder run their scale and rounding in float32, as the kernels do.

Every function is pinned by a CPU test against something other than itself
(closed forms, the worked block table of [P3], brute force on tiny inputs,
library routines on the special cases, invariants).  No function here is
"parity unpinned".

Modules
  kvsize     closed-form KV-cache sizes                     [P1] §1, [P2] §2, [P3]
  widen      stored bytes (f32/f16/bf16/int8/fp8/int4) -> float64  [P1] §4, [P2] §4, [P3]
  paging     slot arithmetic and block-table gather          [P1] §2, [P3]
  attention  paged decode attention = standard attention over the gathered cache
  quant      INT8 / INT4 per-row and FP8 per-tensor quantizers, nibble packing  [P1] §4, [P3]
  append     expected cache after writing new tokens' rows   [P3]
  layout     stored order of the pools <-> logical [NB][Hkv][bs][d] order
  multi      several new query tokens per sequence, causal   [P3]
"""

from . import kvsize, widen, paging, attention, quant, append, layout, multi  # noqa: F401
from .attention import decode_attention, attend, validate_tables  # noqa: F401
from .multi import multi_query_attention  # noqa: F401
from .quant import (quantize_int8_rows, quantize_int4_rows, pack_int4, unpack_int4,  # noqa: F401
                    fp8_tensor_scale, encode_e4m3fn, quantize_fp8)
from .widen import widen_kv  # noqa: F401
