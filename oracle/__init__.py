"""CPU oracle for masked variable-length softmax attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this package: only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library and imports nothing from it.

The oracle is deliberately plain and slow. Every function is the textbook
definition of what the method computes, written in NumPy and evaluated densely
(full ``[Lq, Lk]`` masks, full score matrices). The default floating-point
precision is fp32, the precision of the dense reference the pages test their
kernels against (vLLM PR #50294 page, implementation breakdown step 5; vLLM PR
#49815 page, key code snippets, the test's ``_reference``); every function also
accepts ``dtype=np.float64``.

Sources (the web pages this package restates):
  * [PR50294]  prhub.com.cn, vLLM PR #50294: FA4 mm_prefix range scan replaced
    by an O(1) per-query-row lookup table.
  * [PR49815]  prhub.com.cn, vLLM PR #49815: MiMo vision window attention with a
    per-head sink added to key 0's logit.
  * [PR55624]  prhub.com.cn, vLLM PR #55624 report: sliding-window layers in
    MFU/MBU accounting.
  * [step14_4] mini-vllm tutorial step14_4: causal mask by broadcast, skipped
    at decode.

Pinning status (what fixes each function independently of itself) is listed in
each module's header. Functions with no independent pin say "parity unpinned".
"""

from .table import CapacityError, ref_build_table
from .mask import ref_mask
from .attention import SINK_NONE, SINK_KEY0_BIAS, SINK_NULL_LOGIT, ref_attention, ref_attention_rows
from .decode import ref_gather_paged, ref_paged_decode
from .work import ExecutionContext, ref_useful_pairs, ref_useful_flops, ref_decode_useful_bytes

__all__ = [
    "CapacityError",
    "ref_build_table",
    "ref_mask",
    "SINK_NONE",
    "SINK_KEY0_BIAS",
    "SINK_NULL_LOGIT",
    "ref_attention",
    "ref_attention_rows",
    "ref_gather_paged",
    "ref_paged_decode",
    "ExecutionContext",
    "ref_useful_pairs",
    "ref_useful_flops",
    "ref_decode_useful_bytes",
]
