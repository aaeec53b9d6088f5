"""Oracle for useful-work accounting (FLOPs and bytes that count toward throughput).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Two counters live here.

1. ``ExecutionContext`` restates the per-request accounting of [PR55624]
   ("implementation breakdown" steps 2 and 4, and the ``ExecutionContext``
   snippet): each request adds ``(num_tokens, context_len, is_prefill)``; with
   a window ``W`` every context length is clamped to ``min(context_len, W)``
   before it enters the token-by-context product (attention FLOPs) or the
   decode context sum (KV-cache reads); without a window the unclamped
   aggregates are used. The attention-core FLOPs of one layer are
   ``2 * H * D`` per (token, context) pair for ``Q K^T`` and the same for
   ``P V``. This form ignores the prefill triangle, so it is an upper bound
   for prefill (the page's own risk section says so) and exact for decode.

2. ``ref_useful_pairs`` counts the visible (query, key) pairs exactly, as the
   popcount of the oracle mask of every request. Useful FLOPs are
   ``4 * D`` per visible pair per query head (``2 * D`` for the score, ``2 * D``
   for the value accumulation). Decode useful bytes are the K and V bytes of
   the visible tokens of every kv head.

Pins (tests/test_oracle_decode_work.py): [PR55624]'s closed-form clamp test (a decode
token with context 8192 and window 1024 costs exactly one eighth of the dense
core FLOPs; context 512 under window 1024 costs the same as dense), the 8x and
32x over-estimates the page quotes for 32K and 128K contexts under a 4096
window, and exact popcount never above the page's bound.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .mask import ref_mask


@dataclass
class ExecutionContext:
    """Per-step accounting of scheduled requests ([PR55624], key code snippets)."""

    prefill_num_tokens: int = 0
    prefill_context_len: int = 0
    prefill_token_context_product: int = 0
    decode_num_tokens: int = 0
    decode_context_len: int = 0
    decode_token_context_product: int = 0
    requests: list = field(default_factory=list)

    def add(self, num_tokens: int, context_len: int, is_prefill: bool) -> None:
        self.requests.append((num_tokens, context_len, is_prefill))
        if is_prefill:
            self.prefill_num_tokens += num_tokens
            self.prefill_context_len += context_len
            self.prefill_token_context_product += num_tokens * context_len
        else:
            self.decode_num_tokens += num_tokens
            self.decode_context_len += context_len
            self.decode_token_context_product += num_tokens * context_len

    def total_token_context_product(self, sliding_window=None) -> int:
        if sliding_window is None:
            return self.prefill_token_context_product + self.decode_token_context_product
        return sum(n * min(c, sliding_window) for n, c, _ in self.requests)

    def prefill_context_len_for_window(self, sliding_window=None) -> int:
        if sliding_window is None:
            return self.prefill_context_len
        return sum(min(c, sliding_window) for _, c, pre in self.requests if pre)

    def decode_context_len_for_window(self, sliding_window=None) -> int:
        if sliding_window is None:
            return self.decode_context_len
        return sum(min(c, sliding_window) for _, c, pre in self.requests if not pre)

    def attn_core_flops(self, num_heads: int, head_dim: int, sliding_window=None) -> dict:
        """``attn_qk`` and ``attn_av`` FLOPs of one layer."""
        tc = self.total_token_context_product(sliding_window)
        return {"attn_qk": 2 * num_heads * head_dim * tc, "attn_av": 2 * num_heads * head_dim * tc}


def ref_useful_pairs(cu_q, cu_k, causal=False, wl=-1, wr=-1, table=None) -> int:
    """Number of visible (query, key) pairs of one head, summed over the batch."""
    total = 0
    for b in range(len(cu_q) - 1):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        Lq, Lk = q1 - q0, int(cu_k[b + 1]) - int(cu_k[b])
        if Lq == 0:
            continue
        rows = None if table is None else np.asarray(table)[q0:q1]
        total += int(ref_mask(Lq, Lk, causal, wl, wr, rows).sum())
    return total


def ref_useful_flops(cu_q, cu_k, num_q_heads, head_dim, causal=False, wl=-1, wr=-1, table=None) -> int:
    """Useful FLOPs: ``4 * D`` per visible pair per query head."""
    return 4 * head_dim * num_q_heads * ref_useful_pairs(cu_q, cu_k, causal, wl, wr, table)


def ref_decode_useful_bytes(seq_lens, num_kv_heads, head_dim, elem_bytes, wl=-1) -> int:
    """K plus V bytes of the visible tokens: each sequence sees ``min(L, wl + 1)`` keys."""
    total = 0
    for L in seq_lens:
        L = int(L)
        vis = int(ref_mask(1, L, True, wl, -1).sum()) if L > 0 else 0
        total += vis * num_kv_heads * head_dim * 2 * elem_bytes
    return total
