"""Useful-work accounting for throughput reporting.

Counts only the work the method must do: visible (query, key) pairs for
prefill (``4 * head_dim`` FLOPs per pair per query head: ``2 * D`` for the
score, ``2 * D`` for the value accumulation) and, for decode, the K and V bytes
of visible tokens. Masked pairs, skipped tiles and window-clamped context
never count (vLLM PR #55624 report: attention FLOPs and KV-cache reads of a
sliding-window layer are clamped to the window).

Each query row's visible keys are the union of two key intervals - the base
term (causal/window) and the multimodal range clamped on its past side - so a
row's count is the size of that union, computed here in closed form with
NumPy over all rows at once. (The test suite checks this against a dense
popcount of the mask.)
"""

from __future__ import annotations

import numpy as np


def _interval_sizes(lo, hi):
    return np.maximum(hi - lo + 1, 0)


def visible_pairs_per_request(Lq, Lk, causal, wl, wr, table_rows=None) -> int:
    if Lq <= 0 or Lk <= 0:
        return 0
    p = (Lk - Lq) + np.arange(Lq, dtype=np.int64)
    last = Lk - 1
    blo = np.maximum(p - wl, 0) if wl >= 0 else np.zeros_like(p)
    if causal:
        bhi = p.copy()
    elif wr >= 0:
        bhi = p + wr
    else:
        bhi = np.full_like(p, last)
    bhi = np.minimum(bhi, last)
    base = _interval_sizes(blo, bhi)
    if table_rows is None:
        return int(base.sum())
    t = np.asarray(table_rows, dtype=np.int64).reshape(Lq, 2)
    mlo = np.maximum(t[:, 0], 0)
    if wl >= 0:
        mlo = np.maximum(mlo, p - wl)
    mhi = np.minimum(t[:, 1], last)
    mm = _interval_sizes(mlo, mhi)
    ov = _interval_sizes(np.maximum(blo, mlo), np.minimum(bhi, mhi))
    ov = np.where((base > 0) & (mm > 0), ov, 0)
    return int((base + mm - ov).sum())


def prefill_visible_pairs(cu_q, cu_k, causal, wl, wr, table=None) -> int:
    """Visible pairs of one head over a packed batch."""
    total = 0
    for b in range(len(cu_q) - 1):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        Lk = int(cu_k[b + 1]) - int(cu_k[b])
        rows = None if table is None else np.asarray(table)[q0:q1]
        total += visible_pairs_per_request(q1 - q0, Lk, causal, wl, wr, rows)
    return total


def prefill_useful_flops(cu_q, cu_k, num_q_heads, head_dim, causal, wl, wr, table=None) -> int:
    return 4 * head_dim * num_q_heads * prefill_visible_pairs(cu_q, cu_k, causal, wl, wr, table)


def decode_visible_tokens(seq_lens, wl) -> int:
    L = np.asarray(seq_lens, dtype=np.int64)
    return int(np.minimum(L, wl + 1).sum()) if wl >= 0 else int(L.sum())


def decode_useful_bytes(seq_lens, num_kv_heads, head_dim, elem_bytes, wl) -> int:
    """K + V bytes of the visible tokens of every kv head."""
    return decode_visible_tokens(seq_lens, wl) * num_kv_heads * head_dim * 2 * elem_bytes
