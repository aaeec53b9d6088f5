"""Oracle for paged decode attention.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Decode is the one-query case of prefill: the new token sits at position
``L - 1`` of a sequence of ``L`` keys, so a causal mask hides nothing and only a
window trims the past ([step14_4], "solution": with one query row every key is
visible and the mask is skipped; [PR55624], implementation breakdown step 2:
decode context is clamped to the window). Decode rows never fall inside a
multimodal range ([PR50294], implementation breakdown step 3), so there is no
table.

The cache layout is fixed here (the pages give none): per physical page,
``[Hkv, page_size, D]`` ("HND"); the cache is ``[num_pages, Hkv, page_size, D]``.
``block_table[b, j]`` is the physical page holding tokens
``j*page_size .. (j+1)*page_size - 1`` of sequence ``b``.

The oracle gathers each sequence's keys and values through the block table
into contiguous ``[L, Hkv, D]`` arrays, then evaluates the prefill oracle with
``Lq = 1``, ``Lk = L``, causal, past window ``wl``.

Pins (tests/test_oracle_decode_work.py): equal to the contiguous prefill oracle at
``Lq = 1``; invariant under any permutation of physical pages; a window of
``W`` keeps exactly ``min(L, W)`` keys.
"""

from __future__ import annotations

import numpy as np

from .attention import SINK_NONE, ref_attention


def ref_gather_paged(cache, block_table_row, L: int, page_size: int) -> np.ndarray:
    """Contiguous ``[L, Hkv, D]`` view of one sequence from an HND page cache."""
    Hkv, D = cache.shape[1], cache.shape[3]
    out = np.zeros((L, Hkv, D), dtype=cache.dtype)
    for t in range(L):
        page = int(block_table_row[t // page_size])
        out[t] = cache[page, :, t % page_size, :]
    return out


def ref_paged_decode(q, k_cache, v_cache, block_table, seq_lens, page_size, scale, wl=-1,
                     sinks=None, sink_mode=SINK_NONE, dtype=np.float32, seqs=None):
    """Decode attention for ``q`` ``[B, Hq, D]``; returns (out ``[B, Hq, D]``, lse ``[Hq, B]``).

    ``seqs`` restricts the evaluation to a subset of sequences (others stay 0).
    """
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D), dtype=dtype)
    lse = np.full((Hq, B), -np.inf, dtype=dtype)
    for b in (range(B) if seqs is None else seqs):
        L = int(seq_lens[b])
        kb = ref_gather_paged(k_cache, block_table[b], L, page_size)
        vb = ref_gather_paged(v_cache, block_table[b], L, page_size)
        o, l_ = ref_attention(q[b:b + 1], kb, vb, [0, 1], [0, L], scale, causal=True, wl=wl,
                              wr=-1, table=None, sinks=sinks, sink_mode=sink_mode, dtype=dtype)
        out[b] = o[0]
        lse[:, b] = l_[:, 0]
    return out, lse
