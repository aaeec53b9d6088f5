"""Oracle for the per-query-row multimodal-prefix range table.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the table is ([PR50294], "implementation breakdown" step 1 and the
``fill_mm_prefix_query_ranges`` snippet under "key code snippets"):

  * Request ``b`` schedules ``Lq_b`` query tokens that occupy packed rows
    ``query_start_loc[b] .. query_start_loc[b+1]-1``. Its key count is
    ``seq_lens[b]`` and its context offset is ``ctx_b = seq_lens[b] - Lq_b``,
    so local query ``i`` sits at absolute position ``p = ctx_b + i``.
  * A request owns a list of ``(start, end)`` ranges, both ends inclusive, in
    absolute positions. Ranges of one request never overlap
    ([PR50294], implementation breakdown step 2). A range with
    ``start >= end`` is degenerate and ignored (step 1).
  * Row ``t`` of the table holds the ``(start, end)`` of the valid range whose
    inclusive span contains the row's position ``p``, or ``(-1, -1)`` when no
    range does. The stored pair is the unclipped range; only the rows written
    are limited to the scheduled chunk.
  * The call returns the number of packed rows ``N`` when at least one
    scheduled row lies in a range, and 0 otherwise (no ranges at all, an empty
    batch, or every range outside the scheduled chunk). A return of 0 leaves
    the buffer untouched. A positive return writes exactly rows ``[0, N)``.
  * ``N`` larger than the buffer is an error (the page asserts).

The oracle writes that definition out row by row: for every row it scans the
request's ranges. This is the O(rows x ranges) form; the library computes the
same table from per-range spans in O(rows + ranges). The two share nothing.

When ranges do overlap (outside the contract) the page's fill order makes the
later range in (request, list) order win; the row scan reproduces that by
taking the last matching range.

Pins (tests/test_oracle_table.py): the page's worked example with the
brute-force range scan its test uses, hand-derived clipping and decode-row
cases, degenerate ranges, poison-buffer untouched-row checks.
"""

from __future__ import annotations

import numpy as np


class CapacityError(ValueError):
    """More scheduled rows than the caller's table buffer holds."""


def ref_build_table(out, mm_ranges, query_start_loc, seq_lens) -> int:
    """Fill ``out[:N]`` with each query row's covering range; return N or 0.

    Args:
      out: int32 array ``[capacity, 2]`` owned by the caller. Rows at or past
        the return value are never written.
      mm_ranges: ``dict[request index -> list[(start, end)]]`` or None.
      query_start_loc: ``B+1`` prefix sums of scheduled query counts.
      seq_lens: ``B`` key counts (context plus this chunk) per request.
    """
    if mm_ranges is None:
        return 0
    qsl = [int(x) for x in query_start_loc]
    n_rows = qsl[-1]
    if n_rows <= 0:
        return 0
    if n_rows > out.shape[0]:
        raise CapacityError(f"table holds {out.shape[0]} rows, batch has {n_rows}")

    rows = []  # (row, start, end) for every covered row
    num_reqs = len(qsl) - 1
    for b in range(num_reqs):
        q_len = qsl[b + 1] - qsl[b]
        if q_len <= 0:
            continue
        ctx = int(seq_lens[b]) - q_len
        ranges = mm_ranges.get(b, []) if hasattr(mm_ranges, "get") else []
        for i in range(q_len):
            p = ctx + i
            hit = None
            for start, end in ranges:
                if start < end and start <= p <= end:
                    hit = (int(start), int(end))  # last match wins
            if hit is not None:
                rows.append((qsl[b] + i, hit[0], hit[1]))

    if not rows:
        return 0
    for t in range(n_rows):
        out[t, 0] = -1
        out[t, 1] = -1
    for t, start, end in rows:
        out[t, 0] = start
        out[t, 1] = end
    return n_rows
