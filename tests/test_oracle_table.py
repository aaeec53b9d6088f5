"""Pins for the oracle's range-table builder (CPU only).

The expected values come from the vLLM PR #50294 page (worked example in
"key code snippets"; clipping, degenerate ranges, empty returns and the
capacity assert in "implementation breakdown" step 1 and "risks"), never from
the HIP library.
"""

import os

import numpy as np
import pytest

from oracle import CapacityError, ref_build_table

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example_table.txt")
POISON = 12345


def _load_golden():
    vals = [ln.split() for ln in open(GOLDEN) if ln.strip() and not ln.startswith("#")]
    ret = int(vals[0][0])
    rows = np.array([[int(a), int(b)] for _, a, b in vals[1:]], dtype=np.int32)
    return ret, rows


def _qsl(query_lens):
    return np.concatenate([[0], np.cumsum(query_lens)]).astype(np.int32)


def _scan_keep(ranges, p, k):
    """The range scan the page's test compares against: any valid range holding both."""
    return any(s < e and s <= p <= e and s <= k <= e for s, e in ranges)


def test_worked_example_matches_golden():
    ranges = {0: [(1, 3), (5, 7)], 1: [(2, 4), (9, 12)]}
    out = np.full((16, 2), POISON, dtype=np.int32)
    n = ref_build_table(out, ranges, _qsl([8, 6]), np.array([8, 13]))
    ret, rows = _load_golden()
    assert n == ret
    np.testing.assert_array_equal(out, rows)


def test_worked_example_equals_range_scan():
    """O(1) lookup == brute-force scan for every (query position, key), with a context offset."""
    ranges = {0: [(1, 3), (5, 7)], 1: [(2, 4), (9, 12)]}
    query_lens, seq_lens = [8, 6], [8, 13]
    out = np.full((16, 2), POISON, dtype=np.int32)
    ref_build_table(out, ranges, _qsl(query_lens), np.array(seq_lens))
    row0 = 0
    for b, ql in enumerate(query_lens):
        ctx = seq_lens[b] - ql
        for i in range(ql):
            s, e = out[row0 + i]
            for k in range(seq_lens[b]):
                assert (s <= k <= e) == _scan_keep(ranges[b], ctx + i, k), (b, i, k)
        row0 += ql


@pytest.mark.parametrize("seed", range(12))
def test_random_batches_equal_range_scan(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 6))
    seq_lens = rng.integers(1, 60, size=B)
    query_lens = np.array([int(rng.integers(0, L + 1)) for L in seq_lens])
    ranges = {}
    for b in range(B):
        rs, pos = [], int(rng.integers(0, 4))
        while pos < seq_lens[b] + 6 and len(rs) < 6:  # some ranges run past the scheduled keys
            ln = int(rng.integers(0, 9))
            rs.append((pos, pos + ln) if rng.random() > 0.1 else (pos + ln, pos))  # a few degenerate
            pos += ln + 1 + int(rng.integers(0, 6))
        ranges[b] = rs
    cap = int(query_lens.sum()) + 3
    out = np.full((cap, 2), POISON, dtype=np.int32)
    n = ref_build_table(out, ranges, _qsl(query_lens), seq_lens)
    covered = False
    row0 = 0
    for b in range(B):
        ctx = int(seq_lens[b] - query_lens[b])
        for i in range(int(query_lens[b])):
            p = ctx + i
            in_any = any(s < e and s <= p <= e for s, e in ranges[b])
            covered |= in_any
            if n:
                s, e = out[row0 + i]
                for k in range(int(seq_lens[b])):
                    assert (s <= k <= e) == _scan_keep(ranges[b], p, k)
        row0 += int(query_lens[b])
    assert (n > 0) == covered
    if n:
        assert n == int(query_lens.sum())
        assert (out[n:] == POISON).all()
    else:
        assert (out == POISON).all()


def test_clipping_to_scheduled_chunk():
    """Ranges partly in the context, partly past the chunk, and wholly in the future."""
    out = np.full((8, 2), POISON, dtype=np.int32)
    # ctx 6, 4 queries at positions 6..9: (4,7) covers positions 6,7 -> rows 0,1
    n = ref_build_table(out, {0: [(4, 7)]}, _qsl([4]), np.array([10]))
    assert n == 4
    np.testing.assert_array_equal(out[:4], [[4, 7], [4, 7], [-1, -1], [-1, -1]])
    # ctx 4, positions 4..7: (6,12) runs past the chunk -> rows 2,3 hold the unclipped pair
    out[:] = POISON
    n = ref_build_table(out, {0: [(6, 12)]}, _qsl([4]), np.array([8]))
    assert n == 4
    np.testing.assert_array_equal(out[:4], [[-1, -1], [-1, -1], [6, 12], [6, 12]])
    # a range wholly in the future of the chunk writes nothing: return 0, buffer untouched
    out[:] = POISON
    assert ref_build_table(out, {0: [(9, 11)]}, _qsl([4]), np.array([8])) == 0
    assert (out == POISON).all()


def test_decode_rows_fall_outside_ranges():
    """A decode row (one query at the last position) of a 20-token sequence; range (2,9)."""
    out = np.full((4, 2), POISON, dtype=np.int32)
    for upper_bound in (20, 21, 64, 1 << 20):  # any optimistic upper bound on the length
        assert ref_build_table(out, {0: [(2, 9)]}, _qsl([1]), np.array([upper_bound])) == 0
    assert (out == POISON).all()


def test_degenerate_ranges_skipped():
    out = np.full((8, 2), POISON, dtype=np.int32)
    assert ref_build_table(out, {0: [(5, 5), (6, 5)]}, _qsl([8]), np.array([8])) == 0
    assert (out == POISON).all()
    n = ref_build_table(out, {0: [(5, 5), (1, 2)]}, _qsl([8]), np.array([8]))
    assert n == 8
    np.testing.assert_array_equal(out[:, 0], [-1, 1, 1, -1, -1, -1, -1, -1])


def test_none_and_empty_batches_return_zero():
    out = np.full((4, 2), POISON, dtype=np.int32)
    assert ref_build_table(out, None, _qsl([3]), np.array([3])) == 0
    assert ref_build_table(out, {0: [(0, 2)]}, _qsl([0]), np.array([0])) == 0
    assert ref_build_table(out, {}, _qsl([3]), np.array([3])) == 0
    assert (out == POISON).all()


def test_capacity_overflow_raises():
    out = np.full((4, 2), POISON, dtype=np.int32)
    with pytest.raises(CapacityError):
        ref_build_table(out, {0: [(0, 2)]}, _qsl([5]), np.array([5]))
    assert (out == POISON).all()


def test_stale_rows_are_reset_on_reuse():
    """A reused buffer must not leak the previous step's ranges (page, step 1 comment)."""
    out = np.full((8, 2), POISON, dtype=np.int32)
    assert ref_build_table(out, {0: [(0, 7)]}, _qsl([8]), np.array([8])) == 8
    assert ref_build_table(out, {0: [(6, 7)]}, _qsl([8]), np.array([8])) == 8
    np.testing.assert_array_equal(out[:, 0], [-1] * 6 + [6, 6])
