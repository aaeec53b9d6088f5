"""Pins for the oracle's visibility mask (CPU only).

Independent anchors: the mini-vllm step14_4 tutorial's two equivalent causal
forms; a per-element loop over the predicate written from the vLLM PR #50294
mask_mod description; the range-scan form of the multimodal term used by that
page's test; the 2w+1 key count of the MiMo window (vLLM PR #49815 test
reference); decode rows, where the tutorial skips the mask entirely.
"""

import itertools

import numpy as np
import pytest

from oracle import ref_build_table, ref_mask


def _loop_mask(Lq, Lk, causal, wl, wr, rows=None):
    c = Lk - Lq
    m = np.zeros((Lq, Lk), dtype=bool)
    for i in range(Lq):
        for k in range(Lk):
            delta = c + i - k
            keep = True
            if causal and delta < 0:
                keep = False
            if wl >= 0 and delta > wl:
                keep = False
            if wr >= 0 and -delta > wr:
                keep = False
            mm = False
            if rows is not None:
                s, e = rows[i]
                mm = s <= k <= e and (wl < 0 or delta <= wl)
            m[i, k] = keep or mm
    return m


@pytest.mark.parametrize("total,start", [(4, 0), (9, 3), (16, 15), (7, 6), (12, 0)])
def test_causal_equals_tutorial_forms(total, start):
    seq = total - start
    q_idx = np.arange(seq)[:, None]
    k_idx = np.arange(total)[None, :]
    masked_broadcast = k_idx > (start + q_idx)
    allow_tril = np.tril(np.ones((total, total), dtype=bool))[start:start + seq]
    m = ref_mask(seq, total, True, -1, -1)
    np.testing.assert_array_equal(~m, masked_broadcast)
    np.testing.assert_array_equal(m, allow_tril)


def test_tutorial_four_by_four_picture():
    expect = np.array([[1, 0, 0, 0], [1, 1, 0, 0], [1, 1, 1, 0], [1, 1, 1, 1]], dtype=bool)
    np.testing.assert_array_equal(ref_mask(4, 4, True, -1, -1), expect)


@pytest.mark.parametrize("L", [1, 5, 64, 1000])
def test_decode_row_sees_everything(L):
    assert ref_mask(1, L, True, -1, -1).all()
    assert ref_mask(1, L, False, -1, -1).all()


def test_decode_row_window_keeps_w_keys():
    for L, W in [(8192, 1024), (512, 1024), (4097, 4096), (1, 4096)]:
        assert ref_mask(1, L, True, W - 1, -1).sum() == min(L, W)


@pytest.mark.parametrize("w,L", [(8, 37), (8, 5), (128, 1024), (3, 3)])
def test_bidirectional_window_counts(w, L):
    m = ref_mask(L, L, False, w, w)
    pos = np.arange(L)
    expect = np.abs(pos[:, None] - pos[None, :]) <= w  # the MiMo reference's window
    np.testing.assert_array_equal(m, expect)
    interior = m[w:L - w] if L > 2 * w else m[:0]
    assert (interior.sum(axis=1) == 2 * w + 1).all()


def test_predicate_matches_loop_exhaustively():
    rng = np.random.default_rng(5)
    for Lq, Lk in [(1, 1), (3, 3), (4, 9), (7, 7), (5, 12), (11, 11)]:
        for causal, wl, wr in itertools.product([False, True], [-1, 0, 2, 5], [-1, 0, 3]):
            rows = None
            if rng.random() < 0.6:
                rows = np.full((Lq, 2), -1, dtype=np.int64)
                ranges = [(1, 3), (5, 8)] if Lk > 8 else [(0, Lk - 1)]
                qsl = np.array([0, Lq], dtype=np.int32)
                out = np.full((Lq, 2), -7, dtype=np.int32)
                n = ref_build_table(out, {0: ranges}, qsl, np.array([Lk]))
                rows = out if n else None
            np.testing.assert_array_equal(ref_mask(Lq, Lk, causal, wl, wr, rows),
                                          _loop_mask(Lq, Lk, causal, wl, wr, rows))


def test_mm_term_equals_range_scan_with_window_clamp():
    """mm == any(range holds both query and key), then clamped on the past side only."""
    ranges = [(2, 6), (10, 17)]
    for Lq, Lk, wl in [(20, 20, -1), (8, 20, 3), (20, 20, 1), (5, 18, 0)]:
        out = np.full((Lq, 2), 99, dtype=np.int32)
        n = ref_build_table(out, {0: ranges}, np.array([0, Lq]), np.array([Lk]))
        base = ref_mask(Lq, Lk, True, wl, -1)
        full = ref_mask(Lq, Lk, True, wl, -1, out if n else None)
        c = Lk - Lq
        for i in range(Lq):
            p = c + i
            for k in range(Lk):
                scan = any(s < e and s <= p <= e and s <= k <= e for s, e in ranges)
                clamp = wl < 0 or p - k <= wl
                assert full[i, k] == (base[i, k] or (scan and clamp)), (Lq, Lk, wl, i, k)


def test_future_range_keys_stay_visible_under_window():
    """Inside a range, future keys are visible; the window trims only the past."""
    out = np.full((16, 2), 0, dtype=np.int32)
    ref_build_table(out, {0: [(4, 11)]}, np.array([0, 16]), np.array([16]))
    m = ref_mask(16, 16, True, 2, -1, out)
    assert m[4, 11] and m[6, 11]  # future keys in range
    assert not m[8, 4] and m[6, 4]  # past side clamped: d=4 > 2 hidden, d=2 kept
    assert not m[3, 5]  # query outside the range: plain causal window
