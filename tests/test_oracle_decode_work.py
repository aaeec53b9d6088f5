"""Pins for the paged-decode oracle and the useful-work counters (CPU only).

Anchors: the contiguous prefill oracle at one query (decode is that case, as
the step14_4 tutorial's decode shortcut states); invariance under any
permutation of physical pages; the vLLM PR #55624 report's closed-form clamp
test (context 8192 under window 1024 costs exactly 1/8 of the dense core
FLOPs; context 512 costs the same) and its quoted 8x-30x over-estimates for
32K/128K contexts under a 4096 window.
"""

import numpy as np
import pytest

from masked_varlen_softmax_amd import workloads as W
from oracle import (SINK_KEY0_BIAS, ExecutionContext, ref_attention, ref_decode_useful_bytes,
                    ref_gather_paged, ref_paged_decode, ref_useful_flops, ref_useful_pairs)


def _small_decode(wl, sink_mode=0, seed=3):
    return W.make_decode("d", seed, [1, 16, 17, 40, 93], 8, 2, 32, page_size=16, dtype="f32", wl=wl,
                         sink_mode=sink_mode, extra_pages=3)


@pytest.mark.parametrize("wl,sink_mode", [(-1, 0), (20, 0), (0, 0), (-1, SINK_KEY0_BIAS), (15, SINK_KEY0_BIAS)])
def test_paged_decode_equals_contiguous_prefill(wl, sink_mode):
    c = _small_decode(wl, sink_mode)
    out, lse = ref_paged_decode(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens, c.page_size, c.scale,
                                wl, c.sinks, sink_mode, dtype=np.float64)
    for b, L in enumerate(c.seq_lens):
        # build the contiguous sequence independently of ref_gather_paged
        kb = np.stack([c.k_cache[c.block_table[b][t // 16], :, t % 16] for t in range(L)])
        vb = np.stack([c.v_cache[c.block_table[b][t // 16], :, t % 16] for t in range(L)])
        o, l_ = ref_attention(c.q[b:b + 1], kb, vb, [0, 1], [0, L], c.scale, causal=True, wl=wl, sinks=c.sinks,
                              sink_mode=sink_mode, dtype=np.float64)
        np.testing.assert_allclose(out[b], o[0], atol=1e-14)
        np.testing.assert_allclose(lse[:, b], l_[:, 0], atol=1e-14)


def test_paged_decode_invariant_under_page_permutation():
    c = _small_decode(30)
    out, _ = ref_paged_decode(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens, 16, c.scale, 30,
                              dtype=np.float64)
    rng = np.random.default_rng(0)
    perm = rng.permutation(c.k_cache.shape[0])  # new physical page of old page j is perm[j]
    k2 = np.empty_like(c.k_cache)
    v2 = np.empty_like(c.v_cache)
    k2[perm] = c.k_cache
    v2[perm] = c.v_cache
    bt2 = np.where(c.block_table >= 0, perm[np.maximum(c.block_table, 0)], -1)
    out2, _ = ref_paged_decode(c.q, k2, v2, bt2, c.seq_lens, 16, c.scale, 30, dtype=np.float64)
    np.testing.assert_array_equal(out, out2)


def test_gather_reads_the_right_tokens():
    c = _small_decode(-1)
    b, L = 4, int(c.seq_lens[4])
    g = ref_gather_paged(c.k_cache, c.block_table[b], L, 16)
    assert g.shape == (L, c.Hkv, c.D)
    t = 37
    np.testing.assert_array_equal(g[t], c.k_cache[c.block_table[b][2], :, 5])


def test_window_clamp_is_exactly_eight_times():
    """Decode token, context 8192, window 1024: core FLOPs are 1/8 of dense (PR #55624 test)."""
    H, D, sw = 16, 128, 1024
    ctx = ExecutionContext()
    ctx.add(1, 8192, False)
    dense = ctx.attn_core_flops(H, D)
    swa = ctx.attn_core_flops(H, D, sliding_window=sw)
    assert swa["attn_qk"] * 8 == dense["attn_qk"] and swa["attn_av"] * 8 == dense["attn_av"]
    # the exact count agrees: one query at position 8191 with wl = W - 1 sees 1024 keys
    exact = ref_useful_flops([0, 1], [0, 8192], H, D, causal=True, wl=sw - 1)
    assert exact == swa["attn_qk"] + swa["attn_av"]
    assert exact * 8 == ref_useful_flops([0, 1], [0, 8192], H, D, causal=True)


def test_short_context_equal_to_dense():
    ctx = ExecutionContext()
    ctx.add(1, 512, False)
    assert ctx.attn_core_flops(8, 64, 1024) == ctx.attn_core_flops(8, 64)
    assert ref_useful_pairs([0, 1], [0, 512], True, 1023) == ref_useful_pairs([0, 1], [0, 512], True)


@pytest.mark.parametrize("ctx_len,ratio", [(32768, 8), (131072, 32)])
def test_quoted_overestimates(ctx_len, ratio):
    ctx = ExecutionContext()
    ctx.add(1, ctx_len, False)
    assert ctx.total_token_context_product() == ratio * ctx.total_token_context_product(4096)
    assert ctx.decode_context_len_for_window(4096) * ratio == ctx.decode_context_len_for_window()


def test_exact_prefill_count_never_exceeds_page_bound():
    """The page's formula ignores the causal triangle, so it bounds the exact count from above."""
    rng = np.random.default_rng(4)
    for _ in range(20):
        Lk = int(rng.integers(1, 300))
        Lq = int(rng.integers(1, Lk + 1))
        sw = int(rng.integers(1, 400))
        ctx = ExecutionContext()
        ctx.add(Lq, Lk, True)
        exact = ref_useful_pairs([0, Lq], [0, Lk], True, sw - 1)
        assert exact <= ctx.total_token_context_product(sw)
        assert exact <= Lq * min(Lk, sw)


def test_decode_bytes():
    lens = [8192, 100, 5000]
    assert ref_decode_useful_bytes(lens, 8, 128, 2, wl=4095) == (4096 + 100 + 4096) * 8 * 128 * 2 * 2
    assert ref_decode_useful_bytes(lens, 8, 128, 2) == sum(lens) * 4096


def test_prefill_and_decode_context_len_for_window_by_hand():
    """Per-request window clamp split by request kind ([PR55624], the ``ExecutionContext`` window methods).

    Worked by hand: two prefill requests with contexts 8192 and 512 and one decode request with
    context 32768, under a 4096 window. Prefill: min(8192, 4096) + min(512, 4096) = 4608; decode:
    min(32768, 4096) = 4096. Without a window each method returns its kind's running aggregate
    (8704 and 32768), which ``add`` keeps separately from the per-request list.
    """
    ctx = ExecutionContext()
    ctx.add(2048, 8192, True)
    ctx.add(1, 32768, False)
    ctx.add(512, 512, True)
    assert ctx.prefill_context_len_for_window(4096) == 4608
    assert ctx.decode_context_len_for_window(4096) == 4096
    assert ctx.prefill_context_len_for_window() == 8704
    assert ctx.decode_context_len_for_window() == 32768
    # a window at least as long as every context changes nothing (the page's fast path and slow path agree)
    assert ctx.prefill_context_len_for_window(32768) == ctx.prefill_context_len_for_window()
    assert ctx.decode_context_len_for_window(32768) == ctx.decode_context_len_for_window()
    # the token-context product weighs each clamped context by the request's token count:
    # 2048 * 4096 + 1 * 4096 + 512 * 512
    assert ctx.total_token_context_product(4096) == 2048 * 4096 + 4096 + 512 * 512

