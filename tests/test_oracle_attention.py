"""Pins for the oracle's attention (CPU only).

Anchors that do not come from the oracle itself:
  * closed forms for one and two visible keys under each sink mode;
  * torch's CPU ``scaled_dot_product_attention`` (a library routine) fed the
    same boolean mask, or an additive mask carrying the key-0 sink, in fp64;
  * scipy's ``logsumexp`` for the LSE;
  * structural identities (GQA == MHA on repeated kv heads, sink 0 == no sink,
    a window wider than the sequence == unmasked, probability rows sum to one);
  * on the tiny MiMo configuration (lengths 5 and 37, window 8, 4 heads, D 64),
    the key-0 bias differs from the null-logit sink and from no sink by more
    than 1e-2, as the vLLM PR #49815 page's error figures require.
"""

import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from masked_varlen_softmax_amd import workloads as W
from oracle import (SINK_KEY0_BIAS, SINK_NONE, SINK_NULL_LOGIT, ref_attention, ref_attention_rows,
                    ref_build_table, ref_mask)


def _sigmoid(x):
    return 1.0 / (1.0 + math.exp(-x))


def _case(seed, lens_q, lens_k, Hq, Hkv, D):
    rng = np.random.default_rng(seed)
    nq, nk = sum(lens_q), sum(lens_k)
    q = rng.standard_normal((nq, Hq, D))
    k = rng.standard_normal((nk, Hkv, D))
    v = rng.standard_normal((nk, Hkv, D))
    cu_q = np.concatenate([[0], np.cumsum(lens_q)])
    cu_k = np.concatenate([[0], np.cumsum(lens_k)])
    return q, k, v, cu_q, cu_k


def test_single_key_closed_forms():
    q, k, v, cu_q, cu_k = _case(1, [1], [1], 2, 2, 8)
    sinks = np.array([0.7, -1.3])
    s0 = 0.5 * (q[0] * k[0]).sum(-1)  # per head
    o, lse = ref_attention(q, k, v, cu_q, cu_k, 0.5, sinks=sinks, sink_mode=SINK_KEY0_BIAS, dtype=np.float64)
    np.testing.assert_allclose(o[0], v[0], rtol=0, atol=1e-15)  # one visible key: weight exactly 1
    np.testing.assert_allclose(lse[:, 0], s0 + sinks, atol=1e-12)
    o, lse = ref_attention(q, k, v, cu_q, cu_k, 0.5, sinks=sinks, sink_mode=SINK_NULL_LOGIT, dtype=np.float64)
    for h in range(2):
        np.testing.assert_allclose(o[0, h], _sigmoid(s0[h] - sinks[h]) * v[0, h], atol=1e-12)
        np.testing.assert_allclose(lse[h, 0], np.logaddexp(s0[h], sinks[h]), atol=1e-12)


def test_two_key_closed_form_key0_bias():
    q, k, v, cu_q, cu_k = _case(2, [1], [2], 3, 3, 16)
    sinks = np.array([0.3, 2.0, -0.8])
    o, _ = ref_attention(q, k, v, cu_q, cu_k, 0.25, causal=True, sinks=sinks, sink_mode=SINK_KEY0_BIAS,
                         dtype=np.float64)
    for h in range(3):
        s0 = 0.25 * q[0, h] @ k[0, h]
        s1 = 0.25 * q[0, h] @ k[1, h]
        a = _sigmoid(s0 + sinks[h] - s1)
        np.testing.assert_allclose(o[0, h], a * v[0, h] + (1 - a) * v[1, h], atol=1e-12)


def test_sink_only_where_key0_visible():
    """Window hides key 0 from late queries: the bias must not reach them."""
    q, k, v, cu_q, cu_k = _case(3, [12], [12], 2, 2, 8)
    sinks = np.array([5.0, -5.0])
    with_sink, _ = ref_attention(q, k, v, cu_q, cu_k, 0.3, causal=True, wl=3, sinks=sinks,
                                 sink_mode=SINK_KEY0_BIAS, dtype=np.float64)
    no_sink, _ = ref_attention(q, k, v, cu_q, cu_k, 0.3, causal=True, wl=3, dtype=np.float64)
    np.testing.assert_array_equal(with_sink[4:], no_sink[4:])  # rows 4.. cannot see key 0
    assert np.abs(with_sink[:4] - no_sink[:4]).max() > 1e-3


def _sdpa(q, k, v, cu_q, cu_k, scale, causal, wl, wr, table, sinks, sink_mode):
    """torch CPU SDPA in fp64 on each request, GQA expanded, sink as an additive bias."""
    Hq, Hkv = q.shape[1], k.shape[1]
    out = np.zeros_like(q)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        Lq, Lk = q1 - q0, k1 - k0
        rows = None if table is None else table[q0:q1]
        m = torch.from_numpy(ref_mask(Lq, Lk, causal, wl, wr, rows))
        qt = torch.from_numpy(q[q0:q1]).permute(1, 0, 2)
        kt = torch.from_numpy(k[k0:k1]).repeat_interleave(Hq // Hkv, dim=1).permute(1, 0, 2)
        vt = torch.from_numpy(v[k0:k1]).repeat_interleave(Hq // Hkv, dim=1).permute(1, 0, 2)
        bias = torch.zeros(Hq, Lq, Lk, dtype=torch.float64)
        if sink_mode == SINK_KEY0_BIAS:
            bias[:, :, 0] += torch.from_numpy(sinks).view(Hq, 1)
        bias = bias.masked_fill(~m, float("-inf"))
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=bias, scale=scale)
        out[q0:q1] = o.permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("cfg", [
    dict(causal=True, wl=-1, wr=-1, mm=False, sink=SINK_NONE),
    dict(causal=True, wl=6, wr=-1, mm=True, sink=SINK_NONE),
    dict(causal=False, wl=4, wr=4, mm=False, sink=SINK_KEY0_BIAS),
    dict(causal=True, wl=-1, wr=-1, mm=True, sink=SINK_KEY0_BIAS),
    dict(causal=False, wl=3, wr=7, mm=True, sink=SINK_KEY0_BIAS),
])
def test_matches_torch_sdpa_fp64(cfg):
    lens_q, lens_k = [5, 17, 1, 9], [5, 23, 6, 9]
    q, k, v, cu_q, cu_k = _case(4, lens_q, lens_k, 4, 2, 16)
    sinks = np.random.default_rng(9).standard_normal(4)
    table = None
    if cfg["mm"]:
        table = np.full((sum(lens_q), 2), 0, dtype=np.int32)
        n = ref_build_table(table, {1: [(2, 8), (14, 20)], 2: [(1, 5)], 3: [(0, 3)]},
                            cu_q.astype(np.int32), np.array(lens_k))
        assert n
    o, _ = ref_attention(q, k, v, cu_q, cu_k, 0.4, cfg["causal"], cfg["wl"], cfg["wr"], table, sinks,
                         cfg["sink"], dtype=np.float64)
    ref = _sdpa(q, k, v, cu_q, cu_k, 0.4, cfg["causal"], cfg["wl"], cfg["wr"], table, sinks, cfg["sink"])
    np.testing.assert_allclose(o, ref, atol=1e-12, rtol=0)


def test_lse_matches_logsumexp():
    q, k, v, cu_q, cu_k = _case(5, [7], [11], 2, 1, 8)
    sinks = np.array([0.4, -0.2])
    for mode in (SINK_NONE, SINK_KEY0_BIAS, SINK_NULL_LOGIT):
        _, lse = ref_attention(q, k, v, cu_q, cu_k, 0.6, causal=True, wl=5, sinks=sinks, sink_mode=mode,
                               dtype=np.float64)
        m = ref_mask(7, 11, True, 5, -1)
        for h in range(2):
            s = 0.6 * q[:, h] @ k[:, 0].T
            if mode == SINK_KEY0_BIAS:
                s[:, 0] += sinks[h]
            s = np.where(m, s, -np.inf)
            if mode == SINK_NULL_LOGIT:
                s = np.concatenate([s, np.full((7, 1), sinks[h])], axis=1)
            np.testing.assert_allclose(lse[h], logsumexp(s, axis=1), atol=1e-12)


def test_structural_identities():
    q, k, v, cu_q, cu_k = _case(6, [9, 4], [9, 10], 4, 2, 8)
    zero = np.zeros(4)
    a, _ = ref_attention(q, k, v, cu_q, cu_k, 0.5, causal=True, sinks=zero, sink_mode=SINK_KEY0_BIAS,
                         dtype=np.float64)
    b, _ = ref_attention(q, k, v, cu_q, cu_k, 0.5, causal=True, dtype=np.float64)
    np.testing.assert_array_equal(a, b)  # sink 0 == no sink
    wide, _ = ref_attention(q, k, v, cu_q, cu_k, 0.5, causal=False, wl=50, wr=50, dtype=np.float64)
    full, _ = ref_attention(q, k, v, cu_q, cu_k, 0.5, causal=False, dtype=np.float64)
    np.testing.assert_array_equal(wide, full)  # window wider than the sequence == unmasked
    kr, vr = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    mha, _ = ref_attention(q, kr, vr, cu_q, cu_k, 0.5, causal=True, wl=2, dtype=np.float64)
    gqa, _ = ref_attention(q, k, v, cu_q, cu_k, 0.5, causal=True, wl=2, dtype=np.float64)
    np.testing.assert_allclose(gqa, mha, atol=1e-14)  # query head h reads kv head h // 2


def test_probability_rows_sum_to_one_and_convex_hull():
    Lk = 12
    q, _, _, cu_q, cu_k = _case(7, [Lk], [Lk], 1, 1, 4)
    k = np.random.default_rng(8).standard_normal((Lk, 1, 4))
    eye = np.eye(Lk)[:, None, :]  # value k = e_k: the output row is the probability row
    for mode, sink in [(SINK_NONE, 0.0), (SINK_KEY0_BIAS, 1.5), (SINK_NULL_LOGIT, 1.5)]:
        o, _ = ref_attention(q, k, eye, cu_q, cu_k, 0.7, causal=True, wl=4, sinks=np.array([sink]),
                             sink_mode=mode, dtype=np.float64)
        P = o[:, 0, :]
        vis = ref_mask(Lk, Lk, True, 4, -1)
        assert (P[~vis] == 0).all() and (P >= 0).all()
        if mode == SINK_NULL_LOGIT:
            assert (P.sum(1) < 1).all()  # the null logit takes part of the mass
        else:
            np.testing.assert_allclose(P.sum(1), 1.0, atol=1e-14)


def test_fully_masked_row_convention():
    q, k, v, cu_q, cu_k = _case(9, [1], [3], 1, 1, 4)
    table = None
    # wl=0 keeps only the query's own position; a query left of every key (Lq > Lk not allowed) is
    # emulated with a right window on a non-causal row that sees nothing: wl=0, wr=0 but Lk shifted.
    o, lse = ref_attention(q, k, v, [0, 1], [0, 0], 1.0, causal=True, dtype=np.float64)
    assert (o == 0).all() and np.isneginf(lse).all()
    o, lse = ref_attention(q, k, v, [0, 1], [0, 0], 1.0, causal=True, sinks=np.array([0.5]),
                           sink_mode=SINK_NULL_LOGIT, dtype=np.float64)
    assert (o == 0).all() and lse[0, 0] == 0.5
    del table


@pytest.mark.parametrize("kv", [4, 2])
def test_tiny_mimo_config_distinguishes_sink_semantics(kv):
    """KEY0 bias vs null logit and vs no sink differ by > 1e-2 on seeded inputs."""
    c = W.c1_tiny_window_sinks(kv)
    args = (c.q, c.k, c.v, c.cu_q, c.cu_k, c.scale, c.causal, c.wl, c.wr, None, c.sinks)
    key0, _ = ref_attention(*args, SINK_KEY0_BIAS)
    null, _ = ref_attention(*args, SINK_NULL_LOGIT)
    none, _ = ref_attention(*args, SINK_NONE)
    assert np.abs(key0 - null).max() > 1e-2
    assert np.abs(key0 - none).max() > 1e-2


def test_row_sampler_equals_dense():
    q, k, v, cu_q, cu_k = _case(10, [6, 11], [9, 11], 4, 2, 8)
    sinks = np.random.default_rng(1).standard_normal(4)
    table = np.zeros((17, 2), dtype=np.int32)
    ref_build_table(table, {0: [(3, 7)], 1: [(2, 5)]}, cu_q.astype(np.int32), np.array([9, 11]))
    dense, dlse = ref_attention(q, k, v, cu_q, cu_k, 0.3, True, 4, -1, table, sinks, SINK_KEY0_BIAS,
                                dtype=np.float64)
    samples = [(t, h) for t in range(17) for h in range(4)]
    rows, rlse = ref_attention_rows(q, k, v, cu_q, cu_k, 0.3, samples, True, 4, -1, table, sinks,
                                    SINK_KEY0_BIAS, dtype=np.float64)
    for n, (t, h) in enumerate(samples):
        np.testing.assert_allclose(rows[n], dense[t, h], atol=1e-13)
        np.testing.assert_allclose(rlse[n], dlse[h, t], atol=1e-13)
