"""GPU parity of attn_varlen_fwd against the CPU oracle (needs an MI355X).

Reduced shapes are compared element by element (every output and LSE); they
span several query and key tiles and end in ragged tails. The named
full-size workloads are compared on sampled outputs the oracle evaluates one
by one, on one whole request (every q head, element by element), and on
properties that hold everywhere (finite, written, bounded).
Tolerances: max |err| 1e-2 for bf16, 1e-4 for fp32; LSE 2e-3 / 1e-4.
"""

import zlib

import numpy as np
import pytest

from gpu_helpers import (BF16_TOL, F32_TOL, LSE_TOL_BF16, LSE_TOL_F32, assert_close, assert_lse_close,
                         oracle_prefill, oracle_prefill_rows, run_prefill, table_for, to_dev)
from masked_varlen_softmax_amd import workloads as W
from oracle import ref_attention

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _check(case, dev, table="auto"):
    t = table_for(case) if table == "auto" else table
    got, glse = run_prefill(case, dev, t)
    ref, rlse = oracle_prefill(case, t)
    tol, ltol = (F32_TOL, LSE_TOL_F32) if case.dtype == "f32" else (BF16_TOL, LSE_TOL_BF16)
    err = assert_close(got, ref, tol, case.name)
    assert_lse_close(glse, rlse, ltol, case.name)
    return err


@pytest.mark.parametrize("kv", [4, 2])
def test_c1_tiny_window_sinks_fp32(dev, kv):
    case = W.c1_tiny_window_sinks(kv)
    print(f"case {case.name}", flush=True)
    _check(case, dev)


SWEEP = [
    # name, lens_q, lens_k, Hq, Hkv, D, causal, wl, wr, mm, sink
    ("causal", [300, 1, 77], [300, 1, 77], 4, 2, 128, True, -1, -1, False, 0),
    ("causal_ctx", [130, 64, 5], [400, 64, 300], 4, 4, 128, True, -1, -1, False, 0),
    ("causal_window", [333, 200], [333, 250], 4, 2, 128, True, 63, -1, False, 0),
    ("window_lt_tile", [257, 40], [257, 40], 2, 1, 128, True, 4, -1, False, 0),
    ("bidir_window_key0", [301, 37, 5], [301, 37, 5], 4, 4, 128, False, 8, 8, False, 1),
    ("bidir_asym_null", [190, 66], [190, 66], 4, 2, 128, False, 20, 3, False, 2),
    ("mm_causal_window", [520, 129], [520, 300], 4, 2, 128, True, 100, -1, True, 0),
    ("mm_causal_global", [200, 150], [600, 150], 2, 1, 128, True, -1, -1, True, 0),
    ("mm_key0", [260], [260], 2, 2, 128, True, 50, -1, True, 1),
    ("full_noncausal", [129, 3], [200, 3], 2, 1, 128, False, -1, -1, False, 0),
    ("d64_mm", [300, 17], [300, 90], 4, 2, 64, True, 31, -1, True, 0),
    ("d256_mm_window", [300, 129], [300, 400], 4, 2, 256, True, 127, -1, True, 0),
    ("d256_key0", [200], [200], 2, 2, 256, False, 16, 16, False, 1),
    ("d512_mm_ctx", [150, 64], [500, 64], 2, 1, 512, True, -1, -1, True, 0),
    ("d512_window_null", [140, 33], [140, 100], 2, 2, 512, True, 40, -1, False, 2),
    ("empty_seq_middle", [100, 0, 50], [100, 20, 70], 2, 1, 128, True, -1, -1, True, 0),
    ("single_token", [1, 1, 1], [1, 9, 1000], 2, 2, 128, True, 127, -1, False, 1),
]


@pytest.mark.parametrize("spec", SWEEP, ids=[s[0] for s in SWEEP])
def test_bf16_parity_sweep(dev, spec):
    name, lq, lk, hq, hkv, d, causal, wl, wr, mm, sink = spec
    case = W.make_random_prefill(zlib.crc32(name.encode()) % 1000, lq, lk, hq, hkv, d, "bf16", causal, wl, wr, mm=mm,
                                 sink_mode=sink, max_ranges=4, max_range_len=90)
    case.name = name
    print(f"case {name}", flush=True)
    _check(case, dev)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_fp32_parity(dev, d):
    case = W.make_random_prefill(11, [77, 130], [100, 130], 4, 2, d, "f32", True, 40, -1, mm=True, sink_mode=1)
    print(f"case fp32 d{d}", flush=True)
    _check(case, dev)


def test_all_empty_table_equals_no_table(dev):
    case = W.make_random_prefill(5, [150, 90], [150, 120], 2, 1, 128, "bf16", True, 33, -1)
    empty = np.full((case.q.shape[0], 2), -1, dtype=np.int32)
    a, _ = run_prefill(case, dev, empty)
    b, _ = run_prefill(case, dev, None)
    np.testing.assert_array_equal(a, b)


def test_two_interval_rows(dev):
    """A hand-made table whose ranges do not contain the row's own position."""
    case = W.make_random_prefill(6, [200], [200], 2, 1, 128, "bf16", True, 10, -1)
    t = np.full((200, 2), -1, dtype=np.int32)
    t[20:60] = (150, 190)
    t[100:110] = (0, 3)
    got, _ = run_prefill(case, dev, t)
    ref, _ = oracle_prefill(case, t)
    assert_close(got, ref, BF16_TOL, "two_intervals")


def test_library_table_builder_feeds_kernel(dev):
    import masked_varlen_softmax_amd as mvs

    case = W.make_random_prefill(9, [300, 200], [700, 200], 4, 2, 128, "bf16", True, 255, -1, mm=True)
    host = np.full((600, 2), 7, dtype=np.int32)
    n = mvs.build_query_range_table(host, case.ranges, case.cu_q, case.lens_k)
    t = host[:500] if n else None
    got, _ = run_prefill(case, dev, t)
    ref, _ = oracle_prefill(case, table_for(case))
    assert_close(got, ref, BF16_TOL, "builder->kernel")


def _samples(case, rng, n_rows):
    N = case.q.shape[0]
    rows = set(rng.choice(N, size=n_rows, replace=False).tolist())
    # first and last row of every request, and a row next to each range edge
    for b in range(case.num_seqs):
        q0, q1 = int(case.cu_q[b]), int(case.cu_q[b + 1])
        if q1 > q0:
            rows.update([q0, q1 - 1])
    return [(t, int(rng.integers(0, case.Hq))) for t in sorted(rows)]


@pytest.mark.parametrize("name", ["c2", "c3", "c4"])
def test_full_size_configs_sampled(dev, name):
    import torch

    case = W.PREFILL_CONFIGS[name]()
    print(f"case {name} full size", flush=True)
    t = table_for(case)
    got, glse = run_prefill(case, dev, t)
    assert np.isfinite(got).all(), "unwritten or non-finite outputs"
    assert np.isfinite(glse).all()
    assert np.abs(got).max() < 10.0  # convex combinations of N(0,1) values
    rng = np.random.default_rng(0)
    samples = _samples(case, rng, 48)
    ref, rlse = oracle_prefill_rows(case, samples, t)
    g = np.stack([got[tk, h] for tk, h in samples])
    gl = np.array([glse[h, tk] for tk, h in samples])
    assert_close(g, ref, BF16_TOL, name)
    assert_lse_close(gl, rlse, LSE_TOL_BF16, name)
    # the whole longest request, every q head, element by element (every tile class and every
    # head's place in the launch order of the layer)
    b = int(np.argmax(np.diff(case.cu_q)))
    q0, q1, k0, k1 = int(case.cu_q[b]), int(case.cu_q[b + 1]), int(case.cu_k[b]), int(case.cu_k[b + 1])
    print(f"case {name}: whole request {b} ({q1 - q0} queries x {k1 - k0} keys, {case.Hq} q heads)", flush=True)
    ref_b, rlse_b = ref_attention(W.as_f32(case.q[q0:q1]), W.as_f32(case.k[k0:k1]), W.as_f32(case.v[k0:k1]),
                                  np.array([0, q1 - q0]), np.array([0, k1 - k0]), case.scale, case.causal, case.wl,
                                  case.wr, None if t is None else t[q0:q1], case.sinks, case.sink_mode)
    assert_close(got[q0:q1], ref_b, BF16_TOL, f"{name} request {b}")
    assert_lse_close(glse[:, q0:q1], rlse_b, LSE_TOL_BF16, f"{name} request {b}")
    # the launch bench.py times (no LSE output) gives the same O at every element
    plain, _ = run_prefill(case, dev, t, want_lse=False)
    np.testing.assert_array_equal(plain, got, err_msg=f"{name}: O without the LSE output differs")
    del torch


SCAN = [
    # name, lens_q, lens_k, Hq, Hkv, D, causal, wl, wr, sink
    ("scan_causal_window_ctx", [520, 129], [700, 300], 4, 2, 128, True, 100, -1, 0),
    ("scan_global_d256", [300, 150], [600, 150], 2, 1, 256, True, -1, -1, 2),
    ("scan_bidir_d64_key0", [301, 37], [301, 37], 4, 4, 64, False, 8, 8, 1),
]


@pytest.mark.parametrize("spec", SCAN, ids=[s[0] for s in SCAN])
def test_range_scan_baseline(dev, spec):
    """The range-scan baseline equals the oracle, and the table path bit for bit."""
    import torch

    import masked_varlen_softmax_amd as mvs

    name, lq, lk, hq, hkv, d, causal, wl, wr, sink = spec
    case = W.make_random_prefill(zlib.crc32(name.encode()) % 1000, lq, lk, hq, hkv, d, "bf16", causal, wl, wr,
                                 mm=True, sink_mode=sink, max_ranges=6, max_range_len=90)
    print(f"case {name}", flush=True)
    rp = W.padded_ranges(case, 8)
    q, k, v = to_dev(case.q, dev), to_dev(case.k, dev), to_dev(case.v, dev)
    cu_q, cu_k = to_dev(case.cu_q, dev), to_dev(case.cu_k, dev)
    sinks = None if case.sinks is None else to_dev(case.sinks.astype(np.float32), dev)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((case.Hq, q.shape[0]), float("nan"), dtype=torch.float32, device=dev)
    mvs.attn_varlen_fwd_range_scan(q, k, v, cu_q, cu_k, max(lq), max(lk), case.scale, to_dev(rp, dev), causal, wl,
                                   wr, sinks, case.sink_mode, out=out, lse=lse)
    torch.cuda.synchronize()
    got, glse = out.float().cpu().numpy(), lse.cpu().numpy()
    t = table_for(case)
    ref, rlse = oracle_prefill(case, t)
    assert_close(got, ref, BF16_TOL, name)
    assert_lse_close(glse, rlse, LSE_TOL_BF16, name)
    tab, tlse = run_prefill(case, dev, t)
    np.testing.assert_array_equal(got, tab)
    np.testing.assert_array_equal(glse, tlse)


def test_long_context_chunk(dev):
    """64 new queries after a 131 008-token context (D 128, GQA 2); its ranges lie wholly in the
    context, so the builder clips them all away."""
    case = W.make_random_prefill(31, [64], [131072], 4, 2, 128, "bf16", True, -1, -1, mm=True, sink_mode=2,
                                 max_ranges=4, max_range_len=4000)
    print("case prefill 128K context", flush=True)
    _check(case, dev)
