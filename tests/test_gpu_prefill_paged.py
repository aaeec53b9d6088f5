"""GPU parity of attn_varlen_fwd_paged (prefill reading K/V from a paged cache).

The oracle side gathers each sequence's keys back out of the pages through the
block table (ref_gather_paged) and runs the dense oracle on them, so a wrong
page, slot or head offset in the kernel shows up as a large error. Pages are
assigned in random order, slots past a sequence's end and spare pages hold
random values, and block-table entries past the last page are -1. A second
check runs the contiguous entry point on the same keys: both read identical
tiles, so their outputs must agree bit for bit.
Tolerances: max |err| 1e-2 for bf16 outputs, LSE 2e-3.
"""

import zlib

import numpy as np
import pytest

from gpu_helpers import (BF16_TOL, LSE_TOL_BF16, assert_close, assert_lse_close, run_prefill, table_for, to_dev)
from masked_varlen_softmax_amd import workloads as W
from oracle import ref_attention, ref_attention_rows, ref_gather_paged

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _hnd(cache, nhd):
    return np.transpose(cache, (0, 2, 1, 3)) if nhd else cache


def _gathered(case, kc, vc, bt, page, nhd):
    """Contiguous K and V rebuilt from the pages by the oracle's gather."""
    ks, vs = [], []
    for b in range(case.num_seqs):
        L = int(case.lens_k[b])
        ks.append(ref_gather_paged(_hnd(kc, nhd), bt[b], L, page))
        vs.append(ref_gather_paged(_hnd(vc, nhd), bt[b], L, page))
    return np.concatenate(ks), np.concatenate(vs)


def run_paged(case, dev, kc, vc, bt, page, nhd, table):
    import torch

    import masked_varlen_softmax_amd as mvs

    q = to_dev(case.q, dev)
    kd, vd = to_dev(kc, dev), to_dev(vc, dev)
    if nhd:  # [pages, page, Hkv, D] storage seen as [pages, Hkv, page, D]
        kd, vd = kd.permute(0, 2, 1, 3), vd.permute(0, 2, 1, 3)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((case.Hq, q.shape[0]), float("nan"), dtype=torch.float32, device=dev)
    sinks = None if case.sinks is None else to_dev(case.sinks.astype(np.float32), dev)
    mvs.attn_varlen_fwd_paged(q, kd, vd, to_dev(bt, dev), to_dev(case.cu_q, dev),
                              to_dev(case.lens_k.astype(np.int32), dev), int(case.lens_q.max(initial=0)),
                              int(case.lens_k.max(initial=0)), case.scale, case.causal, case.wl, case.wr,
                              None if table is None else to_dev(table, dev), sinks, case.sink_mode, out=out, lse=lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


PAGED = [
    # name, lens_q, lens_k, Hq, Hkv, D, causal, wl, wr, mm, sink, page, nhd
    ("ctx_d128_p16", [130, 64, 5], [400, 64, 300], 4, 2, 128, True, -1, -1, False, 0, 16, False),
    ("mm_window_d128_p32", [520, 129], [520, 300], 4, 2, 128, True, 100, -1, True, 0, 32, False),
    ("bidir_key0_d64_p64_nhd", [300, 17], [300, 17], 4, 2, 64, False, 31, 31, False, 1, 64, True),
    ("mm_ctx_null_d256_p16", [300, 129], [700, 400], 4, 2, 256, True, 127, -1, True, 2, 16, False),
    ("mm_global_d256_p128_nhd", [200], [900], 2, 1, 256, True, -1, -1, True, 0, 128, True),
    ("mm_ctx_d512_p16", [150, 64], [500, 64], 2, 1, 512, True, -1, -1, True, 0, 16, False),
    ("window_null_d512_p32", [140, 33], [340, 100], 2, 2, 512, True, 40, -1, False, 2, 32, False),
    ("empty_and_single_p16", [100, 0, 1], [100, 20, 1000], 2, 1, 128, True, -1, -1, True, 1, 16, False),
]


@pytest.mark.parametrize("spec", PAGED, ids=[s[0] for s in PAGED])
def test_paged_prefill_parity(dev, spec):
    name, lq, lk, hq, hkv, d, causal, wl, wr, mm, sink, page, nhd = spec
    seed = zlib.crc32(name.encode()) % 1000
    case = W.make_random_prefill(seed, lq, lk, hq, hkv, d, "bf16", causal, wl, wr, mm=mm, sink_mode=sink,
                                 max_ranges=4, max_range_len=90)
    print(f"case paged {name}", flush=True)
    kc, vc, bt = W.paged_kv(case, page, seed + 1, nhd=nhd, extra_pages=3)
    kg, vg = _gathered(case, kc, vc, bt, page, nhd)
    np.testing.assert_array_equal(kg, case.k)  # the scatter put every key where the table says
    t = table_for(case)
    got, glse = run_paged(case, dev, kc, vc, bt, page, nhd, t)
    ref, rlse = ref_attention(W.as_f32(case.q), W.as_f32(kg), W.as_f32(vg), case.cu_q, case.cu_k, case.scale,
                              case.causal, case.wl, case.wr, t, case.sinks, case.sink_mode)
    assert_close(got, ref, BF16_TOL, name)
    assert_lse_close(glse, rlse, LSE_TOL_BF16, name)
    contiguous, clse = run_prefill(case, dev, t)
    np.testing.assert_array_equal(got, contiguous)
    np.testing.assert_array_equal(glse, clse)


def test_paged_prefill_c3_full_size(dev):
    """The chunked-prefill global layer with its context read from 16-token pages."""
    case = W.c3_chunked_global()
    print("case paged c3 full size", flush=True)
    kc, vc, bt = W.paged_kv(case, 16, 77, extra_pages=64)
    t = table_for(case)
    got, glse = run_paged(case, dev, kc, vc, bt, 16, False, t)
    assert np.isfinite(got).all() and np.isfinite(glse).all()
    contiguous, clse = run_prefill(case, dev, t)
    np.testing.assert_array_equal(got, contiguous)
    np.testing.assert_array_equal(glse, clse)
    rng = np.random.default_rng(3)
    rows = sorted(set(rng.choice(case.q.shape[0], size=24, replace=False).tolist())
                  | {int(case.cu_q[b]) for b in range(case.num_seqs)})
    samples = [(r, int(rng.integers(0, case.Hq))) for r in rows]
    kg, vg = _gathered(case, kc, vc, bt, 16, False)
    ref, rlse = ref_attention_rows(W.as_f32(case.q), W.as_f32(kg), W.as_f32(vg), case.cu_q, case.cu_k, case.scale,
                                   samples, case.causal, case.wl, case.wr, t, case.sinks, case.sink_mode)
    assert_close(np.stack([got[r, h] for r, h in samples]), ref, BF16_TOL, "c3 paged")
    assert_lse_close(np.array([glse[h, r] for r, h in samples]), rlse, LSE_TOL_BF16, "c3 paged")
