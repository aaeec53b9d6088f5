"""GPU parity of the prefill entry points at wide GQA groups (needs an MI355X).

Query heads per kv head 4, 8 and 16, the ratios of the pages' global and
sliding layers once their heads are split for serving ([PR49815] key code
snippets: the reference maps query head h to kv head h / group by repeating
K and V). At head_dim 256 the kernel packs two query heads of one kv head
into a workgroup, so a group of 4 or more is split into several such slices;
at 128 and 512 every query head has its own workgroups. The batches have four
requests with ragged tails; in four of them the grid has enough query tiles
that its XCD-aware remap of workgroups is active. Every output and LSE is
compared with the dense oracle, for the contiguous entry point and for the
paged one (K/V scattered into pages in random order; both must agree bit for
bit).
Tolerances: bf16 max |err| 1e-2, LSE 2e-3.
"""

import zlib

import numpy as np
import pytest

from gpu_helpers import (BF16_TOL, LSE_TOL_BF16, assert_close, assert_lse_close, oracle_prefill, run_prefill,
                         table_for, to_dev)
from masked_varlen_softmax_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


GQA = [
    # name, lens_q, lens_k, Hq, Hkv, D, causal, wl, wr, mm, sink
    ("d256_g4_mm_window_key0", [300, 257, 129, 300], [300, 400, 129, 700], 8, 2, 256, True, 127, -1, True, 1),
    ("d256_g8_mm_window", [300, 300, 300, 129], [300, 300, 500, 129], 16, 2, 256, True, 200, -1, True, 0),
    ("d256_g8_bidir_null", [190, 66, 300, 257], [190, 66, 300, 257], 16, 2, 256, False, 40, 9, False, 2),
    ("d256_g16_global_mm", [257, 100, 64, 300], [600, 100, 64, 300], 16, 1, 256, True, -1, -1, True, 0),
    ("d128_g8_mm_window_key0", [300, 257, 129, 300], [300, 400, 129, 300], 16, 2, 128, True, 100, -1, True, 1),
    ("d128_g16_bidir_null", [301, 37, 5, 300], [301, 37, 5, 300], 16, 1, 128, False, 8, 8, False, 2),
    ("d512_g8_mm_ctx", [150, 64, 129, 200], [500, 64, 300, 200], 8, 1, 512, True, -1, -1, True, 0),
    ("d512_g16_window_key0", [140, 33, 129, 200], [140, 100, 129, 333], 16, 1, 512, True, 40, -1, True, 1),
]


def _case(spec):
    name, lq, lk, hq, hkv, d, causal, wl, wr, mm, sink = spec
    case = W.make_random_prefill(zlib.crc32(name.encode()) % 1000, lq, lk, hq, hkv, d, "bf16", causal, wl, wr,
                                 mm=mm, sink_mode=sink, max_ranges=4, max_range_len=90)
    case.name = name
    return case


@pytest.mark.parametrize("spec", GQA, ids=[s[0] for s in GQA])
def test_gqa_parity(dev, spec):
    case = _case(spec)
    print(f"case gqa {case.name}", flush=True)
    t = table_for(case)
    got, glse = run_prefill(case, dev, t)
    ref, rlse = oracle_prefill(case, t)
    assert_close(got, ref, BF16_TOL, case.name)
    assert_lse_close(glse, rlse, LSE_TOL_BF16, case.name)


@pytest.mark.parametrize("spec", GQA[::2] + [GQA[-1]], ids=[s[0] for s in GQA[::2] + [GQA[-1]]])
def test_gqa_paged_parity(dev, spec):
    import torch

    import masked_varlen_softmax_amd as mvs

    case = _case(spec)
    print(f"case gqa paged {case.name}", flush=True)
    page = 16 if case.D == 512 else 32
    kc, vc, bt = W.paged_kv(case, page, 5, extra_pages=3)
    t = table_for(case)
    q = to_dev(case.q, dev)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((case.Hq, q.shape[0]), float("nan"), dtype=torch.float32, device=dev)
    sinks = None if case.sinks is None else to_dev(case.sinks.astype(np.float32), dev)
    mvs.attn_varlen_fwd_paged(q, to_dev(kc, dev), to_dev(vc, dev), to_dev(bt, dev), to_dev(case.cu_q, dev),
                              to_dev(case.lens_k.astype(np.int32), dev), int(case.lens_q.max()),
                              int(case.lens_k.max()), case.scale, case.causal, case.wl, case.wr,
                              None if t is None else to_dev(t, dev), sinks, case.sink_mode, out=out, lse=lse)
    torch.cuda.synchronize()
    got, glse = out.float().cpu().numpy(), lse.cpu().numpy()
    ref, rlse = oracle_prefill(case, t)
    assert_close(got, ref, BF16_TOL, case.name)
    assert_lse_close(glse, rlse, LSE_TOL_BF16, case.name)
    contiguous, clse = run_prefill(case, dev, t)
    np.testing.assert_array_equal(got, contiguous)
    np.testing.assert_array_equal(glse, clse)
