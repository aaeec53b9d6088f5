"""Seeded random prefill configurations against the oracle (needs an MI355X).

Each case draws request lengths (empty, single-token and ragged ones
included), a context offset per request, head_dim, the q/kv head split, the
mask terms (causal, windows on either side, multimodal ranges), the sink mode
and, for bf16, whether K/V come packed or from a paged cache with a random
page size. Every output and LSE is compared with the dense oracle.
Tolerances: bf16 1e-2 (LSE 2e-3), fp32 1e-4.
"""

import numpy as np
import pytest

from gpu_helpers import (BF16_TOL, F32_TOL, LSE_TOL_BF16, LSE_TOL_F32, assert_close, assert_lse_close, run_prefill,
                         table_for, to_dev)
from masked_varlen_softmax_amd import workloads as W
from oracle import ref_attention, ref_gather_paged

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _draw(seed):
    rng = np.random.default_rng(50_000 + seed)
    dtype = "f32" if rng.random() < 0.2 else "bf16"
    D = int(rng.choice([64, 128, 256] if dtype == "f32" else [64, 128, 256, 512]))
    Hkv = int(rng.choice([1, 2, 4]))
    Hq = Hkv * int(rng.choice([1, 2, 3, 4]))
    B = int(rng.integers(1, 5))
    lens_q = [int(x) for x in rng.choice([0, 1, 2, 31, 64, 65, 129, 200, 333], size=B)]
    lens_k = [lq + int(rng.choice([0, 0, 1, 17, 150, 500])) for lq in lens_q]
    if sum(lens_q) == 0:
        lens_q[0], lens_k[0] = 7, max(lens_k[0], 7)
    causal = bool(rng.random() < 0.7)
    wl = int(rng.choice([-1, -1, 0, 5, 40, 200]))
    wr = -1 if causal and rng.random() < 0.8 else int(rng.choice([-1, 0, 3, 64]))
    mm = bool(rng.random() < 0.6)
    sink = int(rng.choice([0, 1, 2]))
    paged = dtype == "bf16" and rng.random() < 0.35
    page = int(rng.choice([16, 32, 64, 256]))
    case = W.make_random_prefill(seed, lens_q, lens_k, Hq, Hkv, D, dtype, causal, wl, wr, mm=mm, sink_mode=sink,
                                 max_ranges=5, max_range_len=120)
    case.name = f"rand{seed}_{dtype}_d{D}_h{Hq}x{Hkv}_{'paged' + str(page) if paged else 'packed'}"
    return case, paged, page


@pytest.mark.parametrize("seed", range(24))
def test_random_prefill_config(dev, seed):
    import torch

    import masked_varlen_softmax_amd as mvs

    case, paged, page = _draw(seed)
    print(f"case {case.name} lens_q {case.lens_q.tolist()} lens_k {case.lens_k.tolist()} causal {case.causal} "
          f"wl {case.wl} wr {case.wr} sink {case.sink_mode}", flush=True)
    t = table_for(case)
    tol, ltol = (F32_TOL, LSE_TOL_F32) if case.dtype == "f32" else (BF16_TOL, LSE_TOL_BF16)
    ref, rlse = ref_attention(W.as_f32(case.q), W.as_f32(case.k), W.as_f32(case.v), case.cu_q, case.cu_k,
                              case.scale, case.causal, case.wl, case.wr, t, case.sinks, case.sink_mode)
    if not paged:
        got, glse = run_prefill(case, dev, t)
    else:
        kc, vc, bt = W.paged_kv(case, page, seed + 3, extra_pages=2)
        for b in range(case.num_seqs):  # the scatter put every key where the table says
            k0, L = int(case.cu_k[b]), int(case.lens_k[b])
            np.testing.assert_array_equal(ref_gather_paged(kc, bt[b], L, page), case.k[k0:k0 + L])
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
    assert_close(got, ref, tol, case.name)
    assert_lse_close(glse, rlse, ltol, case.name)
