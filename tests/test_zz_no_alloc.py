"""GPU test of attn_paged_decode_noalloc, the decode entry point that allocates nothing (needs an MI355X).

Its partials live in the library's per-device buffer instead of a caller workspace; the kernels are
those of attn_paged_decode, so on the same inputs both must give the same outputs and LSE bit for bit.
Two calls in a row, the second smaller (fewer sequences, other head counts, head_dim and page size),
check that nothing left in the shared buffer by the first call leaks into the second. Both are also
compared with the oracle (bf16 max |err| 1e-2, LSE 2e-3).
"""

import numpy as np
import pytest

from gpu_helpers import BF16_TOL, LSE_TOL_BF16, assert_close, assert_lse_close, oracle_decode, run_decode, to_dev
from masked_varlen_softmax_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _run_noalloc(case, dev):
    import torch

    import masked_varlen_softmax_amd as mvs

    q = to_dev(case.q, dev)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((case.Hq, q.shape[0]), float("nan"), dtype=torch.float32, device=dev)
    sinks = None if case.sinks is None else to_dev(case.sinks.astype(np.float32), dev)
    mvs.attn_paged_decode_noalloc(q, to_dev(case.k_cache, dev), to_dev(case.v_cache, dev),
                                  to_dev(case.block_table, dev), to_dev(case.seq_lens, dev),
                                  int(case.seq_lens.max()), case.scale, case.wl, sinks, case.sink_mode, out=out,
                                  lse=lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def test_noalloc_matches_the_workspace_entry_point_on_two_calls(dev):
    first = W.make_decode("noalloc_a", 21, [4100, 37, 9000, 1, 300, 2048], 32, 8, 128, 16, "bf16", wl=-1,
                          sink_mode=2, extra_pages=2)
    second = W.make_decode("noalloc_b", 22, [70, 5, 33], 8, 2, 64, 32, "bf16", wl=40, sink_mode=1)
    for case in (first, second):
        print(f"case {case.name} seq_lens {case.seq_lens.tolist()}", flush=True)
        got, glse = _run_noalloc(case, dev)
        want, wlse = run_decode(case, dev)
        np.testing.assert_array_equal(got, want, err_msg=f"{case.name}: out differs from attn_paged_decode")
        np.testing.assert_array_equal(glse, wlse, err_msg=f"{case.name}: lse differs from attn_paged_decode")
        ref, rlse = oracle_decode(case)
        assert_close(got, ref, BF16_TOL, case.name)
        assert_lse_close(glse, rlse, LSE_TOL_BF16, case.name)
