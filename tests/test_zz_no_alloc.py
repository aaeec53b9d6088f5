"""GPU test of attn_paged_decode_noalloc, the decode entry point that allocates nothing (needs an MI355X).

Its partials live in the library's per-device buffer instead of a caller workspace; the kernels are
those of attn_paged_decode, so on the same inputs both must give the same outputs and LSE bit for bit.
Two calls in a row, the second smaller (fewer sequences, other head counts, head_dim and page size),
check that nothing left in the shared buffer by the first call leaks into the second. Both are also
compared with the oracle (bf16 max |err| 1e-2, LSE 2e-3). A call captured in a graph is replayed
with new inputs and checked against eager calls.
"""

import dataclasses

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


def test_noalloc_replays_from_a_captured_graph(dev):
    """The callers this entry point is for capture it in a HIP graph: capture one call, then replay
    it three times with new query values written in place between replays (eager work and a
    synchronisation in between). Every replay must equal, bit for bit, an eager call of the same
    entry point on the same inputs, and match the oracle."""
    import torch

    import masked_varlen_softmax_amd as mvs

    case = W.make_decode("noalloc_graph", 23, [3000, 17, 700, 4100, 1], 16, 4, 128, 16, "bf16", wl=1023,
                         sink_mode=2, extra_pages=2)
    kc, vc = to_dev(case.k_cache, dev), to_dev(case.v_cache, dev)
    bt, sl = to_dev(case.block_table, dev), to_dev(case.seq_lens, dev)
    sinks = to_dev(case.sinks.astype(np.float32), dev)
    q = to_dev(case.q, dev)
    out = torch.empty_like(q)
    lse = torch.empty((case.Hq, q.shape[0]), dtype=torch.float32, device=dev)
    max_len = int(case.seq_lens.max())

    def call(o, l):
        mvs.attn_paged_decode_noalloc(q, kc, vc, bt, sl, max_len, case.scale, case.wl, sinks, case.sink_mode,
                                      out=o, lse=l)

    call(out, lse)  # outside the capture first: the launcher's per-device state is set up
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream(device=dev)  # default priority
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            call(out, lse)
    torch.cuda.current_stream().wait_stream(stream)
    rng = np.random.default_rng(99)
    for rep in range(3):
        print(f"case noalloc graph replay {rep}", flush=True)
        new_q = rng.standard_normal(case.q.shape, dtype=np.float32)
        q.copy_(torch.from_numpy(new_q).to(dev).to(torch.bfloat16))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got, glse = out.float().cpu().numpy(), lse.cpu().numpy()
        want_o, want_l = torch.empty_like(out), torch.empty_like(lse)
        call(want_o, want_l)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got, want_o.float().cpu().numpy(), err_msg=f"replay {rep}: out")
        np.testing.assert_array_equal(glse, want_l.cpu().numpy(), err_msg=f"replay {rep}: lse")
        rep_case = dataclasses.replace(case, q=q.view(torch.int16).cpu().numpy().view(np.uint16))
        ref, rlse = oracle_decode(rep_case)
        assert_close(got, ref, BF16_TOL, f"replay {rep}")
        assert_lse_close(glse, rlse, LSE_TOL_BF16, f"replay {rep}")
