"""GPU tests of build_query_range_table_device.

The device builder must give bit for bit the oracle builder's table (rows of
a batch with no covered row come out (-1, -1), which the kernels treat like
no table), leave rows past the capacity untouched, and work inside a captured
HIP graph: builder plus attention captured once, replayed with new ranges
written into the same device buffers, each replay checked against the eager
path with a host-built table.
"""

import numpy as np
import pytest

from gpu_helpers import BF16_TOL, assert_close, oracle_prefill, to_dev
from masked_varlen_softmax_amd import workloads as W
from oracle import ref_build_table

pytestmark = pytest.mark.gpu
POISON = -777


@pytest.fixture(scope="module")
def dev():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _qsl(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def _csr(ranges, B):
    offs, pairs = [0], []
    for b in range(B):
        pairs.extend(ranges.get(b, []))
        offs.append(len(pairs))
    return np.asarray(offs, np.int32), np.asarray(pairs, np.int32).reshape(-1, 2)


def _device_table(dev, qsl, seq_lens, offs, pairs, cap):
    import torch

    import masked_varlen_softmax_amd as mvs

    out = torch.full((cap, 2), POISON, dtype=torch.int32, device=dev)
    pr = pairs if len(pairs) else np.zeros((1, 2), np.int32)
    mvs.build_query_range_table_device(out, to_dev(qsl, dev), to_dev(np.asarray(seq_lens, np.int32), dev),
                                       to_dev(offs, dev), to_dev(pr, dev))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _random_batch(rng):
    B = int(rng.integers(1, 7))
    lq = rng.integers(0, 300, B)
    ctx = rng.integers(0, 400, B)
    lk = lq + ctx
    ranges = {}
    for b in range(B):
        rs = []
        for _ in range(int(rng.integers(0, 6))):
            s = int(rng.integers(-5, int(lk[b]) + 5))
            e = s + int(rng.integers(-3, 120))  # degenerate (s >= e), overlapping and out-of-chunk ranges
            rs.append((s, e))
        ranges[b] = rs
    return lq, lk, ranges


@pytest.mark.parametrize("seed", range(8))
def test_device_builder_matches_oracle(dev, seed):
    rng = np.random.default_rng(100 + seed)
    lq, lk, ranges = _random_batch(rng)
    qsl = _qsl(lq)
    N = int(qsl[-1])
    cap = N + 7
    offs, pairs = _csr(ranges, len(lq))
    print(f"case device table seed {seed} rows {N} ranges {len(pairs)}", flush=True)
    got = _device_table(dev, qsl, lk, offs, pairs, cap)
    ref = np.full((cap, 2), POISON, dtype=np.int32)
    n = ref_build_table(ref, ranges, qsl, lk)
    if n == 0:
        ref[:N] = -1  # no covered row: the device writes (-1, -1) where the host writes nothing
    np.testing.assert_array_equal(got, ref)


def test_device_builder_many_ranges_and_capacity(dev):
    rng = np.random.default_rng(7)
    lq, lk = np.array([700, 0, 1500]), np.array([900, 40, 1500])
    ranges = {b: [(int(s), int(s) + int(rng.integers(1, 40))) for s in rng.integers(0, int(lk[b]), 600)]
              for b in range(3)}  # more ranges than one LDS block, many overlapping
    qsl = _qsl(lq)
    offs, pairs = _csr(ranges, 3)
    print("case device table 600 ranges per request", flush=True)
    full = _device_table(dev, qsl, lk, offs, pairs, int(qsl[-1]))
    ref = np.full((int(qsl[-1]), 2), POISON, dtype=np.int32)
    assert ref_build_table(ref, ranges, qsl, lk) == int(qsl[-1])
    np.testing.assert_array_equal(full, ref)
    cap = 1000  # smaller than the batch: rows past it stay untouched
    part = _device_table(dev, qsl, lk, offs, pairs, cap)
    np.testing.assert_array_equal(part, ref[:cap])


@pytest.mark.parametrize("d, hq, hkv", [(128, 4, 2), (256, 8, 4), (512, 4, 2)], ids=["d128", "d256_pairs", "d512"])
def test_graph_captured_builder_and_attention(dev, d, hq, hkv):
    """Each head dim's schedule (kernel 1; its packed-head form at D 256; kernel 3 at D 512)."""
    import torch

    import masked_varlen_softmax_amd as mvs

    lens_q, lens_k = [300, 129], [500, 129]
    case = W.make_random_prefill(21, lens_q, lens_k, hq, hkv, d, "bf16", True, 100, -1)
    B, N = 2, sum(lens_q)
    max_ranges = 8
    q, k, v = to_dev(case.q, dev), to_dev(case.k, dev), to_dev(case.v, dev)
    cu_q, cu_k = to_dev(case.cu_q, dev), to_dev(case.cu_k, dev)
    qsl_d, sl_d = to_dev(case.cu_q, dev), to_dev(np.asarray(lens_k, np.int32), dev)
    offs_d = torch.zeros(B + 1, dtype=torch.int32, device=dev)
    pairs_d = torch.zeros((B * max_ranges, 2), dtype=torch.int32, device=dev)
    table_d = torch.empty((N, 2), dtype=torch.int32, device=dev)
    out = torch.empty_like(q)

    def step():
        mvs.build_query_range_table_device(table_d, qsl_d, sl_d, offs_d, pairs_d)
        mvs.attn_varlen_fwd(q, k, v, cu_q, cu_k, max(lens_q), max(lens_k), case.scale, True, 100, -1, table_d,
                            out=out)

    def load(ranges):
        offs, pairs = _csr(ranges, B)
        offs_d.copy_(torch.from_numpy(offs))
        pairs_d.zero_()
        if len(pairs):
            pairs_d[:len(pairs)].copy_(torch.from_numpy(pairs))

    rng = np.random.default_rng(5)
    s = torch.cuda.Stream()  # default priority
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        load({})
        step()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    print(f"case graph replays d {d}", flush=True)
    for rep in range(3):
        ranges = W.random_ranges(rng, lens_k[0], 4, 90), W.random_ranges(rng, lens_k[1], 4, 40)
        ranges = {0: ranges[0], 1: ranges[1]}
        load(ranges)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        case.ranges = ranges
        t = np.full((N, 2), -1, dtype=np.int32)
        ref_build_table(t, ranges, case.cu_q, case.lens_k)
        np.testing.assert_array_equal(table_d.cpu().numpy(), t)
        ref, _ = oracle_prefill(case, t)
        assert_close(got, ref, BF16_TOL, f"graph replay {rep}")
        # the eager path on the same inputs gives the same bits
        eager = mvs.attn_varlen_fwd(q, k, v, cu_q, cu_k, max(lens_q), max(lens_k), case.scale, True, 100, -1,
                                    to_dev(t, dev))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got, eager.float().cpu().numpy())
