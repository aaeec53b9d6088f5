"""GPU parity of attn_paged_decode against the CPU oracle (needs an MI355X).

Small caches are compared in full; the full-size paged-decode workload (64
sequences, 4K-32K contexts, full and 4096-key window layers) on a sample of
sequences, each evaluated by the oracle on its own pages. Cross-checks:
decode equals the prefill kernel at one query; a permuted block table gives
the same output bit for bit. Tolerance: max |err| 1e-2 (bf16), LSE 2e-3.
"""

import zlib

import numpy as np
import pytest

from gpu_helpers import (BF16_TOL, LSE_TOL_BF16, assert_close, assert_lse_close, oracle_decode, run_decode,
                         run_prefill, to_dev)
from masked_varlen_softmax_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


DECODE = [
    # name, seq_lens, Hq, Hkv, D, page, wl, sink
    ("g4_full", [1, 15, 16, 17, 300, 1000], 8, 2, 128, 16, -1, 0),
    ("g4_window", [1, 15, 100, 1000, 2048], 8, 2, 128, 16, 99, 0),
    ("g4_window_unaligned", [517, 1000, 700], 8, 2, 128, 16, 250, 0),
    ("g1_key0", [5, 600], 4, 4, 128, 16, -1, 1),
    ("g2_null", [33, 900], 4, 2, 128, 16, -1, 2),
    ("g8_window_key0", [40, 400], 16, 2, 128, 16, 63, 1),
    ("g16", [77, 513], 16, 1, 128, 16, -1, 0),
    ("d64", [129, 800], 8, 2, 64, 16, 300, 0),
    ("d256", [129, 800], 8, 2, 256, 16, -1, 1),
    ("page32", [31, 32, 33, 1000], 8, 2, 128, 32, 500, 0),
    ("long_split", [5000, 9000], 8, 2, 128, 16, -1, 0),
    ("empty_seq", [0, 20], 4, 1, 128, 16, -1, 0),
    # more sequences than one wave's lanes: the balanced split scans lengths in batches
    ("many_seqs", [int(x) for x in np.random.default_rng(5).integers(0, 700, 130)], 8, 2, 128, 16, -1, 2),
    ("g16_d256_window", [300, 700], 16, 1, 256, 16, 200, 1),
    ("all_empty", [0, 0, 0], 8, 2, 128, 16, -1, 2),
    # pairs cut over many shares (more segments than a wave has lanes): one query head per kv head at
    # D 64, sixteen at D 256, a window with an empty sequence
    ("g1_d64_split", [3000, 7000], 4, 4, 64, 16, -1, 2),
    ("g16_d256_split", [4000, 6000], 16, 1, 256, 16, -1, 2),
    ("g2_d64_window_split", [9000, 3000, 0, 4500], 4, 2, 64, 16, 4095, 1),
]


@pytest.mark.parametrize("spec", DECODE, ids=[s[0] for s in DECODE])
def test_decode_parity(dev, spec):
    name, lens, hq, hkv, d, page, wl, sink = spec
    case = W.make_decode(name, zlib.crc32(name.encode()) % 997, lens, hq, hkv, d, page, "bf16", wl=wl, sink_mode=sink,
                         extra_pages=5)
    print(f"case {name}", flush=True)
    got, glse = run_decode(case, dev)
    ref, rlse = oracle_decode(case)
    assert_close(got, ref, BF16_TOL, name)
    assert_lse_close(glse, rlse, LSE_TOL_BF16, name)


def test_decode_workspace_reused_across_sizes(dev):
    """One poisoned workspace serves calls of different sizes in turn: the partials and offsets an
    earlier call left behind are never read by a later one."""
    import torch

    import masked_varlen_softmax_amd as mvs

    cases = [W.make_decode("reuse_a", 31, [6000, 2500, 9000], 8, 2, 128, 16, "bf16", wl=-1, sink_mode=2),
             W.make_decode("reuse_b", 32, [int(x) for x in np.random.default_rng(9).integers(0, 3000, 90)], 8, 2,
                           128, 16, "bf16", wl=1023, sink_mode=1),
             W.make_decode("reuse_c", 33, [12000, 40], 16, 4, 128, 16, "bf16", wl=-1, sink_mode=0)]
    need = max(mvs.attn_paged_decode_workspace_size(len(c.seq_lens), c.Hq, c.Hkv, c.D) for c in cases)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=dev)
    for c in cases + cases[:1]:
        print(f"case {c.name} on the shared workspace", flush=True)
        got, glse = run_decode(c, dev, workspace=ws)
        ref, rlse = oracle_decode(c)
        assert_close(got, ref, BF16_TOL, c.name)
        assert_lse_close(glse, rlse, LSE_TOL_BF16, c.name)


def test_decode_invariant_under_page_permutation(dev):
    case = W.make_decode("perm", 3, [300, 1200, 45], 8, 2, 128, 16, "bf16", wl=500, extra_pages=3)
    a, _ = run_decode(case, dev)
    perm = np.random.default_rng(1).permutation(case.k_cache.shape[0])
    k2 = np.empty_like(case.k_cache)
    v2 = np.empty_like(case.v_cache)
    k2[perm] = case.k_cache
    v2[perm] = case.v_cache
    bt2 = np.where(case.block_table >= 0, perm[np.maximum(case.block_table, 0)], -1).astype(np.int32)
    b, _ = run_decode(case, dev, block_table=bt2, k_cache=k2, v_cache=v2)
    np.testing.assert_array_equal(a, b)


def test_decode_equals_prefill_at_one_query(dev):
    """The decode kernel and the prefill kernel agree on a one-query request."""
    case = W.make_decode("x", 4, [700, 64, 1500], 8, 2, 128, 16, "bf16", wl=255, sink_mode=1)
    got, _ = run_decode(case, dev)
    from oracle import ref_gather_paged

    for b, L in enumerate(case.seq_lens):
        L = int(L)
        kb = ref_gather_paged(case.k_cache, case.block_table[b], L, 16)
        vb = ref_gather_paged(case.v_cache, case.block_table[b], L, 16)
        pc = W.PrefillCase("p", "bf16", case.q[b:b + 1], kb, vb, np.array([0, 1], np.int32),
                           np.array([0, L], np.int32), case.scale, True, 255, -1, None, case.sinks, 1)
        pre, _ = run_prefill(pc, dev, None)
        assert np.abs(pre[0] - got[b]).max() <= BF16_TOL


def _subset(case, seqs):
    """The decode case restricted to `seqs`, with only their pages (renumbered)."""
    pages = []
    rows = []
    for b in seqs:
        n = (int(case.seq_lens[b]) + case.page_size - 1) // case.page_size
        rows.append(list(range(len(pages), len(pages) + n)))
        pages.extend(case.block_table[b, :n].tolist())
    mb = max(len(r) for r in rows)
    bt = np.full((len(seqs), mb), -1, dtype=np.int32)
    for i, r in enumerate(rows):
        bt[i, :len(r)] = r
    pages = np.asarray(pages)
    return W.DecodeCase(case.name, case.dtype, case.q[seqs], case.k_cache[pages], case.v_cache[pages], bt,
                        case.seq_lens[seqs], case.page_size, case.scale, case.wl, case.sinks, case.sink_mode)


@pytest.mark.parametrize("window", [False, True])
def test_full_size_paged_decode_sampled(dev, window):
    case = W.c5_paged_decode(window)
    print(f"case {case.name} full size", flush=True)
    got, glse = run_decode(case, dev)
    assert np.isfinite(got).all() and np.isfinite(glse).all()
    rng = np.random.default_rng(2)
    seqs = sorted(set(rng.choice(len(case.seq_lens), size=6, replace=False).tolist())
                  | {int(np.argmax(case.seq_lens)), int(np.argmin(case.seq_lens))})
    sub = _subset(case, seqs)
    ref, rlse = oracle_decode(sub)
    assert_close(got[seqs], ref, BF16_TOL, case.name)
    assert_lse_close(glse[:, seqs], rlse, LSE_TOL_BF16, case.name)


def test_decode_million_token_context(dev):
    """One sequence of 2^20 keys beside a short one: page indices past 2^16, one share per wave
    across the long sequence, null-logit sink and LSE."""
    case = W.make_decode("long", 12, [1 << 20, 77], 8, 2, 128, 16, "bf16", wl=-1, sink_mode=2, extra_pages=3)
    print("case decode 2^20-token context", flush=True)
    got, glse = run_decode(case, dev)
    ref, rlse = oracle_decode(case)
    assert_close(got, ref, BF16_TOL, "long context")
    assert_lse_close(glse, rlse, LSE_TOL_BF16, "long context")


def _draw_decode(seed):
    rng = np.random.default_rng(70_000 + seed)
    D = int(rng.choice([64, 128, 256]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    B = int(rng.integers(1, 70))
    lens = [int(x) for x in rng.choice([0, 1, 15, 16, 17, 255, 1000, 3000], size=B)]
    page = int(rng.choice([16, 32, 48, 64]))
    wl = int(rng.choice([-1, -1, 0, 63, 700]))
    sink = int(rng.choice([0, 1, 2]))
    case = W.make_decode(f"rand_dec{seed}", 900 + seed, lens, Hkv * G, Hkv, D, page, "bf16", wl=wl, sink_mode=sink,
                         extra_pages=3)
    return case


@pytest.mark.parametrize("seed", range(12))
def test_random_decode_config(dev, seed):
    """Seeded random decode batches: 1-69 sequences (empty ones included), D 64-256, groups 1-16,
    pages of 16-64 tokens (48 is not a power of two), windows, both sink modes."""
    case = _draw_decode(seed)
    print(f"case {case.name} B {len(case.seq_lens)} D {case.D} Hq {case.Hq} Hkv {case.Hkv} page {case.page_size} "
          f"wl {case.wl} sink {case.sink_mode}", flush=True)
    got, glse = run_decode(case, dev)
    ref, rlse = oracle_decode(case)
    assert_close(got, ref, BF16_TOL, case.name)
    assert_lse_close(glse, rlse, LSE_TOL_BF16, case.name)
