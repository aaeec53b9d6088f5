"""CPU-only checks of the C ABI: exported symbols, the host range-table builder
(bit-exact against the oracle), argument validation that rejects before any
device work, the decode workspace arithmetic, and the prefill tile plan
checked against the oracle's dense mask. No kernel is launched here.
"""

import ctypes
import os
import re

import numpy as np
import pytest

from masked_varlen_softmax_amd import workloads as W
from oracle import CapacityError, ref_build_table, ref_mask

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
POISON = 12345


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "mvs.h")).read()
    return re.findall(r"MVS_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_library_exports_every_declared_symbol(mvs_lib):
    names = _declared_symbols()
    assert set(names) >= {"build_query_range_table", "build_query_range_table_device", "attn_varlen_fwd",
                          "attn_varlen_fwd_paged", "attn_paged_decode", "attn_paged_decode_workspace_size",
                          "mvs_last_error", "mvs_plan_key_tiles", "mvs_prefill_useful_flops",
                          "mvs_decode_useful_bytes"}
    for name in names:
        assert hasattr(mvs_lib, name), name


def _qsl(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def _both(ranges, query_lens, seq_lens, cap):
    import masked_varlen_softmax_amd as mvs

    a = np.full((cap, 2), POISON, dtype=np.int32)
    b = np.full((cap, 2), POISON, dtype=np.int32)
    try:
        nr = ref_build_table(a, ranges, _qsl(query_lens), np.asarray(seq_lens))
    except CapacityError:
        nr = "capacity"
    try:
        nl = mvs.build_query_range_table(b, ranges, _qsl(query_lens), seq_lens)
    except mvs.MvsError as e:
        nl = "capacity" if e.code == -3 else e
    return nr, nl, a, b


def test_builder_worked_example_bit_exact(mvs_lib):
    golden = [ln.split() for ln in open(os.path.join(ROOT, "tests", "golden", "worked_example_table.txt"))
              if ln.strip() and not ln.startswith("#")]
    rows = np.array([[int(x), int(y)] for _, x, y in golden[1:]], dtype=np.int32)
    nr, nl, a, b = _both({0: [(1, 3), (5, 7)], 1: [(2, 4), (9, 12)]}, [8, 6], [8, 13], 16)
    assert nl == nr == int(golden[0][0])
    np.testing.assert_array_equal(b, rows)
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("seed", range(40))
def test_builder_random_batches_bit_exact(mvs_lib, seed):
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 7))
    seq_lens = rng.integers(0, 200, size=B)
    query_lens = np.array([int(rng.integers(0, L + 1)) if rng.random() > 0.2 else min(1, L) for L in seq_lens])
    ranges = {b: W.random_ranges(rng, int(seq_lens[b]) + 20, 6, 40, allow_degenerate=True) for b in range(B)}
    if rng.random() < 0.2:
        ranges = {}
    cap = int(query_lens.sum()) + int(rng.integers(0, 3))
    if rng.random() < 0.1:
        cap = max(0, int(query_lens.sum()) - 1)
    nr, nl, a, b = _both(ranges, query_lens, seq_lens, cap)
    assert nr == nl
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("seed", range(20))
def test_builder_overlapping_ranges_last_listed_wins(mvs_lib, seed):
    """Outside the contract, but defined: where ranges overlap, the range listed last owns the row, as in
    the oracle's list-order writes. Also a batch whose first request starts past row 0."""
    import masked_varlen_softmax_amd as mvs

    rng = np.random.default_rng(900 + seed)
    B = int(rng.integers(1, 4))
    seq_lens = rng.integers(1, 120, size=B)
    query_lens = np.array([int(rng.integers(1, L + 1)) for L in seq_lens])
    ranges = {}
    for b in range(B):
        rs = []
        for _ in range(int(rng.integers(1, 7))):
            s = int(rng.integers(-5, int(seq_lens[b]) + 5))
            rs.append((s, s + int(rng.integers(-3, 50))))
        ranges[b] = rs
    lead = int(rng.integers(0, 4))
    qsl = _qsl(query_lens) + lead
    cap = int(qsl[-1]) + 2
    a = np.full((cap, 2), POISON, dtype=np.int32)
    b_ = np.full((cap, 2), POISON, dtype=np.int32)
    nr = ref_build_table(a, ranges, qsl, np.asarray(seq_lens))
    nl = mvs.build_query_range_table(b_, ranges, qsl, seq_lens)
    assert nr == nl
    np.testing.assert_array_equal(a, b_)


def test_builder_edge_cases(mvs_lib):
    import masked_varlen_softmax_amd as mvs

    # decode row with an optimistic upper bound never lands in a range
    nr, nl, a, b = _both({0: [(2, 9)]}, [1], [1 << 20], 4)
    assert nr == nl == 0 and (b == POISON).all()
    # clipping past the chunk keeps the unclipped pair
    nr, nl, a, b = _both({0: [(6, 12)]}, [4], [8], 4)
    assert nl == 4
    np.testing.assert_array_equal(b, [[-1, -1], [-1, -1], [6, 12], [6, 12]])
    # None, empty batch, capacity
    out = np.full((2, 2), POISON, dtype=np.int32)
    assert mvs.build_query_range_table(out, None, _qsl([2]), [2]) == 0
    assert mvs.build_query_range_table(out, {0: [(0, 1)]}, _qsl([0]), [0]) == 0
    with pytest.raises(mvs.MvsError) as ei:
        mvs.build_query_range_table(out, {0: [(0, 1)]}, _qsl([3]), [3])
    assert ei.value.code == -3 and (out == POISON).all()
    # CSR input equals dict input
    b1 = np.zeros((14, 2), np.int32)
    b2 = np.zeros((14, 2), np.int32)
    n1 = mvs.build_query_range_table(b1, {0: [(1, 3), (5, 7)], 1: [(2, 4), (9, 12)]}, _qsl([8, 6]), [8, 13])
    n2 = mvs.build_query_range_table(b2, ([0, 2, 4], [[1, 3], [5, 7], [2, 4], [9, 12]]), _qsl([8, 6]), [8, 13])
    assert n1 == n2 == 14 and (b1 == b2).all()


def test_builder_rejects_bad_offsets(mvs_lib):
    import masked_varlen_softmax_amd as mvs

    out = np.zeros((4, 2), np.int32)
    with pytest.raises(mvs.MvsError):
        mvs.build_query_range_table(out, ([0, 2, 1], [[0, 1], [2, 3]]), _qsl([2, 2]), [2, 2])
    with pytest.raises(mvs.MvsError):
        mvs.build_query_range_table(out, {0: [(0, 1)]}, np.array([0, 3, 2], np.int32), [3, 3])


def _call_fwd(lib, **kw):
    args = dict(q=1, k=1, v=1, out=1, dtype=0, qs=1024, ks=512, vs=512, os_=1024, cuq=1, cuk=1, nseq=2, mq=8, mk=8,
                hq=8, hkv=4, d=128, scale=0.1, causal=1, wl=-1, wr=-1, table=None, sinks=None, mode=0, lse=None)
    args.update(kw)
    P = ctypes.c_void_p
    return lib.attn_varlen_fwd(P(args["q"] * 256), P(args["k"] * 256), P(args["v"] * 256), P(int(args["out"] * 256)),
                               args["dtype"], args["qs"], args["ks"], args["vs"], args["os_"], P(args["cuq"] * 256),
                               P(args["cuk"] * 256), args["nseq"], args["mq"], args["mk"], args["hq"], args["hkv"],
                               args["d"], args["scale"], args["causal"], args["wl"], args["wr"], args["table"],
                               args["sinks"], args["mode"], args["lse"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), -2), (dict(d=512, dtype=1), -2), (dict(dtype=7), -1), (dict(hq=6, hkv=4), -1),
    (dict(scale=0.0), -1), (dict(scale=float("nan")), -1), (dict(causal=2), -1), (dict(wl=-2), -1),
    (dict(mode=1), -1), (dict(mode=5), -1), (dict(q=0), -1), (dict(cuk=0), -1), (dict(qs=100), -1),
    (dict(ks=8), -1), (dict(qs=1028), -1), (dict(nseq=-1), -1), (dict(ks=1 << 24), -2), (dict(vs=1 << 25), -2),
])
def test_varlen_fwd_rejects_before_launch(mvs_lib, kw, code):
    assert _call_fwd(mvs_lib, **kw) == code
    assert mvs_lib.mvs_last_error()  # a message is recorded


def test_varlen_fwd_empty_batch_is_a_no_op(mvs_lib):
    assert _call_fwd(mvs_lib, nseq=0) == 0
    assert _call_fwd(mvs_lib, mq=0) == 0


# Sizes beyond one launch grid: 2^24 query tiles x 64 heads x 4096 sequences of bf16 workgroups, or
# more heads or sequences than an fp32 grid's y / z extent. Valid arguments, reported as unsupported
# before anything is queued (the device pointers are never touched).
HUGE_BF16 = dict(mq=2**31 - 1, mk=2**31 - 1, hq=64, hkv=8, nseq=4096, qs=8192, os_=8192, ks=1024, vs=1024)
HUGE_F32 = dict(dtype=1, d=64, hq=70000, hkv=70000, qs=70000 * 64, os_=70000 * 64, ks=70000 * 64, vs=70000 * 64)


@pytest.mark.parametrize("d", [64, 128, 256, 512])
def test_varlen_fwd_rejects_grids_beyond_the_launch_limit(mvs_lib, d):
    kw = dict(HUGE_BF16, d=d, qs=64 * d, os_=64 * d, ks=8 * d, vs=8 * d)
    assert _call_fwd(mvs_lib, **kw) == -2
    assert b"workgroups" in mvs_lib.mvs_last_error()
    # the same call at a size that fits is accepted (nothing is launched for an empty batch)
    assert _call_fwd(mvs_lib, **dict(kw, nseq=0)) == 0


def test_varlen_fwd_fp32_rejects_more_heads_than_a_grid_holds(mvs_lib):
    assert _call_fwd(mvs_lib, **HUGE_F32) == -2
    assert _call_fwd(mvs_lib, **dict(HUGE_F32, nseq=70000, hq=8, hkv=4, qs=512, os_=512, ks=256, vs=256)) == -2


def test_varlen_fwd_bf16_output_needs_16_byte_rows(mvs_lib):
    """Output rows are stored 16 bytes at a time: the stride and the base must allow that."""
    assert _call_fwd(mvs_lib, os_=1028) == -1  # a row starts 8 bytes off a 16-byte boundary
    assert _call_fwd(mvs_lib, out=(256 * 5 + 8) / 256) == -1  # base 8 bytes off
    assert _call_fwd_paged(mvs_lib, os_=1028) == -1


def test_varlen_fwd_paged_rejects_grids_beyond_the_launch_limit(mvs_lib):
    kw = dict(mq=2**31 - 1, mk=2**20, mb=2**16, hq=64, hkv=8, nseq=4096, qs=64 * 128, os_=64 * 128)
    assert _call_fwd_paged(mvs_lib, **kw) == -2
    assert _call_fwd_paged(mvs_lib, **dict(kw, nseq=0)) == 0


def test_varlen_fwd_range_scan_rejects_grids_beyond_the_launch_limit(mvs_lib):
    kw = dict(HUGE_BF16, d=256, qs=64 * 256, os_=64 * 256, ks=8 * 256, vs=8 * 256)
    assert _call_fwd_scan(mvs_lib, **kw) == -2


def test_paged_decode_noalloc_rejects_sizes_beyond_its_buffer(mvs_lib):
    """The library-held workspace is 32 MiB per device; larger sizes are refused before any device call."""
    import masked_varlen_softmax_amd as mvs

    P = ctypes.c_void_p
    B, Hq, Hkv, D = 60000, 32, 8, 256
    assert mvs.attn_paged_decode_workspace_size(B, Hq, Hkv, D) > 32 << 20
    code = mvs_lib.attn_paged_decode_noalloc(P(256), P(512), P(768), P(1024), 0, 16 * 8 * D, 16 * D, D, 100,
                                             P(1280), 64, P(1536), B, 1024, Hq, Hkv, D, 16, 0.1, -1, None, 0,
                                             None, None)
    assert code == -3 and b"library holds" in mvs_lib.mvs_last_error()
    # invalid arguments are reported as for attn_paged_decode
    assert mvs_lib.attn_paged_decode_noalloc(P(256), P(512), P(768), P(1024), 0, 16 * 8 * D, 16 * D, D, 100,
                                             P(1280), 64, P(1536), 4, 1024, Hq, Hkv, 96, 16, 0.1, -1, None, 0,
                                             None, None) == -2


def test_paged_decode_rejects_more_sequences_than_a_grid_holds(mvs_lib):
    assert _call_decode(mvs_lib, nseq=70000) == -2
    assert b"sequences" in mvs_lib.mvs_last_error()


def _call_fwd_scan(lib, **kw):
    a = dict(q=1, k=1, v=1, out=1, dtype=0, qs=1024, ks=512, vs=512, os_=1024, cuq=1, cuk=1, nseq=2, mq=8, mk=8,
             hq=8, hkv=4, d=128, scale=0.1, causal=1, wl=-1, wr=-1, ranges=1, mr=8, sinks=None, mode=0, lse=None)
    a.update(kw)
    P = ctypes.c_void_p
    return lib.attn_varlen_fwd_range_scan(P(a["q"] * 256), P(a["k"] * 256), P(a["v"] * 256), P(a["out"] * 256),
                                          a["dtype"], a["qs"], a["ks"], a["vs"], a["os_"], P(a["cuq"] * 256),
                                          P(a["cuk"] * 256), a["nseq"], a["mq"], a["mk"], a["hq"], a["hkv"], a["d"],
                                          a["scale"], a["causal"], a["wl"], a["wr"], P(a["ranges"] * 256), a["mr"],
                                          a["sinks"], a["mode"], a["lse"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=1), -2), (dict(d=512), -2), (dict(mr=65), -2), (dict(mr=-1), -2), (dict(ranges=0), -1),
    (dict(hq=6, hkv=4), -1), (dict(scale=0.0), -1), (dict(q=0), -1), (dict(ks=1 << 24), -2), (dict(mode=1), -1),
])
def test_varlen_fwd_range_scan_rejects_before_launch(mvs_lib, kw, code):
    assert _call_fwd_scan(mvs_lib, **kw) == code


def _call_fwd_paged(lib, **kw):
    a = dict(q=1, kc=1, vc=1, out=1, dtype=0, qs=1024, os_=1024, bs=16 * 4 * 128, hs=16 * 128, ts=128, nblk=100,
             bt=1, mb=64, page=16, cuq=1, slk=1, nseq=2, mq=8, mk=1024, hq=8, hkv=4, d=128, scale=0.1, causal=1,
             wl=-1, wr=-1, table=None, sinks=None, mode=0, lse=None)
    a.update(kw)
    P = ctypes.c_void_p
    return lib.attn_varlen_fwd_paged(P(a["q"] * 256), P(a["kc"] * 256), P(a["vc"] * 256), P(int(a["out"] * 256)),
                                     a["dtype"], a["qs"], a["os_"], a["bs"], a["hs"], a["ts"], a["nblk"],
                                     P(a["bt"] * 256), a["mb"], a["page"], P(a["cuq"] * 256), P(a["slk"] * 256),
                                     a["nseq"], a["mq"], a["mk"], a["hq"], a["hkv"], a["d"], a["scale"], a["causal"],
                                     a["wl"], a["wr"], a["table"], a["sinks"], a["mode"], a["lse"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=1), -2), (dict(dtype=9), -1), (dict(d=96), -2), (dict(hq=6, hkv=4), -1), (dict(page=8), -2),
    (dict(page=48), -2), (dict(scale=0.0), -1), (dict(causal=3), -1), (dict(wr=-2), -1), (dict(mode=2), -1),
    (dict(bt=0), -1), (dict(slk=0), -1), (dict(kc=0), -1), (dict(nblk=0), -1), (dict(mb=63), -1),
    (dict(ts=64), -1), (dict(ts=1 << 24), -2), (dict(bs=-8), -1), (dict(hs=12), -1), (dict(qs=100), -1),
])
def test_varlen_fwd_paged_rejects_before_launch(mvs_lib, kw, code):
    assert _call_fwd_paged(mvs_lib, **kw) == code
    assert mvs_lib.mvs_last_error()


def test_varlen_fwd_paged_empty_batch_is_a_no_op(mvs_lib):
    assert _call_fwd_paged(mvs_lib, nseq=0) == 0
    assert _call_fwd_paged(mvs_lib, mq=0) == 0


def _call_decode(lib, **kw):
    a = dict(q=1, out=1, kc=1, vc=1, dtype=0, bs=16 * 8 * 128, hs=16 * 128, ts=128, nblk=100, bt=1, mb=64, sl=1,
             nseq=4, msl=1024, hq=32, hkv=8, d=128, page=16, scale=0.1, wl=-1, sinks=None, mode=0, lse=None, ws=1,
             wsb=1 << 30)
    a.update(kw)
    P = ctypes.c_void_p
    return lib.attn_paged_decode(P(a["q"] * 256), P(a["out"] * 256), P(a["kc"] * 256), P(a["vc"] * 256), a["dtype"],
                                 a["bs"], a["hs"], a["ts"], a["nblk"], P(a["bt"] * 256), a["mb"], P(a["sl"] * 256),
                                 a["nseq"], a["msl"], a["hq"], a["hkv"], a["d"], a["page"], a["scale"], a["wl"],
                                 a["sinks"], a["mode"], a["lse"], P(a["ws"] * 256), a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=1), -2), (dict(d=512), -2), (dict(hq=24, hkv=8), -2), (dict(hq=7, hkv=2), -1),
    (dict(page=8), -2), (dict(scale=-1.0), -1), (dict(wl=-3), -1), (dict(mode=2), -1), (dict(bt=0), -1),
    (dict(ws=0), -1), (dict(wsb=1000), -3), (dict(mb=10), -1), (dict(ts=100), -1),
])
def test_paged_decode_rejects_before_launch(mvs_lib, kw, code):
    assert _call_decode(mvs_lib, **kw) == code


def test_decode_workspace_size(mvs_lib):
    import masked_varlen_softmax_amd as mvs

    s = mvs.attn_paged_decode_workspace_size(64, 32, 8, 128)
    assert s > 0 and s % 256 == 0
    # 4096 + 64 * 8 segment slots, 4 query heads each: D floats plus (max, sum); then 65 offsets
    slots = (4096 + 64 * 8) * 4
    assert slots * (128 + 2) * 4 <= s <= slots * (128 + 2) * 4 + 3 * 256 + 65 * 8
    assert mvs.attn_paged_decode_workspace_size(64, 32, 8, 96) == 0
    assert mvs.attn_paged_decode_workspace_size(-1, 32, 8, 128) == 0
    assert mvs.attn_paged_decode_workspace_size(64, 32, 6, 128) == 0
    assert mvs.attn_paged_decode_workspace_size(64, 32, 0, 128) == 0
    # independent of context length: the same call serves any max_seq_len
    assert mvs.attn_paged_decode_workspace_size(0, 4, 4, 64) > 0


TILE_CASES = [
    # (Lq, Lk, causal, wl, wr, ranges)
    (100, 100, True, -1, -1, None),
    (100, 100, True, 30, -1, None),
    (100, 100, True, 5, -1, None),
    (50, 180, True, -1, -1, None),
    (50, 180, True, 63, -1, None),
    (130, 130, False, 8, 8, None),
    (130, 130, False, 40, 3, None),
    (130, 130, False, -1, -1, None),
    (90, 90, True, 20, -1, [(3, 40), (50, 88)]),
    (70, 150, True, 31, -1, [(10, 90), (100, 149)]),
    (70, 150, True, -1, -1, [(0, 5), (79, 120), (130, 140)]),
    (64, 64, False, 4, 4, [(10, 60)]),
    (1, 33, True, -1, -1, None),
    (1, 4097, True, 4095, -1, None),
]


@pytest.mark.parametrize("case", TILE_CASES)
@pytest.mark.parametrize("bm,bn", [(128, 64), (64, 32), (32, 16), (16, 64)])
def test_tile_plan_matches_dense_mask(mvs_lib, case, bm, bn):
    import masked_varlen_softmax_amd as mvs

    Lq, Lk, causal, wl, wr, ranges = case
    table = None
    if ranges is not None:
        table = np.full((Lq, 2), POISON, dtype=np.int32)
        if ref_build_table(table, {0: ranges}, np.array([0, Lq]), np.array([Lk])) == 0:
            table = None
    m = ref_mask(Lq, Lk, causal, wl, wr, table)
    nkt = (Lk + bn - 1) // bn + 1  # one tile past the end must be skipped too
    for row0 in range(0, Lq, bm):
        rows = min(bm, Lq - row0)
        tr = None if table is None else table[row0:row0 + bm]
        cls = mvs.plan_key_tiles(Lq, Lk, row0, bm, causal, wl, wr, tr, bn, nkt)
        blk = m[row0:row0 + rows]
        for j in range(nkt):
            sub = blk[:, j * bn:(j + 1) * bn]
            if cls[j] == 0:
                assert not sub.any(), (row0, j)
            elif cls[j] == 2:
                assert sub.shape[1] == bn and sub.all(), (row0, j)
        # the plan's span is tight: first and last non-skipped tiles hold a visible key
        live = np.nonzero(cls)[0]
        if blk.any():
            assert blk[:, live[0] * bn:(live[0] + 1) * bn].any() and blk[:, live[-1] * bn:(live[-1] + 1) * bn].any()
        else:
            assert live.size == 0


def test_tile_plan_two_disjoint_intervals(mvs_lib):
    """A hand-made table whose range does not hold the row: visible keys split in two."""
    import masked_varlen_softmax_amd as mvs

    Lq = Lk = 64
    table = np.full((Lq, 2), -1, dtype=np.int32)
    table[10:20] = (40, 50)  # rows 10..19 see keys 40..50 as well as their causal window
    m = ref_mask(Lq, Lk, True, 3, -1, table)
    cls = mvs.plan_key_tiles(Lq, Lk, 0, 32, True, 3, -1, table[:32], 8, 8)
    for j in range(8):
        sub = m[:32, 8 * j:8 * j + 8]
        if cls[j] == 0:
            assert not sub.any()
        if cls[j] == 2:
            assert sub.all()
    assert cls[5] != 0  # keys 40..47 are visible to rows 10..19


@pytest.mark.parametrize("case", TILE_CASES)
def test_accounting_matches_oracle_popcount(mvs_lib, case):
    """The library's closed-form visible-pair count equals the oracle mask popcount."""
    import masked_varlen_softmax_amd as mvs
    from oracle import ref_useful_pairs

    Lq, Lk, causal, wl, wr, ranges = case
    table = None
    if ranges is not None:
        table = np.full((Lq, 2), 0, dtype=np.int32)
        if ref_build_table(table, {0: ranges}, np.array([0, Lq]), np.array([Lk])) == 0:
            table = None
    want = ref_useful_pairs([0, Lq], [0, Lk], causal, wl, wr, table)
    # 4 * D FLOPs per visible pair per query head
    assert mvs.prefill_useful_flops([0, Lq], [0, Lk], 3, 64, causal, wl, wr, table) == want * 4 * 64 * 3


def test_accounting_decode_bytes(mvs_lib):
    import masked_varlen_softmax_amd as mvs
    from oracle import ref_decode_useful_bytes

    lens = [1, 4095, 4096, 4097, 30000]
    for wl in (-1, 0, 4095, 100000):
        assert mvs.decode_useful_bytes(lens, 8, 128, 2, wl) == ref_decode_useful_bytes(lens, 8, 128, 2, wl)


def test_library_accounting_matches_oracle(mvs_lib):
    """C accounting on packed batches: prefill pairs and decode bytes against the oracle."""
    import masked_varlen_softmax_amd as mvs
    from oracle import ref_decode_useful_bytes, ref_useful_pairs

    rng = np.random.default_rng(17)
    for trial in range(12):
        B = int(rng.integers(1, 5))
        lq = rng.integers(0, 60, B)
        lk = lq + rng.integers(0, 40, B)
        cu_q, cu_k = _qsl(lq), _qsl(lk)
        causal = bool(trial % 2)
        wl = int(rng.choice([-1, 3, 17]))
        wr = int(rng.choice([-1, 0, 5]))
        ranges = {b: [tuple(sorted(rng.integers(0, max(int(lk[b]), 1), 2).tolist())) for _ in range(2)]
                  for b in range(B)}
        table = np.full((int(cu_q[-1]) + 1, 2), 0, dtype=np.int32)
        if ref_build_table(table, ranges, cu_q, lk) == 0:
            table = None
        else:
            table = table[:int(cu_q[-1])]
        want = ref_useful_pairs(cu_q, cu_k, causal, wl, wr, table)
        assert mvs.prefill_useful_flops(cu_q, cu_k, 2, 128, causal, wl, wr, table) == want * 4 * 128 * 2
    lens = [0, 1, 4095, 4096, 4097, 30000]
    for wl in (-1, 0, 4095):
        assert mvs.decode_useful_bytes(lens, 8, 128, 2, wl) == ref_decode_useful_bytes(lens, 8, 128, 2, wl)
    with pytest.raises(mvs.MvsError):
        mvs.decode_useful_bytes([5, -1], 8, 128, 2, -1)
    with pytest.raises(mvs.MvsError):
        mvs.prefill_useful_flops([0, 5, 3], [0, 5, 9], 2, 64, True)
