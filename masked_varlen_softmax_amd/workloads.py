"""Seeded synthetic inputs for masked varlen attention.

This module only draws random inputs and packs them; it holds none of the
attention arithmetic, so both the HIP library's tests and the CPU oracle can
consume the same arrays. It imports neither.

bf16 tensors are produced as fp32 draws rounded to nearest-even bf16 and
carried as their 16-bit patterns (``*_bits``, ``np.uint16``); ``as_f32`` turns
them back into the exact fp32 values the device sees.

The named workloads mirror the shapes the pages discuss (multimodal frames of a
video as bidirectional ranges, vision-encoder windows with per-head sinks,
long-context decode with sliding windows); every value is synthetic.
"""

from __future__ import annotations

import os
from dataclasses import dataclass, field

import numpy as np

SINK_NONE = 0
SINK_KEY0_BIAS = 1
SINK_NULL_LOGIT = 2


# ----------------------------------------------------------------------------- bf16 storage
_CHUNK = 1 << 22  # elements per independently seeded slab


def _bits_into(x: np.ndarray, out: np.ndarray) -> None:
    """Round a contiguous fp32 slab to bf16 (nearest, ties to even) into ``out`` (uint16)."""
    u = x.view(np.uint32)
    t = np.right_shift(u, 16)
    np.bitwise_and(t, 1, out=t)
    np.add(t, 0x7FFF, out=t)
    np.add(t, u, out=t)
    np.right_shift(t, 16, out=t)
    out[...] = t


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    xf, of = x.reshape(-1), out.reshape(-1)
    for i in range(0, xf.size, _CHUNK):
        _bits_into(xf[i:i + _CHUNK], of[i:i + _CHUNK])
    return out


def as_f32(bits_or_f32: np.ndarray) -> np.ndarray:
    """Exact fp32 values of a bf16 bit array (fp32 arrays pass through)."""
    a = np.asarray(bits_or_f32)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a.astype(np.float32, copy=False)


def draw_normal(seed: int, stream: int, shape, dtype_name: str) -> np.ndarray:
    """N(0,1) draws of ``shape``, as bf16 bit patterns or fp32.

    The flat array is cut into fixed slabs of ``_CHUNK`` elements, each drawn
    from its own child of ``SeedSequence([seed, stream])``, so the values do not
    depend on how many threads fill them.
    """
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    bf16 = dtype_name == "bf16"
    out = np.empty(n, dtype=np.uint16 if bf16 else np.float32)
    nch = (n + _CHUNK - 1) // _CHUNK
    children = np.random.SeedSequence([seed, stream]).spawn(max(nch, 1))

    def work(i):
        g = np.random.Generator(np.random.PCG64(children[i]))
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        x = g.standard_normal(size=hi - lo, dtype=np.float32)
        if bf16:
            _bits_into(x, out[lo:hi])
        else:
            out[lo:hi] = x

    if nch <= 1:
        for i in range(nch):
            work(i)
    else:
        from concurrent.futures import ThreadPoolExecutor

        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(work, range(nch)))
    return out.reshape(shape)


# ----------------------------------------------------------------------------- cases
@dataclass
class PrefillCase:
    name: str
    dtype: str  # "bf16" or "f32"
    q: np.ndarray  # [Nq, Hq, D]   (uint16 bits for bf16, float32 for f32)
    k: np.ndarray  # [Nk, Hkv, D]
    v: np.ndarray  # [Nk, Hkv, D]
    cu_q: np.ndarray  # int32 [B+1]
    cu_k: np.ndarray  # int32 [B+1]
    scale: float
    causal: bool
    wl: int
    wr: int
    ranges: dict | None = None  # request -> list of inclusive (start, end)
    sinks: np.ndarray | None = None  # float32 [Hq]
    sink_mode: int = SINK_NONE
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self):
        return len(self.cu_q) - 1

    @property
    def Hq(self):
        return self.q.shape[1]

    @property
    def Hkv(self):
        return self.k.shape[1]

    @property
    def D(self):
        return self.q.shape[2]

    @property
    def lens_q(self):
        return np.diff(self.cu_q)

    @property
    def lens_k(self):
        return np.diff(self.cu_k)

    def ranges_csr(self):
        """(offsets int32 [B+1], pairs int32 [R, 2]) in request order."""
        offs = [0]
        pairs = []
        for b in range(self.num_seqs):
            rs = (self.ranges or {}).get(b, [])
            pairs.extend(rs)
            offs.append(len(pairs))
        return np.asarray(offs, dtype=np.int32), np.asarray(pairs, dtype=np.int32).reshape(-1, 2)


@dataclass
class DecodeCase:
    name: str
    dtype: str
    q: np.ndarray  # [B, Hq, D]
    k_cache: np.ndarray  # [num_pages, Hkv, page, D]
    v_cache: np.ndarray
    block_table: np.ndarray  # int32 [B, max_blocks], -1 where unused
    seq_lens: np.ndarray  # int32 [B]
    page_size: int
    scale: float
    wl: int
    sinks: np.ndarray | None = None
    sink_mode: int = SINK_NONE
    meta: dict = field(default_factory=dict)

    @property
    def Hq(self):
        return self.q.shape[1]

    @property
    def Hkv(self):
        return self.k_cache.shape[1]

    @property
    def D(self):
        return self.q.shape[2]


def _cu(lens):
    return np.concatenate([[0], np.cumsum(np.asarray(lens, dtype=np.int64))]).astype(np.int32)


def frame_ranges(rng, span: int, n: int, frame: int):
    """``n`` non-overlapping frames of ``frame`` tokens at random offsets in ``[0, span)``.

    The free tokens ``span - n*frame`` are split into ``n + 1`` gaps by a random
    composition; frame ``j`` is stored as the inclusive pair ``(s, s+frame-1)``.
    """
    free = span - n * frame
    assert free >= 0
    cuts = np.sort(rng.integers(0, free + 1, size=n))
    gaps = np.diff(np.concatenate([[0], cuts]))
    out = []
    pos = 0
    for j in range(n):
        pos += int(gaps[j])
        out.append((pos, pos + frame - 1))
        pos += frame
    return out


def random_ranges(rng, Lk: int, max_ranges: int, max_len: int, allow_degenerate=False):
    """Random non-overlapping inclusive ranges inside ``[0, Lk)`` (for parity sweeps)."""
    out = []
    pos = int(rng.integers(0, max(1, Lk // 4) + 1))
    for _ in range(int(rng.integers(0, max_ranges + 1))):
        length = int(rng.integers(1, max_len + 1))
        if pos + length > Lk:
            break
        if allow_degenerate and rng.random() < 0.15:
            out.append((pos + length - 1, pos))  # start >= end: ignored by the method
        else:
            out.append((pos, pos + length - 1))
        pos += length + int(rng.integers(0, max(1, Lk // 3) + 1))
    return out


def make_prefill(name, seed, lens_q, lens_k, Hq, Hkv, D, dtype="bf16", causal=False, wl=-1, wr=-1,
                 ranges=None, sink_mode=SINK_NONE, scale=None) -> PrefillCase:
    cu_q, cu_k = _cu(lens_q), _cu(lens_k)
    nq, nk = int(cu_q[-1]), int(cu_k[-1])
    q = draw_normal(seed, 0, (nq, Hq, D), dtype)
    k = draw_normal(seed, 1, (nk, Hkv, D), dtype)
    v = draw_normal(seed, 2, (nk, Hkv, D), dtype)
    sinks = draw_normal(seed, 3, (Hq,), "f32") if sink_mode != SINK_NONE else None
    if scale is None:
        scale = float(1.0 / np.sqrt(D))
    return PrefillCase(name, dtype, q, k, v, cu_q, cu_k, scale, causal, wl, wr, ranges, sinks, sink_mode)


def make_random_prefill(seed, lens_q, lens_k, Hq, Hkv, D, dtype="bf16", causal=False, wl=-1, wr=-1,
                        mm=False, sink_mode=SINK_NONE, max_ranges=4, max_range_len=64):
    """Generic case for parity sweeps; ``mm`` draws random ranges per request."""
    rng = np.random.default_rng(seed + 7919)
    ranges = None
    if mm:
        ranges = {b: random_ranges(rng, int(lk), max_ranges, max_range_len) for b, lk in enumerate(lens_k)}
    return make_prefill(f"rand{seed}", seed, lens_q, lens_k, Hq, Hkv, D, dtype, causal, wl, wr, ranges, sink_mode)


def padded_ranges(case: PrefillCase, max_ranges: int) -> np.ndarray:
    """The case's ranges as int32 ``[B, max_ranges, 2]`` in list order; unused slots are (0, 0)."""
    out = np.zeros((case.num_seqs, max_ranges, 2), dtype=np.int32)
    for b in range(case.num_seqs):
        rs = (case.ranges or {}).get(b, [])
        assert len(rs) <= max_ranges, (b, len(rs), max_ranges)
        if rs:
            out[b, :len(rs)] = np.asarray(rs, dtype=np.int32)
    return out


def c2_range_count(n: int) -> PrefillCase:
    """The multimodal-prefix sliding layer (4 x 4096, D 256, window 1024) with exactly ``n`` frames per
    request, each ``min(256, 4096 // n)`` tokens long (64 frames of 256 tokens do not fit in 4096)."""
    rng = np.random.default_rng(3000 + n)
    B, L = 4, 4096
    frame = min(256, L // n)
    ranges = {b: frame_ranges(rng, L, n, frame) for b in range(B)}
    case = make_prefill(f"c2_n{n}", 1001, [L] * B, [L] * B, 16, 8, 256, "bf16", causal=True, wl=1023, wr=-1,
                        ranges=ranges)
    return case


def paged_kv(case: PrefillCase, page_size: int, seed: int, nhd: bool = False, extra_pages: int = 0):
    """Scatter a prefill case's packed K and V into pages of ``page_size`` tokens in random page order.

    Returns ``(k_cache, v_cache, block_table)``. The caches are ``[pages, Hkv, page, D]``, or with
    ``nhd`` stored ``[pages, page, Hkv, D]``; block_table is int32 ``[B, max_blocks]`` with -1 past
    each sequence's last page. Slots past a sequence's end and the ``extra_pages`` hold random
    values, so a read of the wrong slot changes the result.
    """
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in case.lens_k]
    pages_per = [(L + page_size - 1) // page_size for L in lens]
    total = max(1, sum(pages_per) + extra_pages)
    perm = rng.permutation(total).astype(np.int32)
    bt = np.full((case.num_seqs, max(1, max(pages_per, default=1))), -1, dtype=np.int32)
    shape = (total, page_size, case.Hkv, case.D) if nhd else (total, case.Hkv, page_size, case.D)
    caches = []
    for stream, src in ((5, case.k), (6, case.v)):
        c = draw_normal(seed, stream, shape, case.dtype)
        pos = 0
        for b, n in enumerate(pages_per):
            k0 = int(case.cu_k[b])
            for j in range(n):
                page = int(perm[pos + j])
                t0, t1 = j * page_size, min(lens[b], (j + 1) * page_size)
                rows = src[k0 + t0:k0 + t1]  # [tokens, Hkv, D]
                if nhd:
                    c[page, :t1 - t0] = rows
                else:
                    c[page, :, :t1 - t0] = rows.transpose(1, 0, 2)
            pos += n
        caches.append(c)
    pos = 0
    for b, n in enumerate(pages_per):
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    return caches[0], caches[1], bt


# ----------------------------------------------------------------------------- named workloads
def c1_tiny_window_sinks(num_kv_heads: int = 4) -> PrefillCase:
    """Tiny non-causal window attention with key-0 sinks, fp32, sequences of 5 and 37 tokens."""
    case = make_prefill("c1", 1000, [5, 37], [5, 37], 4, num_kv_heads, 64, "f32", causal=False, wl=8, wr=8,
                        sink_mode=SINK_KEY0_BIAS, scale=1.0 / 8.0)
    case.name = f"c1_kv{num_kv_heads}"
    return case


def c2_mm_prefix_sliding(frames_max: int = 16) -> PrefillCase:
    """bf16, 4 x 4096 tokens, 16 q / 8 kv heads, D 256, causal, window 1024, 256-token frames.

    Each request holds ``U{8..frames_max}`` frames (at most 16 fit in 4096 tokens).
    """
    rng = np.random.default_rng(2001)
    B, L = 4, 4096
    ranges = {b: frame_ranges(rng, L, int(rng.integers(8, frames_max + 1)), 256) for b in range(B)}
    return make_prefill("c2", 1001, [L] * B, [L] * B, 16, 8, 256, "bf16", causal=True, wl=1023, wr=-1,
                        ranges=ranges)


def c3_chunked_global(frames_max: int = 32) -> PrefillCase:
    """bf16, 8 requests with 6144 cached tokens and a 2048-token chunk, 8 q / 4 kv heads, D 512."""
    rng = np.random.default_rng(2002)
    B, ctx, chunk = 8, 6144, 2048
    ranges = {b: frame_ranges(rng, ctx + chunk, int(rng.integers(8, frames_max + 1)), 256) for b in range(B)}
    return make_prefill("c3", 1002, [chunk] * B, [ctx + chunk] * B, 8, 4, 512, "bf16", causal=True, wl=-1, wr=-1,
                        ranges=ranges)


def c4_vision_window_sinks() -> PrefillCase:
    """bf16, 16 images of U{1024..4096} patches, 16 heads, D 128, window 128 both sides, key-0 sinks."""
    rng = np.random.default_rng(2003)
    lens = [int(x) for x in rng.integers(1024, 4097, size=16)]
    return make_prefill("c4", 1003, lens, lens, 16, 16, 128, "bf16", causal=False, wl=128, wr=128,
                        sink_mode=SINK_KEY0_BIAS)


def make_decode(name, seed, seq_lens, Hq, Hkv, D, page_size=16, dtype="bf16", wl=-1, sink_mode=SINK_NONE,
                extra_pages=0, scale=None) -> DecodeCase:
    """Random-permutation page assignment; unused block-table entries are -1."""
    rng = np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    B = len(seq_lens)
    pages_per = [(int(L) + page_size - 1) // page_size for L in seq_lens]
    total = sum(pages_per) + extra_pages
    perm = rng.permutation(total).astype(np.int32)
    max_blocks = max(1, max(pages_per) if pages_per else 1)
    bt = np.full((B, max_blocks), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(pages_per):
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    q = draw_normal(seed, 0, (B, Hq, D), dtype)
    kc = draw_normal(seed, 1, (total, Hkv, page_size, D), dtype)
    vc = draw_normal(seed, 2, (total, Hkv, page_size, D), dtype)
    sinks = draw_normal(seed, 3, (Hq,), "f32") if sink_mode != SINK_NONE else None
    if scale is None:
        scale = float(1.0 / np.sqrt(D))
    return DecodeCase(name, dtype, q, kc, vc, bt, seq_lens, page_size, scale, wl, sinks, sink_mode)


def c5_paged_decode(window: bool) -> DecodeCase:
    """bf16, 64 sequences, contexts U{4096..32768}, page 16, 32 q / 8 kv heads, D 128.

    ``window`` selects the sliding-window layer (4096 keys) instead of full attention.
    """
    rng = np.random.default_rng(2004)
    lens = rng.integers(4096, 32769, size=64).astype(np.int32)
    case = make_decode("c5_window" if window else "c5_full", 1004, lens, 32, 8, 128, 16, "bf16",
                       wl=4095 if window else -1)
    return case


PREFILL_CONFIGS = {
    "c1_kv4": lambda: c1_tiny_window_sinks(4),
    "c1_kv2": lambda: c1_tiny_window_sinks(2),
    "c2": c2_mm_prefix_sliding,
    "c3": c3_chunked_global,
    "c4": c4_vision_window_sinks,
}
