"""ctypes binding of libmvs.so (the C ABI declared in include/mvs.h).

Argument marshalling only: tensors become raw pointers, strides and the
current HIP stream; every step of the computation runs in the library. Device
entry points require tensors on the GPU and raise otherwise - there is no CPU
fallback. torch supplies device memory and streams.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import library_path

MVS_OK = 0
MVS_ERR_INVALID = -1
MVS_ERR_UNSUPPORTED = -2
MVS_ERR_CAPACITY = -3
MVS_ERR_DEVICE = -4
MVS_BF16 = 0
MVS_F32 = 1
SINK_NONE = 0
SINK_KEY0_BIAS = 1
SINK_NULL_LOGIT = 2

_STATUS = {MVS_ERR_INVALID: "invalid", MVS_ERR_UNSUPPORTED: "unsupported", MVS_ERR_CAPACITY: "capacity",
           MVS_ERR_DEVICE: "device"}


class MvsError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"mvs {_STATUS.get(code, code)} error ({code}): {message}")
        self.code = code


_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F32 = ctypes.c_float
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "build_query_range_table": (_I64, [_P, _I64, _P, _P, _I32, _P, _P]),
    "attn_varlen_fwd": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I64, _I64, _I64, _I64, _P, _P, _I32, _I32, _I32, _I32,
                                       _I32, _I32, _F32, _I32, _I32, _I32, _P, _P, _I32, _P, _P]),
    "attn_varlen_fwd_range_scan": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I64, _I64, _I64, _I64, _P, _P, _I32, _I32,
                                                  _I32, _I32, _I32, _I32, _F32, _I32, _I32, _I32, _P, _I32, _P,
                                                  _I32, _P, _P]),
    "attn_varlen_fwd_paged": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I64, _I64, _I64, _I64, _I64, _I32, _P, _I32,
                                             _I32, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _F32, _I32, _I32,
                                             _I32, _P, _P, _I32, _P, _P]),
    "attn_paged_decode_workspace_size": (_SZ, [_I32, _I32, _I32, _I32]),
    "attn_paged_decode_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I64, _I64, _I64, _I32, _P, _I32, _P, _I32,
                                                 _I32, _I32, _I32, _I32, _I32, _F32, _I32, _P, _I32, _P, _P]),
    "attn_paged_decode": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I64, _I64, _I64, _I32, _P, _I32, _P, _I32, _I32, _I32,
                                         _I32, _I32, _I32, _F32, _I32, _P, _I32, _P, _P, _SZ, _P]),
    "build_query_range_table_device": (ctypes.c_int, [_P, _I64, _P, _P, _I32, _P, _P, _P]),
    "mvs_prefill_useful_flops": (_I64, [_P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _P]),
    "mvs_decode_useful_bytes": (_I64, [_P, _I32, _I32, _I32, _I32, _I32]),
    "mvs_last_error": (ctypes.c_char_p, []),
    "mvs_plan_key_tiles": (ctypes.c_int, [_I32, _I32, _I32, _I32, _I32, _I32, _I32, _P, _I32, _P, _I32]),
}


def lib():
    """The loaded library; raises ImportError when it has not been built."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise ImportError(f"libmvs.so is not built ({path}); run `python masked_varlen_softmax_amd/build.py` "
                              "or __graft_entry__.build()")
        handle = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(code):
    if code != MVS_OK:
        raise MvsError(code, lib().mvs_last_error().decode(errors="replace"))


def _host_i32(x):
    a = np.ascontiguousarray(np.asarray(x), dtype=np.int32)
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# ----------------------------------------------------------------------------- host: range table
def build_query_range_table(out, ranges, query_start_loc, seq_lens) -> int:
    """Fill the caller's ``out`` table (host int32 ``[capacity, 2]``) and return N or 0.

    ``ranges`` is ``dict[request -> list[(start, end)]]`` (inclusive pairs),
    a CSR pair ``(offsets [B+1], pairs [R, 2])``, or None. ``out`` may be a
    NumPy array or a CPU torch tensor (e.g. pinned staging memory).
    """
    qsl = _host_i32(query_start_loc)
    sl = _host_i32(seq_lens)
    B = len(qsl) - 1
    if ranges is None:
        offs, pairs = None, None
    elif isinstance(ranges, dict):
        offs_l, pairs_l = [0], []
        for b in range(B):
            pairs_l.extend(ranges.get(b, []))
            offs_l.append(len(pairs_l))
        offs = np.asarray(offs_l, dtype=np.int32)
        pairs = np.asarray(pairs_l, dtype=np.int32).reshape(-1, 2)
    else:
        offs, pairs = _host_i32(ranges[0]), _host_i32(ranges[1]).reshape(-1, 2)
    if hasattr(out, "data_ptr"):  # torch CPU tensor
        if out.is_cuda or out.dtype.itemsize != 4 or not out.is_contiguous():
            raise ValueError("out must be a contiguous host int32 tensor")
        out_ptr, cap = ctypes.c_void_p(out.data_ptr()), out.shape[0]
    else:
        if out.dtype != np.int32 or not out.flags.c_contiguous:
            raise ValueError("out must be a C-contiguous int32 array")
        out_ptr, cap = out.ctypes.data_as(ctypes.c_void_p), out.shape[0]
    n = lib().build_query_range_table(out_ptr, cap, _ptr(qsl), _ptr(sl), B, _ptr(offs),
                                      _ptr(pairs) if pairs is not None and pairs.size else None)
    if n < 0:
        _check(int(n))
    return int(n)


def prefill_useful_flops(cu_seqlens_q, cu_seqlens_k, num_q_heads, head_dim, causal, window_left=-1,
                         window_right=-1, q_range_table=None) -> int:
    """Useful FLOPs of a prefill call (host arrays), from the library's accounting."""
    cq, ck = _host_i32(cu_seqlens_q), _host_i32(cu_seqlens_k)
    tab = None if q_range_table is None else _host_i32(q_range_table).reshape(-1, 2)
    n = lib().mvs_prefill_useful_flops(_ptr(cq), _ptr(ck), len(cq) - 1, num_q_heads, head_dim, int(bool(causal)),
                                       int(window_left), int(window_right), _ptr(tab))
    if n < 0:
        _check(int(n))
    return int(n)


def decode_useful_bytes(seq_lens, num_kv_heads, head_dim, elem_bytes, window_left=-1) -> int:
    """K + V bytes a decode call must read (host seq_lens), from the library's accounting."""
    sl = _host_i32(seq_lens)
    n = lib().mvs_decode_useful_bytes(_ptr(sl), len(sl), num_kv_heads, head_dim, elem_bytes, int(window_left))
    if n < 0:
        _check(int(n))
    return int(n)


def plan_key_tiles(Lq, Lk, row0, rows, causal, window_left, window_right, table_rows, key_tile, num_key_tiles):
    """Tile classes (0 skip, 1 partial, 2 full) the prefill kernel uses for one query tile."""
    out = np.zeros(num_key_tiles, dtype=np.int8)
    tr = None if table_rows is None else _host_i32(table_rows).reshape(-1, 2)
    _check(lib().mvs_plan_key_tiles(Lq, Lk, row0, rows, int(causal), window_left, window_right, _ptr(tr),
                                    key_tile, _ptr(out), num_key_tiles))
    return out


# ----------------------------------------------------------------------------- device entry points
def _torch():
    import torch

    return torch


def _dev(t, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (no CPU path exists)")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return MVS_BF16
    if t.dtype == torch.float32:
        return MVS_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _token_major(t, name):
    if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
        raise ValueError(f"{name} must be [tokens, heads, head_dim] with heads and head_dim contiguous")


def attn_varlen_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale, causal=False,
                    window_left=-1, window_right=-1, q_range_table=None, sinks=None, sink_mode=SINK_NONE,
                    out=None, lse=None, stream=None):
    """Masked attention prefill; returns ``out`` ``[Nq, Hq, D]`` (and fills ``lse`` ``[Hq, Nq]`` if given)."""
    torch = _torch()
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _token_major(t, nm)
    if out is None:
        out = torch.empty_like(q)
    _token_major(out, "out")
    if k.dtype != q.dtype or v.dtype != q.dtype or out.dtype != q.dtype:
        raise ValueError("q, k, v and out must share a dtype")
    if k.shape[1:] != v.shape[1:] or q.shape[2] != k.shape[2] or k.shape[0] != v.shape[0]:
        raise ValueError("k and v must be [Nk, Hkv, D] with the head_dim of q")
    for t, nm in ((cu_seqlens_q, "cu_seqlens_q"), (cu_seqlens_k, "cu_seqlens_k"), (q_range_table, "q_range_table")):
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
            raise ValueError(f"{nm} must be a contiguous int32 tensor")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    if q_range_table is not None and (q_range_table.dim() != 2 or q_range_table.shape[1] != 2
                                      or q_range_table.shape[0] < q.shape[0]):
        raise ValueError("q_range_table must be [Nq, 2] int32")
    if sinks is not None and (sinks.dtype != torch.float32 or sinks.numel() != q.shape[1] or not sinks.is_contiguous()):
        raise ValueError("sinks must be fp32 [Hq]")
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (q.shape[1], q.shape[0])
                            or not lse.is_contiguous()):
        raise ValueError("lse must be contiguous fp32 [Hq, Nq]")
    code = lib().attn_varlen_fwd(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"), _dtype_code(q), q.stride(0), k.stride(0),
        v.stride(0), out.stride(0), _dev(cu_seqlens_q, "cu_seqlens_q"), _dev(cu_seqlens_k, "cu_seqlens_k"),
        cu_seqlens_q.numel() - 1, int(max_seqlen_q), int(max_seqlen_k), q.shape[1], k.shape[1], q.shape[2],
        float(softmax_scale), int(bool(causal)), int(window_left), int(window_right),
        _dev(q_range_table, "q_range_table"), _dev(sinks, "sinks"), int(sink_mode), _dev(lse, "lse"),
        _stream(stream))
    _check(code)
    return out


def build_query_range_table_device(out, query_start_loc, seq_lens, range_offsets, ranges, stream=None):
    """Fill the device table ``out`` (int32 ``[capacity, 2]``) from device-resident metadata on ``stream``."""
    torch = _torch()
    for t, nm in ((out, "out"), (query_start_loc, "query_start_loc"), (seq_lens, "seq_lens"),
                  (range_offsets, "range_offsets"), (ranges, "ranges")):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{nm} must be a contiguous int32 tensor")
    if out.dim() != 2 or out.shape[1] != 2:
        raise ValueError("out must be [capacity, 2]")
    B = query_start_loc.numel() - 1
    if seq_lens.numel() != B or range_offsets.numel() != B + 1:
        raise ValueError("seq_lens must be [B] and range_offsets [B + 1]")
    code = lib().build_query_range_table_device(
        _dev(out, "out"), out.shape[0], _dev(query_start_loc, "query_start_loc"), _dev(seq_lens, "seq_lens"), B,
        _dev(range_offsets, "range_offsets"), _dev(ranges, "ranges"), _stream(stream))
    _check(code)
    return out


def attn_varlen_fwd_range_scan(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale,
                               ranges, causal=False, window_left=-1, window_right=-1, sinks=None,
                               sink_mode=SINK_NONE, out=None, lse=None, stream=None):
    """The range-scan baseline: like :func:`attn_varlen_fwd` with ``ranges`` (device int32
    ``[B, max_ranges, 2]``, unused slots start >= end) in place of the table."""
    torch = _torch()
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _token_major(t, nm)
    if out is None:
        out = torch.empty_like(q)
    _token_major(out, "out")
    if k.dtype != q.dtype or v.dtype != q.dtype or out.dtype != q.dtype:
        raise ValueError("q, k, v and out must share a dtype")
    B = cu_seqlens_q.numel() - 1
    if ranges.dtype != torch.int32 or not ranges.is_contiguous() or ranges.dim() != 3 or ranges.shape[0] != B \
            or ranges.shape[2] != 2:
        raise ValueError("ranges must be contiguous int32 [B, max_ranges, 2]")
    if sinks is not None and (sinks.dtype != torch.float32 or sinks.numel() != q.shape[1] or not sinks.is_contiguous()):
        raise ValueError("sinks must be fp32 [Hq]")
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (q.shape[1], q.shape[0])
                            or not lse.is_contiguous()):
        raise ValueError("lse must be contiguous fp32 [Hq, Nq]")
    code = lib().attn_varlen_fwd_range_scan(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"), _dtype_code(q), q.stride(0), k.stride(0),
        v.stride(0), out.stride(0), _dev(cu_seqlens_q, "cu_seqlens_q"), _dev(cu_seqlens_k, "cu_seqlens_k"), B,
        int(max_seqlen_q), int(max_seqlen_k), q.shape[1], k.shape[1], q.shape[2], float(softmax_scale),
        int(bool(causal)), int(window_left), int(window_right), _dev(ranges, "ranges"), ranges.shape[1],
        _dev(sinks, "sinks"), int(sink_mode), _dev(lse, "lse"), _stream(stream))
    _check(code)
    return out


def _paged_caches(k_cache, v_cache, block_table):
    torch = _torch()
    if k_cache.dim() != 4 or k_cache.stride(3) != 1 or k_cache.shape != v_cache.shape \
            or k_cache.stride() != v_cache.stride():
        raise ValueError("caches must be 4-D [blocks, Hkv, page, D] views with equal layout and head_dim contiguous")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or not block_table.is_contiguous():
        raise ValueError("block_table must be contiguous int32 [B, max_blocks]")


def attn_varlen_fwd_paged(q, k_cache, v_cache, block_table, cu_seqlens_q, seq_lens_k, max_seqlen_q, max_seqlen_k,
                          softmax_scale, causal=False, window_left=-1, window_right=-1, q_range_table=None,
                          sinks=None, sink_mode=SINK_NONE, out=None, lse=None, stream=None):
    """Prefill with K/V read from a paged cache. ``q`` ``[Nq, Hq, D]`` packed by ``cu_seqlens_q``;
    caches ``[num_blocks, Hkv, page, D]`` views as for :func:`attn_paged_decode`; ``seq_lens_k``
    ``[B]`` counts each sequence's keys (its cached context plus its new tokens)."""
    torch = _torch()
    _token_major(q, "q")
    _paged_caches(k_cache, v_cache, block_table)
    if out is None:
        out = torch.empty_like(q)
    _token_major(out, "out")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype or out.dtype != q.dtype:
        raise ValueError("q, caches and out must share a dtype")
    if k_cache.shape[3] != q.shape[2]:
        raise ValueError("caches must have the head_dim of q")
    for t, nm in ((cu_seqlens_q, "cu_seqlens_q"), (seq_lens_k, "seq_lens_k"), (q_range_table, "q_range_table")):
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
            raise ValueError(f"{nm} must be a contiguous int32 tensor")
    B = cu_seqlens_q.numel() - 1
    if seq_lens_k.numel() != B or block_table.shape[0] < B:
        raise ValueError("seq_lens_k must be [B] and block_table must have B rows")
    if q_range_table is not None and (q_range_table.dim() != 2 or q_range_table.shape[1] != 2
                                      or q_range_table.shape[0] < q.shape[0]):
        raise ValueError("q_range_table must be [Nq, 2] int32")
    if sinks is not None and (sinks.dtype != torch.float32 or sinks.numel() != q.shape[1] or not sinks.is_contiguous()):
        raise ValueError("sinks must be fp32 [Hq]")
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (q.shape[1], q.shape[0])
                            or not lse.is_contiguous()):
        raise ValueError("lse must be contiguous fp32 [Hq, Nq]")
    code = lib().attn_varlen_fwd_paged(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(out, "out"), _dtype_code(q),
        q.stride(0), out.stride(0), k_cache.stride(0), k_cache.stride(1), k_cache.stride(2), k_cache.shape[0],
        _dev(block_table, "block_table"), block_table.shape[1], k_cache.shape[2], _dev(cu_seqlens_q, "cu_seqlens_q"),
        _dev(seq_lens_k, "seq_lens_k"), B, int(max_seqlen_q), int(max_seqlen_k), q.shape[1], k_cache.shape[1],
        q.shape[2], float(softmax_scale), int(bool(causal)), int(window_left), int(window_right),
        _dev(q_range_table, "q_range_table"), _dev(sinks, "sinks"), int(sink_mode), _dev(lse, "lse"),
        _stream(stream))
    _check(code)
    return out


def attn_paged_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim) -> int:
    return int(lib().attn_paged_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim))


def _decode_args(q, k_cache, v_cache, block_table, seq_lens, sinks, lse, out):
    torch = _torch()
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be contiguous [B, Hq, D]")
    _paged_caches(k_cache, v_cache, block_table)
    if seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous() or seq_lens.numel() != q.shape[0]:
        raise ValueError("seq_lens must be contiguous int32 [B]")
    if sinks is not None and (sinks.dtype != torch.float32 or sinks.numel() != q.shape[1] or not sinks.is_contiguous()):
        raise ValueError("sinks must be fp32 [Hq]")
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (q.shape[1], q.shape[0])
                            or not lse.is_contiguous()):
        raise ValueError("lse must be contiguous fp32 [Hq, B]")
    if out is None:
        out = torch.empty_like(q)
    if not out.is_contiguous() or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must be contiguous and shaped like q")
    return out


def attn_paged_decode(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, softmax_scale, window_left=-1,
                      sinks=None, sink_mode=SINK_NONE, out=None, lse=None, workspace=None, stream=None):
    """Paged decode. ``q`` ``[B, Hq, D]``; caches ``[num_blocks, Hkv, page, D]`` (HND) or any
    4-D view with head_dim contiguous, indexed ``[block, kv_head, slot, dim]``."""
    torch = _torch()
    out = _decode_args(q, k_cache, v_cache, block_table, seq_lens, sinks, lse, out)
    B, Hq, D = q.shape
    need = attn_paged_decode_workspace_size(B, Hq, k_cache.shape[1], D)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    code = lib().attn_paged_decode(
        _dev(q, "q"), _dev(out, "out"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dtype_code(q),
        k_cache.stride(0), k_cache.stride(1), k_cache.stride(2), k_cache.shape[0], _dev(block_table, "block_table"),
        block_table.shape[1], _dev(seq_lens, "seq_lens"), B, int(max_seq_len), Hq, k_cache.shape[1], D,
        k_cache.shape[2], float(softmax_scale), int(window_left), _dev(sinks, "sinks"), int(sink_mode),
        _dev(lse, "lse"), _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(code)
    return out


def attn_paged_decode_noalloc(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, softmax_scale, window_left=-1,
                              sinks=None, sink_mode=SINK_NONE, out=None, lse=None, stream=None):
    """attn_paged_decode on the library's per-device workspace: no allocation inside the call
    (``out`` must then be given). Calls that overlap on one device race."""
    if out is None:
        raise ValueError("attn_paged_decode_noalloc allocates nothing: pass out")
    out = _decode_args(q, k_cache, v_cache, block_table, seq_lens, sinks, lse, out)
    B, Hq, D = q.shape
    code = lib().attn_paged_decode_noalloc(
        _dev(q, "q"), _dev(out, "out"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dtype_code(q),
        k_cache.stride(0), k_cache.stride(1), k_cache.stride(2), k_cache.shape[0], _dev(block_table, "block_table"),
        block_table.shape[1], _dev(seq_lens, "seq_lens"), B, int(max_seq_len), Hq, k_cache.shape[1], D,
        k_cache.shape[2], float(softmax_scale), int(window_left), _dev(sinks, "sinks"), int(sink_mode),
        _dev(lse, "lse"), _stream(stream))
    _check(code)
    return out
