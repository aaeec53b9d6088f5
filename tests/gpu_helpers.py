"""Helpers shared by the GPU tests: upload seeded inputs, run the library
through its binding, evaluate the oracle on the same inputs."""

import numpy as np

from masked_varlen_softmax_amd import workloads as W
from oracle import ref_attention, ref_attention_rows, ref_build_table, ref_paged_decode

BF16_TOL = 1e-2
F32_TOL = 1e-4
LSE_TOL_BF16 = 2e-3
LSE_TOL_F32 = 1e-4


def to_dev(a, dev):
    import torch

    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def table_for(case):
    """(table or None) from the oracle's builder; the library builder is checked separately."""
    if case.ranges is None:
        return None
    t = np.full((case.q.shape[0], 2), 0, dtype=np.int32)
    n = ref_build_table(t, case.ranges, case.cu_q, case.lens_k)
    return t if n else None


def run_prefill(case, dev, table=None, want_lse=True, poison=True):
    import torch

    import masked_varlen_softmax_amd as mvs

    q, k, v = to_dev(case.q, dev), to_dev(case.k, dev), to_dev(case.v, dev)
    out = torch.empty_like(q)
    if poison:
        out.fill_(float("nan"))
    lse = None
    if want_lse:
        lse = torch.full((case.Hq, case.q.shape[0]), float("nan"), dtype=torch.float32, device=dev)
    sinks = None if case.sinks is None else to_dev(case.sinks.astype(np.float32), dev)
    mvs.attn_varlen_fwd(q, k, v, to_dev(case.cu_q, dev), to_dev(case.cu_k, dev), int(case.lens_q.max(initial=0)),
                        int(case.lens_k.max(initial=0)), case.scale, case.causal, case.wl, case.wr,
                        None if table is None else to_dev(table, dev), sinks, case.sink_mode, out=out, lse=lse)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    return o, (None if lse is None else lse.cpu().numpy())


def oracle_prefill(case, table=None):
    return ref_attention(W.as_f32(case.q), W.as_f32(case.k), W.as_f32(case.v), case.cu_q, case.cu_k, case.scale,
                         case.causal, case.wl, case.wr, table, case.sinks, case.sink_mode)


def oracle_prefill_rows(case, samples, table=None):
    return ref_attention_rows(W.as_f32(case.q), W.as_f32(case.k), W.as_f32(case.v), case.cu_q, case.cu_k,
                              case.scale, samples, case.causal, case.wl, case.wr, table, case.sinks, case.sink_mode)


def assert_close(got, ref, tol, what):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite outputs (unwritten rows?)"
    err = np.abs(got - ref)
    worst = np.unravel_index(np.argmax(err), err.shape)
    assert err.max() <= tol, f"{what}: max |err| {err.max():.3e} at {worst} (got {got[worst]}, ref {ref[worst]})"
    return float(err.max())


def assert_lse_close(got, ref, tol, what):
    both_inf = np.isneginf(got) & np.isneginf(ref)
    assert (np.isneginf(got) == np.isneginf(ref)).all(), f"{what}: -inf LSE mismatch"
    g, r = np.where(both_inf, 0, got), np.where(both_inf, 0, ref)
    err = np.abs(g - r).max() if g.size else 0.0
    assert err <= tol, f"{what}: LSE max |err| {err:.3e}"


def run_decode(case, dev, want_lse=True, block_table=None, k_cache=None, v_cache=None, workspace=None):
    import torch

    import masked_varlen_softmax_amd as mvs

    q = to_dev(case.q, dev)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((case.Hq, q.shape[0]), float("nan"), dtype=torch.float32, device=dev) if want_lse else None
    kc = to_dev(case.k_cache if k_cache is None else k_cache, dev)
    vc = to_dev(case.v_cache if v_cache is None else v_cache, dev)
    bt = to_dev(case.block_table if block_table is None else block_table, dev)
    sinks = None if case.sinks is None else to_dev(case.sinks.astype(np.float32), dev)
    ws = workspace
    if ws is None:
        ws_bytes = mvs.attn_paged_decode_workspace_size(q.shape[0], case.Hq, case.Hkv, case.D)
        ws = torch.full((ws_bytes // 4,), float("nan"), dtype=torch.float32, device=dev)  # poisoned workspace
    mvs.attn_paged_decode(q, kc, vc, bt, to_dev(case.seq_lens, dev), int(case.seq_lens.max()), case.scale, case.wl,
                          sinks, case.sink_mode, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), (None if lse is None else lse.cpu().numpy())


def oracle_decode(case, seqs=None):
    return ref_paged_decode(W.as_f32(case.q), W.as_f32(case.k_cache), W.as_f32(case.v_cache), case.block_table,
                            case.seq_lens, case.page_size, case.scale, case.wl, case.sinks, case.sink_mode, seqs=seqs)
