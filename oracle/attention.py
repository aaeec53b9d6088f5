"""Oracle for masked softmax attention over packed variable-length sequences.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition ([PR49815], key code snippets: the dense fp32 ``_reference`` of the
MiMo test, and the kernel's sink branch; [PR50294], implementation breakdown
step 5: a dense float32 reference compared element by element):

  for every request b and query head h (kv head h // (Hq / Hkv), the
  ``repeat_interleave`` grouping of the reference):
      S = scale * Q_b[:, h] @ K_b[:, kv]^T                       [Lq, Lk]
      KEY0_BIAS: S[:, 0] += sink[h]   (added after scaling, not scaled)
      S[~visible] = -inf              (visible from oracle.mask.ref_mask)
      P = softmax over keys, with NULL_LOGIT adding exp(sink[h]) to the
          denominator only ([PR49815], key code snippets: the null-logit init
          of the running max at the sink and the running sum at 1)
      O = P @ V_b[:, kv]
      LSE = log of the softmax denominator (natural log)

Sink modes: 0 none, 1 key-0 bias (the MiMo semantics the page adds), 2 null
logit (the GPT-OSS ``s_aux`` semantics the page contrasts it with).

A row with no visible key (never produced by the pages' configurations) has
O = 0 and LSE = -inf, or LSE = sink[h] under NULL_LOGIT: the empty sum
convention. Parity unpinned for such rows beyond that convention.

Inputs are float arrays already rounded to the storage precision (bf16 values
held exactly in fp32); the oracle computes in ``dtype`` (fp32 by default).

Pins (tests/test_oracle_attention.py): torch's CPU scaled_dot_product_attention
in fp64 on the same mask (sink as an additive key-0 bias); scipy's logsumexp
for the LSE; closed forms for one and two visible keys under each sink mode;
sink = 0 equals no sink; a window covering everything equals the unmasked
softmax; GQA equals MHA on repeated kv heads; softmax rows sum to one and
outputs lie in the convex hull of visible values; on the tiny MiMo
configuration KEY0_BIAS differs from NULL_LOGIT and from no sink by more than
1e-2, as the pages' error tables report.
"""

from __future__ import annotations

import numpy as np

from .mask import ref_mask, ref_mask_rows

SINK_NONE = 0
SINK_KEY0_BIAS = 1
SINK_NULL_LOGIT = 2


def _masked_softmax_rows(s, vis, sink, sink_mode, dtype):
    """Softmax of each row of ``s`` over its visible entries.

    Returns (P, lse) with P ``[R, Lk]`` and lse ``[R]`` in ``dtype``.
    """
    s = np.where(vis, s, -np.inf).astype(dtype)
    m = s.max(axis=1) if s.shape[1] > 0 else np.full(s.shape[0], -np.inf, dtype=dtype)
    if sink_mode == SINK_NULL_LOGIT:
        m = np.maximum(m, dtype(sink))
    m_safe = np.where(np.isfinite(m), m, dtype(0.0))
    e = np.exp(s - m_safe[:, None])  # exp(-inf) = 0 for invisible entries
    den = e.sum(axis=1, dtype=dtype)
    if sink_mode == SINK_NULL_LOGIT:
        den = den + np.exp(dtype(sink) - m_safe)
    with np.errstate(divide="ignore", invalid="ignore"):
        P = np.where(den[:, None] > 0, e / den[:, None], dtype(0.0))
        lse = np.where(den > 0, m_safe + np.log(den), -np.inf).astype(dtype)
    return P.astype(dtype), lse


def ref_attention(q, k, v, cu_q, cu_k, scale, causal=False, wl=-1, wr=-1, table=None,
                  sinks=None, sink_mode=SINK_NONE, dtype=np.float32):
    """Dense masked attention for a packed batch.

    Args:
      q: ``[Nq, Hq, D]``; k: ``[Nk, Hkv, D]``; v: ``[Nk, Hkv, Dv]`` (float arrays).
      cu_q, cu_k: ``B+1`` prefix sums of query and key counts.
      scale: softmax scale applied to ``Q K^T``.
      causal, wl, wr: the base predicate (see oracle.mask).
      table: None or int ``[Nq, 2]`` per-query-row range table.
      sinks: None or ``[Hq]`` per-head sink logits; sink_mode as above.
    Returns:
      (out ``[Nq, Hq, Dv]``, lse ``[Hq, Nq]``) in ``dtype``.
    """
    q = np.asarray(q, dtype=dtype)
    k = np.asarray(k, dtype=dtype)
    v = np.asarray(v, dtype=dtype)
    Nq, Hq, D = q.shape
    Hkv = k.shape[1]
    assert Hq % Hkv == 0
    group = Hq // Hkv
    out = np.zeros((Nq, Hq, v.shape[2]), dtype=dtype)
    lse = np.full((Hq, Nq), -np.inf, dtype=dtype)
    for b in range(len(cu_q) - 1):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        k0, k1 = int(cu_k[b]), int(cu_k[b + 1])
        Lq, Lk = q1 - q0, k1 - k0
        if Lq == 0:
            continue
        rows = None if table is None else np.asarray(table)[q0:q1]
        vis = ref_mask(Lq, Lk, causal, wl, wr, rows)
        for h in range(Hq):
            kv = h // group
            s = dtype(scale) * (q[q0:q1, h, :] @ k[k0:k1, kv, :].T)
            sink = 0.0 if sinks is None else float(sinks[h])
            if sink_mode == SINK_KEY0_BIAS and Lk > 0:
                s[:, 0] += dtype(sink)
            P, row_lse = _masked_softmax_rows(s, vis, sink, sink_mode, dtype)
            out[q0:q1, h, :] = P @ v[k0:k1, kv, :]
            lse[h, q0:q1] = row_lse
    return out, lse


def ref_attention_rows(q, k, v, cu_q, cu_k, scale, samples, causal=False, wl=-1, wr=-1,
                       table=None, sinks=None, sink_mode=SINK_NONE, dtype=np.float32):
    """The same definition evaluated only at sampled ``(packed row, head)`` pairs.

    Used for full-size configurations, where the dense oracle would take too
    long: each sampled output is computed alone from its request's keys.
    Returns (out ``[len(samples), D]``, lse ``[len(samples)]``).
    """
    cu_q = [int(x) for x in cu_q]
    cu_k = [int(x) for x in cu_k]
    Hq = q.shape[1]
    group = Hq // k.shape[1]
    out = np.zeros((len(samples), v.shape[2]), dtype=dtype)
    lse = np.full(len(samples), -np.inf, dtype=dtype)
    for n, (t, h) in enumerate(samples):
        b = max(j for j in range(len(cu_q) - 1) if cu_q[j] <= t < cu_q[j + 1])
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        Lq, Lk = q1 - q0, k1 - k0
        i = t - q0
        row = None if table is None else np.asarray(table)[t:t + 1]
        vis = ref_mask_rows([Lk - Lq + i], Lk, causal, wl, wr, row)
        kv = h // group
        qi = np.asarray(q[t, h, :], dtype=dtype)
        kk = np.asarray(k[k0:k1, kv, :], dtype=dtype)
        vv = np.asarray(v[k0:k1, kv, :], dtype=dtype)
        s = (dtype(scale) * (kk @ qi))[None, :]
        sink = 0.0 if sinks is None else float(sinks[h])
        if sink_mode == SINK_KEY0_BIAS and Lk > 0:
            s[:, 0] += dtype(sink)
        P, row_lse = _masked_softmax_rows(s, vis, sink, sink_mode, dtype)
        out[n] = (P @ vv)[0]
        lse[n] = row_lse[0]
    return out, lse
