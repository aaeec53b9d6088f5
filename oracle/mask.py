"""Oracle for the visibility mask of one request.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Notation. Request with ``Lq`` queries and ``Lk`` keys; context offset
``c = Lk - Lq``; local query ``i`` at absolute position ``p = c + i``
([PR50294], the builder snippet and the test snippet under "key code
snippets"; [step14_4], "solution": the query's row is offset by ``start_pos``).
``d = p - k`` is the distance from key ``k`` back to the query.

Windows are given as two bounds: ``wl`` is the largest allowed ``d`` (keys in
the past), ``wr`` the largest allowed ``-d`` (keys in the future); -1 means
unbounded. Readings of the pages:

  * A causal layer with window ``W`` keeps ``W`` keys including the query
    itself: vLLM passes ``1 + layer_window[0]`` as the bound and tests
    ``delta < bound`` ([PR50294], key code snippets, ``forward()`` wiring and
    the mask_mod), so ``wl = layer_window[0] = W - 1``.
  * A bidirectional window ``w`` keeps ``|p - k| <= w`` ([PR49815], key code
    snippets, the test's ``_reference``): ``wl = wr = w``.

The predicate, written out ([PR50294], key code snippets, the mask_mod):

  base(i, k) = 0 <= k < Lk
               and (not causal or d >= 0)
               and (wl < 0 or d <= wl)
               and (wr < 0 or -d <= wr)
  mm(i, k)   = table present and T[i].start <= k <= T[i].end
               and (wl < 0 or d <= wl)        # past side only
  visible    = base or mm

``T[i]`` is this request's table row for query ``i``; the ``(-1, -1)``
sentinel makes ``mm`` false for every real key.

Pins (tests/test_oracle_mask.py): the tutorial's two equivalent causal forms
(broadcast ``k > start_pos + i`` and the ``tril`` slice), a per-element
brute-force loop, the range-scan form of ``mm`` used by the page's test, the
``2w + 1`` key count of a bidirectional window, decode rows with nothing masked.
"""

from __future__ import annotations

import numpy as np


def ref_mask_rows(positions, Lk: int, causal: bool, wl: int, wr: int, table_rows=None) -> np.ndarray:
    """Boolean ``[R, Lk]`` rows for queries at absolute ``positions`` (the predicate above).

    ``table_rows`` is None or an int array ``[R, 2]`` with each query's table row.
    """
    p = np.asarray(positions, dtype=np.int64).reshape(-1, 1)  # [R, 1]
    k = np.arange(Lk, dtype=np.int64)[None, :]  # [1, Lk]
    d = p - k

    base = np.ones((p.shape[0], Lk), dtype=bool)
    if causal:
        base &= d >= 0
    if wl >= 0:
        base &= d <= wl
    if wr >= 0:
        base &= -d <= wr

    if table_rows is None:
        return base
    t = np.asarray(table_rows, dtype=np.int64).reshape(-1, 2)
    mm = (t[:, 0:1] <= k) & (k <= t[:, 1:2])
    if wl >= 0:
        mm &= d <= wl
    return base | mm


def ref_mask(Lq: int, Lk: int, causal: bool, wl: int, wr: int, table_rows=None) -> np.ndarray:
    """Boolean ``[Lq, Lk]`` matrix, True where query ``i`` may attend key ``k``.

    Query ``i`` sits at position ``c + i`` with ``c = Lk - Lq``. ``table_rows``
    is None (no multimodal ranges) or an int array ``[Lq, 2]`` holding this
    request's slice of the per-query-row range table.
    """
    c = Lk - Lq
    return ref_mask_rows(c + np.arange(Lq, dtype=np.int64), Lk, causal, wl, wr, table_rows)
