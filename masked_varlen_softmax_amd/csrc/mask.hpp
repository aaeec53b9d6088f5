// mask.hpp - the visibility predicate as per-row key intervals, and the tile
// plan built from them. Compiled into the HIP kernels and into the host
// diagnostic mvs_plan_key_tiles, so the kernels' skip/partial/full decisions
// can be checked on a CPU against a dense mask.
//
// Predicate (vLLM PR #50294, "key code snippets", the mm-prefix mask_mod; vLLM
// PR #49815, the two-sided window of the MiMo reference): a query at absolute
// position p sees key k (0 <= k < Lk) when
//     base: (!causal || d >= 0) && (wl < 0 || d <= wl) && (wr < 0 || -d <= wr)
//     mm:   start <= k <= end of its table row, and (wl < 0 || d <= wl)
// with d = p - k. For one row each term is an interval of keys, so the row's
// visible set is the union of at most two intervals. When the row's range
// contains p (always true for tables built by build_query_range_table) both
// intervals contain p and the union is one interval; a hand-made table may
// give two disjoint ones, which the kernels handle exactly.
#pragma once

#include "common.hpp"

namespace mvs {

// Visible keys of one row: [a_lo, a_hi] U [b_lo, b_hi]. Empty when lo > hi.
// When both are non-empty and overlap or touch they are merged into `a`.
struct RowKeys {
  int a_lo, a_hi;
  int b_lo, b_hi;
};

MVS_HD inline long long clamp_ll(long long x, long long lo, long long hi) { return x < lo ? lo : (x > hi ? hi : x); }

MVS_HD inline RowKeys row_keys(int causal, int wl, int wr, int p, int Lk, int r_start, int r_end) {
  const long long last = (long long)Lk - 1;
  // base term
  long long blo = (wl >= 0) ? (long long)p - wl : 0;
  long long bhi = causal ? (long long)p : (wr >= 0 ? (long long)p + wr : last);
  if (causal && wr >= 0 && (long long)p + wr < bhi) bhi = (long long)p + wr;
  blo = blo < 0 ? 0 : blo;
  bhi = bhi > last ? last : bhi;
  // multimodal term: the row's own range, past side clamped by the window
  long long mlo = r_start, mhi = r_end;
  if (wl >= 0 && mlo < (long long)p - wl) mlo = (long long)p - wl;
  mlo = mlo < 0 ? 0 : mlo;
  mhi = mhi > last ? last : mhi;
  const bool b_empty = blo > bhi, m_empty = mlo > mhi;
  RowKeys r;
  if (m_empty || (!b_empty && mlo <= bhi + 1 && blo <= mhi + 1)) {
    // one interval (merged, or the base term alone)
    long long lo = blo, hi = bhi;
    if (!m_empty) {
      lo = lo < mlo ? lo : mlo;
      hi = hi > mhi ? hi : mhi;
    }
    r.a_lo = (int)clamp_ll(lo, -1, 0x7fffffff);
    r.a_hi = (int)clamp_ll(hi, -2, 0x7fffffff);
    if (b_empty && m_empty) {
      r.a_lo = 0;
      r.a_hi = -1;
    }
    r.b_lo = 0;
    r.b_hi = -1;
  } else if (b_empty) {
    r.a_lo = (int)mlo;
    r.a_hi = (int)mhi;
    r.b_lo = 0;
    r.b_hi = -1;
  } else {
    r.a_lo = (int)blo;
    r.a_hi = (int)bhi;
    r.b_lo = (int)mlo;
    r.b_hi = (int)mhi;
  }
  return r;
}

MVS_HD inline bool row_sees(const RowKeys& r, int k) {
  return (k >= r.a_lo && k <= r.a_hi) || (k >= r.b_lo && k <= r.b_hi);
}

// Tile plan of one query tile, reduced over its valid rows:
//   [lo, hi]   smallest and largest visible key of any row (empty: lo > hi)
//   [flo, fhi] keys every row sees through its first interval: a key tile
//              inside [flo, fhi] needs no element mask ("full").
struct TilePlan {
  int lo, hi, flo, fhi;
};

MVS_HD inline TilePlan plan_identity() {
  TilePlan t;
  t.lo = 0x7fffffff;
  t.hi = -1;
  t.flo = -0x7fffffff;
  t.fhi = 0x7fffffff;
  return t;
}

MVS_HD inline void plan_add_row(TilePlan& t, const RowKeys& r) {
  if (r.a_lo <= r.a_hi) {
    t.lo = r.a_lo < t.lo ? r.a_lo : t.lo;
    t.hi = r.a_hi > t.hi ? r.a_hi : t.hi;
  }
  if (r.b_lo <= r.b_hi) {
    t.lo = r.b_lo < t.lo ? r.b_lo : t.lo;
    t.hi = r.b_hi > t.hi ? r.b_hi : t.hi;
  }
  // a row with an empty first interval forbids full tiles
  const int flo = r.a_lo <= r.a_hi ? r.a_lo : 0x7fffffff;
  const int fhi = r.a_lo <= r.a_hi ? r.a_hi : -0x7fffffff;
  t.flo = flo > t.flo ? flo : t.flo;
  t.fhi = fhi < t.fhi ? fhi : t.fhi;
}

// 0 = skip, 1 = partial, 2 = full, for key tile [k0, k1].
MVS_HD inline int classify_key_tile(const TilePlan& t, int k0, int k1) {
  if (t.lo > t.hi || k1 < t.lo || k0 > t.hi) return 0;
  if (k0 >= t.flo && k1 <= t.fhi) return 2;
  return 1;
}

}  // namespace mvs
