// host.cpp - host-only entry points of libmvs: the range-table builder, the
// tile-plan diagnostic and the thread-local error message.

#include <cstdarg>
#include <cstdio>

#include "common.hpp"
#include "mask.hpp"

namespace mvs {

static thread_local char g_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof(g_error), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_error[0] = '\0'; }

}  // namespace mvs

using mvs::fail;

extern "C" const char* mvs_last_error(void) { return mvs::g_error; }

// The table of vLLM PR #50294 ("implementation breakdown" step 1): every
// scheduled row gets the inclusive (start, end) of the valid range of its
// request that contains the row's absolute position, else (-1, -1).
//
// Derived per row: row i of request b (position p = ctx + i, ctx = seq_len -
// Lq) belongs to the range that covers p; a valid range (start < end) covers
// the local rows [max(start - ctx, 0), min(end - ctx, Lq - 1)]. If ranges
// overlap (outside the contract) the one listed last owns the row. The rows
// of a request are emitted front to back in runs of equal owner, each row
// written once: a run ends where its owner's span ends or where a range
// listed after the owner begins. Finding a run's owner and end scans the
// request's ranges, so a request with R ranges costs O(Lq + R^2) (R is a
// few dozen frames in the pages' workloads). A first pass only decides
// whether any row is covered, so a batch with no covered row returns 0
// without touching the buffer. Nothing is allocated.
extern "C" int64_t build_query_range_table(int32_t* out_table, int64_t capacity_rows,
                                           const int32_t* query_start_loc, const int32_t* seq_lens,
                                           int32_t num_reqs, const int32_t* range_offsets, const int32_t* ranges) {
  mvs::clear_error();
  if (num_reqs < 0) return fail(MVS_ERR_INVALID, "num_reqs %d < 0", num_reqs);
  if (!query_start_loc) return fail(MVS_ERR_INVALID, "query_start_loc is NULL");
  if (num_reqs > 0 && !seq_lens) return fail(MVS_ERR_INVALID, "seq_lens is NULL");
  if (query_start_loc[0] < 0) return fail(MVS_ERR_INVALID, "query_start_loc[0] = %d < 0", query_start_loc[0]);
  for (int32_t b = 0; b < num_reqs; ++b)
    if (query_start_loc[b + 1] < query_start_loc[b])
      return fail(MVS_ERR_INVALID, "query_start_loc decreases at request %d", b);
  if (!range_offsets) return 0;  // no ranges at all
  if (range_offsets[0] < 0) return fail(MVS_ERR_INVALID, "range_offsets[0] = %d < 0", range_offsets[0]);
  for (int32_t b = 0; b < num_reqs; ++b)
    if (range_offsets[b + 1] < range_offsets[b])
      return fail(MVS_ERR_INVALID, "range_offsets decreases at request %d", b);
  if (num_reqs > 0 && range_offsets[num_reqs] > range_offsets[0] && !ranges)
    return fail(MVS_ERR_INVALID, "ranges is NULL but range_offsets lists %d ranges",
                range_offsets[num_reqs] - range_offsets[0]);

  const int64_t n_rows = query_start_loc[num_reqs];
  if (n_rows <= 0) return 0;
  if (n_rows > capacity_rows)
    return fail(MVS_ERR_CAPACITY, "table holds %lld rows, batch schedules %lld", (long long)capacity_rows,
                (long long)n_rows);

  // Local rows [*lo, *hi] of request b that range r covers; false when none.
  auto local_span = [&](int32_t b, int32_t r, int64_t* lo, int64_t* hi) -> bool {
    const int64_t s = ranges[2 * (int64_t)r], e = ranges[2 * (int64_t)r + 1];
    if (s >= e) return false;  // degenerate
    const int64_t q_len = (int64_t)query_start_loc[b + 1] - query_start_loc[b];
    const int64_t ctx = (int64_t)seq_lens[b] - q_len;
    *lo = s - ctx > 0 ? s - ctx : 0;
    *hi = e - ctx < q_len - 1 ? e - ctx : q_len - 1;
    return *lo <= *hi;
  };

  bool covered = false;
  for (int32_t b = 0; b < num_reqs && !covered; ++b)
    for (int32_t r = range_offsets[b]; r < range_offsets[b + 1] && !covered; ++r) {
      int64_t lo, hi;
      covered = query_start_loc[b + 1] > query_start_loc[b] && local_span(b, r, &lo, &hi);
    }
  if (!covered) return 0;
  if (!out_table) return fail(MVS_ERR_INVALID, "out_table is NULL");

  auto emit = [&](int64_t row0, int64_t i0, int64_t i1, int32_t s, int32_t e) {
    for (int64_t t = row0 + i0; t < row0 + i1; ++t) {
      out_table[2 * t] = s;
      out_table[2 * t + 1] = e;
    }
  };
  emit(0, 0, query_start_loc[0], -1, -1);  // rows before the first request belong to none
  for (int32_t b = 0; b < num_reqs; ++b) {
    const int64_t row0 = query_start_loc[b];
    const int64_t q_len = (int64_t)query_start_loc[b + 1] - row0;
    const int32_t r0 = range_offsets[b], r1 = range_offsets[b + 1];
    int64_t i = 0;
    while (i < q_len) {
      int32_t owner = -1;  // last-listed range covering row i
      int64_t owner_hi = 0, next_lo = q_len;  // next_lo: first start of a span after row i
      for (int32_t r = r0; r < r1; ++r) {
        int64_t lo, hi;
        if (!local_span(b, r, &lo, &hi)) continue;
        if (lo <= i && i <= hi) {
          owner = r;
          owner_hi = hi;
        }
        if (lo > i && lo < next_lo) next_lo = lo;
      }
      if (owner < 0) {  // uncovered up to the next span's first row
        emit(row0, i, next_lo, -1, -1);
        i = next_lo;
        continue;
      }
      int64_t end = owner_hi + 1;  // a range listed after the owner takes over where it begins
      for (int32_t r = owner + 1; r < r1; ++r) {
        int64_t lo, hi;
        if (local_span(b, r, &lo, &hi) && lo > i && lo < end) end = lo;
      }
      emit(row0, i, end, ranges[2 * (int64_t)owner], ranges[2 * (int64_t)owner + 1]);
      i = end;
    }
  }
  return n_rows;
}

extern "C" int mvs_plan_key_tiles(int32_t Lq, int32_t Lk, int32_t row0, int32_t rows, int32_t causal,
                                  int32_t window_left, int32_t window_right, const int32_t* table_rows,
                                  int32_t key_tile, int8_t* tile_class, int32_t num_key_tiles) {
  mvs::clear_error();
  if (Lq < 0 || Lk < 0 || row0 < 0 || rows <= 0 || key_tile <= 0 || num_key_tiles < 0 || !tile_class)
    return fail(MVS_ERR_INVALID, "bad tile-plan arguments");
  if (window_left < -1 || window_right < -1) return fail(MVS_ERR_INVALID, "windows must be >= -1");
  mvs::TilePlan plan = mvs::plan_identity();
  const int c = Lk - Lq;
  for (int32_t r = 0; r < rows; ++r) {
    const int i = row0 + r;
    if (i >= Lq) break;
    const int ts = table_rows ? table_rows[2 * r] : -1;
    const int te = table_rows ? table_rows[2 * r + 1] : -1;
    plan_add_row(plan, mvs::row_keys(causal, window_left, window_right, c + i, Lk, ts, te));
  }
  for (int32_t j = 0; j < num_key_tiles; ++j) {
    const long long k0 = (long long)j * key_tile, k1 = k0 + key_tile - 1;
    tile_class[j] = (int8_t)mvs::classify_key_tile(plan, (int)k0, (int)(k1 > 0x7fffffff ? 0x7fffffff : k1));
  }
  return MVS_OK;
}

// Useful-work accounting (vLLM PR #55624 report: a sliding-window layer's
// attention FLOPs and KV reads count only the keys inside its window). A
// visible (query, key) pair costs 4 * head_dim FLOPs per query head (2D for
// the score, 2D for the value accumulation); each row's visible keys are the
// two disjoint intervals of row_keys, so the count is exact for any table.
extern "C" int64_t mvs_prefill_useful_flops(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                            int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                            int32_t causal, int32_t window_left, int32_t window_right,
                                            const int32_t* q_range_table) {
  mvs::clear_error();
  if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0) return fail(MVS_ERR_INVALID, "bad sizes");
  if (causal != 0 && causal != 1) return fail(MVS_ERR_INVALID, "causal must be 0 or 1");
  if (window_left < -1 || window_right < -1) return fail(MVS_ERR_INVALID, "windows must be >= -1");
  if (num_seqs == 0) return 0;
  if (!cu_seqlens_q || !cu_seqlens_k) return fail(MVS_ERR_INVALID, "NULL cu_seqlens");
  int64_t pairs = 0;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int32_t q0 = cu_seqlens_q[b], Lq = cu_seqlens_q[b + 1] - q0;
    const int32_t Lk = cu_seqlens_k[b + 1] - cu_seqlens_k[b];
    if (Lq < 0 || Lk < 0) return fail(MVS_ERR_INVALID, "cu_seqlens decrease at sequence %d", b);
    for (int32_t i = 0; i < Lq; ++i) {
      const int64_t t = (int64_t)q0 + i;
      const int ts = q_range_table ? q_range_table[2 * t] : -1;
      const int te = q_range_table ? q_range_table[2 * t + 1] : -1;
      const mvs::RowKeys r = mvs::row_keys(causal, window_left, window_right, Lk - Lq + i, Lk, ts, te);
      if (r.a_hi >= r.a_lo) pairs += (int64_t)r.a_hi - r.a_lo + 1;
      if (r.b_hi >= r.b_lo) pairs += (int64_t)r.b_hi - r.b_lo + 1;
    }
  }
  return pairs * 4 * head_dim * num_q_heads;
}

// K and V bytes of the keys each decode query sees: min(L, W) per sequence and
// kv head for a window of W = window_left + 1 keys, L for full attention.
extern "C" int64_t mvs_decode_useful_bytes(const int32_t* seq_lens, int32_t num_seqs, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t elem_bytes, int32_t window_left) {
  mvs::clear_error();
  if (num_seqs < 0 || num_kv_heads <= 0 || head_dim <= 0 || elem_bytes <= 0) return fail(MVS_ERR_INVALID, "bad sizes");
  if (window_left < -1) return fail(MVS_ERR_INVALID, "window_left must be >= -1");
  if (num_seqs == 0) return 0;
  if (!seq_lens) return fail(MVS_ERR_INVALID, "NULL seq_lens");
  int64_t tokens = 0;
  for (int32_t b = 0; b < num_seqs; ++b) {
    if (seq_lens[b] < 0) return fail(MVS_ERR_INVALID, "seq_lens[%d] < 0", b);
    const int64_t L = seq_lens[b];
    tokens += window_left >= 0 && L > (int64_t)window_left + 1 ? (int64_t)window_left + 1 : L;
  }
  return tokens * num_kv_heads * head_dim * 2 * elem_bytes;
}
