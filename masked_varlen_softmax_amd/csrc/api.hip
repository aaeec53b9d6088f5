// api.hip - C-ABI entry points that queue device work: argument checks,
// dispatch to the kernels, error mapping. Nothing here allocates.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "common.hpp"
#include "kernels.hpp"

using mvs::fail;

namespace {

constexpr float kLog2e = 1.4426950408889634f;

bool valid_sink_args(int32_t sink_mode, const float* sinks) {
  if (sink_mode != MVS_SINK_NONE && sink_mode != MVS_SINK_KEY0_BIAS && sink_mode != MVS_SINK_NULL_LOGIT) return false;
  return sink_mode == MVS_SINK_NONE || sinks != nullptr;
}

int device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MVS_OK;
  return fail(MVS_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

namespace {

// Argument checks of attn_varlen_fwd (no launch); MVS_OK when valid.
int check_varlen_args(const void* q, const void* k, const void* v, const void* out, int32_t dtype,
                      int64_t q_stride_tok, int64_t k_stride_tok, int64_t v_stride_tok, int64_t o_stride_tok,
                      const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t num_seqs,
                      int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, float softmax_scale, int32_t causal, int32_t window_left,
                      int32_t window_right, const int32_t* q_range_table, const float* sinks, int32_t sink_mode,
                      const float* lse_out) {
  if (dtype != MVS_BF16 && dtype != MVS_F32) return fail(MVS_ERR_INVALID, "unknown dtype %d", dtype);
  if (num_seqs < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return fail(MVS_ERR_INVALID, "negative sizes (num_seqs %d, max_seqlen_q %d, max_seqlen_k %d)", num_seqs,
                max_seqlen_q, max_seqlen_k);
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(MVS_ERR_INVALID, "num_q_heads %d must be a positive multiple of num_kv_heads %d", num_q_heads,
                num_kv_heads);
  const bool bf16 = dtype == MVS_BF16;
  if (bf16 ? !(head_dim == 64 || head_dim == 128 || head_dim == 256 || head_dim == 512)
           : !(head_dim == 64 || head_dim == 128 || head_dim == 256))
    return fail(MVS_ERR_UNSUPPORTED, "head_dim %d is not built for %s", head_dim, bf16 ? "bf16" : "fp32");
  if (!(std::isfinite(softmax_scale) && softmax_scale > 0.f))
    return fail(MVS_ERR_INVALID, "softmax_scale must be finite and > 0");
  if (causal != 0 && causal != 1) return fail(MVS_ERR_INVALID, "causal must be 0 or 1");
  if (window_left < -1 || window_right < -1) return fail(MVS_ERR_INVALID, "windows must be >= -1");
  if (!valid_sink_args(sink_mode, sinks)) return fail(MVS_ERR_INVALID, "bad sink_mode %d or NULL sinks", sink_mode);
  if (num_seqs == 0 || max_seqlen_q == 0) return MVS_OK;  // nothing to compute
  if (!q || !k || !v || !out || !cu_seqlens_q || !cu_seqlens_k)
    return fail(MVS_ERR_INVALID, "NULL tensor or cu_seqlens pointer");
  if (q_stride_tok < (int64_t)num_q_heads * head_dim || o_stride_tok < (int64_t)num_q_heads * head_dim ||
      k_stride_tok < (int64_t)num_kv_heads * head_dim || v_stride_tok < (int64_t)num_kv_heads * head_dim)
    return fail(MVS_ERR_INVALID, "token strides must cover heads * head_dim");
  // K/V tile loads address a tile as 32-bit byte offsets from its first key row
  if (k_stride_tok >= (int64_t(1) << 24) || v_stride_tok >= (int64_t(1) << 24))
    return fail(MVS_ERR_UNSUPPORTED, "k/v token strides must be below 2^24 elements");
  // bf16: every tensor is read and written in 16-byte vectors (8 elements)
  const uintptr_t vec = bf16 ? 16 : 4;
  const int64_t vec_el = bf16 ? 8 : 1;
  if (!mvs::aligned_to(q, vec) || !mvs::aligned_to(k, vec) || !mvs::aligned_to(v, vec) ||
      !mvs::aligned_to(out, vec) || q_stride_tok % vec_el || k_stride_tok % vec_el || v_stride_tok % vec_el ||
      o_stride_tok % vec_el)
    return fail(MVS_ERR_INVALID, "tensors must be %d-byte aligned with strides in multiples of %lld elements",
                (int)vec, (long long)vec_el);
  if (!mvs::aligned_to(cu_seqlens_q, 4) || !mvs::aligned_to(cu_seqlens_k, 4) ||
      (q_range_table && !mvs::aligned_to(q_range_table, 8)) || (lse_out && !mvs::aligned_to(lse_out, 4)))
    return fail(MVS_ERR_INVALID, "misaligned int32 or fp32 buffer");
  return MVS_OK;
}

// Grids the kernels cannot be launched with: a valid call whose sizes exceed
// them is reported as unsupported before anything is queued.
int check_prefill_grid(int32_t dtype, int32_t head_dim, int32_t num_q_heads, int32_t num_kv_heads, int32_t num_seqs,
                       int32_t max_seqlen_q, bool scan) {
  if (dtype == MVS_F32) {
    if (num_q_heads > mvs::kMaxGridYZ || num_seqs > mvs::kMaxGridYZ)
      return fail(MVS_ERR_UNSUPPORTED, "fp32 prefill launches at most %d heads and %d sequences", mvs::kMaxGridYZ,
                  mvs::kMaxGridYZ);
    return MVS_OK;
  }
  const long long blocks =
      mvs::prefill_bf16_grid(head_dim, num_q_heads / num_kv_heads, num_q_heads, num_seqs, max_seqlen_q, scan);
  if (blocks < 0) return fail(MVS_ERR_UNSUPPORTED, "head_dim %d is not built for bf16", head_dim);
  if (blocks > mvs::kMaxGridBlocks)
    return fail(MVS_ERR_UNSUPPORTED, "the launch needs %lld workgroups, more than one grid holds (%lld)", blocks,
                mvs::kMaxGridBlocks);
  return MVS_OK;
}

mvs::PrefillArgs varlen_args(const void* q, const void* k, const void* v, void* out, int64_t q_stride_tok,
                             int64_t k_stride_tok, int64_t v_stride_tok, int64_t o_stride_tok,
                             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t num_seqs,
                             int32_t num_q_heads, int32_t num_kv_heads, float softmax_scale, int32_t causal,
                             int32_t window_left, int32_t window_right, const int32_t* q_range_table,
                             const float* sinks, int32_t sink_mode, float* lse_out) {
  mvs::PrefillArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = out;
  a.q_st = q_stride_tok;
  a.k_st = k_stride_tok;
  a.v_st = v_stride_tok;
  a.o_st = o_stride_tok;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.num_seqs = num_seqs;
  a.Hq = num_q_heads;
  a.Hkv = num_kv_heads;
  a.group = num_q_heads / num_kv_heads;
  a.scale = softmax_scale;
  a.scale_log2 = softmax_scale * kLog2e;
  a.causal = causal;
  a.wl = window_left;
  a.wr = window_right;
  a.table = q_range_table;
  a.sinks = sinks;
  a.sink_mode = sink_mode;
  a.lse = lse_out;
  return a;
}

}  // namespace

extern "C" int attn_varlen_fwd(const void* q, const void* k, const void* v, void* out, int32_t dtype,
                               int64_t q_stride_tok, int64_t k_stride_tok, int64_t v_stride_tok,
                               int64_t o_stride_tok, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, float softmax_scale, int32_t causal,
                               int32_t window_left, int32_t window_right, const int32_t* q_range_table,
                               const float* sinks, int32_t sink_mode, float* lse_out, void* hip_stream) {
  mvs::clear_error();
  const int rc = check_varlen_args(q, k, v, out, dtype, q_stride_tok, k_stride_tok, v_stride_tok, o_stride_tok,
                                   cu_seqlens_q, cu_seqlens_k, num_seqs, max_seqlen_q, max_seqlen_k, num_q_heads,
                                   num_kv_heads, head_dim, softmax_scale, causal, window_left, window_right,
                                   q_range_table, sinks, sink_mode, lse_out);
  if (rc != MVS_OK || num_seqs == 0 || max_seqlen_q == 0) return rc;
  const int grc = check_prefill_grid(dtype, head_dim, num_q_heads, num_kv_heads, num_seqs, max_seqlen_q, false);
  if (grc != MVS_OK) return grc;
  const mvs::PrefillArgs a = varlen_args(q, k, v, out, q_stride_tok, k_stride_tok, v_stride_tok, o_stride_tok,
                                         cu_seqlens_q, cu_seqlens_k, num_seqs, num_q_heads, num_kv_heads,
                                         softmax_scale, causal, window_left, window_right, q_range_table, sinks,
                                         sink_mode, lse_out);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const hipError_t e = dtype == MVS_BF16 ? mvs::launch_prefill_bf16(a, head_dim, max_seqlen_q, stream)
                                         : mvs::launch_prefill_f32(a, head_dim, max_seqlen_q, stream);
  return device_status(e, "attn_varlen_fwd launch");
}

extern "C" int attn_varlen_fwd_range_scan(const void* q, const void* k, const void* v, void* out, int32_t dtype,
                                          int64_t q_stride_tok, int64_t k_stride_tok, int64_t v_stride_tok,
                                          int64_t o_stride_tok, const int32_t* cu_seqlens_q,
                                          const int32_t* cu_seqlens_k, int32_t num_seqs, int32_t max_seqlen_q,
                                          int32_t max_seqlen_k, int32_t num_q_heads, int32_t num_kv_heads,
                                          int32_t head_dim, float softmax_scale, int32_t causal, int32_t window_left,
                                          int32_t window_right, const int32_t* ranges, int32_t max_ranges,
                                          const float* sinks, int32_t sink_mode, float* lse_out, void* hip_stream) {
  mvs::clear_error();
  if (dtype != MVS_BF16) {
    if (dtype == MVS_F32) return fail(MVS_ERR_UNSUPPORTED, "the range-scan baseline is built for bf16 only");
    return fail(MVS_ERR_INVALID, "unknown dtype %d", dtype);
  }
  if (!(head_dim == 64 || head_dim == 128 || head_dim == 256))
    return fail(MVS_ERR_UNSUPPORTED, "head_dim %d is not built for the range-scan baseline", head_dim);
  if (max_ranges < 0 || max_ranges > mvs::kMaxScanRanges)
    return fail(MVS_ERR_UNSUPPORTED, "max_ranges %d outside [0, %d]", max_ranges, mvs::kMaxScanRanges);
  if (max_ranges > 0 && num_seqs > 0 && max_seqlen_q > 0 && (!ranges || !mvs::aligned_to(ranges, 8)))
    return fail(MVS_ERR_INVALID, "ranges must be a non-NULL 8-byte aligned device array");
  // Everything else is validated as for attn_varlen_fwd; with no ranges the
  // call is attn_varlen_fwd without a table.
  if (max_ranges == 0)
    return attn_varlen_fwd(q, k, v, out, dtype, q_stride_tok, k_stride_tok, v_stride_tok, o_stride_tok, cu_seqlens_q,
                           cu_seqlens_k, num_seqs, max_seqlen_q, max_seqlen_k, num_q_heads, num_kv_heads, head_dim,
                           softmax_scale, causal, window_left, window_right, nullptr, sinks, sink_mode, lse_out,
                           hip_stream);
  const int rc = check_varlen_args(q, k, v, out, dtype, q_stride_tok, k_stride_tok, v_stride_tok, o_stride_tok,
                                   cu_seqlens_q, cu_seqlens_k, num_seqs, max_seqlen_q, max_seqlen_k, num_q_heads,
                                   num_kv_heads, head_dim, softmax_scale, causal, window_left, window_right, nullptr,
                                   sinks, sink_mode, lse_out);
  if (rc != MVS_OK || num_seqs == 0 || max_seqlen_q == 0) return rc;
  const int grc = check_prefill_grid(dtype, head_dim, num_q_heads, num_kv_heads, num_seqs, max_seqlen_q, true);
  if (grc != MVS_OK) return grc;
  mvs::PrefillArgs a = varlen_args(q, k, v, out, q_stride_tok, k_stride_tok, v_stride_tok, o_stride_tok, cu_seqlens_q,
                                   cu_seqlens_k, num_seqs, num_q_heads, num_kv_heads, softmax_scale, causal,
                                   window_left, window_right, nullptr, sinks, sink_mode, lse_out);
  a.scan_ranges = ranges;
  a.max_ranges = max_ranges;
  return device_status(mvs::launch_prefill_bf16(a, head_dim, max_seqlen_q, static_cast<hipStream_t>(hip_stream)),
                       "attn_varlen_fwd_range_scan launch");
}

extern "C" int attn_varlen_fwd_paged(const void* q, const void* k_cache, const void* v_cache, void* out,
                                     int32_t dtype, int64_t q_stride_tok, int64_t o_stride_tok, int64_t blk_stride,
                                     int64_t head_stride, int64_t tok_stride, int32_t num_blocks,
                                     const int32_t* block_table, int32_t max_blocks_per_seq, int32_t page_size,
                                     const int32_t* cu_seqlens_q, const int32_t* seq_lens_k, int32_t num_seqs,
                                     int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim, float softmax_scale, int32_t causal,
                                     int32_t window_left, int32_t window_right, const int32_t* q_range_table,
                                     const float* sinks, int32_t sink_mode, float* lse_out, void* hip_stream) {
  mvs::clear_error();
  if (dtype != MVS_BF16) {
    if (dtype == MVS_F32) return fail(MVS_ERR_UNSUPPORTED, "paged prefill is built for bf16 caches only");
    return fail(MVS_ERR_INVALID, "unknown dtype %d", dtype);
  }
  if (num_seqs < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || num_blocks < 0 || max_blocks_per_seq < 0)
    return fail(MVS_ERR_INVALID, "negative sizes");
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(MVS_ERR_INVALID, "num_q_heads %d must be a positive multiple of num_kv_heads %d", num_q_heads,
                num_kv_heads);
  if (!(head_dim == 64 || head_dim == 128 || head_dim == 256 || head_dim == 512))
    return fail(MVS_ERR_UNSUPPORTED, "head_dim %d is not built for bf16", head_dim);
  if (page_size < 16 || (page_size & (page_size - 1)) != 0)
    return fail(MVS_ERR_UNSUPPORTED, "page_size %d is not a power of two >= 16", page_size);
  if (!(std::isfinite(softmax_scale) && softmax_scale > 0.f))
    return fail(MVS_ERR_INVALID, "softmax_scale must be finite and > 0");
  if (causal != 0 && causal != 1) return fail(MVS_ERR_INVALID, "causal must be 0 or 1");
  if (window_left < -1 || window_right < -1) return fail(MVS_ERR_INVALID, "windows must be >= -1");
  if (!valid_sink_args(sink_mode, sinks)) return fail(MVS_ERR_INVALID, "bad sink_mode %d or NULL sinks", sink_mode);
  if (num_seqs == 0 || max_seqlen_q == 0) return MVS_OK;
  if (!q || !k_cache || !v_cache || !out || !cu_seqlens_q || !seq_lens_k || !block_table)
    return fail(MVS_ERR_INVALID, "NULL tensor, cu_seqlens_q, seq_lens_k or block_table pointer");
  if (num_blocks == 0) return fail(MVS_ERR_INVALID, "empty cache");
  if (max_blocks_per_seq < (int64_t(max_seqlen_k) + page_size - 1) / page_size)
    return fail(MVS_ERR_INVALID, "block table too narrow for max_seqlen_k");
  if (q_stride_tok < (int64_t)num_q_heads * head_dim || o_stride_tok < (int64_t)num_q_heads * head_dim)
    return fail(MVS_ERR_INVALID, "token strides must cover heads * head_dim");
  if (tok_stride < head_dim || head_stride < 0 || blk_stride < 0) return fail(MVS_ERR_INVALID, "bad cache strides");
  if (tok_stride >= (int64_t(1) << 24))
    return fail(MVS_ERR_UNSUPPORTED, "cache token stride must be below 2^24 elements");
  if (!mvs::aligned_to(q, 16) || !mvs::aligned_to(k_cache, 16) || !mvs::aligned_to(v_cache, 16) ||
      !mvs::aligned_to(out, 16) || q_stride_tok % 8 || o_stride_tok % 8 || tok_stride % 8 || head_stride % 8 ||
      blk_stride % 8)
    return fail(MVS_ERR_INVALID, "q, out and caches must be 16-byte aligned with strides in multiples of 8 elements");
  if (!mvs::aligned_to(cu_seqlens_q, 4) || !mvs::aligned_to(seq_lens_k, 4) || !mvs::aligned_to(block_table, 4) ||
      (q_range_table && !mvs::aligned_to(q_range_table, 8)) || (lse_out && !mvs::aligned_to(lse_out, 4)))
    return fail(MVS_ERR_INVALID, "misaligned int32 or fp32 buffer");
  const int grc = check_prefill_grid(dtype, head_dim, num_q_heads, num_kv_heads, num_seqs, max_seqlen_q, false);
  if (grc != MVS_OK) return grc;

  mvs::PrefillArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.o = out;
  a.q_st = q_stride_tok;
  a.k_st = tok_stride;
  a.v_st = tok_stride;
  a.o_st = o_stride_tok;
  a.cu_q = cu_seqlens_q;
  a.cu_k = nullptr;
  a.num_seqs = num_seqs;
  a.Hq = num_q_heads;
  a.Hkv = num_kv_heads;
  a.group = num_q_heads / num_kv_heads;
  a.scale = softmax_scale;
  a.scale_log2 = softmax_scale * kLog2e;
  a.causal = causal;
  a.wl = window_left;
  a.wr = window_right;
  a.table = q_range_table;
  a.sinks = sinks;
  a.sink_mode = sink_mode;
  a.lse = lse_out;
  a.block_table = block_table;
  a.seq_lens_k = seq_lens_k;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  int lg = 0;
  while ((1 << lg) < page_size) ++lg;
  a.page_log2 = lg;
  a.blk_st = blk_stride;
  a.head_st = head_stride;
  return device_status(mvs::launch_prefill_bf16(a, head_dim, max_seqlen_q, static_cast<hipStream_t>(hip_stream)),
                       "attn_varlen_fwd_paged launch");
}

namespace {

bool decode_sizes_ok(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim) {
  return num_seqs >= 0 && num_q_heads > 0 && num_kv_heads > 0 && num_q_heads % num_kv_heads == 0 &&
         (head_dim == 64 || head_dim == 128 || head_dim == 256);
}

struct DecodeLayout {
  size_t o_bytes, ml_bytes, cum_bytes, total;
};

// Workspace: partial O and (max, sum) per slot and query head of the group,
// kDecodeMaxWaves + B * Hkv slots, then the per-sequence offsets.
DecodeLayout decode_layout(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim) {
  DecodeLayout d;
  const size_t slots = (size_t)mvs::kDecodeMaxWaves + (size_t)num_seqs * num_kv_heads;
  const size_t rows = slots * (size_t)(num_q_heads / num_kv_heads);
  d.o_bytes = (rows * head_dim * sizeof(float) + 255) / 256 * 256;
  d.ml_bytes = (rows * 2 * sizeof(float) + 255) / 256 * 256;
  d.cum_bytes = (((size_t)num_seqs + 1) * sizeof(long long) + 255) / 256 * 256;
  d.total = d.o_bytes + d.ml_bytes + d.cum_bytes;
  return d;
}

}  // namespace

extern "C" size_t attn_paged_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                                   int32_t head_dim) {
  if (!decode_sizes_ok(num_seqs, num_q_heads, num_kv_heads, head_dim)) return 0;
  return decode_layout(num_seqs, num_q_heads, num_kv_heads, head_dim).total;
}

namespace {

// attn_paged_decode with the workspace either the caller's (`workspace`,
// `workspace_bytes`) or, with `library_scratch`, the library-held per-device
// buffer of decode.hip.
int paged_decode(const void* q, void* out, const void* k_cache, const void* v_cache, int32_t dtype,
                 int64_t blk_stride, int64_t head_stride, int64_t tok_stride, int32_t num_blocks,
                 const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                 int32_t max_seq_len, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                 float softmax_scale, int32_t window_left, const float* sinks, int32_t sink_mode, float* lse_out,
                 void* workspace, size_t workspace_bytes, bool library_scratch, void* hip_stream) {
  mvs::clear_error();
  if (dtype != MVS_BF16) {
    if (dtype == MVS_F32) return fail(MVS_ERR_UNSUPPORTED, "paged decode is built for bf16 caches only");
    return fail(MVS_ERR_INVALID, "unknown dtype %d", dtype);
  }
  if (num_seqs < 0 || max_seq_len < 0 || num_blocks < 0 || max_blocks_per_seq < 0)
    return fail(MVS_ERR_INVALID, "negative sizes");
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(MVS_ERR_INVALID, "num_q_heads %d must be a positive multiple of num_kv_heads %d", num_q_heads,
                num_kv_heads);
  const int group = num_q_heads / num_kv_heads;
  if (!(group == 1 || group == 2 || group == 4 || group == 8 || group == 16))
    return fail(MVS_ERR_UNSUPPORTED, "query heads per kv head (%d) must be 1, 2, 4, 8 or 16", group);
  if (!(head_dim == 64 || head_dim == 128 || head_dim == 256))
    return fail(MVS_ERR_UNSUPPORTED, "head_dim %d is not built for paged decode", head_dim);
  if (page_size <= 0 || page_size % 16 != 0) return fail(MVS_ERR_UNSUPPORTED, "page_size %d is not a multiple of 16", page_size);
  if (!(std::isfinite(softmax_scale) && softmax_scale > 0.f))
    return fail(MVS_ERR_INVALID, "softmax_scale must be finite and > 0");
  if (window_left < -1) return fail(MVS_ERR_INVALID, "window_left must be >= -1");
  if (!valid_sink_args(sink_mode, sinks)) return fail(MVS_ERR_INVALID, "bad sink_mode %d or NULL sinks", sink_mode);
  if (num_seqs == 0) return MVS_OK;
  if (num_seqs > mvs::kMaxGridYZ)
    return fail(MVS_ERR_UNSUPPORTED, "paged decode launches at most %d sequences per call", mvs::kMaxGridYZ);
  if (max_blocks_per_seq < (max_seq_len + page_size - 1) / page_size)
    return fail(MVS_ERR_INVALID, "max_blocks_per_seq %d cannot hold max_seq_len %d", max_blocks_per_seq,
                max_seq_len);
  if (!q || !out || !k_cache || !v_cache || !block_table || !seq_lens || (!library_scratch && !workspace))
    return fail(MVS_ERR_INVALID, "NULL pointer argument");
  if (blk_stride < 0 || head_stride < 0 || tok_stride < head_dim)
    return fail(MVS_ERR_INVALID, "bad cache strides");
  const size_t dim_span = (size_t)head_dim;
  if ((size_t)head_stride < dim_span && num_kv_heads > 1 && head_stride != 0)
    return fail(MVS_ERR_INVALID, "head_stride smaller than head_dim");
  if (!mvs::aligned_to(q, 16) || !mvs::aligned_to(k_cache, 16) || !mvs::aligned_to(v_cache, 16) ||
      !mvs::aligned_to(out, 4) || blk_stride % 8 || head_stride % 8 || tok_stride % 8)
    return fail(MVS_ERR_INVALID, "q and caches must be 16-byte aligned with strides in multiples of 8 elements");
  const DecodeLayout d = decode_layout(num_seqs, num_q_heads, num_kv_heads, head_dim);
  if (library_scratch) {
    if (d.total > mvs::kDecodeScratchBytes)
      return fail(MVS_ERR_CAPACITY, "these sizes need %zu bytes of workspace; the library holds %zu per device",
                  d.total, mvs::kDecodeScratchBytes);
    const hipError_t e = mvs::decode_scratch(&workspace);
    if (e != hipSuccess) return device_status(e, "library workspace lookup");
    workspace_bytes = mvs::kDecodeScratchBytes;
  } else {
    if (!mvs::aligned_to(workspace, 256)) return fail(MVS_ERR_INVALID, "workspace must be 256-byte aligned");
    if (workspace_bytes < d.total)
      return fail(MVS_ERR_CAPACITY, "workspace holds %zu bytes, needs %zu", workspace_bytes, d.total);
  }

  mvs::DecodeArgs a{};
  a.q = q;
  a.o = out;
  a.kc = k_cache;
  a.vc = v_cache;
  a.blk_st = blk_stride;
  a.head_st = head_stride;
  a.tok_st = tok_stride;
  a.num_blocks = num_blocks;
  a.block_table = block_table;
  a.max_blocks = max_blocks_per_seq;
  a.seq_lens = seq_lens;
  a.num_seqs = num_seqs;
  a.Hq = num_q_heads;
  a.Hkv = num_kv_heads;
  a.group = group;
  a.page_size = page_size;
  a.scale = softmax_scale;
  a.scale_log2 = softmax_scale * kLog2e;
  a.wl = window_left;
  a.sinks = sinks;
  a.sink_mode = sink_mode;
  a.lse = lse_out;
  a.max_seq_len = max_seq_len;
  const long long span = window_left >= 0 ? std::min<long long>(max_seq_len, (long long)window_left + 1) : max_seq_len;
  a.max_pairs = (long long)num_seqs * num_kv_heads * span;
  char* ws = static_cast<char*>(workspace);
  a.ws_o = reinterpret_cast<float*>(ws);
  a.ws_ml = reinterpret_cast<float*>(ws + d.o_bytes);
  a.ws_cum = reinterpret_cast<long long*>(ws + d.o_bytes + d.ml_bytes);
  return device_status(mvs::launch_decode_bf16(a, head_dim, static_cast<hipStream_t>(hip_stream)),
                       "attn_paged_decode launch");
}

}  // namespace

extern "C" int attn_paged_decode(const void* q, void* out, const void* k_cache, const void* v_cache, int32_t dtype,
                                 int64_t blk_stride, int64_t head_stride, int64_t tok_stride, int32_t num_blocks,
                                 const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                 int32_t num_seqs, int32_t max_seq_len, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t page_size, float softmax_scale, int32_t window_left,
                                 const float* sinks, int32_t sink_mode, float* lse_out, void* workspace,
                                 size_t workspace_bytes, void* hip_stream) {
  return paged_decode(q, out, k_cache, v_cache, dtype, blk_stride, head_stride, tok_stride, num_blocks, block_table,
                      max_blocks_per_seq, seq_lens, num_seqs, max_seq_len, num_q_heads, num_kv_heads, head_dim,
                      page_size, softmax_scale, window_left, sinks, sink_mode, lse_out, workspace, workspace_bytes,
                      false, hip_stream);
}

extern "C" int attn_paged_decode_noalloc(const void* q, void* out, const void* k_cache, const void* v_cache,
                                         int32_t dtype, int64_t blk_stride, int64_t head_stride, int64_t tok_stride,
                                         int32_t num_blocks, const int32_t* block_table, int32_t max_blocks_per_seq,
                                         const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                         int32_t page_size, float softmax_scale, int32_t window_left,
                                         const float* sinks, int32_t sink_mode, float* lse_out, void* hip_stream) {
  return paged_decode(q, out, k_cache, v_cache, dtype, blk_stride, head_stride, tok_stride, num_blocks, block_table,
                      max_blocks_per_seq, seq_lens, num_seqs, max_seq_len, num_q_heads, num_kv_heads, head_dim,
                      page_size, softmax_scale, window_left, sinks, sink_mode, lse_out, nullptr, 0, true, hip_stream);
}
