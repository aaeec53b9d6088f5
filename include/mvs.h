/*
 * mvs.h - C ABI of libmvs.so: masked softmax attention over packed
 * variable-length sequences, for AMD Instinct MI355X (gfx950).
 *
 * The library computes softmax(scale * Q K^T + bias, masked) V with one mask
 * predicate shared by prefill and decode. For request b with Lq_b queries and
 * Lk_b keys, query i sits at absolute position p = (Lk_b - Lq_b) + i (the
 * context offset of chunked prefill), and with d = p - k:
 *
 *   base(p, k) = 0 <= k < Lk_b
 *                and (!causal or d >= 0)
 *                and (window_left  < 0 or  d <= window_left)
 *                and (window_right < 0 or -d <= window_right)
 *   mm(t, k)   = table present and T[t].start <= k <= T[t].end
 *                and (window_left < 0 or d <= window_left)
 *   visible    = base or mm,     t = cu_seqlens_q[b] + i (packed row)
 *
 * Sources (web pages restated here, not code):
 *   - vLLM PR #50294 (prhub.com.cn), "FA4 mm_prefix range scan -> O(1)
 *     lookup": the per-query-row range table, its builder, and the mask_mod
 *     (sections "implementation breakdown" and "key code snippets").
 *   - vLLM PR #49815 (prhub.com.cn), "MiMo window attention sinks": the
 *     two-sided window, the per-head sink added to key 0's logit, and the
 *     null-logit sink it is contrasted with ("implementation breakdown",
 *     "key code snippets").
 *   - vLLM PR #55624 report (prhub.com.cn): sliding windows clamp both the
 *     attention FLOPs and the decode KV-cache reads ("implementation
 *     breakdown" steps 2 and 4).
 *   - mini-vllm tutorial step14_4: causal masking with an offset, and decode
 *     (one query) needing no mask.
 *
 * Conventions for every entry point:
 *   - Ownership: every buffer belongs to the caller. The library allocates
 *     nothing and keeps no state between calls apart from a per-device cache
 *     of the decode kernel's occupancy (filled on first use, safe to fill
 *     from several threads); it is safe to call from several host threads. Device buffers must stay valid until the work queued on
 *     the given stream has finished.
 *   - Streams: device work is queued asynchronously on the HIP stream passed
 *     as `hip_stream` (NULL = the default stream). No call synchronises.
 *   - Errors: a non-zero status is returned and a message is stored in a
 *     thread-local buffer readable with mvs_last_error(). Arguments are
 *     checked before anything is queued; a rejected call queues nothing.
 *     MVS_ERR_DEVICE reports a launch failure seen by hipGetLastError.
 *   - Strides are counted in elements, not bytes. Within a token, heads and
 *     head dimensions are contiguous (head stride = head_dim).
 */
#ifndef MVS_H
#define MVS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MVS_API __attribute__((visibility("default")))

/* ---- status codes ---- */
#define MVS_OK 0
#define MVS_ERR_INVALID (-1)     /* bad pointer, size, stride or flag            */
#define MVS_ERR_UNSUPPORTED (-2) /* valid but not built: dtype, head_dim, group  */
#define MVS_ERR_CAPACITY (-3)    /* table buffer or workspace too small          */
#define MVS_ERR_DEVICE (-4)      /* the HIP runtime reported an error            */

/* ---- element types ---- */
#define MVS_BF16 0
#define MVS_F32 1

/* ---- sink modes (vLLM PR #49815, "key code snippets", the kernel's sink branch) ---- */
#define MVS_SINK_NONE 0       /* no sink                                                */
#define MVS_SINK_KEY0_BIAS 1  /* sink[h] is added to the logit of key 0 where visible   */
#define MVS_SINK_NULL_LOGIT 2 /* exp(sink[h]) joins the denominator only (GPT-OSS)      */

/*
 * build_query_range_table - per-query-row multimodal-prefix range table.
 *
 * vLLM PR #50294, "implementation breakdown" step 1 and the builder under
 * "key code snippets". Host function; touches no GPU.
 *
 * Row t = query_start_loc[b] + i of the table receives the inclusive (start,
 * end) of the request's valid range that contains the row's position
 * p = (seq_lens[b] - Lq_b) + i, or (-1, -1) if none does. The stored pair is
 * the unclipped range; only rows of the scheduled chunk are written.
 *
 *   out_table       host int32 [capacity_rows][2], caller-owned.
 *   capacity_rows   rows available in out_table.
 *   query_start_loc host int32 [num_reqs + 1], prefix sums of query counts.
 *   seq_lens        host int32 [num_reqs], key counts (context + chunk). Any
 *                   upper bound is allowed for decode rows: they stay outside
 *                   every range (PR #50294, step 3).
 *   range_offsets   host int32 [num_reqs + 1] CSR offsets into `ranges`, or
 *                   NULL for "no ranges at all".
 *   ranges          host int32 [R][2] inclusive (start, end) pairs per request,
 *                   non-overlapping within a request; start >= end is a
 *                   degenerate range and is skipped.
 *
 * Returns N = query_start_loc[num_reqs] when at least one scheduled row lies in
 * a range; then rows [0, N) are fully rewritten and rows >= N are untouched.
 * Returns 0 (table untouched, pass NULL as q_range_table so the kernels skip
 * the multimodal term) when there are no ranges, no scheduled rows, or no
 * scheduled row inside a range. Returns MVS_ERR_CAPACITY if N > capacity_rows
 * and MVS_ERR_INVALID for bad arguments; on error the table is untouched.
 * Overlapping ranges break the contract; the later range in (request, list)
 * order then wins.
 */
MVS_API int64_t build_query_range_table(int32_t* out_table, int64_t capacity_rows, const int32_t* query_start_loc,
                                const int32_t* seq_lens, int32_t num_reqs, const int32_t* range_offsets,
                                const int32_t* ranges);

/*
 * build_query_range_table_device - build_query_range_table with every buffer
 * in device memory, queued on hip_stream: no host pass, no copy, no
 * allocation, so a step that refills the table from device-resident range
 * metadata can be captured in a HIP graph (vLLM PR #50294, "implementation
 * breakdown" step 3: the table lives in a persistent buffer refilled every
 * step).
 *
 *   out_table       device int32 [capacity_rows][2], caller-owned.
 *   query_start_loc device int32 [num_reqs + 1]; seq_lens device int32
 *                   [num_reqs]; range_offsets device int32 [num_reqs + 1];
 *                   ranges device int32 [range_offsets[num_reqs]][2], inclusive
 *                   (start, end) pairs in list order.
 *
 * Rows [query_start_loc[0], min(query_start_loc[num_reqs], capacity_rows)) are
 * written with exactly the values build_query_range_table gives them; when no
 * row is covered they are all (-1, -1), which the attention kernels treat
 * like no table. Inputs are trusted: a request whose query_start_loc or
 * range_offsets decrease gets no rows or no ranges instead of an error, and
 * rows past capacity_rows are not written. Host-side argument checks only:
 * MVS_OK once queued, MVS_ERR_INVALID for NULL or misaligned pointers,
 * MVS_ERR_DEVICE if the launch fails.
 */
MVS_API int build_query_range_table_device(int32_t* out_table, int64_t capacity_rows, const int32_t* query_start_loc,
                                   const int32_t* seq_lens, int32_t num_reqs, const int32_t* range_offsets,
                                   const int32_t* ranges, void* hip_stream);

/*
 * attn_varlen_fwd - masked attention prefill over packed variable-length
 * sequences (the predicate above; vLLM PR #50294 mask_mod and forward wiring,
 * vLLM PR #49815 window and sink semantics).
 *
 *   q, out        device [Nq tokens][num_q_heads][head_dim], token strides
 *                 q_stride_tok / o_stride_tok (elements, >= Hq * head_dim).
 *   k, v          device [Nk tokens][num_kv_heads][head_dim], strides
 *                 k_stride_tok / v_stride_tok (below 2^24 elements, else
 *                 MVS_ERR_UNSUPPORTED). Query head h reads kv head
 *                 h / (num_q_heads / num_kv_heads).
 *   dtype         MVS_BF16 (head_dim 64, 128, 256, 512) or MVS_F32 (head_dim
 *                 64, 128, 256). bf16 pointers and strides must be multiples
 *                 of 8 elements (16-byte vectors).
 *   cu_seqlens_q/k device int32 [num_seqs + 1] prefix sums; Lk_b >= Lq_b.
 *   max_seqlen_q  host-known upper bound of Lq_b (sizes the grid; no device
 *                 read-back happens, so a smaller value is not detected: rows
 *                 past it are not computed and their output is left as it
 *                 was). max_seqlen_k: upper bound of Lk_b.
 *   softmax_scale finite and > 0; applied to Q K^T (sinks are not scaled).
 *   causal        0 or 1. window_left / window_right: -1 = unbounded. A causal
 *                 window of W keys is window_left = W - 1 (vLLM passes
 *                 1 + left window and tests delta < bound); a bidirectional
 *                 window w is window_left = window_right = w.
 *   q_range_table device int32 [Nq][2] from build_query_range_table, or NULL.
 *   sinks         device fp32 [num_q_heads], or NULL when sink_mode is NONE.
 *   lse_out       device fp32 [num_q_heads][Nq] natural-log LSE, or NULL.
 *
 * A row with no visible key gets out = 0 and lse = -inf (sink under
 * NULL_LOGIT). Sequences with Lq_b = 0 produce nothing. Sizes whose launch
 * would need more workgroups than one grid holds (2^31 - 1; for MVS_F32 at
 * most 65535 heads and 65535 sequences) return MVS_ERR_UNSUPPORTED before
 * anything is queued.
 */
MVS_API int attn_varlen_fwd(const void* q, const void* k, const void* v, void* out, int32_t dtype, int64_t q_stride_tok,
                    int64_t k_stride_tok, int64_t v_stride_tok, int64_t o_stride_tok, const int32_t* cu_seqlens_q,
                    const int32_t* cu_seqlens_k, int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float softmax_scale, int32_t causal,
                    int32_t window_left, int32_t window_right, const int32_t* q_range_table, const float* sinks,
                    int32_t sink_mode, float* lse_out, void* hip_stream);

/*
 * attn_varlen_fwd_range_scan - attn_varlen_fwd with the multimodal term read
 * from each request's padded range list instead of the per-row table: the
 * layout the table replaced (vLLM PR #50294, "functionality and motivation":
 * a [num_seqs, max_ranges, 2] tensor scanned in the mask, O(max_ranges) per
 * score). A query and a key are visible through the term when one valid
 * range (start < end) holds both positions. Kept as a measurement baseline
 * for the table path, not as a faster path; with non-overlapping ranges (the
 * pages' invariant) the result equals attn_varlen_fwd with the table that
 * build_query_range_table makes from the same ranges, bit for bit.
 *
 *   ranges        device int32 [num_seqs][max_ranges][2], inclusive (start,
 *                 end) absolute key positions; unused slots hold start >= end.
 *   max_ranges    0..64 (0: no multimodal term).
 *   dtype         MVS_BF16; head_dim 64, 128 or 256.
 * All other arguments, errors and outputs as for attn_varlen_fwd.
 */
MVS_API int attn_varlen_fwd_range_scan(const void* q, const void* k, const void* v, void* out, int32_t dtype,
                               int64_t q_stride_tok, int64_t k_stride_tok, int64_t v_stride_tok,
                               int64_t o_stride_tok, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, float softmax_scale, int32_t causal,
                               int32_t window_left, int32_t window_right, const int32_t* ranges, int32_t max_ranges,
                               const float* sinks, int32_t sink_mode, float* lse_out, void* hip_stream);

/*
 * attn_varlen_fwd_paged - attn_varlen_fwd with K and V read from a paged
 * cache through a block table instead of packed contiguous rows: chunked
 * prefill whose earlier tokens already sit in the cache (vLLM PR #50294, the
 * real-kernel test matrix lists a paged FA4 variant; the mask is unchanged).
 *
 *   q, out, q_stride_tok, o_stride_tok, cu_seqlens_q, max_seqlen_q, heads,
 *   softmax_scale, causal, windows, q_range_table, sinks, sink_mode, lse_out
 *                 as for attn_varlen_fwd.
 *   k_cache,v_cache device pages laid out as for attn_paged_decode: key t of
 *                 sequence b is at cache + block_table[b][t >> log2(page_size)]
 *                 * blk_stride + kv_head * head_stride + (t % page_size) *
 *                 tok_stride (elements; multiples of 8, tok_stride below 2^24).
 *   num_blocks    pages in each cache; a table entry outside [0, num_blocks)
 *                 reads page 0 instead of faulting (the result is then wrong
 *                 but defined).
 *   block_table   device int32 [num_seqs][max_blocks_per_seq]; entries past a
 *                 sequence's last page are never used.
 *   page_size     a power of two >= 16.
 *   seq_lens_k    device int32 [num_seqs]: Lk_b, the keys of sequence b
 *                 (cached context plus its Lq_b new tokens), Lk_b >= Lq_b and
 *                 <= max_seqlen_k <= max_blocks_per_seq * page_size.
 *   dtype         MVS_BF16 only (MVS_F32 is MVS_ERR_UNSUPPORTED); head_dim 64,
 *                 128, 256 or 512.
 *
 * The query rows are the last Lq_b of the sequence's Lk_b positions, exactly
 * as with attn_varlen_fwd. Status codes as for attn_varlen_fwd; rejected
 * arguments launch nothing.
 */
MVS_API int attn_varlen_fwd_paged(const void* q, const void* k_cache, const void* v_cache, void* out, int32_t dtype,
                          int64_t q_stride_tok, int64_t o_stride_tok, int64_t blk_stride, int64_t head_stride,
                          int64_t tok_stride, int32_t num_blocks, const int32_t* block_table,
                          int32_t max_blocks_per_seq, int32_t page_size, const int32_t* cu_seqlens_q,
                          const int32_t* seq_lens_k, int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float softmax_scale,
                          int32_t causal, int32_t window_left, int32_t window_right, const int32_t* q_range_table,
                          const float* sinks, int32_t sink_mode, float* lse_out, void* hip_stream);

/*
 * attn_paged_decode_workspace_size - bytes of device workspace that
 * attn_paged_decode needs for these sizes: partial outputs with their running
 * max and sum for up to 4096 + num_seqs * num_kv_heads segments, and the
 * per-sequence offsets of the balanced split. Pure host arithmetic,
 * independent of sequence lengths; 0 for invalid sizes.
 */
MVS_API size_t attn_paged_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim);

/*
 * attn_paged_decode - one new query per sequence against a paged KV cache.
 *
 * Decode is the one-query case of the predicate: the query sits at position
 * seq_lens[b] - 1, so nothing is masked except keys older than the window
 * (mini-vllm step14_4, "solution"; vLLM PR #55624 report, decode KV reads
 * clamped to the window). Decode rows never fall in a multimodal range
 * (vLLM PR #50294, step 3), so there is no table argument.
 *
 *   q, out        device [num_seqs][num_q_heads][head_dim], contiguous.
 *   k_cache,v_cache device pages; token t of sequence b is at
 *                 cache + block_table[b][t / page_size] * blk_stride
 *                       + kv_head * head_stride + (t % page_size) * tok_stride
 *                 (elements). HND pages [blocks][Hkv][page][D] are the tuned
 *                 layout; head_dim is contiguous.
 *   num_blocks    number of pages in each cache; table entries of tokens below
 *                 seq_len must lie in [0, num_blocks).
 *   block_table   device int32 [num_seqs][max_blocks_per_seq].
 *   seq_lens      device int32 [num_seqs], each <= max_seq_len (host-known;
 *                 longer ones are treated as max_seq_len).
 *   dtype         MVS_BF16. head_dim 64, 128 or 256. num_q_heads / num_kv_heads
 *                 in {1, 2, 4, 8, 16}. page_size a multiple of 16.
 *   window_left   -1 (full attention) or W - 1 for a window of W keys.
 *   sinks/sink_mode as for attn_varlen_fwd. lse_out: fp32 [num_q_heads][num_seqs]
 *                 or NULL.
 *   workspace     device buffer of at least
 *                 attn_paged_decode_workspace_size(num_seqs, num_q_heads,
 *                 num_kv_heads, head_dim) bytes, 256-byte aligned,
 *                 caller-owned; its contents need no initialisation. Calls
 *                 that share a workspace must be ordered on one stream.
 * At most 65535 sequences per call (MVS_ERR_UNSUPPORTED beyond).
 */
MVS_API int attn_paged_decode(const void* q, void* out, const void* k_cache, const void* v_cache, int32_t dtype,
                      int64_t blk_stride, int64_t head_stride, int64_t tok_stride, int32_t num_blocks,
                      const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                      int32_t num_seqs, int32_t max_seq_len, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t page_size, float softmax_scale, int32_t window_left,
                      const float* sinks, int32_t sink_mode, float* lse_out, void* workspace,
                      size_t workspace_bytes, void* hip_stream);

/*
 * attn_paged_decode_noalloc - attn_paged_decode without a caller workspace and
 * without any allocation, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. The split partials go to a buffer the library holds in each
 * device's memory for the life of the process (32 MiB per device); sizes whose
 * workspace (attn_paged_decode_workspace_size) exceeds it return
 * MVS_ERR_CAPACITY. Every call on a device shares that device's buffer, so
 * calls that overlap on one device (different streams, or host threads not
 * ordered on one stream) race and give undefined results; calls ordered on
 * one stream are safe. Arguments, outputs and other status codes as for
 * attn_paged_decode.
 */
MVS_API int attn_paged_decode_noalloc(const void* q, void* out, const void* k_cache, const void* v_cache, int32_t dtype,
                              int64_t blk_stride, int64_t head_stride, int64_t tok_stride, int32_t num_blocks,
                              const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                              int32_t num_seqs, int32_t max_seq_len, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t page_size, float softmax_scale, int32_t window_left,
                              const float* sinks, int32_t sink_mode, float* lse_out, void* hip_stream);

/* mvs_last_error - message of the last non-zero status on this thread ("" if none). */
MVS_API const char* mvs_last_error(void);

/*
 * mvs_plan_key_tiles - host evaluation of the prefill kernel's tile plan, for
 * checking it against a dense mask (diagnostic; touches no GPU).
 *
 * For one query tile - rows [row0, row0 + rows) of a request with Lq queries
 * and Lk keys - and key tiles of key_tile keys, writes one class per key tile
 * into tile_class[num_key_tiles]: 0 = skipped (no visible pair), 1 = partial
 * (the element predicate runs), 2 = full (every valid row sees every key).
 * table_rows is the host int32 [rows][2] slice of the range table or NULL.
 * Rows past Lq are ignored, as in the kernel. Returns MVS_OK or
 * MVS_ERR_INVALID.
 */
MVS_API int mvs_plan_key_tiles(int32_t Lq, int32_t Lk, int32_t row0, int32_t rows, int32_t causal, int32_t window_left,
                       int32_t window_right, const int32_t* table_rows, int32_t key_tile, int8_t* tile_class,
                       int32_t num_key_tiles);

/*
 * mvs_prefill_useful_flops - useful FLOPs of one prefill call: 4 * head_dim
 * per visible (query, key) pair per query head, where "visible" is the
 * predicate above with the window clamp (vLLM PR #55624 report: attention
 * FLOPs of a sliding-window layer count only the keys in the window). Host
 * arrays: cu_seqlens_q/k [num_seqs + 1], q_range_table [Nq][2] or NULL.
 * Returns the count, or a negative status for invalid arguments.
 */
MVS_API int64_t mvs_prefill_useful_flops(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t head_dim, int32_t causal, int32_t window_left,
                                 int32_t window_right, const int32_t* q_range_table);

/*
 * mvs_decode_useful_bytes - K and V bytes one decode call must read: for
 * each sequence min(seq_len, window_left + 1) keys (all keys when
 * window_left is -1) per kv head, head_dim * elem_bytes each for K and for V
 * (vLLM PR #55624 report: decode KV reads are clamped to the window). Host
 * seq_lens [num_seqs]. Returns the count, or a negative status.
 */
MVS_API int64_t mvs_decode_useful_bytes(const int32_t* seq_lens, int32_t num_seqs, int32_t num_kv_heads,
                                int32_t head_dim, int32_t elem_bytes, int32_t window_left);

#ifdef __cplusplus
}
#endif

#endif /* MVS_H */
