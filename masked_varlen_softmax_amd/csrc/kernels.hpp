// kernels.hpp - argument blocks and launchers shared between the C-ABI layer
// (api.hip) and the kernel sources.
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace mvs {

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  long long q_st, k_st, v_st, o_st;  // token strides, elements
  const int* cu_q;
  const int* cu_k;
  int num_seqs;
  int Hq, Hkv, group;  // group = Hq / Hkv
  int n_mtiles;        // query tiles per (sequence, head) for max_seqlen_q
  float scale;         // softmax scale
  float scale_log2;    // scale * log2(e)
  int causal, wl, wr;
  const int* table;  // [N][2] or null
  const float* sinks;
  int sink_mode;
  float* lse;  // [Hq][N] or null
  // Paged K/V (chunked prefill from the cache) when block_table is set: k and
  // v are the cache bases, k_st / v_st the token stride within a page,
  // seq_lens_k the key counts (cu_k unused).
  const int* block_table;  // [num_seqs][max_blocks]
  const int* seq_lens_k;
  int max_blocks, num_blocks, page_log2;
  long long blk_st, head_st;  // elements
};

// bf16 prefill, head_dim 64/128/256/512 (contiguous or paged K/V). Returns a HIP error code.
hipError_t launch_prefill_bf16(PrefillArgs a, int head_dim, int max_seqlen_q, hipStream_t stream);
// fp32 prefill, head_dim 64/128/256.
hipError_t launch_prefill_f32(PrefillArgs a, int head_dim, int max_seqlen_q, hipStream_t stream);

struct DecodeArgs {
  const void* q;
  void* o;
  const void* kc;
  const void* vc;
  long long blk_st, head_st, tok_st;  // elements
  int num_blocks;
  const int* block_table;
  int max_blocks;
  const int* seq_lens;
  int num_seqs, Hq, Hkv, group;
  int page_size;
  float scale, scale_log2;
  int wl;
  const float* sinks;
  int sink_mode;
  float* lse;  // [Hq][B] or null
  int split_tokens, num_splits;
  int grid_splits;  // blocks along x; below num_splits they count back from each sequence's last split
  float* ws_o;   // [B][Hq][S][D]
  float* ws_ml;  // [B][Hq][S][2]  (running max in log2 units, running sum)
};

// Tokens per split-K partition for a maximum context length: a power of two
// between MVS_DECODE_SPLIT_MIN and 1024, aiming at no more than 128
// partitions. A split then spans at most 64 pages of 16 tokens.
#ifndef MVS_DECODE_SPLIT_MIN
#define MVS_DECODE_SPLIT_MIN 256
#endif
constexpr int kDecodeMaxSplitTokens = 1024;
constexpr int kDecodeMaxSplits = 4096;  // partitions the combine kernel merges
MVS_HD inline int decode_split_tokens(int max_seq_len) {
  int need = (max_seq_len + 127) / 128;
  int s = MVS_DECODE_SPLIT_MIN;
  while (s < need && s < kDecodeMaxSplitTokens) s <<= 1;
  return s;
}

hipError_t launch_decode_bf16(DecodeArgs a, int head_dim, hipStream_t stream);

}  // namespace mvs
