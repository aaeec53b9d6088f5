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
  // Range-scan mode (a measurement baseline for the table): when set, the
  // multimodal term comes from each request's padded range list
  // [num_seqs][max_ranges][2], scanned for every masked score, and table is
  // unused.
  const int* scan_ranges;
  int max_ranges;
};

constexpr int kMaxScanRanges = 64;

// bf16 prefill, head_dim 64/128/256/512 (contiguous or paged K/V). Returns a HIP error code.
hipError_t launch_prefill_bf16(PrefillArgs a, int head_dim, int max_seqlen_q, hipStream_t stream);
// Workgroups launch_prefill_bf16 would launch for these sizes (-1: head_dim not
// built); the entry points reject grids beyond kMaxGridBlocks before launching.
long long prefill_bf16_grid(int head_dim, int group, int Hq, int num_seqs, int max_seqlen_q, bool scan);
constexpr long long kMaxGridBlocks = 0x7fffffffLL;
// Largest grid y / z extent (fp32 prefill: heads and sequences; decode combine: sequences).
constexpr int kMaxGridYZ = 65535;
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
  int max_seq_len;  // sequence lengths are clamped to it
  float scale, scale_log2;
  int wl;
  const float* sinks;
  int sink_mode;
  float* lse;  // [Hq][B] or null
  // Balanced split: the visible keys of every (sequence, kv head), laid end to
  // end, are cut into `waves` equal shares, one per workgroup. A share that
  // touches several (sequence, kv head) pairs leaves one partial per pair, in
  // slot share + sequence * Hkv + kv head (unique along the sequence of cuts).
  int waves;            // set by the launcher
  long long max_pairs;  // host bound on the visible (token, kv head) pairs of the batch
  float* ws_o;         // [waves + B * Hkv][group][D]: unnormalised O
  float* ws_ml;        // [waves + B * Hkv][group][2]: running max (log2 units), running sum
  long long* ws_cum;   // [B + 1]: visible (token, kv head) pairs before each sequence
};

// Upper bound on the workgroups of the balanced decode split; the workspace
// holds kDecodeMaxWaves + B * Hkv partial slots.
constexpr int kDecodeMaxWaves = 4096;

hipError_t launch_decode_bf16(DecodeArgs a, int head_dim, hipStream_t stream);

// Size of the library-held decode workspace (one copy per device), and the
// device address of the current device's copy.
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
hipError_t decode_scratch(void** ptr);

}  // namespace mvs
