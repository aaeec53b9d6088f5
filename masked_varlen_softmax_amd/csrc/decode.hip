// decode.hip - split-K paged decode attention (bf16 cache, fp32 math) and the
// split combine, for gfx950.
//
// Decode is the one-query case of the shared predicate: the new token sits at
// position L - 1, so every older key is visible unless a window trims the
// past (mini-vllm step14_4, "solution": no mask at one query; vLLM PR #55624
// report: decode KV reads are clamped to the window). Only the keys in
// [max(0, L - 1 - window_left), L - 1] are read, so a window layer reads
// exactly W keys per kv head.
//
// The pass is bound by HBM bandwidth (about 4 FLOP per byte of K+V), so the
// design goal is many bytes in flight, not matrix-core throughput:
//   * Grid (split, kv head, sequence). A split covers a fixed, 16-aligned
//     token range; splits outside the visible range exit at once. One wave
//     per workgroup; splits are small (>= 256 tokens), so tens of thousands
//     of waves keep every CU busy with independent loads.
//   * The wave walks its range in 16-token chunks (one chunk lies inside one
//     page). The next chunk's K and V loads are issued before the current
//     chunk is computed.
//   * Scores: one v_mfma_f32_16x16x32_bf16 per 32 dims gives the 16 tokens x
//     G query heads of the kv head's group (G <= 16) in one shot; K rows are
//     the A operand loaded straight from HBM (lane: token, 8 dims), Q the B
//     operand held in registers. Lane (head n, g) then holds 4 tokens of
//     head n: the per-head max needs two exchanges.
//   * Values: lane l owns dims D/64 * l .. of every token; the chunk's
//     probabilities and rescale factors are broadcast through 320 bytes of LDS
//     and accumulated with fp32 FMAs (V is read in its natural [token][dim]
//     order, fully coalesced).
//   * Each split writes its unnormalised O, running max (base 2) and sum to
//     the workspace; the combine kernel merges the splits of each (sequence,
//     head) by their max, adds a null-logit sink once, and writes bf16 O and
//     the natural-log LSE.

#include <hip/hip_runtime.h>

#include "common.hpp"
#include "kernels.hpp"
#include "mask.hpp"

namespace mvs {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Visible key range of the decode query of a sequence of L keys.
__device__ inline void decode_keys(int L, int wl, int* lo, int* hi) {
  const RowKeys rk = row_keys(1, wl, -1, L - 1, L, -1, -1);
  *lo = rk.a_lo;
  *hi = rk.a_hi;
}

// One 16-token chunk of one kv head, as loaded: K rows for the score MFMA
// (lane (token n, g): dims 32*s + 8*g ..) and V rows in 16-byte pieces
// (lane (token group tv, piece dv): tokens TPI*i + tv, dims 8*dv ..).
template <int D>
struct Chunk {
  static constexpr int QS = D / 32;     // 16x16x32 MFMAs per chunk
  static constexpr int LPR = D / 8;     // lanes per V row
  static constexpr int TPI = 64 / LPR;  // V rows per load instruction
  static constexpr int VL = 16 / TPI;   // V loads per chunk
  u32x4_t k[QS];
  u32x4_t v[VL];
  bool ok;  // the chunk's page is mapped (uniform)
};

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// PD chunks are in flight while one is computed. The chunk ring lives in
// registers with compile-time slots (the loop is unrolled by PD + 1), so a
// chunk is consumed where it was loaded, never copied while in flight.
template <int D, int G, int PD>
__global__ __launch_bounds__(64) void decode_split_kernel(const DecodeArgs a) {
  using C = Chunk<D>;
  constexpr int QS = C::QS, LPR = C::LPR, TPI = C::TPI, VL = C::VL;
  __shared__ __attribute__((aligned(16))) float xs[16 * G + G];  // p[token][head], then alpha[head]

  const int lane = threadIdx.x;
  const int n = lane & 15, g4 = lane >> 4;
  const int tv = lane / LPR, dv = lane % LPR;
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int* bt = a.block_table + (long long)b * a.max_blocks;
  // Page ids of the split's nominal token range [sp * split, sp * split + split),
  // one per lane (a split spans at most 64 pages: decode_split_tokens caps it
  // at 1024 tokens and pages hold at least 16).
  int pid = -1;
  auto load_pids = [&](int sp_) {
    const int pg_nom = sp_ * a.split_tokens / a.page_size;
    const int np = (sp_ * a.split_tokens + a.split_tokens - 1) / a.page_size - pg_nom + 1;
    if (lane < np && pg_nom + lane < a.max_blocks) pid = bt[pg_nom + lane];
  };
  // A grid over every split knows its split before the sequence length: its
  // page ids load alongside the length. A grid counted back from the end
  // (window layers) needs the length first.
  const bool from_end = a.grid_splits < a.num_splits;  // uniform
  if (!from_end) load_pids(blockIdx.x);
  const int L = a.seq_lens[b];
  const int sp = from_end ? (L - 1) / a.split_tokens - (int)blockIdx.x : (int)blockIdx.x;
  if (sp < 0) return;
  if (from_end) load_pids(sp);
  int lo, hi;
  decode_keys(L, a.wl, &lo, &hi);
  const int t_begin = max(lo, sp * a.split_tokens);
  const int t_end = min(hi, sp * a.split_tokens + a.split_tokens - 1);
  if (lo > hi || t_begin > t_end) return;  // the combine applies the same rule

  const int head = kvh * G + n;  // this lane's query head in the score layout
  bf16x8_t qf[QS];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((long long)b * a.Hq + (n < G ? head : 0)) * D + 8 * g4;
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      u32x4_t raw = {0u, 0u, 0u, 0u};
      if (n < G) raw = *reinterpret_cast<const u32x4_t*>(qp + 32 * s);
      qf[s] = __builtin_bit_cast(bf16x8_t, raw);
    }
  }
  // Consumed here, so the compiler's memory-counter waits in the chunk loop
  // only ever count chunk loads.
#pragma unroll
  for (int s = 0; s < QS; ++s) asm volatile("" ::"v"(qf[s]));
  const float c2 = a.scale_log2;
  const float sink_raw = (a.sink_mode == MVS_SINK_KEY0_BIAS && n < G) ? a.sinks[head] / a.scale : 0.f;

  float o[G][8];
#pragma unroll
  for (int hq = 0; hq < G; ++hq)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[hq][e] = 0.f;
  float m2 = -INFINITY, l = 0.f;

  const uint16_t* kc = static_cast<const uint16_t*>(a.kc);
  const uint16_t* vc = static_cast<const uint16_t*>(a.vc);
  const int cs0 = t_begin & ~15;
  const int nchunks = ((t_end - cs0) >> 4) + 1;

  const int pg0 = sp * a.split_tokens / a.page_size;  // lane 0's page in pid
  asm volatile("" ::"v"(pid));
  // Every chunk issues the same loads, whatever its state, so the memory
  // counter always holds exactly the chunks in flight: an unmapped page reads
  // block 0 instead (its scores and values are masked below).
  auto load_chunk = [&](int cs, C& c) {
    int phys = __builtin_amdgcn_readlane(pid, min(cs / a.page_size - pg0, 63));
    c.ok = phys >= 0 && phys < a.num_blocks;
    if (!c.ok) phys = 0;
    const long long base = (long long)phys * a.blk_st + (long long)kvh * a.head_st + (long long)(cs % a.page_size) * a.tok_st;
    const uint16_t* kp = kc + base + (long long)n * a.tok_st + 8 * g4;
#pragma unroll
    for (int s = 0; s < QS; ++s) c.k[s] = *reinterpret_cast<const u32x4_t*>(kp + 32 * s);
    const uint16_t* vp = vc + base + (long long)tv * a.tok_st + 8 * dv;
#pragma unroll
    for (int i = 0; i < VL; ++i) c.v[i] = *reinterpret_cast<const u32x4_t*>(vp + (long long)(TPI * i) * a.tok_st);
  };

  auto compute = [&](const C& c, int cs) {
    // scores of 16 tokens x 16 head columns (lane (n, g4): tokens 4*g4 + r of head n)
    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
    if (c.ok) {
#pragma unroll
      for (int s = 0; s < QS; ++s)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, c.k[s]), qf[s], sc, 0, 0, 0);
    }
    const bool partial = !c.ok || cs < t_begin || cs + 15 > t_end;  // uniform
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = cs + 4 * g4 + r;
      if (partial && (!c.ok || tok < t_begin || tok > t_end)) sc[r] = -INFINITY;
      if (tok == 0) sc[r] += sink_raw;
    }
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(m2, mx * c2);
    const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m2 - mn);
    const float mb = mn == -INFINITY ? 0.f : mn;
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sc[r] = __builtin_amdgcn_exp2f(fmaf(sc[r], c2, -mb));
      ps += sc[r];
    }
    l = l * alpha + ps;
    m2 = mn;
    if (n < G) {
#pragma unroll
      for (int r = 0; r < 4; ++r) xs[(4 * g4 + r) * G + n] = sc[r];
      if (g4 == 0) xs[16 * G + n] = alpha;
    }
    __syncthreads();
#pragma unroll
    for (int hq = 0; hq < G; ++hq) {
      const float al = xs[16 * G + hq];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[hq][e] *= al;
    }
#pragma unroll
    for (int i = 0; i < VL; ++i) {
      const int t = TPI * i + tv;
      u32x4_t w = c.v[i];
      // tokens outside the range may be unwritten cache slots: never let them reach O
      if (partial && (!c.ok || cs + t < t_begin || cs + t > t_end)) w = u32x4_t{0u, 0u, 0u, 0u};
      float vv[8];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        vv[2 * x] = bf16_lo(w[x]);
        vv[2 * x + 1] = bf16_hi(w[x]);
      }
#pragma unroll
      for (int hq = 0; hq < G; ++hq) {
        const float p = xs[t * G + hq];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hq][e] = fmaf(p, vv[e], o[hq][e]);
      }
    }
    __syncthreads();
  };

  // Chunks past the last one reload the last chunk (never computed), so that
  // every step issues the same loads.
  C ring[PD + 1];
#pragma unroll
  for (int u = 0; u < PD; ++u) load_chunk(cs0 + 16 * min(u, nchunks - 1), ring[u]);
  for (int c0 = 0; c0 < nchunks; c0 += PD + 1) {
#pragma unroll
    for (int u = 0; u <= PD; ++u) {
      const int c = c0 + u;
      if (c >= nchunks) break;  // uniform
      load_chunk(cs0 + 16 * min(c + PD, nchunks - 1), ring[(u + PD) % (PD + 1)]);
      compute(ring[u], cs0 + 16 * c);
    }
  }

  // ---- partial results of this split: sum the token groups, then store
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
    for (int hq = 0; hq < G; ++hq)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[hq][e] += __shfl_xor(o[hq][e], off);
  const long long row = (long long)b * a.Hq + kvh * G;  // first head of the group
  if (n < G && g4 == 0) {
    float* ml = a.ws_ml + ((row + n) * a.num_splits + sp) * 2;
    ml[0] = m2;
    ml[1] = l;
  }
  if (tv == 0) {
#pragma unroll
    for (int hq = 0; hq < G; ++hq) {
      float* op = a.ws_o + ((row + hq) * a.num_splits + sp) * D + 8 * dv;
      *reinterpret_cast<f32x4_t*>(op) = f32x4_t{o[hq][0], o[hq][1], o[hq][2], o[hq][3]};
      *reinterpret_cast<f32x4_t*>(op + 4) = f32x4_t{o[hq][4], o[hq][5], o[hq][6], o[hq][7]};
    }
  }
}

template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(const DecodeArgs a) {
  // One wave per (head, sequence). The active splits' maxima are reduced
  // across lanes, their weights staged in LDS, then every lane accumulates
  // its D/64 dims over the splits with several loads in flight.
  constexpr int DPL = D / 64;
  constexpr int MAXS = kDecodeMaxSplits;  // the API bounds max_seq_len accordingly
  __shared__ float wsh[MAXS];
  const int lane = threadIdx.x;
  const int h = blockIdx.x, b = blockIdx.y;
  const int L = a.seq_lens[b];
  int lo, hi;
  decode_keys(L, a.wl, &lo, &hi);
  const long long row = (long long)b * a.Hq + h;
  int s_lo = 0, ns = 0;
  if (lo <= hi) {
    s_lo = lo / a.split_tokens;
    ns = min(hi / a.split_tokens, a.num_splits - 1) - s_lo + 1;  // seq_len beyond max_seq_len: clipped
  }
  ns = min(ns, MAXS);
  const float* ml = a.ws_ml + (row * a.num_splits + s_lo) * 2;
  float M = a.sink_mode == MVS_SINK_NULL_LOGIT ? a.sinks[h] * kLog2e : -INFINITY;
  for (int s = lane; s < ns; s += 64) M = fmaxf(M, ml[2 * s]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float lt = 0.f;
  for (int s = lane; s < ns; s += 64) {
    const float m = ml[2 * s];
    const float wgt = (m == -INFINITY || M == -INFINITY) ? 0.f : exp2f(m - M);
    wsh[s] = wgt;
    lt += wgt * ml[2 * s + 1];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lt += __shfl_xor(lt, off);
  if (a.sink_mode == MVS_SINK_NULL_LOGIT && M != -INFINITY) lt += exp2f(a.sinks[h] * kLog2e - M);
  __syncthreads();
  float o[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = 0.f;
  const float* op = a.ws_o + (row * a.num_splits + s_lo) * D + DPL * lane;
  int s = 0;
  for (; s + 4 <= ns; s += 4) {
    float v[4][DPL];
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int e = 0; e < DPL; ++e) v[x][e] = op[(long long)(s + x) * D + e];
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[e] = fmaf(wsh[s + x], v[x][e], o[e]);
  }
  for (; s < ns; ++s)
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] = fmaf(wsh[s], op[(long long)s * D + e], o[e]);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  uint16_t* out = static_cast<uint16_t*>(a.o) + row * D + DPL * lane;
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    const __bf16 x = (__bf16)(o[e] * inv);
    out[e] = __builtin_bit_cast(uint16_t, x);
  }
  if (a.lse != nullptr && lane == 0) a.lse[(long long)h * a.num_seqs + b] = lt > 0.f ? (M + log2f(lt)) * kLn2 : -INFINITY;
}

#ifndef MVS_DECODE_PREFETCH
#define MVS_DECODE_PREFETCH 2
#endif

template <int D, int G>
hipError_t launch(const DecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((decode_split_kernel<D, G, MVS_DECODE_PREFETCH>), dim3(a.grid_splits, a.Hkv, a.num_seqs), dim3(64),
                     0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(a.Hq, a.num_seqs), dim3(64), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t stream) {
  switch (a.group) {
    case 1:
      return launch<D, 1>(a, stream);
    case 2:
      return launch<D, 2>(a, stream);
    case 4:
      return launch<D, 4>(a, stream);
    case 8:
      return launch<D, 8>(a, stream);
    case 16:
      return launch<D, 16>(a, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_bf16(DecodeArgs a, int head_dim, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  if (a.num_seqs > 65535 || a.Hkv > 65535 || a.Hq > 65535) return hipErrorInvalidValue;
  switch (head_dim) {
    case 64:
      return launch_d<64>(a, stream);
    case 128:
      return launch_d<128>(a, stream);
    case 256:
      return launch_d<256>(a, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace mvs
