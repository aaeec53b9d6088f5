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
// design goal is a steady stream of bytes in flight on every CU, with no
// start-up gaps and no tail:
//   * Balanced split. The visible keys of all (sequence, kv head) pairs, laid
//     end to end, are cut into as many equal shares as the chip holds
//     workgroups at once (one wave each). Every wave streams the same number
//     of keys, so all finish together, and a wave pays its start-up (sequence
//     lengths, first loads) once, not once per fixed-size split. A share that
//     crosses pair boundaries processes one segment per pair.
//   * A segment walks its keys in 16-token chunks (one chunk lies inside one
//     page). The next chunks' K and V loads are issued before the current
//     chunk is computed; the page id of the chunk after those is read one
//     chunk ahead with a scalar load, so address formation never waits.
//   * Scores: one v_mfma_f32_16x16x32_bf16 per 32 dims gives the 16 tokens x
//     G query heads of the kv head's group (G <= 16) in one shot; K rows are
//     the A operand loaded straight from HBM (lane: token, 8 dims), Q the B
//     operand held in registers. Lane (head n, g) then holds 4 tokens of
//     head n: the per-head max needs two exchanges.
//   * Values: lane l owns dims D/64 * l .. of every token; the chunk's
//     probabilities and rescale factors are broadcast through 320 bytes of LDS
//     and accumulated with fp32 FMAs (V is read in its natural [token][dim]
//     order, fully coalesced).
//   * Each segment writes its unnormalised O, running max (base 2) and sum to
//     the workspace; the combine kernel merges the segments of each
//     (sequence, head) by their max, adds a null-logit sink once, and writes
//     bf16 O and the natural-log LSE.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>

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

// Keys of sequence b that the decode query sees (0 when the sequence is
// empty); the length is clamped to max_seq_len.
__device__ inline int seq_span(const DecodeArgs& a, int b, int* lo_out) {
  int L = a.seq_lens[b];
  L = max(0, min(L, a.max_seq_len));
  int lo, hi;
  decode_keys(L, a.wl, &lo, &hi);
  *lo_out = lo;
  return hi >= lo ? hi - lo + 1 : 0;
}

__device__ inline long long wave_incl_scan(long long x) {
  const int lane = threadIdx.x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const long long y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}

__device__ inline long long uniform64(long long x) {
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)x);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)((unsigned long long)x >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}

// Share boundaries. Workgroup w runs on XCD w % 8, and streaming from HBM the
// odd XCDs ran 5-9 % slower than the even ones on every board measured, so
// with equal shares the layer ended with the odd XCDs' waves alone. Long
// shares are therefore weighted 27 (even XCD) : 25 (odd): share s starts at
// floor(T * q(s) / q(W)), q(s) the summed weights of shares 0 .. s-1 (26 per
// share on average); every share is then non-empty, as the combine, which
// counts every share between a pair's first and last, needs. Shares under
// 4096 pairs on average keep equal cuts of ceil(T / W) (the empty ones all at
// the end): measured, the weights paid off for long shares only (full layer
// of 64 contexts of 4K-32K: 0.8218 -> 0.8089 ms; the 4096-key window layer,
// 2048 pairs per share: 0.1915 -> 0.1929 ms, and slower still with heavier
// weights, although its weighted cuts still fall one per pair).
#ifndef MVS_DECODE_XCD_WEIGHT
#define MVS_DECODE_XCD_WEIGHT 1
#endif
#ifndef MVS_DECODE_W_EVEN
#define MVS_DECODE_W_EVEN 27
#endif
#ifndef MVS_DECODE_W_ODD
#define MVS_DECODE_W_ODD 25
#endif
__device__ inline long long share_q(long long s) {
  constexpr long long WE = MVS_DECODE_W_EVEN, WO = MVS_DECODE_W_ODD;
  static_assert(WO >= 1 && WE >= WO, "share weights");
  const long long k = s & 7;
  return 4 * (WE + WO) * (s >> 3) + (WE + WO) * (k >> 1) + WE * (k & 1);  // 0, 27, 52, 79, 104, ...
}
__device__ inline bool share_weighted(long long T, int waves) {
  return MVS_DECODE_XCD_WEIGHT && T >= 4096LL * waves && T * MVS_DECODE_W_ODD >= share_q(waves);
}
__device__ inline long long share_begin(long long T, int waves, long long s) {
  if (share_weighted(T, waves)) return T * share_q(s) / share_q(waves);
  const long long per = (T + waves - 1) / waves;
  return min(T, s * per);
}
// The share holding pair position p (0 <= p < T): the last s with
// share_begin(s) <= p, i.e. T * q(s) < (p + 1) * q(W) when weighted.
__device__ inline int share_of(long long T, int waves, long long p) {
  if (!share_weighted(T, waves)) return (int)(p / ((T + waves - 1) / waves));
  const long long lim = (p + 1) * share_q(waves);
  int lo = 0, hi = waves - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (T * share_q(mid) < lim)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// Lane l's value of v, broadcast (l uniform); the bits travel as an integer.
__device__ inline float lane_f(float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); }

using cint = __attribute__((address_space(4))) const int;

// PD chunks are in flight while one is computed. The chunk ring lives in
// registers with compile-time slots (the loop is unrolled by PD + 1), so a
// chunk is consumed where it was loaded, never copied while in flight.
template <int D, int G, int PD>
struct Segment {
  using C = Chunk<D>;
  static constexpr int QS = C::QS, LPR = C::LPR, TPI = C::TPI, VL = C::VL;

  // Keys [t_begin, t_end] of kv head kvh of sequence b; results go to `slot`.
  __device__ static void run(const DecodeArgs& a, float* xs, int b, int kvh, int t_begin, int t_end, int slot) {
    const int lane = threadIdx.x;
    const int n = lane & 15, g4 = lane >> 4;
    const int tv = lane / LPR, dv = lane % LPR;
    const cint* bt = (const cint*)(a.block_table + (long long)b * a.max_blocks);
    const int head = kvh * G + n;  // this lane's query head in the score layout

    const uint16_t* kc = static_cast<const uint16_t*>(a.kc);
    const uint16_t* vc = static_cast<const uint16_t*>(a.vc);
    const int cs0 = t_begin & ~15;
    const int nchunks = ((t_end - cs0) >> 4) + 1;
    auto page_of = [&](int c) {  // page id of chunk c (clamped to the last chunk)
      const int cs = cs0 + 16 * min(c, nchunks - 1);
      return bt[min(cs / a.page_size, a.max_blocks - 1)];
    };
    // Every chunk issues the same loads, whatever its state, so the memory
    // counter always holds exactly the chunks in flight: an unmapped page reads
    // block 0 instead (its scores and values are masked below).
    auto load_chunk = [&](int c, int phys, C& ch) {
      const int cs = cs0 + 16 * min(c, nchunks - 1);
      ch.ok = phys >= 0 && phys < a.num_blocks;
      if (!ch.ok) phys = 0;
      const long long base =
          (long long)phys * a.blk_st + (long long)kvh * a.head_st + (long long)(cs % a.page_size) * a.tok_st;
      const uint16_t* kp = kc + base + (long long)n * a.tok_st + 8 * g4;
#pragma unroll
      for (int s = 0; s < QS; ++s) ch.k[s] = *reinterpret_cast<const u32x4_t*>(kp + 32 * s);
      const uint16_t* vp = vc + base + (long long)tv * a.tok_st + 8 * dv;
#pragma unroll
      for (int i = 0; i < VL; ++i) ch.v[i] = *reinterpret_cast<const u32x4_t*>(vp + (long long)(TPI * i) * a.tok_st);
    };

    // Q loads go out first and the first chunks' loads behind them; Q is
    // consumed once those are queued, so its latency overlaps theirs and the
    // compiler's memory-counter waits in the chunk loop only count chunk loads.
    bf16x8_t qf[QS];
    {
      const uint16_t* qp =
          static_cast<const uint16_t*>(a.q) + ((long long)b * a.Hq + (n < G ? head : kvh * G)) * D + 8 * g4;
#pragma unroll
      for (int s = 0; s < QS; ++s) qf[s] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(qp + 32 * s));
    }
    C ring[PD + 1];
    int ph = page_of(0);
#pragma unroll
    for (int u = 0; u < PD; ++u) {
      const int nx = page_of(u + 1);
      load_chunk(u, ph, ring[u]);
      ph = nx;
    }
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

    auto compute = [&](const C& ch, int cs) {
      // scores of 16 tokens x 16 head columns (lane (n, g4): tokens 4*g4 + r of head n)
      f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
      if (ch.ok) {
#pragma unroll
        for (int s = 0; s < QS; ++s)
          sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ch.k[s]), qf[s], sc, 0, 0, 0);
      }
      const bool partial = !ch.ok || cs < t_begin || cs + 15 > t_end;  // uniform
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = cs + 4 * g4 + r;
        if (partial && (!ch.ok || tok < t_begin || tok > t_end)) sc[r] = -INFINITY;
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
        u32x4_t w = ch.v[i];
        // tokens outside the range may be unwritten cache slots: never let them reach O
        if (partial && (!ch.ok || cs + t < t_begin || cs + t > t_end)) w = u32x4_t{0u, 0u, 0u, 0u};
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
    for (int c0 = 0; c0 < nchunks; c0 += PD + 1) {
#pragma unroll
      for (int u = 0; u <= PD; ++u) {
        const int c = c0 + u;
        if (c >= nchunks) break;  // uniform
        const int nx = page_of(c + PD + 1);
        load_chunk(c + PD, ph, ring[(u + PD) % (PD + 1)]);
        ph = nx;
        compute(ring[u], cs0 + 16 * c);
      }
    }

    // ---- partial results of this segment: sum the token groups, then store
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
      for (int hq = 0; hq < G; ++hq)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hq][e] += __shfl_xor(o[hq][e], off);
    if (n < G && g4 == 0) {
      float* ml = a.ws_ml + ((long long)slot * G + n) * 2;
      ml[0] = m2;
      ml[1] = l;
    }
    if (tv == 0) {
#pragma unroll
      for (int hq = 0; hq < G; ++hq) {
        float* op = a.ws_o + ((long long)slot * G + hq) * D + 8 * dv;
        *reinterpret_cast<f32x4_t*>(op) = f32x4_t{o[hq][0], o[hq][1], o[hq][2], o[hq][3]};
        *reinterpret_cast<f32x4_t*>(op + 4) = f32x4_t{o[hq][4], o[hq][5], o[hq][6], o[hq][7]};
      }
    }
  }
};

// One wave per share of the visible (token, kv head) pairs of the batch.
template <int D, int G, int PD>
__global__ __launch_bounds__(64) void decode_split_kernel(const DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) float xs[16 * G + G];  // p[token][head], then alpha[head]
  const int lane = threadIdx.x;
  const int w = blockIdx.x;
  const int Hkv = a.Hkv;
  // Visible pairs of the whole batch, in (sequence, kv head, key) order. The
  // first wave also stores each sequence's offset for the combine kernel.
  // Lane i keeps sequence i's span, window start and pairs up to its end, so
  // a batch of at most 64 sequences is read once.
  long long T = 0;
  int my_span = 0, my_lo = 0;
  long long my_incl = 0;
  for (int b0 = 0; b0 < a.num_seqs; b0 += 64) {
    int lo = 0;
    const int sp = b0 + lane < a.num_seqs ? seq_span(a, b0 + lane, &lo) : 0;
    const long long x = (long long)sp * Hkv;
    const long long s = wave_incl_scan(x);
    if (w == 0 && b0 + lane < a.num_seqs) a.ws_cum[b0 + lane] = T + s - x;
    if (b0 == 0) {
      my_span = sp;
      my_lo = lo;
      my_incl = s;
    }
    T += __shfl(s, 63);
  }
  T = uniform64(T);
  if (w == 0 && lane == 0) a.ws_cum[a.num_seqs] = T;
  long long pos = share_begin(T, a.waves, w);
  const long long end = share_begin(T, a.waves, w + 1);
  if (pos >= end) return;
  const bool small = a.num_seqs <= 64;
  auto seq_at = [&](int bb, int* lo_out) -> int {  // span and window start of sequence bb (uniform)
    if (small) {
      *lo_out = __builtin_amdgcn_readlane(my_lo, bb);
      return __builtin_amdgcn_readlane(my_span, bb);
    }
    int l;
    const int sp = seq_span(a, bb, &l);
    *lo_out = __builtin_amdgcn_readfirstlane(l);
    return __builtin_amdgcn_readfirstlane(sp);
  };

  // the sequence holding pair `pos`, and the pairs before it
  int b = 0;
  long long base = 0;
  if (small) {
    b = __builtin_amdgcn_readfirstlane(__builtin_ctzll(__ballot(my_incl > pos)));
    base = uniform64(__shfl(my_incl - (long long)my_span * Hkv, b));
  } else {
    for (int b0 = 0; b0 < a.num_seqs; b0 += 64) {
      int lo;
      const long long x = b0 + lane < a.num_seqs ? (long long)seq_span(a, b0 + lane, &lo) * Hkv : 0;
      const long long s = wave_incl_scan(x);
      const long long tot = uniform64(__shfl(s, 63));
      if (pos < base + tot) {
        const unsigned long long hit = __ballot(base + s > pos);
        const int l = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
        b = b0 + l;
        base += uniform64(__shfl(s - x, l));
        break;
      }
      base += tot;
    }
  }
  int lo;
  int span = seq_at(b, &lo);
  const long long off = pos - base;
  int kvh = (int)(off / span);
  int toff = (int)(off % span);
  while (true) {
    const int seg = (int)min(end - pos, (long long)(span - toff));
    Segment<D, G, PD>::run(a, xs, b, kvh, lo + toff, lo + toff + seg - 1, w + b * Hkv + kvh);
    pos += seg;
    if (pos >= end) break;
    toff = 0;
    if (++kvh == Hkv) {
      kvh = 0;
      do {  // a later sequence has visible keys, since pos < T
        ++b;
        span = seq_at(b, &lo);
      } while (span == 0);
    }
  }
}

template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(const DecodeArgs a) {
  // One wave per (head, sequence). The pair's segments are those of the
  // shares its visible keys fall in. Lane s holds segment s's (max, sum) for
  // the first 64; their O rows are requested together with them, four at a
  // time, and weighted once the maxima are reduced (weights broadcast from
  // the lane that holds them). Longer lists go on 64 segments at a time.
  constexpr int DPL = D / 64;
  const int lane = threadIdx.x;
  const int h = blockIdx.x, b = blockIdx.y;
  const int G = a.group, kvh = h / G, g = h % G;
  const long long T = a.ws_cum[a.num_seqs];
  const long long c0 = a.ws_cum[b];
  const long long span = (a.ws_cum[b + 1] - c0) / a.Hkv;
  int ns = 0;
  long long w_lo = 0;
  if (span > 0) {
    const long long start = c0 + kvh * span;
    w_lo = share_of(T, a.waves, start);
    ns = share_of(T, a.waves, start + span - 1) - (int)w_lo + 1;  // at most `waves`
  }
  const long long slot0 = w_lo + (long long)b * a.Hkv + kvh;  // consecutive shares: consecutive slots
  const float* ml = a.ws_ml + (slot0 * G + g) * 2;
  const long long sst = 2LL * G;  // floats between the same head's entries of consecutive slots
  const float* op = a.ws_o + (slot0 * G + g) * D + DPL * lane;
  const long long ost = (long long)G * D;
  const float m0 = lane < ns ? ml[lane * sst] : -INFINITY;
  const float l0 = lane < ns ? ml[lane * sst + 1] : 0.f;
  float v[4][DPL];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int e = 0; e < DPL; ++e) v[x][e] = x < ns ? op[x * ost + e] : 0.f;
  float M = a.sink_mode == MVS_SINK_NULL_LOGIT ? a.sinks[h] * kLog2e : -INFINITY;
  M = fmaxf(M, m0);
  for (int s = lane + 64; s < ns; s += 64) M = fmaxf(M, ml[s * sst]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float o[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = 0.f;
  float lt = 0.f;
  for (int s0 = 0; s0 < ns; s0 += 64) {
    const float m = s0 == 0 ? m0 : (s0 + lane < ns ? ml[(s0 + lane) * sst] : -INFINITY);
    const float l = s0 == 0 ? l0 : (s0 + lane < ns ? ml[(s0 + lane) * sst + 1] : 0.f);
    const float wgt = (m == -INFINITY || M == -INFINITY) ? 0.f : exp2f(m - M);
    lt = fmaf(wgt, l, lt);
    const int cnt = min(64, ns - s0);
    int s = 0;
    if (s0 == 0) {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const float wx = lane_f(wgt, x);  // 0 past ns
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[e] = fmaf(wx, v[x][e], o[e]);
      }
      s = 4;
    }
    const float* p = op + s0 * ost;
    for (; s + 4 <= cnt; s += 4) {
      float u[4][DPL];
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int e = 0; e < DPL; ++e) u[x][e] = p[(s + x) * ost + e];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const float wx = lane_f(wgt, s + x);
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[e] = fmaf(wx, u[x][e], o[e]);
      }
    }
    for (; s < cnt; ++s) {
      const float wx = lane_f(wgt, s);
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[e] = fmaf(wx, p[s * ost + e], o[e]);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lt += __shfl_xor(lt, off);
  if (a.sink_mode == MVS_SINK_NULL_LOGIT && M != -INFINITY) lt += exp2f(a.sinks[h] * kLog2e - M);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  uint16_t* out = static_cast<uint16_t*>(a.o) + ((long long)b * a.Hq + h) * D + DPL * lane;
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    const __bf16 x = (__bf16)(o[e] * inv);
    out[e] = __builtin_bit_cast(uint16_t, x);
  }
  if (a.lse != nullptr && lane == 0) a.lse[(long long)h * a.num_seqs + b] = lt > 0.f ? (M + log2f(lt)) * kLn2 : -INFINITY;
}

#ifndef MVS_DECODE_PREFETCH
#define MVS_DECODE_PREFETCH 3
#endif

// Chunks in flight per wave: the register ring holds (PD + 1) chunks of
// 16 tokens beside a D x G accumulator, so wide groups keep one chunk ahead.
// Three chunks ahead leave room for one wave per SIMD at head_dim 128 and
// group 4; two waves on one SIMD stream at unequal rates (the first-issued
// one about a fifth faster), so a CU's equal shares end apart.
template <int D, int G>
constexpr int decode_prefetch() {
  return D * G >= 2048 ? 1 : MVS_DECODE_PREFETCH;
}

// Workgroups of the split kernel resident at once on the current device
// (CUs x occupancy), cached per device. Several host threads may fill an
// entry at once; they all compute the same value, and the relaxed atomic
// store and load make that benign.
template <int D, int G>
int resident_waves() {
  static std::atomic<int> cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_split_kernel<D, G, decode_prefetch<D, G>()>, 64, 0) !=
      hipSuccess)
    return 0;
  const int n = cus * per_cu;
  if (dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <int D, int G>
hipError_t launch(DecodeArgs a, hipStream_t stream) {
  const int res = resident_waves<D, G>();
  if (res <= 0) return hipErrorInvalidDevice;
  // one share per resident workgroup, each of at least 256 (token, kv head)
  // pairs of the largest batch the sizes allow
  a.waves = (int)std::min<long long>({(long long)res, (long long)kDecodeMaxWaves, std::max(1LL, a.max_pairs / 256)});
  hipLaunchKernelGGL((decode_split_kernel<D, G, decode_prefetch<D, G>()>), dim3(a.waves), dim3(64), 0, stream, a);
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

// Library-held workspace of attn_paged_decode_noalloc, for callers that cannot
// allocate device memory. Each device holds its own copy for the life of the
// process. In host code `scratch` names a host-side stand-in, not device
// memory: its device address comes from hipGetSymbolAddress, fetched once per
// device (with that device current) and kept below; only that address is
// ever passed to a kernel.
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mutex;
}  // namespace

hipError_t decode_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_decode_bf16(DecodeArgs a, int head_dim, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  if (a.num_seqs > kMaxGridYZ) return hipErrorInvalidValue;  // rejected by attn_paged_decode already
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
