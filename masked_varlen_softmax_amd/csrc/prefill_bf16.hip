// prefill_bf16.hip - masked varlen attention prefill, bf16 in/out, fp32
// accumulation, for gfx950 (MI355X).
//
// What it computes: for every packed query row and query head,
// softmax(scale * q K^T + key-0 sink, masked) V over the keys of its own
// request, under the predicate of mask.hpp (vLLM PR #50294 mask_mod: causal,
// window, multimodal-prefix table; vLLM PR #49815: two-sided window, key-0
// sink bias and null-logit sink). The per-row table lookup is hoisted out of
// the key loop, as the PR #50294 page describes for its FA4 kernel.
//
// Work decomposition. One workgroup = NW waves = one query head and
// BM = WM * NW consecutive query rows of one request. Each wave owns WM rows
// (32, or 16 where the fp32 O accumulator of 32 rows would not fit in
// registers, i.e. head_dim 512).
// The workgroup walks the key tiles (BN keys each) between the smallest and
// largest key any of its rows can see, skipping everything else (the window
// path of vLLM PR #49815 visits only blocks inside the window; the
// multimodal ranges widen the upper end, never the lower one). A key tile
// that every row sees whole skips the element mask.
//
// Matrix-core layout. WM = 32 uses v_mfma_f32_32x32x16_bf16, WM = 16 uses
// v_mfma_f32_16x16x32_bf16; lane = WM * gq + col, gq < 64 / WM:
//   S^T[key][query] = K Q^T: A = K tile rows from LDS (lane: key col, 8
//     consecutive dims), B = the wave's Q rows held in registers (lane: query
//     col). The result gives lane (col, gq) the scores of query `col` only
//     (WM = 32: keys 8*(r/4) + 4*gq + r%4, r < 16; WM = 16: keys 4*gq + r,
//     r < 4), so the row max is an in-lane max plus one or two exchanges
//     across gq, and the online-softmax rescale is one scalar per lane.
//   O^T[dim][query] += V^T P^T: B = P^T straight from the S^T registers
//     (rounded to bf16); A = V^T read from a transposed V tile in LDS in the
//     key order the S^T registers use (the sum over keys does not care about
//     that order as long as both operands share it). O^T leaves lane
//     (col, gq) holding query `col` and four consecutive dims per group.
//
// Memory: K and V tiles go straight from global memory to LDS
// (global_load_lds_dwordx4: no staging registers, no ALU), double buffered
// with one barrier per tile; the loads of tile j+1 are in flight while tile j
// is computed. Both tiles are row-major with a 16-byte-chunk XOR swizzle so
// the matrix-core operand reads are free of bank conflicts: K rows are read
// with ds_read_b128, and the V^T operand is read from the row-major V tile
// with the gfx950 transposing read ds_read_b64_tr_b16 (each 16-lane group
// receives a 4-key x 16-dim block transposed: lane i gets dim i of 4 keys).
// Keys past the end of the request are loaded from its last key (valid
// memory) and masked, so no load is conditional.
//
// Online softmax in base 2 with scale * log2(e) folded into one FMA per
// score. The running max is only raised when a new tile's max exceeds it by
// more than 8 (factor 256), so the O rescale is rare; the result is the same
// softmax (the max only guards the exponent range). P is rounded to bf16 for
// the matrix cores; the normalising sum adds the same rounded values, so each
// output is a convex combination of its values, while the LSE uses the exact
// fp32 sum.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.hpp"
#include "kernels.hpp"
#include "mask.hpp"

namespace mvs {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ constexpr bf16x2_t kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;  // log2 units

template <int D, int BN, int NW, int WM>
struct Tile {
  static constexpr int BM = WM * NW;
  static constexpr int THREADS = 64 * NW;
  static constexpr int ROWB = 2 * D;             // bytes per K or V row in LDS (no pad: swizzled)
  static constexpr int TILEB = BN * ROWB;        // bytes of one K or V tile
  static constexpr int BUFB = 2 * TILEB;         // K tile then V tile
  static constexpr int CHUNKS = D / 8;           // 16-byte chunks per row
  static constexpr int SLOTS = BN * CHUNKS;      // 16-byte slots per tile
  static constexpr int LOADS = SLOTS / THREADS;  // direct loads per thread per tensor per tile
  static_assert(SLOTS % THREADS == 0, "tile must split evenly over the workgroup");
  static_assert(CHUNKS >= 8, "swizzle needs 8 chunks per row");
};

// 16-byte-chunk swizzles (position of logical chunk c in row r).
__device__ inline int k_chunk(int r, int c) { return c ^ (r & 7); }
__device__ inline int v_chunk(int r, int c) { return c ^ ((r & 3) << 1); }

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4v_t;

__device__ inline int xcd_remap(int bid, int n) {
  // Workgroups are dispatched round-robin over the 8 XCDs. Give each XCD a
  // contiguous range of work items so the query tiles of one (request, kv
  // head) - which read the same K and V - share one XCD's L2.
  constexpr int X = 8;
  const int per = n / X;
  if (bid >= per * X) return bid;
  return (bid % X) * per + bid / X;
}

__device__ inline int wave_min(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = min(x, __shfl_xor(x, off));
  return x;
}

__device__ inline int wave_max(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = max(x, __shfl_xor(x, off));
  return x;
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// One matrix-core shape: WM x WM outputs, KD-deep reduction, per wave.
template <int WM>
struct Mfma;

template <>
struct Mfma<32> {
  static constexpr int KD = 16;     // reduction depth per instruction
  static constexpr int REGS = 16;   // fp32 accumulators per lane
  typedef f32x16_t acc_t;
  __device__ static acc_t mma(bf16x8_t a, bf16x8_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // row (M index) of accumulator r in lane group gq
  __device__ static constexpr int row(int r, int gq) { return 8 * (r >> 2) + 4 * gq + (r & 3); }
};

template <>
struct Mfma<16> {
  static constexpr int KD = 32;
  static constexpr int REGS = 4;
  typedef f32x4_t acc_t;
  __device__ static acc_t mma(bf16x8_t a, bf16x8_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static constexpr int row(int r, int gq) { return 4 * gq + r; }
};


template <int D, int BN, int NW, int WM, int MINW>
__global__ __launch_bounds__(64 * NW, MINW) void prefill_bf16_kernel(const PrefillArgs a) {
  using T = Tile<D, BN, NW, WM>;
  using M = Mfma<WM>;
  typedef typename M::acc_t acc_t;
  constexpr int SB = BN / WM;     // score blocks per key tile
  constexpr int OT = D / WM;      // output tiles per wave
  constexpr int QS = D / M::KD;   // Q fragments (reduction steps of K Q^T)
  constexpr int PS = BN / M::KD;  // reduction steps of V^T P^T per key tile
  static_assert(D % M::KD == 0 && BN % M::KD == 0 && BN % WM == 0, "tile shape");
  __shared__ __attribute__((aligned(1024))) char smem[2 * T::BUFB];
  __shared__ int red[4 * NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane % WM, gq = lane / WM;

  // ---- work item: (request b, kv head, query head in group, query tile), heavy tiles first
  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int m_rev = w % a.n_mtiles;
  int rest = w / a.n_mtiles;
  const int g = rest % a.group;
  rest /= a.group;
  const int kvh = rest % a.Hkv;
  const int b = rest / a.Hkv;
  const int h = kvh * a.group + g;
  const int mt = a.n_mtiles - 1 - m_rev;

  const int q0 = a.cu_q[b];
  const int Lq = a.cu_q[b + 1] - q0;
  const int kbase = a.cu_k[b];
  const int Lk = a.cu_k[b + 1] - kbase;
  const int i0 = mt * T::BM;
  if (i0 >= Lq) return;  // whole workgroup: tile past this request's queries
  const int c = Lk - Lq;

  // ---- this lane's query row and its visible keys (table row loaded once)
  const int i = i0 + wave * WM + col;
  const bool valid = i < Lq;
  int ts = -1, te = -1;
  if (a.table != nullptr && valid) {
    ts = a.table[2 * (long long)(q0 + i)];
    te = a.table[2 * (long long)(q0 + i) + 1];
  }
  RowKeys rk = row_keys(a.causal, a.wl, a.wr, c + i, Lk, ts, te);
  TilePlan tp = plan_identity();
  if (valid) {
    plan_add_row(tp, rk);
  } else {
    rk.a_lo = 0;
    rk.a_hi = -1;
    rk.b_lo = 0;
    rk.b_hi = -1;
  }
  const bool two_intervals = __any(rk.b_lo <= rk.b_hi);
  {
    const int lo = wave_min(tp.lo), hi = wave_max(tp.hi), flo = wave_max(tp.flo), fhi = wave_min(tp.fhi);
    if (lane == 0) {
      red[wave] = lo;
      red[NW + wave] = hi;
      red[2 * NW + wave] = flo;
      red[3 * NW + wave] = fhi;
    }
  }
  __syncthreads();
  TilePlan plan = plan_identity();
#pragma unroll
  for (int x = 0; x < NW; ++x) {
    plan.lo = min(plan.lo, red[x]);
    plan.hi = max(plan.hi, red[NW + x]);
    plan.flo = max(plan.flo, red[2 * NW + x]);
    plan.fhi = min(plan.fhi, red[3 * NW + x]);
  }
  // identical in every lane: keep in scalar registers
  plan.lo = __builtin_amdgcn_readfirstlane(plan.lo);
  plan.hi = __builtin_amdgcn_readfirstlane(plan.hi);
  plan.flo = __builtin_amdgcn_readfirstlane(plan.flo);
  plan.fhi = __builtin_amdgcn_readfirstlane(plan.fhi);
  const int kt_lo = plan.lo <= plan.hi ? plan.lo / BN : 0;
  const int ntiles = plan.lo <= plan.hi ? plan.hi / BN - kt_lo + 1 : 0;

  // ---- Q rows of this wave as MFMA B operands (lane: query col, dims KD*s + 8*gq ..)
  bf16x8_t qf[QS];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (long long)(q0 + (valid ? i : 0)) * a.q_st +
                         (long long)h * D + 8 * gq;
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      u32x4_t raw = {0u, 0u, 0u, 0u};
      if (valid) raw = *reinterpret_cast<const u32x4_t*>(qp + M::KD * s);
      qf[s] = __builtin_bit_cast(bf16x8_t, raw);
    }
  }

  // ---- direct global -> LDS tile loads. Load round j of the workgroup fills
  // the 16-byte slots j * THREADS + tid of the tile (each wave 64 consecutive
  // slots); slot (row r, position p) holds logical chunk p ^ swizzle(r) of key
  // row r. With RPL rows per round, thread tid always lands on position
  // p0 = tid % CHUNKS of rows r0 + j * RPL, r0 = tid / CHUNKS.
  static_assert(T::THREADS % T::CHUNKS == 0, "a load round covers whole rows");
  constexpr int RPL = T::THREADS / T::CHUNKS;
  const int r0 = tid / T::CHUNKS, p0 = tid % T::CHUNKS;
  const uint16_t* kg = static_cast<const uint16_t*>(a.k) + (long long)kbase * a.k_st + (long long)kvh * D;
  const uint16_t* vg = static_cast<const uint16_t*>(a.v) + (long long)kbase * a.v_st + (long long)kvh * D;
  const int k_st = (int)a.k_st, v_st = (int)a.v_st;  // token strides fit 32 bits (heads * D)
  auto load_tile = [&](int kt, int buf) {
    char* kb_lds = smem + buf * T::BUFB;
    char* vb_lds = kb_lds + T::TILEB;
    const int key0 = kt * BN;
    const uint16_t* kt_g = kg + (long long)key0 * a.k_st;
    const uint16_t* vt_g = vg + (long long)key0 * a.v_st;
    const bool whole = key0 + BN <= Lk;  // uniform: no key of the tile is past the end
#pragma unroll
    for (int j = 0; j < T::LOADS; ++j) {
      const int r = j * RPL + r0;
      int rk_ = r;
      if (!whole) rk_ = min(key0 + r, Lk - 1) - key0;  // past the end: reload the last key (masked)
      const int dst = (j * NW + wave) * 64 * 16;
      __builtin_amdgcn_global_load_lds(kt_g + rk_ * k_st + k_chunk(r, p0) * 8, (lds_void_t*)(kb_lds + dst), 16, 0,
                                       0);
      __builtin_amdgcn_global_load_lds(vt_g + rk_ * v_st + v_chunk(r, p0) * 8, (lds_void_t*)(vb_lds + dst), 16, 0,
                                       0);
    }
  };

  // ---- per-lane LDS read offsets (bytes within a tile). XOR swizzles only
  // touch the low 3 bits of a chunk index, so every operand address is one of
  // a few per-lane bases plus a compile-time offset.
  // K operand of step st, block kb: row WM*kb + col, logical chunk
  // c = KD*st/8 + gq; its low 3 bits cycle with period KV = 64 / KD.
  constexpr int KV = 64 / M::KD;
  int kbase_off[KV];
#pragma unroll
  for (int x = 0; x < KV; ++x) kbase_off[x] = col * T::ROWB + ((((M::KD / 8) * x + gq) & 7) ^ (col & 7)) * 16;
  // V^T operand (transposing read): this lane's 16-lane group covers dims
  // d0 .. d0+15 of 4 consecutive keys; the lane supplies the 8 bytes at dims
  // d0 + 4*(lane%4) of key k0 + (lane%16)/4. For WM = 32 the groups split the
  // 32 output dims in halves (lanes 16..31, 48..63 hold dims 16..31); the key
  // offset is 4*gq. Key rows keep their index mod 4 (= (lane%16)/4), so the V
  // swizzle is a per-lane constant; the low chunk bits then depend only on
  // the parity of the output tile.
  const int tr_row = (lane & 15) >> 2;
  const int tr_dim = ((WM == 32) ? 16 * ((lane >> 4) & 1) : 0) + 4 * (lane & 3);  // within a WM-dim tile
  const int tr_key = 4 * gq + tr_row;
  constexpr int TPB = 64 / WM;  // output tiles per 8-chunk (128-byte) group of a V row
  int vbase_off[TPB];
#pragma unroll
  for (int x = 0; x < TPB; ++x) {
    const int dim = WM * x + tr_dim;  // < 64: chunk index < 8
    vbase_off[x] = tr_key * T::ROWB + (((dim >> 3) & 7) ^ (tr_row << 1)) * 16 + (dim & 7) * 2;
  }

  // ---- running state
  acc_t o[OT];
#pragma unroll
  for (int dt = 0; dt < OT; ++dt)
#pragma unroll
    for (int r = 0; r < M::REGS; ++r) o[dt][r] = 0.f;
  const float c2 = a.scale_log2;
  float m2 = -INFINITY, l = 0.f, lx = 0.f;  // running max (log2), rounded sum, exact sum
  float sink_raw = 0.f;
  if (a.sink_mode == MVS_SINK_NULL_LOGIT) {
    m2 = a.sinks[h] * kLog2e;
    l = lx = gq == 0 ? 1.f : 0.f;  // the null term is counted once per row
  } else if (a.sink_mode == MVS_SINK_KEY0_BIAS) {
    sink_raw = a.sinks[h] / a.scale;  // scaled below with the scores
  }

  if (ntiles > 0) load_tile(kt_lo, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int kt = kt_lo + j;
    const char* Kt = smem + (j & 1) * T::BUFB;
    const char* Vt = Kt + T::TILEB;
    if (j + 1 < ntiles) load_tile(kt + 1, (j + 1) & 1);

    // S^T = K Q^T
    acc_t s[SB];
#pragma unroll
    for (int kb = 0; kb < SB; ++kb)
#pragma unroll
      for (int r = 0; r < M::REGS; ++r) s[kb][r] = 0.f;
#pragma unroll
    for (int st = 0; st < QS; ++st) {
#pragma unroll
      for (int kb = 0; kb < SB; ++kb) {
        const int off = kbase_off[st % KV] + WM * kb * T::ROWB + ((M::KD * st / 8) & ~7) * 16;
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(Kt + off);
        s[kb] = M::mma(kf, qf[st], s[kb]);
      }
    }

    // element mask on partial tiles only
    const int key0 = kt * BN;
    if (classify_key_tile(plan, key0, key0 + BN - 1) != 2) {
#pragma unroll
      for (int kb = 0; kb < SB; ++kb)
#pragma unroll
        for (int r = 0; r < M::REGS; ++r) {
          const int key = key0 + WM * kb + M::row(r, gq);
          bool vis = key >= rk.a_lo && key <= rk.a_hi;
          if (two_intervals) vis = vis || (key >= rk.b_lo && key <= rk.b_hi);
          s[kb][r] = vis ? s[kb][r] : -INFINITY;
        }
    }
    if (a.sink_mode == MVS_SINK_KEY0_BIAS && kt == 0 && gq == 0) s[0][0] += sink_raw;  // key 0

    // online softmax (base 2)
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < SB; ++kb)
#pragma unroll
      for (int r = 0; r < M::REGS; ++r) mx = fmaxf(mx, s[kb][r]);
#pragma unroll
    for (int off = WM; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    const float mnew = mx * c2;
    const bool raise = mnew > m2 + kRescaleSlack;
    if (__any(raise)) {
      const float mu = raise ? mnew : m2;
      const float alpha = raise ? __builtin_amdgcn_exp2f(m2 - mu) : 1.f;
      l *= alpha;
      lx *= alpha;
#pragma unroll
      for (int dt = 0; dt < OT; ++dt)
#pragma unroll
        for (int r = 0; r < M::REGS; ++r) o[dt][r] *= alpha;
      m2 = mu;
    }
    const float mb = m2 == -INFINITY ? 0.f : m2;
    float rsx = 0.f;
#pragma unroll
    for (int kb = 0; kb < SB; ++kb)
#pragma unroll
      for (int r = 0; r < M::REGS; ++r) {
        s[kb][r] = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c2, -mb));
        rsx += s[kb][r];
      }
    lx += rsx;

    // P^T as bf16 B operands. Step u covers keys KD*u .. KD*u + KD-1; its 8
    // values per lane are accumulators (8u .. 8u+7) of the flattened score
    // blocks, whose keys are KD*u + {4*gq + 0..3, KD/2 + 4*gq + 0..3}.
    bf16x8_t pb[PS];
    float rs = 0.f;
#pragma unroll
    for (int u = 0; u < PS; ++u) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int flat = 8 * u + e;
        pb[u][e] = (__bf16)s[flat / M::REGS][flat % M::REGS];
      }
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        bf16x2_t pair = {pb[u][e], pb[u][e + 1]};
        rs = __builtin_amdgcn_fdot2_f32_bf16(pair, kOnes2, rs, false);
      }
    }
    l += rs;

    // O^T += V^T P^T; A operand by transposing reads of the row-major V tile
#pragma unroll
    for (int dt = 0; dt < OT; ++dt) {
      // tile dt: low chunk bits repeat with period TPB, the rest is an immediate
      const int hi_off = (dt / TPB) * 128;
#pragma unroll
      for (int u = 0; u < PS; ++u) {
        short4v half[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int krow = M::KD * u + hf * (M::KD / 2);
          const int off = vbase_off[dt % TPB] + hi_off + krow * T::ROWB;
          half[hf] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v_t*)(Vt + off));
        }
        const u32x4_t vv = {__builtin_bit_cast(u32x2_t, half[0]).x, __builtin_bit_cast(u32x2_t, half[0]).y,
                            __builtin_bit_cast(u32x2_t, half[1]).x, __builtin_bit_cast(u32x2_t, half[1]).y};
        o[dt] = M::mma(__builtin_bit_cast(bf16x8_t, vv), pb[u], o[dt]);
      }
    }

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // tile j+1 has landed in LDS
    __syncthreads();
  }

  // ---- epilogue
  float lt = l, ltx = lx;
#pragma unroll
  for (int off = WM; off < 64; off <<= 1) {
    lt += __shfl_xor(lt, off);
    ltx += __shfl_xor(ltx, off);
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (valid) {
    uint16_t* op = static_cast<uint16_t*>(a.o) + (long long)(q0 + i) * a.o_st + (long long)h * D;
#pragma unroll
    for (int dt = 0; dt < OT; ++dt)
#pragma unroll
      for (int grp = 0; grp < M::REGS / 4; ++grp) {
        bf16x4_t val;
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] = (__bf16)(o[dt][4 * grp + e] * inv);
        *reinterpret_cast<bf16x4_t*>(op + WM * dt + M::row(4 * grp, gq)) = val;
      }
    if (a.lse != nullptr && gq == 0) {
      const int n_total = a.cu_q[a.num_seqs];
      a.lse[(long long)h * n_total + q0 + i] = ltx > 0.f ? (m2 + __log2f(ltx)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, int BN, int NW, int WM, int MINW>
hipError_t launch(PrefillArgs a, int max_seqlen_q, hipStream_t stream) {
  using T = Tile<D, BN, NW, WM>;
  a.n_mtiles = (max_seqlen_q + T::BM - 1) / T::BM;
  const long long blocks = (long long)a.n_mtiles * a.Hq * a.num_seqs;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, BN, NW, WM, MINW>), dim3((unsigned)blocks), dim3(T::THREADS), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

int prefill_bf16_block_m(int head_dim) { return head_dim == 512 ? 64 : 128; }

int prefill_bf16_block_n(int head_dim) { return head_dim >= 256 ? 32 : 64; }

hipError_t launch_prefill_bf16(PrefillArgs a, int head_dim, int max_seqlen_q, hipStream_t stream) {
  switch (head_dim) {
    case 64:
      return launch<64, 64, 4, 32, 1>(a, max_seqlen_q, stream);
    case 128:
      return launch<128, 64, 4, 32, 1>(a, max_seqlen_q, stream);
    case 256:
      return launch<256, 32, 4, 32, 2>(a, max_seqlen_q, stream);
    case 512:
      return launch<512, 32, 4, 16, 1>(a, max_seqlen_q, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace mvs
