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
// Work decomposition. One workgroup = NW waves = HPW query heads of one kv
// head and BM = WM * NW / HPW consecutive query rows of one request; each
// wave owns WM rows of one of the heads (32, or 16 where the fp32 O
// accumulator of 32 rows would not fit in registers). With HPW > 1 the
// heads that share a kv head share every K/V tile load of the workgroup.
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
#include <type_traits>

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

// Build option (schedule experiments; the default is the measured best).
#ifndef MVS_PREFILL_QLDS
#define MVS_PREFILL_QLDS 1
#endif
// Output rows are written with nontemporal (streaming) stores: O is never
// read back by the kernel, and ordinary stores leave it dirty in L2, where it
// displaces K/V tiles other workgroups still read and must be written back
// when the kernel ends, before the next launch starts.
// Kernel 1 waves skip the key tiles none of their own rows see (the
// workgroup's tile range is the union over all its waves), and mask only the
// tiles some of their own rows see in part.
#ifndef MVS_PREFILL_WAVE_FULL
#define MVS_PREFILL_WAVE_FULL 1
#endif
#ifndef MVS_PREFILL_WAVE_SKIP
#define MVS_PREFILL_WAVE_SKIP 1
#endif
#ifndef MVS_PREFILL_NT_STORE
#define MVS_PREFILL_NT_STORE 1
#endif


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

// 16-byte-chunk swizzles: logical chunk c of row r sits at position c ^ sw(r)
// (an involution, so the same formula maps positions back to chunks). Rows
// are a multiple of 256 bytes, so only the position decides the LDS bank. K
// rows are read 16 at a time (ds_read_b128, one row per lane): a 4-bit XOR
// gives 16 rows 16 distinct 16-byte slots of a 256-byte bank window. V is
// read by transposing 8-byte reads, 4 rows x 32 bytes per 16-lane group; the
// XOR values below give every row/chunk pair that is read together its own
// slot, for both 32- and 64-bank LDS.
template <int CHUNKS>
__device__ inline int k_swz(int r) {
  return CHUNKS >= 16 ? (r & 15) : (r & 7);
}
template <int WM, int CHUNKS>
__device__ inline int v_swz(int r) {
  if constexpr (CHUNKS < 16) return (r & 3) << 1;
  if constexpr (WM == 32) return ((r & 3) << 1) ^ ((r & 1) << 3);
  return (r & 7) << 1;
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4v_t;

__device__ inline int xcd_remap(int bid, int n, int chunk) {
  // Workgroups are dispatched round-robin over the 8 XCDs. Work items come
  // in chunks of `chunk` consecutive items that read the same K and V (the
  // query tiles of every q head of one (request, kv head)); each chunk goes
  // whole to one XCD, so its K/V stays in that XCD's L2, and chunks are dealt
  // round-robin over the XCDs, so every XCD gets the same mix of long and
  // short requests (query tiles past a short request's end exit at once).
  constexpr int X = 8;
  const long long span = (long long)X * chunk;  // a chunk may be large when one request is very long
  const int full = chunk > 0 ? (int)(n / span * span) : 0;
  if (bid >= full) return bid;
  const int xcd = bid % X, slot = bid / X;
  return ((slot / chunk) * X + xcd) * chunk + slot % chunk;
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

// Max over the lanes that hold the same query row: lane l and l ^ off for
// off = WM .. 32. The 32-lane step is a VALU lane swap (no LDS round trip).
template <int WM>
__device__ inline float cross_group_max(float x) {
#pragma unroll
  for (int off = WM; off < 32; off <<= 1) x = fmaxf(x, __shfl_xor(x, off));
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

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


// ---------------------------------------------------------------- shared pieces

// Everything a workgroup knows about its query tile after the setup phase.
struct QTile {
  int h, kvh, b, q0, Lq, kbase, Lk, i;
  bool valid;
  RowKeys rk;          // this lane's visible keys (first interval, optional second)
  unsigned wa, wb;     // interval widths (0 = empty)
  bool two_intervals;  // some lane of the wave has a second interval
  TilePlan plan;       // reduced over the workgroup's valid rows (uniform)
  int kt_lo, ntiles;   // key tiles to visit
  int wk_lo, wk_hi;    // lowest and highest key any row of this wave sees (lo > hi: none)
  int wf_lo, wf_hi;    // keys every valid row of this wave sees (its tiles inside need no mask)
};

// Key tile [k0, k1] seen whole by every row that masks with this tile plan:
// with MVS_PREFILL_WAVE_FULL by every row of the wave, else of the workgroup.
__device__ inline bool tile_full(const QTile& t, int k0, int k1) {
  if constexpr (MVS_PREFILL_WAVE_FULL) return k0 >= t.wf_lo && k1 <= t.wf_hi;
  return classify_key_tile(t.plan, k0, k1) == 2;
}

// Work-item decode, per-row key intervals and the workgroup tile plan.
// Returns false when the workgroup has no query rows (whole-workgroup exit).
template <int D, int WM>
__device__ inline void load_q(const PrefillArgs& a, const QTile& t, bf16x8_t* qf);

template <int D, int WM>
__device__ inline void load_q_lds(const PrefillArgs& a, const QTile& t, char* blk);

// Also issues the wave's Q loads as soon as its rows are known: with QLDS
// into the wave's LDS block qblk (ahead of the table loads; the caller waits
// for them, reads the fragments and synchronises before the LDS is reused),
// else into qf (the caller waits with consume_q).
template <int NW, int WM, int BM, int BN, int D, bool SCAN = false, int HPW = 1, bool QLDS = false>
__device__ inline bool setup_qtile(const PrefillArgs& a, int* red, QTile& t, bf16x8_t* qf, int2* rsh = nullptr,
                                   char* qblk = nullptr) {
  constexpr int RW = NW / HPW;  // waves per query head
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane % WM;
  // (request b, kv head, HPW-head slice of the group, query tile), heavy tiles first
  const int slices = a.group / HPW;
  const int w = xcd_remap(blockIdx.x, gridDim.x, slices * a.n_mtiles);
  const int m_rev = w % a.n_mtiles;
  int rest = w / a.n_mtiles;
  const int g = rest % slices;
  rest /= slices;
  t.kvh = rest % a.Hkv;
  const int b = rest / a.Hkv;
  t.b = b;
  t.h = t.kvh * a.group + g * HPW + wave / RW;
  const int mt = a.n_mtiles - 1 - m_rev;
  t.q0 = a.cu_q[b];
  t.Lq = a.cu_q[b + 1] - t.q0;
  if (a.block_table != nullptr) {
    t.kbase = 0;
    t.Lk = a.seq_lens_k[b];
  } else {
    t.kbase = a.cu_k[b];
    t.Lk = a.cu_k[b + 1] - t.kbase;
  }
  const int i0 = mt * BM;
  if (i0 >= t.Lq) return false;
  t.i = i0 + (wave % RW) * WM + col;
  t.valid = t.i < t.Lq;
  if constexpr (QLDS)
    load_q_lds<D, WM>(a, t, qblk);
  else if constexpr (SCAN)
    load_q<D, WM>(a, t, qf);
  int ts = -1, te = -1;
  if constexpr (SCAN) {
    // the request's range list into LDS; each row takes the last valid range
    // holding its position (what the table builder stores)
    const int* src = a.scan_ranges + 2 * (long long)b * a.max_ranges;
    for (int r = tid; r < a.max_ranges; r += 64 * NW) rsh[r] = make_int2(src[2 * r], src[2 * r + 1]);
    __syncthreads();
    const int p = (t.Lk - t.Lq) + t.i;
    for (int r = 0; r < a.max_ranges; ++r) {
      const int2 x = rsh[r];
      if (t.valid && x.x < x.y && x.x <= p && p <= x.y) {
        ts = x.x;
        te = x.y;
      }
    }
  } else if (a.table != nullptr && t.valid) {  // the row's range, loaded once
    ts = a.table[2 * (long long)(t.q0 + t.i)];
    te = a.table[2 * (long long)(t.q0 + t.i) + 1];
  }
  if constexpr (!QLDS && !SCAN) {
    // Q after the table: the plan waits only for the table rows, and the Q
    // loads land while the plan is reduced and the first tiles are requested
    __builtin_amdgcn_sched_barrier(0);
    load_q<D, WM>(a, t, qf);
  }
  t.rk = row_keys(a.causal, a.wl, a.wr, (t.Lk - t.Lq) + t.i, t.Lk, ts, te);
  TilePlan tp = plan_identity();
  if (t.valid) {
    plan_add_row(tp, t.rk);
  } else {
    t.rk.a_lo = 0;
    t.rk.a_hi = -1;
    t.rk.b_lo = 0;
    t.rk.b_hi = -1;
  }
  t.two_intervals = __any(t.rk.b_lo <= t.rk.b_hi);
  t.wa = (unsigned)max(t.rk.a_hi - t.rk.a_lo + 1, 0);
  t.wb = (unsigned)max(t.rk.b_hi - t.rk.b_lo + 1, 0);
  {
    const int lo = wave_min(tp.lo), hi = wave_max(tp.hi), flo = wave_max(tp.flo), fhi = wave_min(tp.fhi);
    t.wk_lo = __builtin_amdgcn_readfirstlane(lo);
    t.wk_hi = __builtin_amdgcn_readfirstlane(hi);
    t.wf_lo = __builtin_amdgcn_readfirstlane(flo);
    t.wf_hi = __builtin_amdgcn_readfirstlane(fhi);
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
  t.plan.lo = __builtin_amdgcn_readfirstlane(plan.lo);
  t.plan.hi = __builtin_amdgcn_readfirstlane(plan.hi);
  t.plan.flo = __builtin_amdgcn_readfirstlane(plan.flo);
  t.plan.fhi = __builtin_amdgcn_readfirstlane(plan.fhi);
  t.kt_lo = t.plan.lo <= t.plan.hi ? t.plan.lo / BN : 0;
  t.ntiles = t.plan.lo <= t.plan.hi ? t.plan.hi / BN - t.kt_lo + 1 : 0;
  return true;
}

// The wave's Q rows as MFMA B operands (lane: query col, dims KD*s + 8*gq ..).
template <int D, int WM>
__device__ inline void load_q(const PrefillArgs& a, const QTile& t, bf16x8_t* qf) {
  using M = Mfma<WM>;
  const int gq = (threadIdx.x & 63) / WM;
  const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (long long)(t.q0 + (t.valid ? t.i : 0)) * a.q_st +
                       (long long)t.h * D + 8 * gq;
#pragma unroll
  for (int s = 0; s < D / M::KD; ++s) {
    u32x4_t raw = {0u, 0u, 0u, 0u};
    if (t.valid) raw = *reinterpret_cast<const u32x4_t*>(qp + M::KD * s);
    qf[s] = __builtin_bit_cast(bf16x8_t, raw);
  }
}

// Make the compiler wait for the Q loads here (called after the first tile
// loads are issued, so the two latencies overlap), so that it never re-checks
// the memory counter inside the key loop, where the tile loads it does not
// track are in flight.
template <int N>
__device__ inline void consume_q(const bf16x8_t* qf) {
#pragma unroll
  for (int s = 0; s < N; ++s) asm volatile("" ::"v"(qf[s]));
}

// Direct global -> LDS load of one K or V tile. Load round j of the workgroup
// fills the 16-byte slots j * THREADS + tid (each wave 64 consecutive slots,
// one instruction); slot (row r, position p) receives logical chunk
// p ^ swizzle(r) of key row r. Thread tid always lands on position
// p0 = tid % CHUNKS of rows r0 + j * RPL, so its byte offset from the tile's
// first key row is a per-thread constant (computed once) and the tile base is
// uniform (scalar registers). Keys past the end of the request reload its
// last key (valid memory; masked later).
//
// The load is issued as global_load_lds_dwordx4 in its scalar-base form
// (64-bit base in SGPRs, 32-bit per-lane offset). It is written as inline
// assembly so that the compiler does not treat it as an LDS store that every
// later LDS read must wait for: the kernels order these loads explicitly
// with "s_waitcnt vmcnt(0)" and a workgroup barrier before the tile is read,
// and the tile being loaded is never the one being read. M0 holds the LDS
// destination of the wave's 64 slots; nothing else in these kernels uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is listed as clobbered on purpose
__device__ inline void lds_dma16(unsigned voff, const char* sbase, unsigned lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(lds_addr)
      : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ inline unsigned lds_u32(const char* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Wait until at most N of this wave's vector memory loads are in flight.
// Loads complete in issue order, so this waits for everything but the last N.
template <int N>
__device__ inline void vm_wait() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Where the key rows of one tensor (K or V) of this (request, kv head) live.
struct KVSrc {
  const char* base;   // contiguous: the request's first key row; paged: the cache plus the kv head offset
  int tok_stb;        // bytes between consecutive tokens (rows, or slots of a page)
  long long blk_stb;  // paged: bytes between pages
  const int* bt;      // paged: the request's block-table row
  int max_blocks, num_blocks, page_log2;
};

template <int D>
__device__ inline KVSrc kv_src(const PrefillArgs& a, int kvh, int b, int kbase, bool is_v) {
  KVSrc s;
  const char* t = static_cast<const char*>(is_v ? a.v : a.k);
  const long long st = is_v ? a.v_st : a.k_st;
  s.tok_stb = (int)(st * 2);
  if (a.block_table != nullptr) {
    s.base = t + 2 * (long long)kvh * a.head_st;
    s.blk_stb = 2 * a.blk_st;
    const unsigned long long row = reinterpret_cast<unsigned long long>(a.block_table + (long long)b * a.max_blocks);
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)row);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(row >> 32));
    s.bt = reinterpret_cast<const int*>(((unsigned long long)hi << 32) | lo);
    s.max_blocks = a.max_blocks;
    s.num_blocks = a.num_blocks;
    s.page_log2 = a.page_log2;
  } else {
    s.base = t + 2 * ((long long)kbase * st + (long long)kvh * D);
    s.blk_stb = 0;
    s.bt = nullptr;
    s.max_blocks = s.num_blocks = s.page_log2 = 0;
  }
  return s;
}

// global_load_lds_dwordx4 with a full 64-bit address per lane (paged rows).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is listed as clobbered on purpose
__device__ inline void lds_dma16_v(const char* vaddr, unsigned lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(vaddr), "s"(lds_addr)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// The wave's WM query rows of head t.h into its own LDS block blk, laid out
// like a K tile (row-major, 16-byte chunks permuted by k_swz), so that the
// B-operand fragments read back with OperandAddr::k_off. Each direct
// global->LDS load moves 64 consecutive 16-byte chunks of whole rows; loads
// straight into the MFMA register layout would touch 32 rows per
// instruction, 16 bytes of each, and take the address unit several times as
// long. Rows past the request's end repeat its last row (finite values; the
// outputs of those rows are never stored).
template <int D, int WM>
__device__ inline void load_q_lds(const PrefillArgs& a, const QTile& t, char* blk) {
  constexpr int ROWB = 2 * D, CH = ROWB / 16;  // bytes, 16-byte chunks per row
  static_assert(CH <= 64 && 64 % CH == 0, "whole rows per load");
  constexpr int RPL = 64 / CH;          // rows per load
  constexpr int NL = WM * ROWB / 1024;  // loads per wave
  const int lane = threadIdx.x & 63;
  const int row0 = __builtin_amdgcn_readfirstlane(t.i - lane % WM);  // the wave's first row
  const uint16_t* qh = static_cast<const uint16_t*>(a.q) + (long long)t.q0 * a.q_st + (long long)t.h * D;
  const unsigned l0 = lds_u32(blk);
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    const int r = j * RPL + lane / CH;
    const int row = min(row0 + r, t.Lq - 1);
    const int c = (lane % CH) ^ k_swz<CH>(r);
    lds_dma16_v(reinterpret_cast<const char*>(qh + (long long)row * a.q_st + c * 8), l0 + j * 1024);
  }
}

template <int D, int BN, int NW, int WM, bool IS_V>
struct TileLoader {
  using T = Tile<D, BN, NW, WM>;
  static_assert(T::THREADS % T::CHUNKS == 0, "a load round covers whole rows");
  static constexpr int RPL = T::THREADS / T::CHUNKS;  // rows per load round
  // The swizzles depend on the row index mod 16 at most, so the per-thread
  // offset of round j repeats every P rounds up to a uniform row offset, which
  // goes into the scalar base instead of a register.
  static constexpr int P = (RPL >= 16 ? 1 : 16 / RPL) < T::LOADS ? (RPL >= 16 ? 1 : 16 / RPL) : T::LOADS;
  static_assert(T::LOADS % P == 0, "load rounds split into whole periods");
  unsigned voff[P];  // per-thread offsets from the first row of rounds 0..P-1
  __device__ static int swz(int r) { return IS_V ? v_swz<WM, T::CHUNKS>(r) : k_swz<T::CHUNKS>(r); }
  __device__ explicit TileLoader(int stb) {
    const int tid = threadIdx.x;
    const int r0 = tid / T::CHUNKS, p0 = tid % T::CHUNKS;
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const int r = j * RPL + r0;
      voff[j] = (unsigned)(r * stb + ((p0 ^ swz(r)) << 4));
    }
  }
  // Paged rows: each row's page comes from the block table; rows past the end
  // reload the last key; an entry outside [0, num_blocks) reads page 0. key0
  // is a multiple of BN and pages are powers of two >= 16, so a tile spans at
  // most BN / 16 pages, and the rows of a 16-row group share a page. The
  // table is read with scalar loads through the constant address space: a
  // vector load would join the DMA loads' vmcnt queue and its wait would
  // drain the tiles in flight.
  __device__ void load_paged(const KVSrc& s, int key0, int Lk, char* lds) const {
    constexpr int NP = BN / 16;
    const int wave_u = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const unsigned l0 = lds_u32(lds) + wave_u * 1024;
    const int lg = s.page_log2, pmask = (1 << lg) - 1;
    const int pg0 = __builtin_amdgcn_readfirstlane(key0 >> lg);
    const int last_pg = min((Lk - 1) >> lg, s.max_blocks - 1);  // never past the table row
    using cint = __attribute__((address_space(4))) const int;
    const cint* bt = (const cint*)s.bt;
    int pids[NP];
#pragma unroll
    for (int x = 0; x < NP; ++x) {
      const int v = bt[max(min(pg0 + x, last_pg), 0)];
      pids[x] = (v >= 0 && v < s.num_blocks) ? v : 0;
    }
    if (key0 + BN <= Lk && (RPL <= 16 || (1 << lg) >= RPL)) {
      // whole tile inside the request and every load round within one page:
      // a uniform base per round plus the contiguous loader's lane offsets
#pragma unroll
      for (int j = 0; j < T::LOADS; ++j) {
        const int kj = key0 + (j - j % P) * RPL;  // first key of round j's row group
        const int rel = (kj >> lg) - pg0;
        int phys = pids[0];
#pragma unroll
        for (int x = 1; x < NP; ++x) phys = rel == x ? pids[x] : phys;
        const char* base = s.base + (long long)phys * s.blk_stb + (long long)(kj & pmask) * s.tok_stb;
        lds_dma16(voff[j % P], base, l0 + j * NW * 1024);
      }
      return;
    }
    const int tid = threadIdx.x;
    const int r0 = tid / T::CHUNKS, p0 = tid % T::CHUNKS;
#pragma unroll
    for (int j = 0; j < T::LOADS; ++j) {
      const int r = j * RPL + r0;
      const int key = min(key0 + r, Lk - 1);
      const int rel = (key >> lg) - pg0;
      int phys = pids[0];
#pragma unroll
      for (int x = 1; x < NP; ++x) phys = rel == x ? pids[x] : phys;
      const char* addr = s.base + (long long)phys * s.blk_stb + (long long)(key & pmask) * s.tok_stb +
                         ((p0 ^ swz(r)) << 4);
      lds_dma16_v(addr, l0 + j * NW * 1024);
    }
  }
  template <bool PAGED>
  __device__ void load_src(const KVSrc& s, int key0, int Lk, char* lds) const {
    if constexpr (PAGED)
      load_paged(s, key0, Lk, lds);
    else
      load(s.base, s.tok_stb, key0, Lk, lds);
  }
  // g: the request's first key row of this kv head; key0: first key of the tile.
  __device__ void load(const char* g, int stb, int key0, int Lk, char* lds) const {
    const int wave_u = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const char* base = g + (long long)key0 * stb;
    const unsigned l0 = lds_u32(lds) + wave_u * 1024;
    if (key0 + BN <= Lk) {  // uniform: the whole tile is inside the request
#pragma unroll
      for (int j = 0; j < T::LOADS; ++j)
        lds_dma16(voff[j % P], base + (long long)(j - j % P) * RPL * stb, l0 + j * NW * 1024);
    } else {
      const int tid = threadIdx.x;
      const int r0 = tid / T::CHUNKS, p0 = tid % T::CHUNKS;
      const int last = Lk - 1 - key0;
#pragma unroll
      for (int j = 0; j < T::LOADS; ++j) {
        const int r = j * RPL + r0;
        const unsigned off = (unsigned)(min(r, last) * stb + ((p0 ^ swz(r)) << 4));
        lds_dma16(off, base, l0 + j * NW * 1024);
      }
    }
  }
};

// Per-lane LDS read offsets (bytes within a tile). Rows are multiples of 256
// bytes and the swizzles only touch chunk bits 0..3, so an operand address is
// (per-lane base) XOR (compile-time bits 4..7) plus a compile-time multiple
// of 256.
//  K operand, step st, block kb: row WM*kb + col, logical chunk (KD/8)*st + gq
//    (gq < KD/8: the two terms occupy disjoint bits).
//  V^T operand (transposing read): this lane's 16-lane group covers dims
//    d0 .. d0+15 of 4 consecutive keys; the lane supplies the 8 bytes at dims
//    d0 + 4*(lane%4) of key k0 + (lane%16)/4. For WM = 32 the groups split
//    the 32 output dims in halves (lanes 16..31, 48..63 hold dims 16..31);
//    the key offset is 4*gq. Key rows read together share their index mod 8
//    with tr_key, so the V swizzle is a per-lane constant.
template <int D, int WM>
struct OperandAddr {
  static constexpr int ROWB = 2 * D, CHUNKS = D / 8;
  static_assert(ROWB % 256 == 0 || CHUNKS == 8, "rows must be whole bank windows (or 8-chunk rows)");
  int k_rd, v_rd;
  __device__ OperandAddr() {
    const int lane = threadIdx.x & 63;
    const int col = lane % WM, gq = lane / WM;
    k_rd = col * ROWB + ((gq ^ k_swz<CHUNKS>(col)) << 4);
    const int tr_row = (lane & 15) >> 2;
    const int tr_dim = ((WM == 32) ? 16 * ((lane >> 4) & 1) : 0) + 4 * (lane & 3);  // within a WM-dim tile
    const int tr_key = 4 * gq + tr_row;
    v_rd = tr_key * ROWB + (((tr_dim >> 3) ^ v_swz<WM, CHUNKS>(tr_key)) << 4) + (tr_dim & 7) * 2;
  }
  // K fragment of reduction step st for score block kb
  __device__ static int k_off(int k_rd_, int st, int kb) {
    constexpr int CPS = Mfma<WM>::KD / 8;  // chunks per step
    const int c = CPS * st;
    return (k_rd_ ^ ((c & 15) << 4)) + (c >> 4) * 256 + WM * kb * ROWB;
  }
  // V^T fragment half hf of reduction step u for output tile dt
  __device__ static int v_off(int v_rd_, int dt, int u, int hf) {
    constexpr int CPT = WM / 8;  // chunks per output tile
    const int c = CPT * dt;
    const int krow = Mfma<WM>::KD * u + hf * (Mfma<WM>::KD / 2);
    return (v_rd_ ^ ((c & 15) << 4)) + (c >> 4) * 256 + krow * ROWB;
  }
};

// Initial score accumulator of a key tile: 0 where the key is visible, -inf
// where it is not (finite products keep -inf through the MFMA sums), plus the
// key-0 sink. Full tiles start from 0.
template <int WM, int SB, bool SCAN = false>
__device__ inline void init_scores(typename Mfma<WM>::acc_t* s, const PrefillArgs& a, const QTile& t, int kt,
                                   int BN_, float sink_raw, const int2* rsh = nullptr) {
  using M = Mfma<WM>;
  const int gq = (threadIdx.x & 63) / WM;
  const int key0 = kt * BN_;
  if (!SCAN && tile_full(t, key0, key0 + BN_ - 1)) {
#pragma unroll
    for (int kb = 0; kb < SB; ++kb)
#pragma unroll
      for (int r = 0; r < M::REGS; ++r) s[kb][r] = 0.f;
  } else if (SCAN && classify_key_tile(t.plan, key0, key0 + BN_ - 1) == 2) {
#pragma unroll
    for (int kb = 0; kb < SB; ++kb)
#pragma unroll
      for (int r = 0; r < M::REGS; ++r) s[kb][r] = 0.f;
  } else {
    // key k is in [lo, lo + width) iff (unsigned)(k - lo) < width. (The empty
    // asm keeps this uniform branch a branch: without it the compiler
    // evaluates both sides on every tile.)
    asm volatile("; partial key tile" ::);
    if constexpr (SCAN) {
      // Range-scan baseline: base term, then every range of the request for
      // every score: visible when the query's position and the key lie in the
      // same range (past side clamped by the window).
      const int p = (t.Lk - t.Lq) + t.i;
      const RowKeys bk = row_keys(a.causal, a.wl, a.wr, p, t.Lk, -1, -1);
      const int tb0 = key0 - bk.a_lo;
      const unsigned wb0 = t.valid ? (unsigned)max(bk.a_hi - bk.a_lo + 1, 0) : 0u;
      bool vis[SB][M::REGS];
#pragma unroll
      for (int kb = 0; kb < SB; ++kb)
#pragma unroll
        for (int r = 0; r < M::REGS; ++r) vis[kb][r] = (unsigned)(tb0 + WM * kb + M::row(r, gq)) < wb0;
      for (int q = 0; q < a.max_ranges; ++q) {
        const int2 x = rsh[q];
        const bool in = t.valid && x.x < x.y && x.x <= p && p <= x.y;
        const int lo = max(a.wl >= 0 ? max(x.x, p - a.wl) : x.x, 0);
        const int hi = min(x.y, t.Lk - 1);
        const unsigned w = in ? (unsigned)max(hi - lo + 1, 0) : 0u;
        const int tm = key0 - lo;
#pragma unroll
        for (int kb = 0; kb < SB; ++kb)
#pragma unroll
          for (int r = 0; r < M::REGS; ++r) vis[kb][r] |= (unsigned)(tm + WM * kb + M::row(r, gq)) < w;
      }
#pragma unroll
      for (int kb = 0; kb < SB; ++kb)
#pragma unroll
        for (int r = 0; r < M::REGS; ++r) s[kb][r] = vis[kb][r] ? 0.f : -INFINITY;
      if (a.sink_mode == MVS_SINK_KEY0_BIAS && kt == 0 && gq == 0) s[0][0] += sink_raw;  // key 0
      return;
    }
    const int ta = key0 - t.rk.a_lo;
    if (!t.two_intervals) {  // uniform; every table built by build_query_range_table lands here
#pragma unroll
      for (int kb = 0; kb < SB; ++kb)
#pragma unroll
        for (int r = 0; r < M::REGS; ++r) s[kb][r] = (unsigned)(ta + WM * kb + M::row(r, gq)) < t.wa ? 0.f : -INFINITY;
    } else {
      const int tb = key0 - t.rk.b_lo;
#pragma unroll
      for (int kb = 0; kb < SB; ++kb)
#pragma unroll
        for (int r = 0; r < M::REGS; ++r) {
          const int off = WM * kb + M::row(r, gq);
          const bool vis = ((unsigned)(ta + off) < t.wa) | ((unsigned)(tb + off) < t.wb);
          s[kb][r] = vis ? 0.f : -INFINITY;
        }
    }
  }
  if (a.sink_mode == MVS_SINK_KEY0_BIAS && kt == 0 && gq == 0) s[0][0] += sink_raw;  // key 0
}

// Running online-softmax state of one lane (one query row, base 2).
struct RowState {
  float m2;  // running max (log2 units)
  float l;   // sum of the bf16-rounded weights (normalises O)
  float lx;  // exact fp32 sum (LSE only)
};

// O accumulator rescale for the pipelined kernel, whose accumulators live in
// AGPRs: read, multiply, write back in place, so the register allocator never
// has to move O into VGPRs for the (rare) rescale. The leading wait states
// cover a matrix-core result still in flight into the accumulator; the
// trailing ones cover the next MFMA reading the rewritten value.
template <int REGS, typename Acc>
__device__ inline void rescale_agpr(Acc& o, float alpha) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::);
#pragma unroll
  for (int r = 0; r < REGS; ++r) {
    float tmp;
    asm volatile(
        "v_accvgpr_read_b32 %1, %0\n\t"
        "v_mul_f32 %1, %1, %2\n\t"
        "v_accvgpr_write_b32 %0, %1"
        : "+a"(o[r]), "=&v"(tmp)
        : "v"(alpha));
  }
  asm volatile("s_nop 4" ::);
}

// Epilogue: normalise and store O (bf16) and the LSE.
// store_out for 32-row waves, staged through LDS so that every global store
// writes 16 contiguous bytes per lane along whole output rows: the O^T
// registers hold 4 dims of one row per group, so direct stores scatter 8-byte
// pieces over 32 rows per instruction. `stage` is this wave's kStageBytes of
// LDS (free once the key loop is done); the wave writes and reads only its
// own stage, 64 dims per pass.
constexpr int kStageRowB = 64 * 2 + 16;   // a 64-dim bf16 row plus padding (bank spread)
constexpr int kStageBytes = 32 * kStageRowB;

// Rows i - i % 32 .. of head h in the request starting at packed row q0 (Lq rows).
template <int D, bool LSE>
__device__ inline void store_out_staged(const PrefillArgs& a, int h, int q0, int Lq, int i, bool valid,
                                        const f32x16_t* o, const RowState& st, char* stage) {
  using M = Mfma<32>;
  const int lane = threadIdx.x & 63;
  const int col = lane % 32, gq = lane / 32;
  float lt = st.l, ltx = st.lx;
  lt += __shfl_xor(lt, 32);
  ltx += __shfl_xor(ltx, 32);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const int base = i - col;  // the wave's first row (may be past Lq)
  uint16_t* obase = static_cast<uint16_t*>(a.o) + (long long)q0 * a.o_st + (long long)h * D;
#pragma unroll
  for (int p = 0; p < D / 64; ++p) {
#pragma unroll
    for (int dl = 0; dl < 2; ++dl) {
      const int dt = 2 * p + dl;
#pragma unroll
      for (int grp = 0; grp < M::REGS / 4; ++grp) {
        bf16x4_t val;
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] = (__bf16)(o[dt][4 * grp + e] * inv);
        *reinterpret_cast<bf16x4_t*>(stage + col * kStageRowB + (32 * dl + M::row(4 * grp, gq)) * 2) = val;
      }
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int r = 8 * it + lane / 8, c = lane % 8;  // row, 16-byte chunk of its 128 bytes
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stage + r * kStageRowB + c * 16);
      if (base + r < Lq) {
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(obase + (long long)(base + r) * a.o_st + 64 * p + 8 * c);
        if constexpr (MVS_PREFILL_NT_STORE)
          __builtin_nontemporal_store(v, dst);
        else
          *dst = v;
      }
    }
  }
  if (LSE && gq == 0 && valid) {
    const int n_total = a.cu_q[a.num_seqs];
    a.lse[(long long)h * n_total + q0 + i] = ltx > 0.f ? (st.m2 + __log2f(ltx)) * kLn2 : -INFINITY;
  }
}

template <int D, int WM, bool LSE>
__device__ inline void store_out(const PrefillArgs& a, const QTile& t, typename Mfma<WM>::acc_t* o,
                                 const RowState& st) {
  using M = Mfma<WM>;
  const int gq = (threadIdx.x & 63) / WM;
  float lt = st.l, ltx = st.lx;
#pragma unroll
  for (int off = WM; off < 64; off <<= 1) {
    lt += __shfl_xor(lt, off);
    ltx += __shfl_xor(ltx, off);
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (!t.valid) return;
  uint16_t* op = static_cast<uint16_t*>(a.o) + (long long)(t.q0 + t.i) * a.o_st + (long long)t.h * D;
#pragma unroll
  for (int dt = 0; dt < D / WM; ++dt)
#pragma unroll
    for (int grp = 0; grp < M::REGS / 4; ++grp) {
      bf16x4_t val;
#pragma unroll
      for (int e = 0; e < 4; ++e) val[e] = (__bf16)(o[dt][4 * grp + e] * inv);
      *reinterpret_cast<bf16x4_t*>(op + WM * dt + M::row(4 * grp, gq)) = val;
    }
  if (LSE && gq == 0) {
    const int n_total = a.cu_q[a.num_seqs];
    a.lse[(long long)t.h * n_total + t.q0 + t.i] = ltx > 0.f ? (st.m2 + __log2f(ltx)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------- wide-wave pieces
// A wave of the wide kernel owns NB blocks of 32 query rows: block b of wave
// w holds rows i0 + 32 * (NB * w + b) + (lane % 32), i0 = 128 * NB * tile.
template <int NB>
struct QTileN {
  int h, kvh, b, q0, Lq, kbase, Lk;
  int i[NB];
  bool valid[NB];
  RowKeys rk[NB];          // this lane's visible keys in each block
  unsigned wa[NB], wb[NB];  // interval widths (0 = empty)
  bool two_intervals;      // some lane of the wave has a second interval
  TilePlan plan;           // reduced over the workgroup's valid rows (uniform)
  int kt_lo, ntiles;
};

template <int D>
__device__ inline void load_q_row(const PrefillArgs& a, int h, int q0, int i, bool valid, bf16x8_t* qf);

// Work item w (query tile, q head, request; heaviest query tiles first within
// each (request, kv head)). Also issues the Q loads of every block (into qf)
// before the table loads.
template <int NB, int BN, int D>
__device__ inline bool setup_qtile_n(const PrefillArgs& a, int* red, QTileN<NB>& t, bf16x8_t (*qf)[D / 16], int w) {
  constexpr int NW = 4, WM = 32, BM = NW * WM * NB;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane % WM;
  const int m_rev = w % a.n_mtiles;
  int rest = w / a.n_mtiles;
  const int g = rest % a.group;
  rest /= a.group;
  t.kvh = rest % a.Hkv;
  const int bq = rest / a.Hkv;
  t.b = bq;
  t.h = t.kvh * a.group + g;
  const int mt = a.n_mtiles - 1 - m_rev;
  t.q0 = a.cu_q[bq];
  t.Lq = a.cu_q[bq + 1] - t.q0;
  if (a.block_table != nullptr) {
    t.kbase = 0;
    t.Lk = a.seq_lens_k[bq];
  } else {
    t.kbase = a.cu_k[bq];
    t.Lk = a.cu_k[bq + 1] - t.kbase;
  }
  const int i0 = mt * BM;
  if (i0 >= t.Lq) return false;
  TilePlan tp = plan_identity();
  bool two = false;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    t.i[b] = i0 + WM * (NB * wave + b) + col;
    t.valid[b] = t.i[b] < t.Lq;
    load_q_row<D>(a, t.h, t.q0, t.i[b], t.valid[b], qf[b]);
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    int ts = -1, te = -1;
    if (a.table != nullptr && t.valid[b]) {
      ts = a.table[2 * (long long)(t.q0 + t.i[b])];
      te = a.table[2 * (long long)(t.q0 + t.i[b]) + 1];
    }
    RowKeys rk = row_keys(a.causal, a.wl, a.wr, (t.Lk - t.Lq) + t.i[b], t.Lk, ts, te);
    if (t.valid[b]) {
      plan_add_row(tp, rk);
    } else {
      rk.a_lo = 0;
      rk.a_hi = -1;
      rk.b_lo = 0;
      rk.b_hi = -1;
    }
    two |= rk.b_lo <= rk.b_hi;
    t.rk[b] = rk;
    t.wa[b] = (unsigned)max(rk.a_hi - rk.a_lo + 1, 0);
    t.wb[b] = (unsigned)max(rk.b_hi - rk.b_lo + 1, 0);
  }
  t.two_intervals = __any(two);
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
  t.plan.lo = __builtin_amdgcn_readfirstlane(plan.lo);
  t.plan.hi = __builtin_amdgcn_readfirstlane(plan.hi);
  t.plan.flo = __builtin_amdgcn_readfirstlane(plan.flo);
  t.plan.fhi = __builtin_amdgcn_readfirstlane(plan.fhi);
  t.kt_lo = t.plan.lo <= t.plan.hi ? t.plan.lo / BN : 0;
  t.ntiles = t.plan.lo <= t.plan.hi ? t.plan.hi / BN - t.kt_lo + 1 : 0;
  return true;
}

// One 32-row block's Q as B operands of the 32x32x16 MFMA (lane: query col,
// dims 16 * s + 8 * gq ..), waited for before the key loop.
template <int D>
__device__ inline void load_q_row(const PrefillArgs& a, int h, int q0, int i, bool valid, bf16x8_t* qf) {
  const int gq = (threadIdx.x & 63) / 32;
  const uint16_t* qp =
      static_cast<const uint16_t*>(a.q) + (long long)(q0 + (valid ? i : 0)) * a.q_st + (long long)h * D + 8 * gq;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    u32x4_t raw = {0u, 0u, 0u, 0u};
    if (valid) raw = *reinterpret_cast<const u32x4_t*>(qp + 16 * s);
    qf[s] = __builtin_bit_cast(bf16x8_t, raw);
  }
}


}  // namespace

namespace detail {

// Operand prefetch distance (in MFMAs) of kernel 1, and the wave priority
// raised around its matrix-core loops (0 = off): a wave inside its MFMA
// chain wins issue over the SIMD's other wave, which is in its softmax or
// load phase, so the matrix core sees fewer gaps.
#ifndef MVS_PREFILL_PREFETCH
#define MVS_PREFILL_PREFETCH 2
#endif
#ifndef MVS_PREFILL_PRIO
#define MVS_PREFILL_PRIO 1
#endif

#if MVS_PREFILL_PRIO > 0
#define MVS_PRIO_HI() __builtin_amdgcn_s_setprio(MVS_PREFILL_PRIO)
#define MVS_PRIO_LO() __builtin_amdgcn_s_setprio(0)
#else
#define MVS_PRIO_HI()
#define MVS_PRIO_LO()
#endif

// ---------------------------------------------------------------- kernel 1
// One schedule for every shape: per key tile, K Q^T, softmax, then V^T P^T,
// all in one wave; latency is hidden by running two or more waves per SIMD.
template <int D, int BN, int NW, int WM, int MINW, int NS, bool PAGED, bool LSE, bool SCAN, int HPW>
__global__ __launch_bounds__(64 * NW, MINW) void prefill_bf16_kernel(const PrefillArgs a) {
  using T = Tile<D, BN, NW, WM>;
  using M = Mfma<WM>;
  using A = OperandAddr<D, WM>;
  typedef typename M::acc_t acc_t;
  constexpr int SB = BN / WM;     // score blocks per key tile
  constexpr int OT = D / WM;      // output tiles per wave
  constexpr int QS = D / M::KD;   // Q fragments (reduction steps of K Q^T)
  constexpr int PS = BN / M::KD;  // reduction steps of V^T P^T per key tile
  static_assert(D % M::KD == 0 && BN % M::KD == 0 && BN % WM == 0, "tile shape");
  static_assert(NS >= 2, "at least double buffering");
  constexpr int LPT = 2 * T::LOADS;  // loads per wave per key tile (K and V)
  // Q comes in through LDS (one block of WM rows per wave, before the K/V
  // ring takes the space over) for 32-row waves whose blocks fit the ring.
  // (The 8-wave D 256 schedule would need twice the ring; measured there,
  // the larger allocation cancels the shorter setup.)
  constexpr int QBLK = WM * 2 * D;
  constexpr bool QLDS = MVS_PREFILL_QLDS && WM == 32 && NW * QBLK <= NS * T::BUFB;
  __shared__ __attribute__((aligned(1024))) char smem[NS * T::BUFB];
  __shared__ int red[4 * NW];
  __shared__ int2 rsh[SCAN ? kMaxScanRanges : 1];

  QTile t;
  bf16x8_t qf[QS];
  char* const qblk = smem + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * QBLK;
  if (!setup_qtile<NW, WM, T::BM / HPW, BN, D, SCAN, HPW, QLDS>(a, red, t, qf, rsh, qblk)) return;
  const int gq = (threadIdx.x & 63) / WM;
  const A addr;
  if constexpr (QLDS) {
    vm_wait<0>();  // this wave's Q block has landed
#pragma unroll
    for (int s = 0; s < QS; ++s) qf[s] = *reinterpret_cast<const bf16x8_t*>(qblk + A::k_off(addr.k_rd, s, 0));
    consume_q<QS>(qf);
    __syncthreads();  // every wave holds its Q before the tile loads reuse the LDS
  }
  const KVSrc ksrc = kv_src<D>(a, t.kvh, t.b, t.kbase, false);
  const KVSrc vsrc = kv_src<D>(a, t.kvh, t.b, t.kbase, true);
  const TileLoader<D, BN, NW, WM, false> kld(ksrc.tok_stb);
  const TileLoader<D, BN, NW, WM, true> vld(vsrc.tok_stb);
  auto load_tile = [&](int kt, int buf) {
    char* kb_lds = smem + buf * T::BUFB;
    kld.template load_src<PAGED>(ksrc, kt * BN, t.Lk, kb_lds);
    vld.template load_src<PAGED>(vsrc, kt * BN, t.Lk, kb_lds + T::TILEB);
  };

  acc_t o[OT];
#pragma unroll
  for (int dt = 0; dt < OT; ++dt)
#pragma unroll
    for (int r = 0; r < M::REGS; ++r) o[dt][r] = 0.f;
  const float c2 = a.scale_log2;
  RowState rs{-INFINITY, 0.f, 0.f};
  float sink_raw = 0.f;
  if (a.sink_mode == MVS_SINK_NULL_LOGIT) {
    rs.m2 = a.sinks[t.h] * kLog2e;
    rs.l = rs.lx = gq == 0 ? 1.f : 0.f;  // the null term is counted once per row
  } else if (a.sink_mode == MVS_SINK_KEY0_BIAS) {
    sink_raw = a.sinks[t.h] / a.scale;  // scaled below with the scores
  }

  // Key tile visited at step j: the tile whose index is j modulo the tile
  // count, so that workgroups whose key ranges overlap (neighbouring query
  // tiles under a sliding window) read each shared tile at the same step,
  // while it is in L2. The online softmax does not depend on the order.
  const int ntl = t.ntiles;
  const int kt_rot = ntl > 0 ? ((-t.kt_lo) % ntl + ntl) % ntl : 0;
  auto tile_at = [&](int j) {
    int x = j + kt_rot;
    x = x >= ntl ? x - ntl : x;
    return t.kt_lo + x;
  };
  // NS-stage ring: tiles j+1 .. j+NS-1 are in flight while tile j is
  // computed. Tile j+NS-1 goes into the buffer tile j-1 used, which every
  // wave released at the barrier that ended iteration j-1.
#pragma unroll
  for (int p = 0; p < NS - 1; ++p)
    if (p < t.ntiles) load_tile(tile_at(p), p);
  consume_q<QS>(qf);
  if (t.ntiles >= NS - 1)
    vm_wait<(NS - 2) * LPT>();  // tile 0 has landed; tiles 1 .. NS-2 may still be in flight
  else
    vm_wait<0>();
  __syncthreads();

  int buf = 0;
  for (int j = 0; j < t.ntiles; ++j) {
    const int kt = tile_at(j);
    static_assert(T::TILEB % 4096 == 0, "ring slots leave the swizzled address bits alone");
    const bool refill = j + NS - 1 < t.ntiles;  // uniform
    if (refill) load_tile(tile_at(j + NS - 1), buf == 0 ? NS - 1 : buf - 1);

    // A tile no row of this wave sees is skipped by the wave (it still takes
    // its share of the loads and the barrier); the SIMD's other wave has the
    // matrix core meanwhile.
    const bool wave_sees = !MVS_PREFILL_WAVE_SKIP || (kt * BN <= t.wk_hi && kt * BN + BN - 1 >= t.wk_lo);
    if (wave_sees) {
    acc_t s[SB];
    // Per-tile lane addresses including the ring slot: the swizzle XORs only
    // bits 4-7 and slot offsets are multiples of 4 KB, so adding the slot
    // before the XOR equals adding it after, and each fragment read is one
    // XOR plus an immediate offset. Re-materialised per tile (no pinned
    // registers).
    int k_rd_t = addr.k_rd + buf * T::BUFB;
    asm volatile("" : "+v"(k_rd_t));
    // K fragments read two MFMAs ahead (three in registers); the first reads
    // go out before the score initialisation, which hides their latency
    constexpr int NQK = QS * SB;
    constexpr int PF = MVS_PREFILL_PREFETCH;
    bf16x8_t kf[PF + 1];
    auto kread = [&](int n) {
      kf[n % (PF + 1)] = *reinterpret_cast<const bf16x8_t*>(smem + A::k_off(k_rd_t, n / SB, n % SB));
    };
#pragma unroll
    for (int n = 0; n < PF && n < NQK; ++n) kread(n);
    // A tile every row of the workgroup sees whole (and not carrying the
    // key-0 sink) starts its score chains from the MFMA's zero operand
    // instead of register moves; other tiles start from the mask.
    const bool zinit = !SCAN && tile_full(t, kt * BN, kt * BN + BN - 1) &&
                       !(a.sink_mode == MVS_SINK_KEY0_BIAS && kt == 0);
    // raised from the score initialisation through the last K Q^T MFMA
    MVS_PRIO_HI();
    if (zinit) {
#pragma unroll
      for (int n = 0; n < SB; ++n) {
        if (n + PF < NQK) kread(n + PF);
        s[n] = M::mma(kf[n % (PF + 1)], qf[0], acc_t{});
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      init_scores<WM, SB, SCAN>(s, a, t, kt, BN, sink_raw, rsh);
#pragma unroll
      for (int n = 0; n < SB; ++n) {
        if (n + PF < NQK) kread(n + PF);
        s[n] = M::mma(kf[n % (PF + 1)], qf[0], s[n]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    {
      // the scheduling fences keep the compiler from hoisting every read
#pragma unroll
      for (int n = SB; n < NQK; ++n) {
        if (n + PF < NQK) kread(n + PF);
        s[n % SB] = M::mma(kf[n % (PF + 1)], qf[n / SB], s[n % SB]);
        __builtin_amdgcn_sched_barrier(0);
      }
      MVS_PRIO_LO();
    }

    // V^T fragments (transposing reads of the row-major V tile) are read two
    // MFMAs ahead, as for K
    int v_rd_t = addr.v_rd + buf * T::BUFB + T::TILEB;
    asm volatile("" : "+v"(v_rd_t));
    constexpr int NPV = OT * PS;
    u32x4_t vf[PF + 1];
    auto vread = [&](int n) {
      const int dt = n / PS, u = n % PS;
      short4v half[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        half[hf] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v_t*)(smem + A::v_off(v_rd_t, dt, u, hf)));
      vf[n % (PF + 1)] = u32x4_t{__builtin_bit_cast(u32x2_t, half[0]).x, __builtin_bit_cast(u32x2_t, half[0]).y,
                                 __builtin_bit_cast(u32x2_t, half[1]).x, __builtin_bit_cast(u32x2_t, half[1]).y};
    };

    // online softmax (base 2)
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < SB; ++kb)
#pragma unroll
      for (int r = 0; r < M::REGS; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = cross_group_max<WM>(mx);
    const float mnew = mx * c2;
    const bool raise = mnew > rs.m2 + kRescaleSlack;
    if (__any(raise)) {
      asm volatile("; raise running max" ::);  // keep the rare rescale out of the common path
      const float mu = raise ? mnew : rs.m2;
      const float alpha = raise ? __builtin_amdgcn_exp2f(rs.m2 - mu) : 1.f;
      rs.l *= alpha;
      rs.lx *= alpha;
#pragma unroll
      for (int dt = 0; dt < OT; ++dt)
#pragma unroll
        for (int r = 0; r < M::REGS; ++r) o[dt][r] *= alpha;
      rs.m2 = mu;
    }
    const float mb = rs.m2 == -INFINITY ? 0.f : rs.m2;
    float rsx = 0.f;
#pragma unroll
    for (int kb = 0; kb < SB; ++kb)
#pragma unroll
      for (int r = 0; r < M::REGS; ++r) {
        s[kb][r] = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c2, -mb));
        if constexpr (LSE) rsx += s[kb][r];
      }
    if constexpr (LSE) rs.lx += rsx;

    // P^T as bf16 B operands. Step u covers keys KD*u .. KD*u + KD-1; its 8
    // values per lane are accumulators (8u .. 8u+7) of the flattened score
    // blocks, whose keys are KD*u + {4*gq + 0..3, KD/2 + 4*gq + 0..3}. The
    // row sum adds the rounded weights, so numerator and denominator agree.
    bf16x8_t pb[PS];
    float rsum = 0.f;
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
        rsum = __builtin_amdgcn_fdot2_f32_bf16(pair, kOnes2, rsum, false);
      }
    }
    rs.l += rsum;

    // O^T += V^T P^T
    {
#pragma unroll
      for (int n = 0; n < PF && n < NPV; ++n) vread(n);
      MVS_PRIO_HI();
#pragma unroll
      for (int n = 0; n < NPV; ++n) {
        if (n + PF < NPV) vread(n + PF);
        o[n / PS] = M::mma(__builtin_bit_cast(bf16x8_t, vf[n % (PF + 1)]), pb[n % PS], o[n / PS]);
        __builtin_amdgcn_sched_barrier(0);
      }
      MVS_PRIO_LO();
    }
    }  // wave_sees

    // tile j+1 has landed in LDS (only tiles j+2 .. j+NS-1 may be in flight)
    if (refill)
      vm_wait<(NS - 2) * LPT>();
    else
      vm_wait<0>();
    __syncthreads();
    buf = buf == NS - 1 ? 0 : buf + 1;
  }
  if constexpr (WM == 32) {
    static_assert(NW * kStageBytes <= NS * T::BUFB, "output staging fits the K/V ring");
    store_out_staged<D, LSE>(a, t.h, t.q0, t.Lq, t.i, t.valid, o, rs, smem + (threadIdx.x >> 6) * kStageBytes);
  } else {
    store_out<D, WM, LSE>(a, t, o, rs);
  }
}

// ---------------------------------------------------------------- kernel 3
// Wide waves, one per SIMD, with the K/V tile loads spread over the matrix-core
// work. Each wave owns NB blocks of 32 query rows (the workgroup 128 * NB rows
// of one query head); O lives in AGPRs, Q and the scores in VGPRs.
//
// On MI355X the K/V tiles come from L2 into LDS at about 25 bytes per clock
// per CU, and a wave stalled on issuing a load also stops issuing MFMAs. One
// 32-key tile of K and V feeds 2048 cycles of matrix-core work per SIMD (at
// 128 * NB query rows per workgroup) and is 32 KB (D 256) or 64 KB (D 512), so
// the tile's loads are issued a round at a time between the MFMAs, with a
// whole iteration between a load and its use. Iteration j (KS K slots):
//   S^T(j) = K(j) Q^T (chains start from the MFMA zero operand), with the
//     wave's share of K(j+KS-1) issued between the MFMAs;
//   mask (partial tiles only) and row max of S(j), raise of the running max;
//   O^T += V(j-1)^T P(j-1)^T, with the exponentials of S(j) between the MFMAs
//     and the wave's share of V(j) issued between them; then P(j) in bf16.
// The barrier before the value MFMAs makes every wave's V(j-1) rounds visible.
// With two K slots a second barrier at the end makes K(j+1) visible and frees
// slot j % 2. With three (D 512: three K and two V slots fill the 160 KB of
// LDS) the first barrier does both: K(j+1) was issued before V(j-1), so it has
// landed too, and slot j % 3 is refilled only in the next iteration's score
// chain, after every wave has left this one. V has two slots; loads past the
// last tile refill a slot no wave reads again (with the last tile), so every
// iteration issues the same loads and the memory-counter waits are constants.
// Direct loads of one K or V tile, a round at a time: round j fills rows
// j * RPL .. j * RPL + RPL - 1 (each wave 1 KB); rows past `last` (the tile's
// last key inside the request) repeat row `last`.
template <int D, int BN, bool IS_V>
struct PipeLoader {
  using T = Tile<D, BN, 4, 32>;
  static constexpr int RPL = T::THREADS / T::CHUNKS;  // rows per round
  // tile: first key row of the tile; stb: bytes per key row; lds: the slot.
  // (The lane's row and chunk are recomputed per round rather than kept in
  // registers: the loop that calls this has no VGPR to spare.)
  __device__ static void round(const char* tile, int stb, int last, unsigned lds, int j) {
    const int tid = threadIdx.x;
    const int r = j * RPL + tid / T::CHUNKS, p0 = tid % T::CHUNKS;
    const int sw = IS_V ? v_swz<32, T::CHUNKS>(r) : k_swz<T::CHUNKS>(r);
    const unsigned wave_u = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    lds_dma16((unsigned)(min(r, last) * stb) + (unsigned)((p0 ^ sw) << 4), tile,
              lds + j * T::THREADS * 16 + wave_u * 1024);
  }
  // With 64-chunk rows (D 512) a paged round gives each wave one whole row,
  // so the row, its clamp, its page offset and its swizzle are uniform: they
  // go into the scalar base, and a lane adds only its chunk position.
  // (Measured: c3 from pages 2.055 -> 2.024 ms; the same form for contiguous
  // K/V was 1.9 % slower, so that path keeps the per-lane row offset.)
  static constexpr bool ROW_PER_WAVE = T::CHUNKS == 64;
  // Paged round j of the tile whose first key is key0 (pages of 2^lg >= 16
  // keys): a round's rows lie in one 16-key group, hence in one page, whose
  // base (cache + kv head + page * page stride) is page[rel] for the tile's
  // rel-th page. Rows past the request's last key (Lk - 1) repeat it; it lies
  // in the same page as the round's first row, or the whole round is past it.
  template <int NP>
  __device__ static void round_paged(const char* const* page, int key0, int Lk, int lg, int stb, unsigned lds, int j) {
    const int tid = threadIdx.x;
    const int r = j * RPL + tid / T::CHUNKS, p0 = tid % T::CHUNKS;
    const int sw = IS_V ? v_swz<32, T::CHUNKS>(r) : k_swz<T::CHUNKS>(r);
    const int kfirst = min(key0 + j * RPL, Lk - 1);  // uniform
    const int rel = (kfirst >> lg) - (key0 >> lg);
    const char* base = page[0];
#pragma unroll
    for (int x = 1; x < NP; ++x) base = rel == x ? page[x] : base;
    const unsigned wave_u = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if constexpr (ROW_PER_WAVE) {
      const int key = min(key0 + j * RPL + (int)wave_u, Lk - 1);
      const int swu = IS_V ? v_swz<32, T::CHUNKS>(j * RPL + (int)wave_u) : k_swz<T::CHUNKS>(j * RPL + (int)wave_u);
      lds_dma16((unsigned)(((threadIdx.x & 63) ^ swu) << 4), base + (long long)(key & ((1 << lg) - 1)) * stb,
                lds + j * T::THREADS * 16 + wave_u * 1024);
    } else {
      const int key = min(key0 + r, Lk - 1);
      lds_dma16((unsigned)((key & ((1 << lg) - 1)) * stb) + (unsigned)((p0 ^ sw) << 4), base,
                lds + j * T::THREADS * 16 + wave_u * 1024);
    }
  }
};

// K slots of kernel 3: three when three K and two V tiles fill at most the
// 160 KB of LDS (D 512: 5 x 32 KB), else two. With three, K(j+2) is loaded
// during iteration j and one barrier per iteration suffices.
#ifndef MVS_PREFILL_KSLOTS
#define MVS_PREFILL_KSLOTS 3
#endif
template <int D, int BN>
constexpr int pipe_kslots() {
  return MVS_PREFILL_KSLOTS >= 3 && 5 * Tile<D, BN, 4, 32>::TILEB <= 160 * 1024 ? 3 : 2;
}

// One work item of kernel 3: the key loop of one 128-row query tile and its
// output; `desc` walks the key tiles from the last down.
template <int D, int NB, int BN, int PFK, int PFV, bool PAGED, bool LSE>
__device__ __attribute__((always_inline)) inline void pipe_item(const PrefillArgs& a, char* smem, int* red, int w,
                                                                 bool desc) {
  constexpr int NW = 4, WM = 32;
  using T = Tile<D, BN, NW, WM>;
  using M = Mfma<WM>;
  using A = OperandAddr<D, WM>;
  typedef typename M::acc_t acc_t;
  constexpr int SB = BN / WM, OT = D / WM, QS = D / M::KD, PS = BN / M::KD;
  static_assert(SB == 1, "one 32-key score block per tile");
  constexpr int NQK = QS * NB;       // score MFMAs per tile
  constexpr int NVF = OT * PS;       // V fragments per tile
  constexpr int NPV = NVF * NB;      // value MFMAs per tile
  constexpr int LD = T::LOADS;       // loads per wave per tensor per tile
  constexpr int NSC = NB * M::REGS;  // scores per lane per tile
  static_assert(NQK % LD == 0 && NPV % LD == 0, "loads spread evenly over the MFMAs");
  static_assert(T::TILEB % 4096 == 0, "slot offsets leave the swizzled address bits alone");
  constexpr int KS = pipe_kslots<D, BN>();  // K slots; V has two, after them
  QTileN<NB> t;
  bf16x8_t qf[NB][QS];
  if (!setup_qtile_n<NB, BN, D>(a, red, t, qf, w)) return;
  const int gq = (threadIdx.x & 63) / WM;
  const A addr;
  const KVSrc ksrc = kv_src<D>(a, t.kvh, t.b, t.kbase, false);
  const KVSrc vsrc = kv_src<D>(a, t.kvh, t.b, t.kbase, true);
  using KLoad = PipeLoader<D, BN, false>;
  using VLoad = PipeLoader<D, BN, true>;
  const int ntiles = t.ntiles;
  // key tile visited at step jt (past the last step, the last one again); the
  // online softmax does not depend on the order
  auto tile_of = [&](int jt) {
    const int x = min(jt, ntiles - 1);
    return t.kt_lo + (desc ? ntiles - 1 - x : x);
  };
  const unsigned lds0 = lds_u32(smem);
  // Paged K/V: the bases of the (at most NP) pages of the tiles whose loads an
  // iteration issues (K(j+1), V(j)), read with scalar loads through the
  // constant address space (a vector load would join the tile loads' memory
  // counter) at the top of the iteration; an entry outside [0, num_blocks)
  // reads page 0.
  constexpr int NP = BN / 16 > 0 ? BN / 16 : 1;
  const char* kpage[NP];
  const char* vpage[NP];
  auto page_bases = [&](const KVSrc& src, int jt, const char** page) {
    using cint = __attribute__((address_space(4))) const int;
    const cint* bt = (const cint*)src.bt;
    const int key0 = tile_of(jt) * BN;
    const int pg0 = key0 >> src.page_log2;
    const int last_pg = min((t.Lk - 1) >> src.page_log2, src.max_blocks - 1);
#pragma unroll
    for (int x = 0; x < NP; ++x) {
      const int v = bt[max(min(pg0 + x, last_pg), 0)];
      page[x] = src.base + (long long)((v >= 0 && v < src.num_blocks) ? v : 0) * src.blk_stb;
    }
  };
  // the page bases are needed before the tile's first MFMA: wait for them here,
  // while no LDS read is in flight, rather than in the middle of the MFMA chain
  auto settle_pages = [&](const char** page) {
#pragma unroll
    for (int x = 0; x < NP; ++x) asm volatile("" ::"s"(page[x]));
  };
  // round r of the loads of tile jt into its slot; past the last tile, the last tile again
  auto kload = [&](int jt, int r) {
    const int key0 = tile_of(jt) * BN;
    if constexpr (PAGED)
      KLoad::template round_paged<NP>(kpage, key0, t.Lk, ksrc.page_log2, ksrc.tok_stb, lds0 + (jt % KS) * T::TILEB,
                                      r);
    else
      KLoad::round(ksrc.base + (long long)key0 * ksrc.tok_stb, ksrc.tok_stb, t.Lk - 1 - key0,
                   lds0 + (jt % KS) * T::TILEB, r);
  };
  auto vload = [&](int jt, int r) {
    const int key0 = tile_of(jt) * BN;
    if constexpr (PAGED)
      VLoad::template round_paged<NP>(vpage, key0, t.Lk, vsrc.page_log2, vsrc.tok_stb,
                                      lds0 + (KS + (jt & 1)) * T::TILEB, r);
    else
      VLoad::round(vsrc.base + (long long)key0 * vsrc.tok_stb, vsrc.tok_stb, t.Lk - 1 - key0,
                   lds0 + (KS + (jt & 1)) * T::TILEB, r);
  };

  acc_t o[NB][OT];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int dt = 0; dt < OT; ++dt)
#pragma unroll
      for (int r = 0; r < M::REGS; ++r) o[b][dt][r] = 0.f;
  const float c2 = a.scale_log2;
  RowState rs[NB];
  float sink_raw = 0.f;
#pragma unroll
  for (int b = 0; b < NB; ++b) rs[b] = RowState{-INFINITY, 0.f, 0.f};
  if (a.sink_mode == MVS_SINK_NULL_LOGIT) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      rs[b].m2 = a.sinks[t.h] * kLog2e;
      rs[b].l = rs[b].lx = gq == 0 ? 1.f : 0.f;  // the null term is counted once per row
    }
  } else if (a.sink_mode == MVS_SINK_KEY0_BIAS) {
    sink_raw = a.sinks[t.h] / a.scale;  // scaled with the scores
  }

  // prologue: K(0) .. K(KS-2). Iteration j issues K(j+KS-1) and V(j); at its
  // barriers the oldest outstanding groups are the ones needed next (V(j-1)
  // before the value MFMAs; with two K slots K(j+1) at the end), the newest
  // LD loads may still be in flight.
#pragma unroll
  for (int jk = 0; jk < KS - 1; ++jk) {
    if constexpr (PAGED) {
      page_bases(ksrc, jk, kpage);
      settle_pages(kpage);
    }
#pragma unroll
    for (int r = 0; r < LD; ++r) kload(jk, r);
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) consume_q<QS>(qf[b]);
  vm_wait<0>();
  __syncthreads();

  bf16x8_t pb[NB][PS];  // P of the previous tile, bf16 B operands
  // V^T P^T of tile jv for every block; V fragments read PF ahead, each feeding NB MFMAs.
  auto pv = [&](int jv, auto&& extra) {
    int v_rd_t = addr.v_rd + (KS + (jv & 1)) * T::TILEB;  // slot added before the swizzle XOR (bits 4-7 only)
    asm volatile("" : "+v"(v_rd_t));
    u32x4_t vf[PFV + 1];
    auto vread = [&](int n) {
      const int dt = n / PS, u = n % PS;
      short4v half[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        half[hf] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v_t*)(smem + A::v_off(v_rd_t, dt, u, hf)));
      vf[n % (PFV + 1)] = u32x4_t{__builtin_bit_cast(u32x2_t, half[0]).x, __builtin_bit_cast(u32x2_t, half[0]).y,
                                 __builtin_bit_cast(u32x2_t, half[1]).x, __builtin_bit_cast(u32x2_t, half[1]).y};
    };
#pragma unroll
    for (int n = 0; n < PFV && n < NVF; ++n) vread(n);
#pragma unroll
    for (int n = 0; n < NVF; ++n) {
      if (n + PFV < NVF) vread(n + PFV);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        o[b][n / PS] = M::mma(__builtin_bit_cast(bf16x8_t, vf[n % (PFV + 1)]), pb[b][n % PS], o[b][n / PS]);
        extra(n * NB + b);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  constexpr int KEVERY = NQK / LD;  // score MFMAs per K load round
  constexpr int VEVERY = NPV / LD;  // value MFMAs per V load round
  for (int j = 0; j < ntiles; ++j) {
    const int kt = tile_of(j);
    if constexpr (PAGED) {
      page_bases(ksrc, j + KS - 1, kpage);
      page_bases(vsrc, j, vpage);
      settle_pages(kpage);
      settle_pages(vpage);
    }
    // scores of tile j: S^T = K Q^T for every block, K fragments PF ahead; K(j+KS-1) rounds between
    acc_t s[NB];
    {
      int k_rd_t = addr.k_rd + (j % KS) * T::TILEB;
      asm volatile("" : "+v"(k_rd_t));
      bf16x8_t kf[PFK + 1];
      auto kread = [&](int st) {
        kf[st % (PFK + 1)] = *reinterpret_cast<const bf16x8_t*>(smem + A::k_off(k_rd_t, st, 0));
      };
#pragma unroll
      for (int st = 0; st < PFK && st < QS; ++st) kread(st);
#pragma unroll
      for (int st = 0; st < QS; ++st) {
        if (st + PFK < QS) kread(st + PFK);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          s[b] = st == 0 ? M::mma(kf[0], qf[b][0], acc_t{}) : M::mma(kf[st % (PFK + 1)], qf[b][st], s[b]);
          const int n = st * NB + b;
          if (n % KEVERY == 1 % KEVERY) kload(j + KS - 1, n / KEVERY);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // mask of partial tiles (the predicate as two key intervals per row), key-0 sink
    if (classify_key_tile(t.plan, kt * BN, kt * BN + BN - 1) != 2) {
      asm volatile("; partial key tile" ::);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int ta = kt * BN - t.rk[b].a_lo, tb = kt * BN - t.rk[b].b_lo;
#pragma unroll
        for (int r = 0; r < M::REGS; ++r) {
          const int off = M::row(r, gq);
          const bool vis = ((unsigned)(ta + off) < t.wa[b]) | ((unsigned)(tb + off) < t.wb[b]);
          s[b][r] = vis ? s[b][r] : -INFINITY;
        }
      }
    }
    if (a.sink_mode == MVS_SINK_KEY0_BIAS && kt == 0 && gq == 0) {
#pragma unroll
      for (int b = 0; b < NB; ++b) s[b][0] += sink_raw;  // key 0 (-inf stays -inf where masked)
    }

    // row max of tile j (the two 32-lane halves hold the same query rows)
    float mb[NB];
    bool raise_any = false;
    bool raise[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < M::REGS; ++r) mx = fmaxf(mx, s[b][r]);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      raise[b] = mx * c2 > rs[b].m2 + kRescaleSlack;
      raise_any |= raise[b];
      mb[b] = mx * c2;
    }
    // V(j-1) has landed in every wave's share (only K(j+KS-1) may still be in
    // flight; with three K slots K(j+1), issued before V(j-1), has landed too)
    vm_wait<LD>();
    __syncthreads();
    bool pv_pending = j > 0;
    if (__any(raise_any)) {
      asm volatile("; raise running max" ::);
      // O must hold tile j-1's contribution before it is rescaled; V(j) rounds go out with it
      if (pv_pending) pv(j - 1, [&](int n) {
        if (n % VEVERY == 1 % VEVERY) vload(j, n / VEVERY);
      });
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float mu = raise[b] ? mb[b] : rs[b].m2;
        const float alpha = raise[b] ? __builtin_amdgcn_exp2f(rs[b].m2 - mu) : 1.f;
        rs[b].l *= alpha;
        rs[b].lx *= alpha;
#pragma unroll
        for (int dt = 0; dt < OT; ++dt) rescale_agpr<M::REGS>(o[b][dt], alpha);
        rs[b].m2 = mu;
      }
      pv_pending = false;
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) mb[b] = rs[b].m2 == -INFINITY ? 0.f : rs[b].m2;

    // exponentials of tile j, interleaved with V^T P^T of tile j-1 and the V(j) rounds
    constexpr int EPS = (NSC + NPV - 1) / NPV;
    float rsx[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) rsx[b] = 0.f;
    auto exp_range = [&](int e0, int e1) {
#pragma unroll
      for (int e = e0; e < e1; ++e) {
        const int b = e / M::REGS, r = e % M::REGS;
        const float x = __builtin_amdgcn_exp2f(fmaf(s[b][r], c2, -mb[b]));
        s[b][r] = x;
        if constexpr (LSE) rsx[b] += x;
      }
    };
    if (pv_pending) {
      pv(j - 1, [&](int n) {
        exp_range(min(n * EPS, NSC), min((n + 1) * EPS, NSC));
        if (n % VEVERY == 1 % VEVERY) vload(j, n / VEVERY);
      });
    } else {
      exp_range(0, NSC);
      if (j == 0) {  // no value MFMAs in the first iteration: V(0) goes out in one burst
#pragma unroll
        for (int r = 0; r < LD; ++r) vload(0, r);
      }
    }

    // P of tile j as bf16 B operands; the row sums add the rounded values
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if constexpr (LSE) rs[b].lx += rsx[b];
      float rsum = 0.f;
#pragma unroll
      for (int u = 0; u < PS; ++u) {
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[b][u][e] = (__bf16)s[b][8 * u + e];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          bf16x2_t pair = {pb[b][u][e], pb[b][u][e + 1]};
          rsum = __builtin_amdgcn_fdot2_f32_bf16(pair, kOnes2, rsum, false);
        }
      }
      rs[b].l += rsum;
    }

    // Two K slots: K(j+1) has landed in every wave's share (only V(j) may
    // still be in flight), and slot j % 2 is free for K(j+2). With three the
    // barrier before the value MFMAs did both: K(j+1) landed before V(j-1),
    // and every wave had finished reading slot j % 3 (refilled with K(j+3)
    // next iteration) and V slot (j-1) % 2 (refilled with V(j+1) after the
    // next such barrier).
    if constexpr (KS == 2) {
      vm_wait<LD>();
      __syncthreads();
    }
  }
  if (ntiles > 0) {
    vm_wait<0>();  // V(last) was issued by the last iteration
    __syncthreads();
    pv(ntiles - 1, [](int) {});
  }
  // the K slots are free now (the last V tile is still being read from its slot)
  static_assert(4 * kStageBytes <= 2 * T::TILEB, "output staging fits the K slots");
  char* stage = smem + (threadIdx.x >> 6) * kStageBytes;
#pragma unroll
  for (int b = 0; b < NB; ++b) store_out_staged<D, LSE>(a, t.h, t.q0, t.Lq, t.i[b], t.valid[b], o[b], rs[b], stage);
}

template <int D, int NB, int BN, int PFK, int PFV, bool PAGED, bool LSE>
__global__ __launch_bounds__(256, 1) void prefill_bf16_pipe_kernel(const PrefillArgs a) {
  constexpr int KS = pipe_kslots<D, BN>();
  constexpr int TILEB = Tile<D, BN, 4, 32>::TILEB;
  __shared__ __attribute__((aligned(1024))) char smem[(KS + 2) * TILEB];  // K slots, then two V slots
  // The setup's 64-byte reduction lives in K slot 2 when there is one (the
  // slots then fill the LDS): K(2), its first tile, is issued only after the
  // prologue's barrier, by when every wave has read the reduction.
  __shared__ int red_own[KS == 3 ? 1 : 4 * 4];
  int* red = KS == 3 ? reinterpret_cast<int*>(smem + 2 * TILEB) : red_own;
  // Each workgroup takes two query tiles of one (request, q head): the
  // longest and the shortest of the pairs (tile m and tile n - 1 - m), the
  // first walking its keys upward, the second downward. Under a causal mask
  // every pair then holds the same number of keys, so the workgroups of one
  // (request, kv head) on an XCD finish together, and in both halves they
  // read the same key tile at the same time: the tiles stay in that XCD's L2.
  const int np = (a.n_mtiles + 1) / 2;
  const int wp = xcd_remap(blockIdx.x, gridDim.x, a.group * np);
  const int pr = wp % np, rest = wp / np;
  pipe_item<D, NB, BN, PFK, PFV, PAGED, LSE>(a, smem, red, rest * a.n_mtiles + pr, false);
  if (a.n_mtiles - 1 - pr != pr) {
    __syncthreads();  // the first tile's output staging used the K slots
    pipe_item<D, NB, BN, PFK, PFV, PAGED, LSE>(a, smem, red, rest * a.n_mtiles + a.n_mtiles - 1 - pr, true);
  }
}

}  // namespace detail

namespace {

// Workgroups of a kernel-1 launch: query tiles x head slices x sequences.
template <int D, int BN, int NW, int WM, int HPW>
long long k1_blocks(int Hq, int num_seqs, int max_seqlen_q) {
  constexpr int BM = Tile<D, BN, NW, WM>::BM / HPW;  // query rows per workgroup
  return (long long)((int)(((long long)max_seqlen_q + BM - 1) / BM)) * (Hq / HPW) * num_seqs;
}

template <int D, int BN, int NW, int WM, int MINW, int NS, bool PAGED, bool SCAN, int HPW>
hipError_t launch_k1(PrefillArgs a, int max_seqlen_q, hipStream_t stream) {
  using T = Tile<D, BN, NW, WM>;
  constexpr int BM = T::BM / HPW;  // query rows per workgroup
  a.n_mtiles = (int)(((long long)max_seqlen_q + BM - 1) / BM);
  const long long blocks = (long long)a.n_mtiles * (a.Hq / HPW) * a.num_seqs;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (a.lse != nullptr)
    hipLaunchKernelGGL((detail::prefill_bf16_kernel<D, BN, NW, WM, MINW, NS, PAGED, true, SCAN, HPW>),
                       dim3((unsigned)blocks), dim3(T::THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL((detail::prefill_bf16_kernel<D, BN, NW, WM, MINW, NS, PAGED, false, SCAN, HPW>),
                       dim3((unsigned)blocks), dim3(T::THREADS), 0, stream, a);
  return hipGetLastError();
}

// HPW query heads of one kv head per workgroup (NW waves in all, NW / HPW per
// head) when the group divides evenly, else one head per workgroup with
// NW / HPW waves, at least 4.
template <int D, int BN, int NW, int WM, int MINW, int NS, int HPW = 1>
long long grid_launch(int group, int Hq, int num_seqs, int max_seqlen_q, bool scan) {
  constexpr int NW1 = NW / HPW < 4 ? 4 : NW / HPW;
  if (HPW > 1 && !scan && group % HPW == 0) return k1_blocks<D, BN, NW, WM, HPW>(Hq, num_seqs, max_seqlen_q);
  return k1_blocks<D, BN, NW1, WM, 1>(Hq, num_seqs, max_seqlen_q);
}

template <int D, int BN, int NW, int WM, int MINW, int NS, int HPW = 1>
hipError_t launch(PrefillArgs a, int max_seqlen_q, hipStream_t stream) {
  constexpr int NW1 = NW / HPW < 4 ? 4 : NW / HPW;  // one head per workgroup
  if (a.scan_ranges != nullptr) {  // contiguous K/V only
    if (a.block_table != nullptr || a.max_ranges > kMaxScanRanges) return hipErrorInvalidValue;
    return launch_k1<D, BN, NW1, WM, MINW, NS, false, true, 1>(a, max_seqlen_q, stream);
  }
  if constexpr (HPW > 1) {
    if (a.group % HPW == 0)
      return a.block_table != nullptr ? launch_k1<D, BN, NW, WM, MINW, NS, true, false, HPW>(a, max_seqlen_q, stream)
                                      : launch_k1<D, BN, NW, WM, MINW, NS, false, false, HPW>(a, max_seqlen_q, stream);
  }
  return a.block_table != nullptr
             ? launch_k1<D, BN, NW1, WM, MINW, NS, true, false, 1>(a, max_seqlen_q, stream)
             : launch_k1<D, BN, NW1, WM, MINW, NS, false, false, 1>(a, max_seqlen_q, stream);
}

// The kernel-1 schedule of head_dim D, for the calls kernel 3 does not take
// (the range-scan baseline, which the library accepts for D <= 256 only).
template <int D>
hipError_t launch_fallback(PrefillArgs a, int max_seqlen_q, hipStream_t stream) {
  if constexpr (D == 512)
    return hipErrorInvalidValue;  // every D 512 call the library accepts runs kernel 3
  else if constexpr (D == 256)
    return launch<256, 32, 4, 32, 2, 2, 2>(a, max_seqlen_q, stream);
  else if constexpr (D == 128)
    return launch<128, 32, 4, 32, 2, 3>(a, max_seqlen_q, stream);
  else
    return launch<64, 64, 4, 32, 1, 2>(a, max_seqlen_q, stream);
}

template <int D>
long long grid_fallback(int group, int Hq, int num_seqs, int max_seqlen_q, bool scan) {
  if constexpr (D == 512)
    return 0;
  else if constexpr (D == 256)
    return grid_launch<256, 32, 4, 32, 2, 2, 2>(group, Hq, num_seqs, max_seqlen_q, scan);
  else if constexpr (D == 128)
    return grid_launch<128, 32, 4, 32, 2, 3>(group, Hq, num_seqs, max_seqlen_q, scan);
  else
    return grid_launch<64, 64, 4, 32, 1, 2>(group, Hq, num_seqs, max_seqlen_q, scan);
}

// Kernel 3 (the software-pipelined wide schedule): 4 waves of NB * 32 rows.
template <int D, int BN, int NB, int PFK, int PFV, bool PAGED>
hipError_t launch_pipe_impl(PrefillArgs a, int max_seqlen_q, hipStream_t stream) {
  constexpr int BM = 128 * NB;
  a.n_mtiles = (int)(((long long)max_seqlen_q + BM - 1) / BM);
  const long long blocks = (long long)((a.n_mtiles + 1) / 2) * a.Hq * a.num_seqs;  // a pair of query tiles each
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (a.lse != nullptr)
    hipLaunchKernelGGL((detail::prefill_bf16_pipe_kernel<D, NB, BN, PFK, PFV, PAGED, true>), dim3((unsigned)blocks),
                       dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((detail::prefill_bf16_pipe_kernel<D, NB, BN, PFK, PFV, PAGED, false>), dim3((unsigned)blocks),
                       dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int D, int BN, int NB, int PFK, int PFV>
hipError_t launch_pipe(PrefillArgs a, int max_seqlen_q, hipStream_t stream) {
  if (a.scan_ranges != nullptr) return launch_fallback<D>(a, max_seqlen_q, stream);
  return a.block_table != nullptr ? launch_pipe_impl<D, BN, NB, PFK, PFV, true>(a, max_seqlen_q, stream)
                                  : launch_pipe_impl<D, BN, NB, PFK, PFV, false>(a, max_seqlen_q, stream);
}

template <int D, int BN, int NB, int PFK, int PFV>
long long grid_launch_pipe(int group, int Hq, int num_seqs, int max_seqlen_q, bool scan) {
  constexpr int BM = 128 * NB;
  const long long mt = ((long long)max_seqlen_q + BM - 1) / BM;
  const long long own = (mt + 1) / 2 * Hq * num_seqs;
  const long long fb = grid_fallback<D>(group, Hq, num_seqs, max_seqlen_q, scan);
  return own > fb ? own : fb;
}

}  // namespace

// Tile configuration per head_dim and the schedule: launch = kernel 1 (key-tile
// width BN, waves per workgroup NW, query rows per wave WM, minimum waves per
// SIMD MINW, K/V pipeline stages NS, optionally the query heads per workgroup
// HPW, NW counting the waves of all of them), launch_pipe = kernel 3 (BN,
// 32-row blocks per wave NB, K and V fragment prefetch depths). A build may
// override one with -DMVS_PREFILL_CFG_<D>=... and -DMVS_PREFILL_SCHED_<D>=...
// D 256: the two q heads of a kv head share one workgroup, so each K/V tile
// is loaded once for both (sliding layer: 0.393 -> 0.375 ms with 8 waves),
// and 4-wave workgroups of 64 rows per head let two workgroups share a CU,
// one's setup and epilogue overlapping the other's key loop (0.324 -> 0.317
// ms at steady clocks). D 512: K fragments read three MFMAs ahead and V^T
// fragments four (c3 1.803 -> 1.786 ms against two and two, 24 interleaved
// rounds; one K fragment ahead was 10 % slower).
#ifndef MVS_PREFILL_CFG_64
#define MVS_PREFILL_CFG_64 64, 4, 32, 1, 2
#endif
#ifndef MVS_PREFILL_CFG_128
#define MVS_PREFILL_CFG_128 32, 4, 32, 2, 3
#endif
#ifndef MVS_PREFILL_CFG_256
#define MVS_PREFILL_CFG_256 32, 4, 32, 2, 2, 2
#endif
#ifndef MVS_PREFILL_CFG_512
#define MVS_PREFILL_CFG_512 32, 1, 3, 4
#endif
#ifndef MVS_PREFILL_SCHED_64
#define MVS_PREFILL_SCHED_64 launch
#endif
#ifndef MVS_PREFILL_SCHED_128
#define MVS_PREFILL_SCHED_128 launch
#endif
#ifndef MVS_PREFILL_SCHED_256
#define MVS_PREFILL_SCHED_256 launch
#endif
#ifndef MVS_PREFILL_SCHED_512
#define MVS_PREFILL_SCHED_512 launch_pipe
#endif

#define MVS_CAT2(a, b) a##b
#define MVS_CAT(a, b) MVS_CAT2(a, b)

long long prefill_bf16_grid(int head_dim, int group, int Hq, int num_seqs, int max_seqlen_q, bool scan) {
  switch (head_dim) {
    case 64:
      return MVS_CAT(grid_, MVS_PREFILL_SCHED_64)<64, MVS_PREFILL_CFG_64>(group, Hq, num_seqs, max_seqlen_q, scan);
    case 128:
      return MVS_CAT(grid_, MVS_PREFILL_SCHED_128)<128, MVS_PREFILL_CFG_128>(group, Hq, num_seqs, max_seqlen_q, scan);
    case 256:
      return MVS_CAT(grid_, MVS_PREFILL_SCHED_256)<256, MVS_PREFILL_CFG_256>(group, Hq, num_seqs, max_seqlen_q, scan);
    case 512:
      return MVS_CAT(grid_, MVS_PREFILL_SCHED_512)<512, MVS_PREFILL_CFG_512>(group, Hq, num_seqs, max_seqlen_q, scan);
    default:
      return -1;
  }
}

hipError_t launch_prefill_bf16(PrefillArgs a, int head_dim, int max_seqlen_q, hipStream_t stream) {
  switch (head_dim) {
    case 64:
      return MVS_PREFILL_SCHED_64<64, MVS_PREFILL_CFG_64>(a, max_seqlen_q, stream);
    case 128:
      return MVS_PREFILL_SCHED_128<128, MVS_PREFILL_CFG_128>(a, max_seqlen_q, stream);
    case 256:
      return MVS_PREFILL_SCHED_256<256, MVS_PREFILL_CFG_256>(a, max_seqlen_q, stream);
    case 512:
      return MVS_PREFILL_SCHED_512<512, MVS_PREFILL_CFG_512>(a, max_seqlen_q, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace mvs
