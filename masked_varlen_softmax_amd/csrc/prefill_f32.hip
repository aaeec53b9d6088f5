// prefill_f32.hip - masked varlen attention prefill in fp32 (inputs, math and
// outputs), for gfx950.
//
// Same predicate, sinks and outputs as the bf16 kernel (mask.hpp; vLLM PR
// #49815 sink semantics, vLLM PR #50294 mask). This path serves fp32 callers
// and small problems (the MiMo vision window of the PR #49815 test is fp32 on
// 5- and 37-token sequences), so it favours exactness over speed: vector ALU
// arithmetic, exact exp2, one online-softmax update per key.
//
// One workgroup = 64 query rows of one head; 4 lanes per row, each holding a
// quarter of the head dimension. Key tiles of 32 keys are staged in LDS; the
// workgroup visits only the key tiles its rows can see (mask.hpp tile plan).

#include <hip/hip_runtime.h>

#include "common.hpp"
#include "kernels.hpp"
#include "mask.hpp"

namespace mvs {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D>
__global__ __launch_bounds__(256) void prefill_f32_kernel(const PrefillArgs a) {
  constexpr int BM = 64, BN = 32, DPT = D / 4;
  __shared__ float ks[BN * D];
  __shared__ float vs[BN * D];
  __shared__ int plan_s[4];

  const int tid = threadIdx.x;
  const int r = tid >> 2, part = tid & 3;
  const int mt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int kvh = h / a.group;

  const int q0 = a.cu_q[b];
  const int Lq = a.cu_q[b + 1] - q0;
  const int kbase = a.cu_k[b];
  const int Lk = a.cu_k[b + 1] - kbase;
  const int i0 = mt * BM;
  if (i0 >= Lq) return;
  const int i = i0 + r;
  const bool valid = i < Lq;

  int ts = -1, te = -1;
  if (a.table != nullptr && valid) {
    ts = a.table[2 * (long long)(q0 + i)];
    te = a.table[2 * (long long)(q0 + i) + 1];
  }
  const RowKeys rk = row_keys(a.causal, a.wl, a.wr, (Lk - Lq) + i, Lk, ts, te);
  if (tid == 0) {
    const TilePlan id = plan_identity();
    plan_s[0] = id.lo;
    plan_s[1] = id.hi;
  }
  __syncthreads();
  if (valid && part == 0) {
    TilePlan tp = plan_identity();
    plan_add_row(tp, rk);
    atomicMin(&plan_s[0], tp.lo);
    atomicMax(&plan_s[1], tp.hi);
  }
  __syncthreads();
  const int lo = plan_s[0], hi = plan_s[1];

  const float* qp = static_cast<const float*>(a.q) + (long long)(q0 + (valid ? i : 0)) * a.q_st +
                    (long long)h * D + part * DPT;
  float q[DPT], o[DPT];
#pragma unroll
  for (int d = 0; d < DPT; ++d) {
    q[d] = valid ? qp[d] : 0.f;
    o[d] = 0.f;
  }
  float m2 = -INFINITY, l = 0.f;
  if (a.sink_mode == MVS_SINK_NULL_LOGIT) {
    m2 = a.sinks[h] * kLog2e;
    l = 1.f;
  }
  const float sink2 = a.sink_mode == MVS_SINK_KEY0_BIAS ? a.sinks[h] * kLog2e : 0.f;

  const float* kg = static_cast<const float*>(a.k) + (long long)kbase * a.k_st + (long long)kvh * D;
  const float* vg = static_cast<const float*>(a.v) + (long long)kbase * a.v_st + (long long)kvh * D;

  if (lo <= hi) {
    for (int kt = lo / BN; kt <= hi / BN; ++kt) {
      __syncthreads();
      for (int e = tid; e < BN * D; e += 256) {
        const int kk = e / D, d = e % D;
        const int key = kt * BN + kk;
        ks[e] = key < Lk ? kg[(long long)key * a.k_st + d] : 0.f;
        vs[e] = key < Lk ? vg[(long long)key * a.v_st + d] : 0.f;
      }
      __syncthreads();
      for (int kk = 0; kk < BN; ++kk) {
        const int key = kt * BN + kk;
        float dot = 0.f;
#pragma unroll
        for (int d = 0; d < DPT; ++d) dot = fmaf(q[d], ks[kk * D + part * DPT + d], dot);
        dot += __shfl_xor(dot, 1);
        dot += __shfl_xor(dot, 2);
        if (!valid || !row_sees(rk, key)) continue;
        float sc = dot * a.scale_log2;
        if (key == 0) sc += sink2;
        const float mn = fmaxf(m2, sc);
        const float alpha = m2 == -INFINITY ? 0.f : exp2f(m2 - mn);
        const float p = exp2f(sc - mn);
        l = l * alpha + p;
#pragma unroll
        for (int d = 0; d < DPT; ++d) o[d] = fmaf(p, vs[kk * D + part * DPT + d], o[d] * alpha);
        m2 = mn;
      }
    }
  }

  if (valid) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* op = static_cast<float*>(a.o) + (long long)(q0 + i) * a.o_st + (long long)h * D + part * DPT;
#pragma unroll
    for (int d = 0; d < DPT; ++d) op[d] = o[d] * inv;
    if (a.lse != nullptr && part == 0) {
      const int n_total = a.cu_q[a.num_seqs];
      a.lse[(long long)h * n_total + q0 + i] = l > 0.f ? (m2 + log2f(l)) * kLn2 : -INFINITY;
    }
  }
}

template <int D>
hipError_t launch(PrefillArgs a, int max_seqlen_q, hipStream_t stream) {
  const int mt = (int)(((long long)max_seqlen_q + 63) / 64);
  if (mt == 0 || a.num_seqs == 0) return hipSuccess;
  if (a.num_seqs > kMaxGridYZ || a.Hq > kMaxGridYZ) return hipErrorInvalidValue;  // rejected by the entry points
  hipLaunchKernelGGL(prefill_f32_kernel<D>, dim3(mt, a.Hq, a.num_seqs), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(PrefillArgs a, int head_dim, int max_seqlen_q, hipStream_t stream) {
  switch (head_dim) {
    case 64:
      return launch<64>(a, max_seqlen_q, stream);
    case 128:
      return launch<128>(a, max_seqlen_q, stream);
    case 256:
      return launch<256>(a, max_seqlen_q, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace mvs
