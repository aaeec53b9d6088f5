// table_device.hip - the query-range table built on the device.
//
// Same table as build_query_range_table (vLLM PR #50294, "implementation
// breakdown" step 1: each scheduled row holds the inclusive (start, end) of
// the valid range of its request that contains the row's absolute position,
// else (-1, -1)), but every input is device-resident and nothing runs on the
// host. The pages keep the table in a persistent buffer sized for the largest
// batch and refill it every step so the step stays free of allocation and can
// be captured in a graph (step 3, pinned staging plus a persistent device
// buffer); building it on the device removes the host pass and the copy from
// that loop as well.
//
// Sixteen workgroups per request, each taking every sixteenth block of 256
// rows. Each thread owns rows of the request and scans the request's ranges
// in list order, keeping the last one that covers the row: exactly the host
// builder's order, where later ranges overwrite earlier ones. The ranges pass
// through LDS in blocks of 256.

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace mvs {
namespace {

constexpr int kThreads = 256;
constexpr int kRowBlocks = 16;  // workgroups per request; each takes every 16th block of 256 rows

__global__ __launch_bounds__(kThreads) void build_table_kernel(int32_t* table, long long capacity,
                                                               const int32_t* qsl, const int32_t* seq_lens,
                                                               const int32_t* offs, const int32_t* ranges) {
  __shared__ int2 rs[kThreads];
  const int b = blockIdx.x;
  const long long t0 = qsl[b], t1 = qsl[b + 1];
  if (t0 < 0 || t1 <= t0) return;  // no rows (a decreasing offset counts as none)
  const long long q_len = t1 - t0;
  const long long ctx = (long long)seq_lens[b] - q_len;
  int r0 = offs[b], r1 = offs[b + 1];
  if (r0 < 0 || r1 < r0) r1 = r0 = 0;  // malformed range offsets: the request gets no range
  const long long rows_end = t1 < capacity ? t1 : capacity;
  for (long long row_base = t0 + (long long)blockIdx.y * kThreads; row_base < rows_end;
       row_base += (long long)kThreads * kRowBlocks) {
    const long long t = row_base + threadIdx.x;
    const long long p = ctx + (t - t0);  // absolute position of the row
    int s_out = -1, e_out = -1;
    for (int rb = r0; rb < r1; rb += kThreads) {
      __syncthreads();
      if (rb + (int)threadIdx.x < r1) {
        const long long r = rb + threadIdx.x;
        rs[threadIdx.x] = make_int2(ranges[2 * r], ranges[2 * r + 1]);
      }
      __syncthreads();
      const int n = min(kThreads, r1 - rb);
      for (int j = 0; j < n; ++j) {
        const int2 x = rs[j];
        if (x.x < x.y && x.x <= p && p <= x.y) {  // valid (start < end) and holds the row
          s_out = x.x;
          e_out = x.y;
        }
      }
    }
    if (t < rows_end) {
      table[2 * t] = s_out;
      table[2 * t + 1] = e_out;
    }
  }
}

}  // namespace
}  // namespace mvs

using mvs::fail;

extern "C" int build_query_range_table_device(int32_t* out_table, int64_t capacity_rows,
                                              const int32_t* query_start_loc, const int32_t* seq_lens,
                                              int32_t num_reqs, const int32_t* range_offsets, const int32_t* ranges,
                                              void* hip_stream) {
  mvs::clear_error();
  if (num_reqs < 0 || capacity_rows < 0) return fail(MVS_ERR_INVALID, "negative sizes");
  if (num_reqs == 0 || capacity_rows == 0) return MVS_OK;
  if (num_reqs > 0x7fffffff - 1) return fail(MVS_ERR_INVALID, "too many requests");
  if (!out_table || !query_start_loc || !seq_lens || !range_offsets || !ranges)
    return fail(MVS_ERR_INVALID, "NULL pointer argument");
  if (!mvs::aligned_to(out_table, 8) || !mvs::aligned_to(query_start_loc, 4) || !mvs::aligned_to(seq_lens, 4) ||
      !mvs::aligned_to(range_offsets, 4) || !mvs::aligned_to(ranges, 4))
    return fail(MVS_ERR_INVALID, "misaligned buffer");
  hipLaunchKernelGGL(mvs::build_table_kernel, dim3((unsigned)num_reqs, mvs::kRowBlocks), dim3(mvs::kThreads), 0,
                     static_cast<hipStream_t>(hip_stream), out_table, (long long)capacity_rows, query_start_loc,
                     seq_lens, range_offsets, ranges);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MVS_ERR_DEVICE, "build_query_range_table_device launch: %s", hipGetErrorString(e));
  return MVS_OK;
}
