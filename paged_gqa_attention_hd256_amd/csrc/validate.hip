// Device-side check of the data-dependent preconditions that the attention
// calls leave unchecked (checking them inside a call would need a host
// synchronisation): sequence lengths, block-table entries and index lists.
// Every read stays inside the extents the host arguments describe, whatever
// the device data hold, so garbage lengths cannot push a read out of bounds.
#include <algorithm>

#include "pga_args.h"
#include "pga_device.h"

namespace pga {
namespace {

constexpr int kValidateThreads = 256;

__global__ void validate_zero_kernel(int32_t* counts) {
  if (threadIdx.x < kValidateCounts) counts[threadIdx.x] = 0;
}

__device__ __forceinline__ int block_sum(int x, int* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  if (lane_id() == 0) red[wave_id()] = x;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int w = 0; w < kValidateThreads / 64; ++w) s += red[w];
  return s;
}

__device__ __forceinline__ int32_t kv_len(const ValidateArgs& a, int b) {
  return a.lens_k ? a.lens_k[b] : a.cu_k[b + 1] - a.cu_k[b];
}

// One workgroup per sequence: its lengths, and the block-table entries of its
// keys (never more columns than the table row holds).
__global__ __launch_bounds__(kValidateThreads) void validate_seq_kernel(ValidateArgs a) {
  __shared__ int red[kValidateThreads / 64];
  const int b = blockIdx.x;
  const int32_t q0 = a.cu_q[b], q1 = a.cu_q[b + 1];
  const int32_t lq = q1 - q0, lk = kv_len(a, b);
  if (threadIdx.x == 0) {
    bool bad = lq < 0 || lk < 0 || lk < lq || (b == 0 && q0 != 0);
    if (a.cu_k) bad = bad || a.cu_k[b + 1] < a.cu_k[b] || (b == 0 && a.cu_k[0] != 0);
    if (b == a.num_seqs - 1 && a.num_q_tokens >= 0) bad = bad || q1 != a.num_q_tokens;
    const int64_t pages = lk > 0 ? (int64_t(lk) + a.page_size - 1) / a.page_size : 0;
    const bool over = (a.max_q_len > 0 && lq > a.max_q_len) || (a.max_kv_len > 0 && lk > a.max_kv_len) ||
                      pages > a.bt_stride;
    if (bad) atomicAdd(&a.counts[0], 1);
    if (over) atomicAdd(&a.counts[1], 1);
  }
  const int64_t pages = lk > 0 ? (int64_t(lk) + a.page_size - 1) / a.page_size : 0;
  const int64_t cols = pages < a.bt_stride ? pages : a.bt_stride;
  int n = 0;
  for (int64_t j = threadIdx.x; j < cols; j += kValidateThreads) {
    const int32_t page = a.bt[int64_t(b) * a.bt_stride + j];
    n += page < 0 || page >= a.num_pages;
  }
  n = block_sum(n, red);
  if (threadIdx.x == 0 && n > 0) atomicAdd(&a.counts[2], n);
}

// Index lists: one wave per row, rows strided over the grid.  Entries below
// zero are padding; entries at or past the row's Lk_b are counted.
__global__ __launch_bounds__(kValidateThreads) void validate_idx_kernel(ValidateArgs a) {
  const int64_t wave = int64_t(blockIdx.x) * (kValidateThreads / 64) + wave_id();
  const int64_t waves = int64_t(gridDim.x) * (kValidateThreads / 64);
  int n = 0;
  for (int64_t row = wave; row < a.num_q_tokens; row += waves) {
    int lo = 0, hi = a.num_seqs - 1;  // sequence of this row: largest b with cu_q[b] <= row
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.cu_q[mid] <= row) lo = mid; else hi = mid - 1;
    }
    const int32_t lk = kv_len(a, lo);
    for (int e = lane_id(); e < a.num_selected; e += 64) n += a.idx[row * a.idx_stride + e] >= lk;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) n += __shfl_xor(n, off);
  if (lane_id() == 0 && n > 0) atomicAdd(&a.counts[3], n);
}

}  // namespace

hipError_t launch_validate(const ValidateArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(validate_zero_kernel, dim3(1), dim3(64), 0, s, a.counts);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  if (a.num_seqs > 0) {
    hipLaunchKernelGGL(validate_seq_kernel, dim3(a.num_seqs), dim3(kValidateThreads), 0, s, a);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  if (a.idx && a.num_q_tokens > 0 && a.num_seqs > 0 && a.num_selected > 0) {
    const int64_t rows_per_block = kValidateThreads / 64;
    const int64_t blocks = std::min<int64_t>(4096, (a.num_q_tokens + rows_per_block - 1) / rows_per_block);
    hipLaunchKernelGGL(validate_idx_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kValidateThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace pga
