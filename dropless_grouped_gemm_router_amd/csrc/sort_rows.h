// Token rows copied into expert order, x_sorted[j] = x[perm[j] / k]: the
// "sorted" dispatch of the forward (kernel_gmm_gpu.json "layer" suite,
// field "dispatch") and the row-range operand of the backward's bf16
// dW_gate / dW_up. Each wave moves kSortRows rows in 16-byte pieces with all
// of a piece's row loads issued before its stores.
#pragma once

#include "common.h"

namespace moe {

constexpr int kSortRows = 4;
constexpr int kSortThreads = 256;

template <typename T>
__global__ __launch_bounds__(kSortThreads) void sort_rows_kernel(const T* __restrict__ x,
                                                                 const int32_t* __restrict__ perm,
                                                                 int k, int64_t S, int d,
                                                                 T* __restrict__ xs) {
  constexpr int V = 16 / static_cast<int>(sizeof(T));
  const int64_t j0 =
      (static_cast<int64_t>(blockIdx.x) * (kSortThreads / 64) + (threadIdx.x >> 6)) * kSortRows;
  int64_t t[kSortRows];
#pragma unroll
  for (int q = 0; q < kSortRows; ++q) t[q] = j0 + q < S ? perm[j0 + q] / k : -1;
  for (int c = (threadIdx.x & 63) * V; c < d; c += 64 * V) {
    u32x4 v[kSortRows];
#pragma unroll
    for (int q = 0; q < kSortRows; ++q)
      if (t[q] >= 0) v[q] = *reinterpret_cast<const u32x4*>(x + t[q] * d + c);
#pragma unroll
    for (int q = 0; q < kSortRows; ++q)
      if (t[q] >= 0) *reinterpret_cast<u32x4*>(xs + (j0 + q) * d + c) = v[q];
  }
}

// Blocks of sort_rows_kernel for S rows.
inline unsigned sort_rows_blocks(int64_t S) {
  constexpr int64_t per = (kSortThreads / 64) * kSortRows;
  return static_cast<unsigned>((S + per - 1) / per);
}

}  // namespace moe
