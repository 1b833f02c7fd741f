// Page range of one KV split ("L3 hints: split-KV decode and LSE merge",
// section 2): pages are dealt to splits in contiguous runs of
// ceil(num_pages / splits); trailing splits may be empty (p_end <= p_start).
// Shared by the host planner and the decode kernel so both use one formula.
#pragma once

#include <hip/hip_runtime.h>

namespace mi {

__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

__host__ __device__ __forceinline__ void split_pages(int ctx, int page_size, int num_splits,
                                                     int split, int* p_start, int* p_end) {
  const int num_pages = ceil_div(ctx, page_size);
  const int per_split = ceil_div(num_pages, num_splits);
  const int start = split * per_split;
  const int end = start + per_split;
  *p_start = start;
  *p_end = end < num_pages ? end : num_pages;
}

}  // namespace mi
