// Device helpers shared by the attention kernels (included by .hip sources only).
#pragma once

#include "lra_internal.h"

namespace lra {

// Request that owns work item w (wave-uniform): lane i compares the start of request i, and
// the count of requests starting at or before w, less one, is the owner.  Work starts are
// strictly increasing (every request has at least one work item).
__device__ __forceinline__ int find_request(const AttnArgs* A, int w) {
  const int lane = threadIdx.x & 63;
  const int start = lane < A->n_req ? A->reqs[lane].work_start : 0x7fffffff;
  return __builtin_amdgcn_readfirstlane(__popcll(__ballot(start <= w)) - 1);
}

// Unit of the shared-context decode kernel that owns work item w (wave-uniform): the last
// request whose work start is <= w.  Unit members other than the first hold INT32_MAX and
// never match; the starts of the first members increase strictly.
__device__ __forceinline__ int find_unit(const AttnArgs* A, int w) {
  const int lane = threadIdx.x & 63;
  const int start = lane < A->n_req ? A->reqs[lane].work_start : 0x7fffffff;
  const unsigned long long m = __ballot(start <= w);
  return __builtin_amdgcn_readfirstlane(63 - __clzll(m));
}

// Request that owns combine row `row` (per thread): combine starts are a non-decreasing
// prefix sum over requests (zero rows for requests without key splits), so the owner is
// the last request whose start is <= row.  Binary search over the starts held one per
// lane; every lane of the wave must call it.
__device__ __forceinline__ int find_combine_request(const AttnArgs* A, int row) {
  const int lane = threadIdx.x & 63;
  const int n = A->n_req;
  const int start = lane < n ? A->reqs[lane].comb_start : 0x7fffffff;
  int count = 0;   // requests whose start is <= row
#pragma unroll
  for (int step = 64; step > 0; step >>= 1) {
    const int cand = count + step;
    const int v = __shfl(start, min(cand, 64) - 1);
    if (cand <= n && v <= row) count = cand;
  }
  return count - 1;
}

}  // namespace lra
