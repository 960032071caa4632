// Radix-select step shared by the top-k kernels and the decode scoring
// kernel's per-workgroup candidate cut.
#pragma once

#include "common.hpp"

namespace misa {

// Finds the bin of a histogram (NBINS bins, bin NBINS-1 = largest keys) that
// holds the K-th largest element.  With clamp_total, K = min(K, total) first.
// All NT threads call it; results in `res`: [0] digit, [1] rank inside the
// digit's bin (1-based), [2] K, [3] total.  K == 0 leaves digit/rank 0.
template <int NT, int NBINS>
__device__ __forceinline__ void find_digit(const uint32_t* hist, uint32_t K, bool clamp_total, uint32_t* sm,
                           uint32_t* res) {
  constexpr int PER = NBINS >= NT ? NBINS / NT : 1;
  const int t = static_cast<int>(threadIdx.x);
  const bool owner = NBINS >= NT || t < NBINS;
  const int lo = NBINS - (t + 1) * PER;                 // this thread's lowest bin
  uint32_t v[PER];
  if (owner) {
    if constexpr (PER % 4 == 0) {
      const uint4* p4 = reinterpret_cast<const uint4*>(hist + lo);
#pragma unroll
      for (int q = 0; q < PER / 4; ++q) {
        const uint4 x = p4[q];
        v[4 * q] = x.x;
        v[4 * q + 1] = x.y;
        v[4 * q + 2] = x.z;
        v[4 * q + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int q = 0; q < PER; ++q) v[q] = hist[lo + q];
    }
  } else {
#pragma unroll
    for (int q = 0; q < PER; ++q) v[q] = 0u;
  }
  uint32_t c = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) c += v[q];
  uint32_t total;
  const uint32_t above = block_excl_scan<NT>(c, sm, total);
  if (clamp_total && K > total) K = total;
  if (t == 0) {
    res[0] = 0;
    res[1] = 0;
    res[2] = K;
    res[3] = total;
  }
  __syncthreads();
  if (K > 0 && above < K && K <= above + c) {
    uint32_t acc = above;
#pragma unroll
    for (int q = PER - 1; q >= 0; --q) {
      if (acc < K && acc + v[q] >= K) {
        res[0] = static_cast<uint32_t>(lo + q);
        res[1] = K - acc;
      }
      acc += v[q];
    }
  }
  __syncthreads();
}

}  // namespace misa
