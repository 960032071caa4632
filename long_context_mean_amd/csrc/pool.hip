// Block mean-pooling of index keys, gfx950.
//
// MISA's router summarises the prefix by M = ceil(L/B) blocks of mean-pooled
// index keys (MISA technical summary, gist.science, "Methodology" item 1).
// One workgroup pools one block of one sequence: its 256 threads stream the
// block's key rows with 16-byte loads (consecutive threads read consecutive
// 16-byte pieces of a row, so a wavefront reads whole rows), accumulate in
// fp32 registers, and reduce the row groups through LDS.  The pass is one
// HBM read of the keys: bandwidth bound.
//
// Incremental mode (a decode loop appending tokens to its key cache): the
// router only reads blocks a row sees completely and computes a row's
// partial last block from the keys themselves, so the cached table needs
// only the complete blocks.  Each call pools exactly the blocks that the
// newly appended tokens complete (one workgroup per candidate block; those
// that complete nothing exit at once): O(B d) work per B appended tokens.
// Keys may live in a paged cache (KeyIndex).
#include "common.hpp"
#include "kernels.hpp"

namespace misa {
namespace {

template <int KT, int D>
__global__ __launch_bounds__(256) void pool_kernel(const uint8_t* __restrict__ k,
                                                   const float* __restrict__ k_scale, int L,
                                                   int B, float* __restrict__ kbar, KeyIndex ki,
                                                   const int32_t* __restrict__ len_old,
                                                   const int32_t* __restrict__ len_new) {
  constexpr int EB = KeyBytes<KT>::value;
  constexpr int ROW_BYTES = D * EB;
  constexpr int CPR = ROW_BYTES / 16;          // 16-byte pieces per row
  constexpr int EPC = 16 / EB;                 // elements per piece
  constexpr int RG = 256 / CPR;                // row groups
  __shared__ float part[RG][D + 1];

  const int s = blockIdx.y, M = (L + B - 1) / B;
  int b = blockIdx.x, t1;
  if (len_new) {
    // the (blockIdx.x)-th block at or after the one holding token len_old[s]
    b += len_old[s] / B;
    t1 = (b + 1) * B;
    if (t1 > len_new[s] || (b + 1) * B <= len_old[s]) return;   // not completed by this call
  } else {
    t1 = (b * B + B < L) ? b * B + B : L;
  }
  const int t0 = b * B;
  const int c = threadIdx.x % CPR, g = threadIdx.x / CPR;

  float acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.f;

  constexpr int U = 8;
  for (int t = t0 + g; t < t1; t += U * RG) {
    uint4 x[U];
    float sc[U];
#pragma unroll
    for (int r = 0; r < U; ++r) {
      const int tt = t + r * RG;
      const int tc = tt < t1 ? tt : t;           // stay in bounds; masked below
      const size_t row = ki.row(s, tc);
      x[r] = *reinterpret_cast<const uint4*>(k + row * ROW_BYTES + c * 16);
      sc[r] = 1.f;
      if constexpr (KT == DT_E4M3) sc[r] = k_scale[row];
    }
#pragma unroll
    for (int r = 0; r < U; ++r) {
      if (t + r * RG < t1) {
        float v[EPC];
        unpack16<KT>(x[r], v);
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          if constexpr (KT == DT_E4M3)
            acc[e] += v[e] * sc[r];
          else
            acc[e] += v[e];
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < EPC; ++e) part[g][c * EPC + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    float sum = 0.f;
#pragma unroll 8
    for (int r = 0; r < RG; ++r) sum += part[r][threadIdx.x];
    kbar[(static_cast<size_t>(s) * M + b) * D + threadIdx.x] = sum / static_cast<float>(t1 - t0);
  }
}

template <int KT, int D>
hipError_t launch_pool_t(const PoolArgs& a, hipStream_t st) {
  if (a.len_new) {
    // blocks that max_new appended tokens can complete: floor(max_new / B) + 1
    const int nb = a.max_new / a.B + 1;
    MISA_LAUNCH(K_POOL_UPDATE, (pool_kernel<KT, D>), dim3(nb, a.S), dim3(256), 0, st,
                static_cast<const uint8_t*>(a.k), a.k_scale, a.L, a.B, a.kbar, a.kidx,
                a.len_old, a.len_new);
  } else {
    const int M = (a.L + a.B - 1) / a.B;
    MISA_LAUNCH(K_POOL, (pool_kernel<KT, D>), dim3(M, a.S), dim3(256), 0, st,
                static_cast<const uint8_t*>(a.k), a.k_scale, a.L, a.B, a.kbar, a.kidx,
                nullptr, nullptr);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool(const PoolArgs& a, hipStream_t st) {
  if (a.d == 64) {
    if (a.k_dt == DT_F32) return launch_pool_t<DT_F32, 64>(a, st);
    if (a.k_dt == DT_BF16) return launch_pool_t<DT_BF16, 64>(a, st);
    return launch_pool_t<DT_E4M3, 64>(a, st);
  }
  if (a.k_dt == DT_F32) return launch_pool_t<DT_F32, 128>(a, st);
  if (a.k_dt == DT_BF16) return launch_pool_t<DT_BF16, 128>(a, st);
  return launch_pool_t<DT_E4M3, 128>(a, st);
}

}  // namespace misa
