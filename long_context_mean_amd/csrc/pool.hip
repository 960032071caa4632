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
#include "pool_block.hpp"

namespace misa {
namespace {

template <int KT, int D>
__global__ __launch_bounds__(256) void pool_kernel(const uint8_t* __restrict__ k,
                                                   const float* __restrict__ k_scale, int L,
                                                   int B, float* __restrict__ kbar, KeyIndex ki,
                                                   const int32_t* __restrict__ len_old,
                                                   const int32_t* __restrict__ len_new) {
  __shared__ float part[PoolMap<KT, D>::RG][D + 1];

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
  const float m = pool_block_mean<KT, D>(k, k_scale, ki, s, b * B, t1, part);
  if (threadIdx.x < D) kbar[(static_cast<size_t>(s) * M + b) * D + threadIdx.x] = m;
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
