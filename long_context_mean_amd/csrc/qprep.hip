// fp8 query preparation for the kernels that read bf16 queries (decode
// scoring, the router, the MISA-dagger rerank), gfx950.
//
// An e4m3 query head is q = s * c with codes c and a positive fp32 head scale
// s.  Every e4m3 value is exact in bf16 (at most 4 significant bits, exponent
// range inside bf16's), and a positive scale leaves ReLU's sign test alone:
//   w * ReLU(s * (c . k)) = (w * s) * ReLU(c . k),   |w| * s = |w * s|.
// So the indexer score and the router term of the fp8 problem are those of
// the bf16 problem (codes as bf16, weights w * s).
#include "common.hpp"
#include "kernels.hpp"

namespace misa {
namespace {

// One thread per 16 codes (one 16-byte load, two 16-byte stores); the first
// `rows` threads also write one folded weight.
__global__ __launch_bounds__(256) void q8_prep_kernel(Q8PrepArgs a) {
  const int64_t n16 = a.rows * (a.d / 16);
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16;
       i += stride) {
    const uint4 x = reinterpret_cast<const uint4*>(a.q)[i];
    uint4 lo, hi;
    e4m3x4_to_bf16x4(x.x, lo.x, lo.y);
    e4m3x4_to_bf16x4(x.y, lo.z, lo.w);
    e4m3x4_to_bf16x4(x.z, hi.x, hi.y);
    e4m3x4_to_bf16x4(x.w, hi.z, hi.w);
    uint4* dst = reinterpret_cast<uint4*>(a.qb) + 2 * i;
    dst[0] = lo;
    dst[1] = hi;
    if (i < a.rows) a.wq[i] = a.w[i] * a.q_scale[i];
  }
}

}  // namespace

hipError_t launch_q8_prep(const Q8PrepArgs& a, hipStream_t st) {
  const int64_t n16 = a.rows * (a.d / 16);          // >= rows (d >= 16)
  const int64_t blocks = (n16 + 255) / 256;
  const int grid = static_cast<int>(blocks < 4096 ? blocks : 4096);
  MISA_LAUNCH(K_Q8_PREP, q8_prep_kernel, dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace misa
