// Device-side helpers shared by the gfx950 kernels of the MISA indexer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace misa {

enum : int { DT_F32 = 0, DT_BF16 = 1, DT_E4M3 = 2 };

// Radix select on 32-bit order keys: 12 + 12 + 8 bit digits.
constexpr int kDigit0Bits = 12, kDigit1Bits = 12, kDigit2Bits = 8;
constexpr int kBins0 = 1 << kDigit0Bits, kBins1 = 1 << kDigit1Bits, kBins2 = 1 << kDigit2Bits;
constexpr int kShift0 = 32 - kDigit0Bits;                 // 20
constexpr int kShift1 = kShift0 - kDigit1Bits;            // 8
// Per-row words of the level-0 histogram region in the workspace: 4096 bins,
// then the candidate count and the selection's level-0 digit, its rank and K
// (written by the collect step), padded to keep rows 256-byte aligned.
constexpr int kHistWords = kBins0 + 64;
constexpr int kCandCountOffset = kBins0;
constexpr int kMetaOffset = kCandCountOffset + 1;

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) {
  return __uint_as_float(packed & 0xFFFF0000u);
}

// Four OCP e4m3 codes (one 32-bit word) -> four bf16 values (two packed
// words).  The conversion is exact: an e4m3 value has at most 4 significant
// bits and its exponent range lies inside bf16's.
__device__ __forceinline__ void e4m3x4_to_bf16x4(uint32_t codes, uint32_t& lo, uint32_t& hi) {
  bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, false);
  bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, true);
  lo = __builtin_bit_cast(uint32_t, a);
  hi = __builtin_bit_cast(uint32_t, b);
}

// Row of token t of key sequence s in the key storage (key bytes and fp8
// scales share the numbering): contiguous sequences [S, L], or pages of
// 2^page_shift tokens whose physical page numbers a block table
// [S, max_pages] lists per sequence (paged KV cache).
struct KeyIndex {
  const int32_t* table;   // NULL: contiguous
  int L;
  int page_shift;
  int max_pages;

  __device__ __forceinline__ size_t row(int s, int t) const {
    if (table == nullptr) return static_cast<size_t>(s) * L + t;
    return row_in_page(page(s, t), t);
  }
  // paged: the page holding token t of sequence s, and the row of token t in
  // page pg (split so that a caller can have many page reads in flight)
  __device__ __forceinline__ int page(int s, int t) const {
    return table[static_cast<size_t>(s) * max_pages + (t >> page_shift)];
  }
  __device__ __forceinline__ size_t row_in_page(int pg, int t) const {
    return (static_cast<size_t>(pg) << page_shift) + (t & ((1 << page_shift) - 1));
  }
};

template <int KT>
struct KeyBytes;
template <>
struct KeyBytes<DT_F32> { static constexpr int value = 4; };
template <>
struct KeyBytes<DT_BF16> { static constexpr int value = 2; };
template <>
struct KeyBytes<DT_E4M3> { static constexpr int value = 1; };

// Unpacks one 16-byte piece of key storage into 16 / bytes fp32 values.
template <int KT>
__device__ __forceinline__ void unpack16(uint4 x, float* out) {
  const uint32_t wds[4] = {x.x, x.y, x.z, x.w};
  if constexpr (KT == DT_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(wds[i]);
  } else if constexpr (KT == DT_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = bf16_lo(wds[i]);
      out[2 * i + 1] = bf16_hi(wds[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t lo, hi;
      e4m3x4_to_bf16x4(wds[i], lo, hi);
      out[4 * i + 0] = bf16_lo(lo);
      out[4 * i + 1] = bf16_hi(lo);
      out[4 * i + 2] = bf16_lo(hi);
      out[4 * i + 3] = bf16_hi(hi);
    }
  }
}

// Total order on fp32 scores as unsigned keys: larger score <-> larger key,
// -0.0 and +0.0 map to the same key (adding +0.0 turns -0.0 into +0.0).  Key
// 0 (a negative NaN pattern) is never produced for a finite score and marks
// an empty slot.
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t b = __float_as_uint(v + 0.0f);
  return b ^ (static_cast<uint32_t>(static_cast<int32_t>(b) >> 31) | 0x80000000u);
}

// ReLU in one instruction (median of x, 0 and the largest finite float).
__device__ __forceinline__ float relu(float x) {
  return __builtin_amdgcn_fmed3f(x, 0.0f, 3.4028234663852886e38f);
}

__device__ __forceinline__ float key_score(uint32_t u) {
  const uint32_t b = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(b);
}

// Inclusive scan across the 64 lanes of a wavefront.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Exclusive scan over the NT threads of a workgroup; `sm` holds NT/64 words.
// Every thread must call it.  Returns the exclusive prefix, sets `total`.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sm, uint32_t& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(v);
  if (lane == 63) sm[wid] = incl;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const uint32_t s = sm[i];
    before += (i < wid) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return before + incl - v;
}

// Block-wide sum over NT threads; `sm` holds NT/64 words.
template <int NT>
__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t* sm) {
  uint32_t total;
  (void)block_excl_scan<NT>(v, sm, total);
  return total;
}

}  // namespace misa
