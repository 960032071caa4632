// Sparse attention over the selected tokens, gfx950: the consumer of the
// indexer's top-k (the indexer picks the tokens the main attention reads,
// MISA abstract, HF Daily Papers digest).  The attention is ordinary softmax
// attention of every query head over the row's selected cache rows; value
// rows are the first d_v elements of the same rows (latent attention's
// shared key/value cache), so one gathered row serves both products.
//
//   s_t = scale * q_h . kv_t,   out_h = sum_t softmax(s)_t kv_t[0:d_v],
//   lse_h = log sum_t exp(s_t)
//
// attn_split_kernel: one workgroup per (split of the selection, block of 32
// heads, row).  A split is a few chunks of 64 selected tokens, handled in
// turn with an online softmax (running max, rescaled sum and output); each
// chunk's rows are gathered into LDS (padded rows: conflict-free for both
// read patterns below).  Wavefront w owns heads 16*(w/2) .. +15 of the block
// and half of d_v, whose output stays in registers across the chunks.
//  - S^T = K Q^T on v_mfma_f32_16x16x32_bf16: A = 16 cached rows from LDS,
//    B = the wavefront's query heads (registers).  Output lane (g, c) holds
//    tokens 4g..4g+3 of head c, so each head's max and sum over the split
//    take two cross-lane steps.
//  - O^T += V^T P^T on v_mfma_f32_16x16x16_bf16: P^T is the S^T output layout
//    as it stands (lane (g, c): tokens 4g..4g+3 of head c, the K = 16 slice of
//    lane group g), and V^T comes from ds_read_b64_tr_b16: lane 4m+q of a
//    16-lane group points at 4 values of row 4g+m, and the transpose hands
//    lane c the values of rows 4g..4g+3 in column c.  P is split into bf16
//    hi + lo parts (two MFMAs), so the products carry ~2^-17 relative error.
// The split's partial (sum_t p_t v_t, max, sum_t p_t) goes to the workspace;
// attn_combine_kernel merges the splits of each (row, head).

#include "common.hpp"
#include "kernels.hpp"

namespace misa {
namespace {

typedef short bf16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kChunkTok = 64;          // selected tokens per chunk (one LDS fill)
// chunks per split: 2 measured best against 1 and 4 at 128 heads x 2048
// selected tokens
constexpr int kChunksPerSplit = 2;
constexpr int kHeadBlock = 32;         // heads per workgroup (16 per wavefront pair)
constexpr float kLog2e = 1.4426950408889634f;

struct AttnParams {
  const uint16_t* q;        // [N, H, dqk] bf16
  const uint8_t* kv;        // cache rows of dqk bf16
  KeyIndex ki;
  const int32_t* q_seq;
  const int32_t* idx;       // [N, topk]
  int N, H, dv, topk, splits, chunks;   // chunks of kChunkTok tokens per split
  float scale2;             // softmax scale * log2(e)
  float* o_part;            // [N, H, splits, dv]: sum_t p_t v_t over the split
  float2* ml_part;          // [N, H, splits]: (max in log2 units, sum_t p_t)
};

__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// DVF: value tiles per wavefront (d_v / 32) fixed at compile time, or 0 to
// take them from d_v at run time.  With DVF fixed the value products run as
// DVF independent accumulation chains side by side; the run-time form
// handles one tile's chain at a time.
template <int KK, int DVF>
__global__ __launch_bounds__(256) void attn_split_kernel(AttnParams p) {
  constexpr int DQK = KK * 32;
  constexpr int ROWP = DQK * 2 + 16;                    // padded LDS row (bytes)
  constexpr int PIECES = DQK * 2 / 16;                  // 16-byte pieces per row
  constexpr int MAXDVT = 16;                            // value tiles per wavefront (d_v <= 512)
  __shared__ __align__(16) uint8_t kvt[kChunkTok * ROWP];
  __shared__ int tok_lds[kChunkTok];

  const int sp = blockIdx.x, hb = blockIdx.y, n = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(tid >> 6));
  const int g = lane >> 4, c = lane & 15;
  const int s = p.q_seq[n];

  // this wavefront's query heads as the B operand: lane (g, c) = head c,
  // d elements 32kk + 8g .. +7
  const int head = hb * kHeadBlock + 16 * (wave >> 1) + c;
  const bool hv = head < p.H;
  bf16x8_t qf[KK];
  {
    const uint16_t* qr = p.q + (static_cast<size_t>(n) * p.H + (hv ? head : 0)) * DQK;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4_t v = *reinterpret_cast<const u32x4_t*>(qr + 32 * kk + 8 * g);
      if (!hv) v = u32x4_t{0u, 0u, 0u, 0u};
      qf[kk] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  const int half = p.dv / 2;
  const int dvt = DVF > 0 ? DVF : half / 16;            // value tiles of this wavefront
  const int dv0 = (wave & 1) * half;
  const int r4 = lane & 15;                             // 4m + q within the lane group
  f32x4_t o[MAXDVT];
#pragma unroll
  for (int j = 0; j < MAXDVT; ++j) o[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff(), l_run = 0.f;         // per head c, in log2 units

  for (int ch = 0; ch < p.chunks; ++ch) {
    const int e0 = (sp * p.chunks + ch) * kChunkTok;
    if (e0 >= p.topk) break;                            // uniform over the workgroup
    __syncthreads();                                    // the previous chunk's reads are done
    if (tid < kChunkTok) {
      const int e = e0 + tid;
      tok_lds[tid] = e < p.topk ? p.idx[static_cast<size_t>(n) * p.topk + e] : -1;
    }
    __syncthreads();
    // gather the chunk's cache rows (unselected slots read token 0, masked below)
    constexpr int TOTAL = kChunkTok * PIECES;
    constexpr int BATCH = 6;
    for (int base = 0; base < TOTAL; base += 256 * BATCH) {
      // every read issued (pieces past the chunk re-read its last one and
      // are not stored), page numbers first for a paged cache, so a batch is
      // one round trip (two paged) rather than one per guarded read
      u32x4_t x[BATCH];
      int tk[BATCH];
      size_t row[BATCH];
#pragma unroll
      for (int b = 0; b < BATCH; ++b) {
        const int f = base + b * 256 + tid;
        const int t = tok_lds[(f < TOTAL ? f : TOTAL - 1) / PIECES];
        tk[b] = t >= 0 ? t : 0;
      }
      if (p.ki.table) {
        int pg[BATCH];
#pragma unroll
        for (int b = 0; b < BATCH; ++b) pg[b] = p.ki.page(s, tk[b]);
#pragma unroll
        for (int b = 0; b < BATCH; ++b) row[b] = p.ki.row_in_page(pg[b], tk[b]);
      } else {
#pragma unroll
        for (int b = 0; b < BATCH; ++b) row[b] = static_cast<size_t>(s) * p.ki.L + tk[b];
      }
#pragma unroll
      for (int b = 0; b < BATCH; ++b) {
        const int f = base + b * 256 + tid;
        const int pc = (f < TOTAL ? f : TOTAL - 1) % PIECES;
        x[b] = *reinterpret_cast<const u32x4_t*>(p.kv + row[b] * (DQK * 2) + 16 * pc);
      }
#pragma unroll
      for (int b = 0; b < BATCH; ++b) {
        const int f = base + b * 256 + tid;
        if (f < TOTAL) {
          const int r = f / PIECES, pc = f % PIECES;
          *reinterpret_cast<u32x4_t*>(kvt + r * ROWP + 16 * pc) = x[b];
        }
      }
    }
    __syncthreads();

    // S^T for the chunk's 4 tiles of 16 tokens, in log2 units; unselected
    // -inf.  The 4 tiles' accumulation chains (over d, in order) run side by
    // side.
    float sv[4][4];
    {
      f32x4_t acc[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bf16x8_t a = __builtin_bit_cast(
              bf16x8_t, *reinterpret_cast<const u32x4_t*>(kvt + (16 * t + c) * ROWP + 16 * g +
                                                          64 * kk));
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[kk], acc[t], 0, 0, 0);
        }
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sv[t][i] = tok_lds[16 * t + 4 * g + i] >= 0 ? acc[t][i] * p.scale2 : -__builtin_inff();
    }
    float m_c = -__builtin_inff();
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) m_c = fmaxf(m_c, sv[t][i]);
    m_c = fmaxf(m_c, __shfl_xor(m_c, 16, 64));
    m_c = fmaxf(m_c, __shfl_xor(m_c, 32, 64));
    const float m_new = fmaxf(m_run, m_c);
    if (m_new == -__builtin_inff()) continue;           // nothing selected so far (uniform per head)
    const float alpha = exp2f(m_run - m_new);           // 0 when m_run is -inf
    // P^T as bf16 hi + lo (B operand of the 16x16x16 MFMA: k = tokens 4g..4g+3)
    float lc = 0.f;
    bf16x4_t phi[4], plo[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint32_t h[4], lo[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = exp2f(sv[t][i] - m_new);
        lc += pv;
        h[i] = bf16_rne(pv);
        lo[i] = bf16_rne(pv - __uint_as_float(h[i] << 16));
      }
      phi[t] = bf16x4_t{static_cast<short>(h[0]), static_cast<short>(h[1]),
                        static_cast<short>(h[2]), static_cast<short>(h[3])};
      plo[t] = bf16x4_t{static_cast<short>(lo[0]), static_cast<short>(lo[1]),
                        static_cast<short>(lo[2]), static_cast<short>(lo[3])};
    }
    lc += __shfl_xor(lc, 16, 64);
    lc += __shfl_xor(lc, 32, 64);
    l_run = l_run * alpha + lc;
    m_run = m_new;

    // O^T (this wavefront's half of d_v, 16 value columns per tile) += V^T P^T;
    // per tile j: rescale, then the 4 token tiles' hi and lo products in order
    typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
    if constexpr (DVF > 0) {
#pragma unroll
      for (int j = 0; j < DVF; ++j) o[j] = o[j] * alpha;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int row = 16 * t + 4 * g + (r4 >> 2);
        bf16x4_t av[DVF];
#pragma unroll
        for (int j = 0; j < DVF; ++j) {
          const int col = dv0 + 16 * j + 4 * (r4 & 3);
          lds_bf16x4_t* ap = (lds_bf16x4_t*)((__attribute__((address_space(3))) uint8_t*)kvt +
                                             row * ROWP + col * 2);
          av[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(ap);
        }
#pragma unroll
        for (int j = 0; j < DVF; ++j) {
          o[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av[j], phi[t], o[j], 0, 0, 0);
          o[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av[j], plo[t], o[j], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < MAXDVT; ++j) {
        if (j < dvt) {
          f32x4_t acc = o[j] * alpha;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int row = 16 * t + 4 * g + (r4 >> 2);
            const int col = dv0 + 16 * j + 4 * (r4 & 3);
            // generic -> LDS address space (a C-style cast is the address-space cast)
            lds_bf16x4_t* ap = (lds_bf16x4_t*)((__attribute__((address_space(3))) uint8_t*)kvt +
                                               row * ROWP + col * 2);
            const bf16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(ap);
            acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, phi[t], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, plo[t], acc, 0, 0, 0);
          }
          o[j] = acc;
        }
      }
    }
  }
  if (hv) {
    // the partials are read once, by the combine kernel: non-temporal stores
    // keep them from displacing cached data
    float* op = p.o_part + ((static_cast<size_t>(n) * p.H + head) * p.splits + sp) * p.dv +
                dv0 + 4 * g;
#pragma unroll
    for (int j = 0; j < (DVF > 0 ? DVF : MAXDVT); ++j)
      if (j < dvt) __builtin_nontemporal_store(o[j], reinterpret_cast<f32x4_t*>(op + 16 * j));
    if (g == 0 && (wave & 1) == 0)
      p.ml_part[(static_cast<size_t>(n) * p.H + head) * p.splits + sp] = make_float2(m_run, l_run);
  }
}

// One workgroup per (row, head): out = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ o_part,
                                                           const float2* __restrict__ ml_part,
                                                           int splits, int dv,
                                                           float* __restrict__ out,
                                                           float* __restrict__ lse) {
  __shared__ float wsh[1024];
  __shared__ float red[4];
  const size_t nh = blockIdx.x;
  const float2* ml = ml_part + nh * splits;
  const float* op = o_part + nh * splits * dv;
  // the first PS splits of this thread's (at most two: d_v <= 512) output
  // columns, loaded before the weights are known: unconditional loads of
  // clamped (valid) addresses, so they are all in flight together; the
  // partials are read once, non-temporally
  constexpr int PS = 16;
  float pv[2][PS];
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) {
    const int d = min(static_cast<int>(threadIdx.x) + 256 * c2, dv - 1);
#pragma unroll
    for (int u = 0; u < PS; ++u)
      pv[c2][u] = __builtin_nontemporal_load(&op[static_cast<size_t>(min(u, splits - 1)) * dv + d]);
  }
  float M = -__builtin_inff();
  for (int i = threadIdx.x; i < splits; i += 256) M = fmaxf(M, ml[i].x);
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float Ls = 0.f;
  for (int i = threadIdx.x; i < splits; i += 256) {
    const float wgt = M == -__builtin_inff() ? 0.f : exp2f(ml[i].x - M);
    if (i < 1024) wsh[i] = wgt;
    Ls += wgt * ml[i].y;
  }
  for (int o = 32; o > 0; o >>= 1) Ls += __shfl_xor(Ls, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = Ls;
  __syncthreads();
  Ls = red[0] + red[1] + red[2] + red[3];
  const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
  auto weight = [&](int k) {
    return k < 1024 ? wsh[k] : (M == -__builtin_inff() ? 0.f : exp2f(ml[k].x - M));
  };
  // splits in order (a split with no selected token holds zeros, so its
  // weight may be anything finite); past the prefetched ones in groups of 8
  // independent loads
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) {
    const int d = static_cast<int>(threadIdx.x) + 256 * c2;
    if (d >= dv) break;
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < PS; ++u)
      if (u < splits) acc += weight(u) * pv[c2][u];
    int i = PS;
    for (; i + 8 <= splits; i += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = __builtin_nontemporal_load(&op[static_cast<size_t>(i + u) * dv + d]);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += weight(i + u) * v[u];
    }
    for (; i < splits; ++i)
      acc += weight(i) * __builtin_nontemporal_load(&op[static_cast<size_t>(i) * dv + d]);
    out[nh * dv + d] = acc * inv;
  }
  if (threadIdx.x == 0)
    lse[nh] = Ls > 0.f ? (M + log2f(Ls)) * 0.6931471805599453f : -__builtin_inff();
}

template <int KK, int DVF>
hipError_t launch_attn_t(const AttnArgs& a, hipStream_t st) {
  AttnParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.kv = static_cast<const uint8_t*>(a.kv);
  p.ki = a.kidx;
  p.q_seq = a.q_seq;
  p.idx = a.idx;
  p.N = a.N;
  p.H = a.H;
  p.dv = a.d_v;
  p.topk = a.topk;
  p.splits = attn_splits(a.topk);
  p.chunks = attn_chunks_per_split(a.topk);
  p.scale2 = a.scale * kLog2e;
  p.o_part = a.o_part;
  p.ml_part = reinterpret_cast<float2*>(a.ml_part);
  const dim3 grid(p.splits, (a.H + kHeadBlock - 1) / kHeadBlock, a.N);
  MISA_LAUNCH(K_ATTN_SPLIT, (attn_split_kernel<KK, DVF>), grid, dim3(256), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  MISA_LAUNCH(K_ATTN_COMBINE, attn_combine_kernel, dim3(a.N * a.H), dim3(256), 0, st,
              a.o_part, reinterpret_cast<const float2*>(a.ml_part), p.splits, a.d_v, a.out,
              a.lse);
  return hipGetLastError();
}

}  // namespace

int attn_chunks_per_split(int topk) {
  const int chunks = (topk + kChunkTok - 1) / kChunkTok;
  return kChunksPerSplit < chunks ? kChunksPerSplit : chunks;
}

int attn_splits(int topk) {
  const int chunks = (topk + kChunkTok - 1) / kChunkTok;
  const int per = attn_chunks_per_split(topk);
  return (chunks + per - 1) / per;
}

// d_v of 64, 128, 256 or 512 (value tiles per wavefront 2, 4, 8 or 16) take
// the fixed forms; other d_v the run-time one.
template <int KK>
hipError_t launch_attn_kk(const AttnArgs& a, hipStream_t st) {
  const int dvt = a.d_v / 32;
  if (dvt == 2) return launch_attn_t<KK, 2>(a, st);
  if constexpr (KK >= 4)
    if (dvt == 4) return launch_attn_t<KK, 4>(a, st);
  if constexpr (KK >= 8)
    if (dvt == 8) return launch_attn_t<KK, 8>(a, st);
  if constexpr (KK >= 16)
    if (dvt == 16) return launch_attn_t<KK, 16>(a, st);
  return launch_attn_t<KK, 0>(a, st);
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
  switch (a.d_qk) {
    case 64: return launch_attn_kk<2>(a, st);
    case 128: return launch_attn_kk<4>(a, st);
    case 256: return launch_attn_kk<8>(a, st);
    default: return launch_attn_kk<18>(a, st);
  }
}

}  // namespace misa
