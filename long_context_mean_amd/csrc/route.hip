// Block-pooled head router, gfx950.
//
// For query row n the router scores every indexer head j against the pooled
// block keys and keeps the top-h heads (MISA technical summary, gist.science,
// "Methodology" item 1; cost O(H_I M)).  The head importance is
//   r[n,j] = |w[n,j]| * sum_{b < M_n} ReLU(q[n,j,:] . kbar_n[b]),
// the indexer's own ReLU term at block granularity.  Blocks fully visible to
// the row are read from the pooled table; the row's partial last block (when
// L_n is not a multiple of B) is the mean of its visible keys only.
//
//  route_partial: grid (chunk of 16 full blocks, row); per-chunk sums go to
//    the workspace (no float atomics: the final sum runs in a fixed order and
//    is deterministic).  bf16 q: an MFMA product of the heads against the
//    chunk's pooled keys split into two bf16 parts.  fp32 q: lane j holds
//    head j's query row in registers and reads the pooled keys from LDS as
//    broadcasts.
//  route_select: one workgroup per row.  Sums the chunk partials, adds the
//    partial-block term, applies |w|, and routes every head that fewer than
//    h heads beat under (r desc, head index asc); heads are written in
//    ascending order.
#include "common.hpp"
#include "kernels.hpp"
#include "pool_block.hpp"
#include "route_select.hpp"

namespace misa {
namespace {

constexpr int kRouteBlocks = 16;     // pooled blocks per route_partial workgroup

template <int QT, int D>
__global__ __launch_bounds__(256) void route_partial_kernel(
    const void* __restrict__ q, const float* __restrict__ kbar, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int L, int B, int H_I, int nchunks,
    float* __restrict__ partial) {
  __shared__ __align__(16) float kb_lds[kRouteBlocks][D];
  __shared__ float red[4][64];

  const int n = blockIdx.y, chunk = blockIdx.x;
  const int Ln = q_pos[n] + 1;
  const int Mf = Ln / B;                       // blocks fully visible to row n
  const int M = (L + B - 1) / B;               // rows of the pooled table
  const int b0 = chunk * kRouteBlocks;
  const int b1 = (b0 + kRouteBlocks < Mf) ? b0 + kRouteBlocks : Mf;
  float* out = partial + (static_cast<size_t>(n) * nchunks + chunk) * H_I;
  if (b0 >= b1) {
    for (int j = threadIdx.x; j < H_I; j += 256) out[j] = 0.f;
    return;
  }
  const int s = q_seq[n];
  const int nb = b1 - b0;
  // all loads in flight at once: pooled keys of the chunk, then the head row
  constexpr int NF = kRouteBlocks * D / 4 / 256;      // float4 per thread
  const float4* src = reinterpret_cast<const float4*>(kbar + (static_cast<size_t>(s) * M + b0) * D);
  float4 tmp[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int e = threadIdx.x + f * 256;
    tmp[f] = e < nb * D / 4 ? src[e] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float qr[D];
  if (lane < H_I) load_q_row<QT, D>(q, static_cast<size_t>(n) * H_I + lane, qr);
#pragma unroll
  for (int f = 0; f < NF; ++f)
    reinterpret_cast<float4*>(&kb_lds[0][0])[threadIdx.x + f * 256] = tmp[f];
  __syncthreads();

  float acc = 0.f;
  if (lane < H_I) {
    for (int b = wave; b < nb; b += 8) {
      const int b2 = b + 4 < nb ? b + 4 : b;
      float d0 = 0.f, d1 = 0.f;
#pragma unroll
      for (int i = 0; i < D; i += 4) {
        const float4 x = *reinterpret_cast<const float4*>(&kb_lds[b][i]);
        const float4 y = *reinterpret_cast<const float4*>(&kb_lds[b2][i]);
        d0 += qr[i] * x.x + qr[i + 1] * x.y + qr[i + 2] * x.z + qr[i + 3] * x.w;
        d1 += qr[i] * y.x + qr[i + 1] * y.y + qr[i + 2] * y.z + qr[i + 3] * y.w;
      }
      acc += fmaxf(d0, 0.f);
      if (b + 4 < nb) acc += fmaxf(d1, 0.f);
    }
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (threadIdx.x < H_I)
    out[threadIdx.x] = (red[0][threadIdx.x] + red[1][threadIdx.x]) +
                       (red[2][threadIdx.x] + red[3][threadIdx.x]);
}

// route_partial on the matrix cores (bf16 q): grid (chunk of 16 full
// blocks, row).  Wavefront w takes heads 16w..16w+15 as the A operand of
// v_mfma_f32_16x16x32_bf16 (straight from q); the chunk's 16 pooled keys are
// split as kbar = hi + lo (both bf16, round to nearest, so each product is
// exact and the dot carries ~2^-17 relative error) and laid out in LDS as
// the B operand, one column per block.  Lane (g, c) gets heads 4g..4g+3
// against block c; ReLU, the visibility mask and the sum over the 16 blocks
// (across lanes) give the chunk's partial for every head.
//
// For the routed decode step that selects heads inside the scoring kernel
// (RoutePartialExtra), the grid has one more workgroup per row: it writes the
// row's partial-block term ReLU(q_j . mean of the visible keys of the last,
// incomplete block) to chunk slot nchunks (0 when the row ends on a block
// boundary), and chunk 0 of each row clears that row's level-0 histogram for
// the scoring kernel.
//
// With the incremental pooling folded in (the blocks completed by the tokens
// len_old[s] .. len_new[s] - 1), workgroups nchunks + 1 .. of row 0 pool
// those blocks into the table, as the pooling kernel does, and a chunk
// holding such a block pools it for itself from the keys with the same
// function instead of using the table's entry (which it may read while it is
// rewritten, and discards): the routes equal those after a separate pooling
// call.
struct RoutePartialExtra {
  const void* k;
  const float* k_scale;
  KeyIndex ki;
  uint32_t* hist0;         // [N, kHistWords] cleared by chunk 0 (NULL: no extra work)
  const int32_t* len_old = nullptr;   // [S] (NULL: no pooling)
  const int32_t* len_new = nullptr;   // [S]
  float* kbar_out = nullptr;          // the table (the kbar the chunks read)
  int npool = 0;                      // pooling workgroups per sequence
  int S = 0;                          // sequences (len_old / len_new entries)
};

// Zeroes row n's level-0 histogram region (the scoring kernel's atomics add
// into it).
__device__ __forceinline__ void clear_hist_row(uint32_t* hist0, int n) {
  uint32_t* h = hist0 + static_cast<size_t>(n) * kHistWords;
  for (int i = threadIdx.x; i < kHistWords; i += 256) h[i] = 0u;
}

template <int KT, int D>
__global__ __launch_bounds__(256) void route_partial_mfma_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ kbar,
    const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int L, int B, int H_I,
    int nchunks, int pstride, float* __restrict__ partial, RoutePartialExtra x) {
  using PM = PieceMap<KT, D>;
  constexpr int KK = D / 32;
  constexpr int STRIDE = D * 2 + 16;                   // padded bf16 row (bytes)
  __shared__ __align__(16) uint8_t hi_t[kRouteBlocks * STRIDE];
  __shared__ __align__(16) uint8_t lo_t[kRouteBlocks * STRIDE];
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

  // key-row sums of the pooling paths (one array for all of them)
  static_assert(PoolMap<KT, D>::RG == PM::RG, "pooling and partial-block maps agree");
  __shared__ float kpart[PM::RG][D + 1];

  const int n = blockIdx.y, chunk = blockIdx.x;
  const int M = (L + B - 1) / B;
  if (chunk > nchunks) {
    // pooling workgroup: block (pb % npool)-th at or after the one holding
    // token len_old[s] of sequence s = pb / npool, if this call completes it
    if (n != 0) return;
    const int pb = chunk - (nchunks + 1);
    const int s = pb / x.npool;
    const int lo = x.len_old[s], hi = x.len_new[s];    // one round trip for both
    const int b = pb % x.npool + lo / B;
    const int t1 = (b + 1) * B;
    if (t1 > hi || t1 <= lo) return;
    const float m = pool_block_mean<KT, D>(static_cast<const uint8_t*>(x.k), x.k_scale, x.ki, s,
                                           b * B, t1, kpart);
    if (threadIdx.x < D) x.kbar_out[(static_cast<size_t>(s) * M + b) * D + threadIdx.x] = m;
    return;
  }
  float* out = partial + (static_cast<size_t>(n) * pstride + chunk) * H_I;
  if (chunk == nchunks) {
    // the partial block's term, exactly as the router's selection step forms it
    __shared__ float mean[D];
    __shared__ float part[4][64];
    QQuarter<DT_BF16, D> qq;
    load_q_quarter<DT_BF16, D>(q, static_cast<size_t>(n) * H_I, H_I, qq);
    const int s = q_seq[n];
    const int Ln = q_pos[n] + 1;
    const int Mf = Ln / B;
    const int cp = Ln - Mf * B;
    if (cp > 0) {
      partial_block_mean<KT, D>(x.k, x.k_scale, x.ki, s, Mf * B, Ln, kpart, mean);
      partial_block_terms<DT_BF16, D>(qq, H_I, mean, part);
    }
    if (x.hist0 && chunk == 0) clear_hist_row(x.hist0, n);
    if (threadIdx.x < H_I)
      out[threadIdx.x] = cp > 0 ? partial_block_term_sum(part, threadIdx.x) : 0.f;
    return;
  }
  // loads in the order of their dependences, none behind a store of this
  // workgroup: the query heads (the row alone), the chunk's table entries
  // (the row's sequence), then the row's length and the sequence's lengths
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  // A operand: head 16 * wave + c, elements 32 kk + 8 g .. + 8
  const int j = wave * 16 + c;
  bf16x8_t a[KK];
  {
    const uint16_t* qr = q + (static_cast<size_t>(n) * H_I + (j < H_I ? j : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4_t x = *reinterpret_cast<const u32x4_t*>(qr + 32 * kk + 8 * g);
      if (j >= H_I) x = u32x4_t{0u, 0u, 0u, 0u};
      a[kk] = __builtin_bit_cast(bf16x8_t, x);
    }
  }
  // the chunk's table entries, every load issued (entries past the table's
  // end read its last one; entries past the row's visible blocks are zeroed
  // below); those of blocks completed by this call ([nlo, nhi)) are replaced
  // below
  // with few sequences each lane reads one sequence's lengths alongside the
  // row's sequence, so the lengths of a block this call completes do not
  // wait for it (one round trip fewer before that block's keys are read)
  int lo_v = 0, hi_v = 0;
  if (x.len_new && x.S <= 64) {
    const int l = lane < x.S ? lane : 0;
    lo_v = x.len_old[l];
    hi_v = x.len_new[l];
  }
  const int s = q_seq[n];
  const int b0 = chunk * kRouteBlocks;
  constexpr int PER = kRouteBlocks * D / 4 / 256;      // table float4s per thread
  const float* tab = kbar + static_cast<size_t>(s) * M * D;
  float4 kx[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int f = tid + 256 * i;
    const int blk = f / (D / 4), col = (f % (D / 4)) * 4;
    const int e = min(b0 + blk, M - 1);
    kx[i] = *reinterpret_cast<const float4*>(tab + static_cast<size_t>(e) * D + col);
  }
  const int Mf = (q_pos[n] + 1) / B;                   // blocks fully visible to row n
  const int nb = min(kRouteBlocks, Mf - b0);
  int len_old = 0, len_new = 0;
  if (x.len_new) {
    if (x.S <= 64) {
      len_old = __builtin_amdgcn_readlane(lo_v, s);
      len_new = __builtin_amdgcn_readlane(hi_v, s);
    } else {
      len_old = x.len_old[s];
      len_new = x.len_new[s];
    }
  }
  if (x.hist0 && chunk == 0) clear_hist_row(x.hist0, n);
  if (nb <= 0) {
    for (int jj = threadIdx.x; jj < H_I; jj += 256) out[jj] = 0.f;
    return;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int blk = (tid + 256 * i) / (D / 4);
    if (blk >= nb) kx[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // blocks [nlo, nhi) of this chunk are completed by this call: pooled here
  // (the loads of the query and of the table go out first, so their round
  // trips overlap the key reads)
  int nlo = 0, nhi = 0;
  if (x.len_new) {
    nlo = max(b0, len_old / B);
    nhi = min(b0 + nb, len_new / B);
  }
  __shared__ __align__(16) float fresh[kRouteBlocks][D];
  for (int b = nlo; b < nhi; ++b) {
    const float m = pool_block_mean<KT, D>(static_cast<const uint8_t*>(x.k), x.k_scale, x.ki,
                                           s, b * B, (b + 1) * B, kpart);
    if (tid < D) fresh[b - b0][tid] = m;
    __syncthreads();
  }
  // the chunk's pooled keys, split into hi / lo bf16 rows
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int f = tid + 256 * i;
    const int blk = f / (D / 4), col = (f % (D / 4)) * 4;
    const float4 xv = (b0 + blk >= nlo && b0 + blk < nhi)
                          ? *reinterpret_cast<const float4*>(&fresh[blk][col])
                          : kx[i];
    const float xs[4] = {xv.x, xv.y, xv.z, xv.w};
    uint32_t hb[4], lb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t u = __float_as_uint(xs[e]);
      hb[e] = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
      const uint32_t ul = __float_as_uint(xs[e] - __uint_as_float(hb[e] << 16));
      lb[e] = (ul + 0x7FFFu + ((ul >> 16) & 1u)) >> 16;
    }
    *reinterpret_cast<uint2*>(hi_t + blk * STRIDE + col * 2) =
        make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
    *reinterpret_cast<uint2*>(lo_t + blk * STRIDE + col * 2) =
        make_uint2(lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16));
  }
  __syncthreads();
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const int off = c * STRIDE + 64 * kk + 16 * g;
    const bf16x8_t bh = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(hi_t + off));
    const bf16x8_t bl = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(lo_t + off));
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[kk], bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[kk], bl, acc, 0, 0, 0);
  }
  // ReLU over the visible blocks, then the sum over the 16 block columns
  const bool vis = c < nb;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v = vis ? relu(acc[i]) : 0.f;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, 64);
    const int jj = wave * 16 + 4 * g + i;
    if (c == 0 && jj < H_I) out[jj] = v;
  }
}

// Many query rows over one key sequence (prefill): the router dots are a
// GEMM, [rows x H_I, d] x [d, M], run on v_mfma_f32_16x16x32_bf16.  q is
// exact in bf16; each pooled key is split as kbar = hi + lo with hi, lo
// bf16 (round to nearest), so q.kbar = q.hi + q.lo with both products exact
// and fp32 accumulation (relative error ~2^-17 of |q||kbar|).  One
// workgroup owns 256 / HPI query rows (HPI = H_I padded to 16, 32 or 64
// rows, 64 head rows per wavefront) and streams the pooled blocks visible to
// them in tiles of 64 through LDS; each lane sums ReLU(dot) over the blocks
// of its output column, masked per row to the row's fully visible blocks,
// and the 16 columns are reduced across lanes at the end.  The partial
// visible block is added by route_select.
constexpr int kRouteTile = 64;       // pooled blocks per LDS tile

// The pooled table of one sequence as bf16 hi / lo halves: kbar = hi + lo,
// hi = RNE(kbar), lo = RNE(kbar - hi).
__global__ __launch_bounds__(256) void route_split_kernel(const float* __restrict__ kbar,
                                                          size_t n4, uint16_t* __restrict__ hi,
                                                          uint16_t* __restrict__ lo) {
  for (size_t f = blockIdx.x * static_cast<size_t>(256) + threadIdx.x; f < n4;
       f += static_cast<size_t>(gridDim.x) * 256) {
    const float4 x = reinterpret_cast<const float4*>(kbar)[f];
    const float xs[4] = {x.x, x.y, x.z, x.w};
    uint32_t hb[4], lb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t u = __float_as_uint(xs[e]);
      hb[e] = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
      const uint32_t ul = __float_as_uint(xs[e] - __uint_as_float(hb[e] << 16));
      lb[e] = (ul + 0x7FFFu + ((ul >> 16) & 1u)) >> 16;
    }
    reinterpret_cast<uint2*>(hi)[f] = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
    reinterpret_cast<uint2*>(lo)[f] = make_uint2(lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16));
  }
}

template <int HPI, bool QF8>
__global__ __launch_bounds__(256, 4) void route_mfma_kernel(const void* __restrict__ q,
                                                         const uint16_t* __restrict__ kb_hi,
                                                         const uint16_t* __restrict__ kb_lo,
                                                         const int32_t* __restrict__ q_pos,
                                                         int N, int L, int B, int H_I,
                                                         float* __restrict__ partial) {
  constexpr int D = 128;
  constexpr int KK = D / 32;
  constexpr int STRIDE = D * 2 + 16;                   // padded bf16 row in LDS (bytes)
  constexpr int QB = 256 / HPI;                        // query rows per workgroup
  __shared__ __align__(16) uint8_t hi_t[kRouteTile * STRIDE];
  __shared__ __align__(16) uint8_t lo_t[kRouteTile * STRIDE];
  __shared__ int mf_lds[QB];
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int q0 = blockIdx.x * QB;
  const int M = (L + B - 1) / B;
  for (int i = tid; i < QB; i += 256) mf_lds[i] = q0 + i < N ? (q_pos[q0 + i] + 1) / B : 0;
  __syncthreads();
  int mmax = 0;
  for (int i = 0; i < QB; ++i) mmax = max(mmax, mf_lds[i]);

  // A operand: 4 row tiles of head rows; row r of the workgroup is head r % HPI
  // of query row r / HPI
  bf16x8_t a[4][KK];
  int mf_row[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int r = wave * 64 + rt * 16 + c;
    const int t = q0 + r / HPI, j = r % HPI;
    const bool rv = t < N && j < H_I;
    const size_t qrow = static_cast<size_t>(rv ? t : 0) * H_I + (rv ? j : 0);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4_t x;
      if constexpr (QF8) {
        // 8 e4m3 codes widened to bf16 (exact); the head scale is folded
        // into the router weight
        const uint2 c8 = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(q) +
                                                         qrow * D + 32 * kk + 8 * g);
        uint32_t b0, b1, b2, b3;
        e4m3x4_to_bf16x4(c8.x, b0, b1);
        e4m3x4_to_bf16x4(c8.y, b2, b3);
        x = u32x4_t{b0, b1, b2, b3};
      } else {
        x = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(q) + qrow * D +
                                              32 * kk + 8 * g);
      }
      if (!rv) x = u32x4_t{0u, 0u, 0u, 0u};
      a[rt][kk] = __builtin_bit_cast(bf16x8_t, x);
    }
    // rows 4g..4g+3 of the tile all belong to one query row (HPI >= 16)
    mf_row[rt] = mf_lds[(wave * 64 + rt * 16) / HPI];
  }
  float acc_rows[4][4] = {};

  for (int b0 = 0; b0 < mmax; b0 += kRouteTile) {
    __syncthreads();
    // the tile's pooled keys (bf16 hi / lo rows) into LDS
    constexpr int PIECES = kRouteTile * D * 2 / 16;     // 16-byte pieces per half
#pragma unroll
    for (int i = 0; i < PIECES / 256; ++i) {
      const int f = tid + 256 * i;
      const int blk = f / (D / 8), col = (f % (D / 8)) * 8;
      const size_t src = static_cast<size_t>(b0 + blk < M ? b0 + blk : 0) * D + col;
      const u32x4_t h = *reinterpret_cast<const u32x4_t*>(kb_hi + src);
      const u32x4_t l = *reinterpret_cast<const u32x4_t*>(kb_lo + src);
      *reinterpret_cast<u32x4_t*>(hi_t + blk * STRIDE + col * 2) = h;
      *reinterpret_cast<u32x4_t*>(lo_t + blk * STRIDE + col * 2) = l;
    }
  __syncthreads();
#pragma unroll
    for (int ct = 0; ct < kRouteTile / 16; ++ct) {
      const int blk = b0 + ct * 16 + c;                // this lane's output column
      // one K step of B (hi and lo) at a time against all 4 row tiles keeps
      // the live B fragments to two (the register budget allows 4 waves/SIMD)
      f32x4_t acc[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int off = (ct * 16 + c) * STRIDE + 64 * kk + 16 * g;
        const bf16x8_t bh =
            __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(hi_t + off));
        const bf16x8_t bl =
            __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(lo_t + off));
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rt][kk], bh, acc[rt], 0, 0, 0);
          acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rt][kk], bl, acc[rt], 0, 0, 0);
        }
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const bool vis = blk < mf_row[rt];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc_rows[rt][i] += vis ? relu(acc[rt][i]) : 0.f;
      }
    }
  }
  // sum the 16 output columns held by lanes c = 0..15 of each lane group
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = acc_rows[rt][i];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, 64);
      const int r = wave * 64 + rt * 16 + 4 * g + i;
      const int t = q0 + r / HPI, j = r % HPI;
      if (c == 0 && t < N && j < H_I) partial[static_cast<size_t>(t) * H_I + j] = v;
    }
  }
}

// NP: the chunk partials each thread loads up front (1 when the partials
// come from the MFMA router, which leaves one chunk per row).
template <int QT, int KT, int D, int NP>
__global__ __launch_bounds__(256) void route_select_kernel(
    const void* __restrict__ q, const float* __restrict__ w, const void* __restrict__ k,
    const float* __restrict__ k_scale, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int L, int B, int H_I, int h, int nchunks,
    const float* __restrict__ partial, int32_t* __restrict__ heads,
    float* __restrict__ head_score, KeyIndex ki, const float* __restrict__ q_scale) {
  using PM = PieceMap<KT, D>;
  __shared__ float psum[PM::RG][D + 1];
  __shared__ float mean[D];
  __shared__ float red[4][64];
  __shared__ float part[4][64];

  const int n = blockIdx.x;
  const int Ln = q_pos[n] + 1;
  const int Mf = Ln / B;
  const int cp = Ln - Mf * B;                 // visible keys of the partial block
  const int s = q_seq[n];

  // the loads that need nothing else (partials, this thread's quarter of a
  // query head, the head's weight) go out together, ahead of the key reads
  const float* prow = partial + static_cast<size_t>(n) * nchunks * H_I;
  float pv[NP];
  load_chunk_partials<NP>(prow, nchunks, H_I, pv);
  QQuarter<QT, D> qq;
  load_q_quarter<QT, D>(q, static_cast<size_t>(n) * H_I, H_I, qq);
  const int jc = (threadIdx.x & 63) < H_I ? (threadIdx.x & 63) : H_I - 1;
  float wj = w[static_cast<size_t>(n) * H_I + jc];
  if (QT == DT_E4M3) wj *= q_scale[static_cast<size_t>(n) * H_I + jc];
  finish_chunk_partials<NP>(prow, nchunks, H_I, pv, red);
  if (cp > 0) {
    partial_block_mean<KT, D>(k, k_scale, ki, s, Mf * B, Ln, psum, mean);
    partial_block_terms<QT, D>(qq, H_I, mean, part);
  } else {
    __syncthreads();
  }
  if (threadIdx.x < 64) {
    const int j = threadIdx.x;
    float r = -1.f;
    if (j < H_I) {
      float a = combine_partials(red, j);
      if (cp > 0) a += partial_block_term_sum(part, j);
      r = fabsf(wj) * a;
      if (head_score) head_score[static_cast<size_t>(n) * H_I + j] = r;
    }
    rank_heads(r, H_I, h, heads + static_cast<size_t>(n) * h);
  }
}

template <int QT, int KT, int D>
hipError_t launch_route_t(const RouteArgs& a, hipStream_t st) {
  int nchunks = a.nchunks;
  if (a.partials_only && route_uses_mfma(a)) return hipErrorInvalidValue;
  if (route_uses_mfma(a)) {
    nchunks = 1;
    const int M = (a.L + a.B - 1) / a.B;
    const size_t n4 = static_cast<size_t>(M) * 128 / 4;
    uint16_t* hi = a.kb_split;
    uint16_t* lo = a.kb_split + static_cast<size_t>(M) * 128;
    const size_t nblk = (n4 + 255) / 256;
    const unsigned sb = static_cast<unsigned>(nblk < 1024 ? nblk : 1024);
    MISA_LAUNCH(K_ROUTE_SPLIT, route_split_kernel, dim3(sb), dim3(256), 0, st, a.kbar, n4, hi,
                lo);
    const int hpi = a.H_I <= 16 ? 16 : (a.H_I <= 32 ? 32 : 64);
    const dim3 grid((a.N + 256 / hpi - 1) / (256 / hpi));
    constexpr bool QF8 = QT == DT_E4M3;
    if (hpi == 16)
      MISA_LAUNCH(K_ROUTE_PARTIAL, (route_mfma_kernel<16, QF8>), grid, dim3(256), 0, st, a.q,
                  hi, lo, a.q_pos, a.N, a.L, a.B, a.H_I, a.partial);
    else if (hpi == 32)
      MISA_LAUNCH(K_ROUTE_PARTIAL, (route_mfma_kernel<32, QF8>), grid, dim3(256), 0, st, a.q,
                  hi, lo, a.q_pos, a.N, a.L, a.B, a.H_I, a.partial);
    else
      MISA_LAUNCH(K_ROUTE_PARTIAL, (route_mfma_kernel<64, QF8>), grid, dim3(256), 0, st, a.q,
                  hi, lo, a.q_pos, a.N, a.L, a.B, a.H_I, a.partial);
  } else if constexpr (QT == DT_E4M3) {
    return hipErrorInvalidValue;   // e4m3 queries reach the router only on the GEMM path
  } else {
    if constexpr (QT == DT_BF16) {
      // the routed decode step: partials plus the partial-block slot, heads
      // picked by the scoring kernel
      const bool fused = a.partials_only;
      RoutePartialExtra x{a.k, a.k_scale, a.kidx, a.hist0};
      int gx = a.nchunks + (fused ? 1 : 0);
      if (fused && a.len_new && a.max_new > 0) {
        x.len_old = a.len_old;
        x.len_new = a.len_new;
        x.kbar_out = a.kbar_out;
        x.npool = a.max_new / a.B + 1;     // blocks max_new tokens can complete
        x.S = a.S;
        gx += x.npool * a.S;
      }
      MISA_LAUNCH(K_ROUTE_PARTIAL, (route_partial_mfma_kernel<KT, D>), dim3(gx, a.N), dim3(256),
                  0, st,
                  static_cast<const uint16_t*>(a.q), a.kbar, a.q_seq, a.q_pos, a.L, a.B, a.H_I,
                  a.nchunks, a.nchunks + (fused ? 1 : 0), a.partial, x);
      if (fused) return hipGetLastError();
    } else if (a.partials_only) {
      return hipErrorInvalidValue;     // the fused decode step takes bf16 queries only
    } else
      MISA_LAUNCH(K_ROUTE_PARTIAL, (route_partial_kernel<QT, D>), dim3(a.nchunks, a.N),
                  dim3(256), 0, st, a.q, a.kbar, a.q_seq, a.q_pos, a.L, a.B, a.H_I, a.nchunks,
                  a.partial);
  }
  if constexpr (D == 128 && QT != DT_F32) {
    if (nchunks == 1) {
      MISA_LAUNCH(K_ROUTE_SELECT, (route_select_kernel<QT, KT, D, 1>), dim3(a.N), dim3(256), 0,
                  st, a.q, a.w, a.k, a.k_scale, a.q_seq, a.q_pos, a.L, a.B, a.H_I, a.h, nchunks,
                  a.partial, a.heads, a.head_score, a.kidx, a.q_scale);
      return hipGetLastError();
    }
  }
  MISA_LAUNCH(K_ROUTE_SELECT, (route_select_kernel<QT, KT, D, 16>), dim3(a.N), dim3(256), 0, st,
              a.q, a.w, a.k, a.k_scale, a.q_seq, a.q_pos, a.L, a.B, a.H_I, a.h, nchunks,
              a.partial, a.heads, a.head_score, a.kidx, a.q_scale);
  return hipGetLastError();
}

template <int D>
hipError_t launch_route_d(const RouteArgs& a, hipStream_t st) {
  if (a.q_dt == DT_F32) return launch_route_t<DT_F32, DT_F32, D>(a, st);
  if (a.q_dt == DT_E4M3) {
    if constexpr (D == 128) return launch_route_t<DT_E4M3, DT_E4M3, D>(a, st);
    return hipErrorInvalidValue;
  }
  if (a.k_dt == DT_BF16) return launch_route_t<DT_BF16, DT_BF16, D>(a, st);
  return launch_route_t<DT_BF16, DT_E4M3, D>(a, st);
}

}  // namespace

int route_blocks_per_chunk() { return kRouteBlocks; }

bool route_uses_mfma(const RouteArgs& a) {
  return a.S == 1 && a.N >= 128 && (a.q_dt == DT_BF16 || a.q_dt == DT_E4M3) && a.d == 128;
}

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
  return a.d == 64 ? launch_route_d<64>(a, st) : launch_route_d<128>(a, st);
}

}  // namespace misa
