// Token scoring for the MISA indexer (routed or all-head), gfx950.
//
//   I_n(s) = sum over the row's heads j of w[n,j] * ReLU(q[n,j,:] . key_s)
// (DSA token-wise indexer score; MISA scores only the h routed heads, MISA
// technical summary, gist.science, "Methodology" item 2.)
//
// score_mfma_kernel (bf16 or fp8 keys): one query row against a stream of
// keys.  The row's heads form the A operand of v_mfma_f32_16x16x32_bf16
// (16 head rows per tile, zero-padded), 16 keys form the B operand, so one
// MFMA per 32 elements of d yields 16 heads x 16 keys of dot products in fp32
// from exact bf16 products.  Keys are read with flat 16-byte loads (a load
// instruction covers whole key rows) into two register buffers that
// ping-pong, so the next group of tiles is in flight while the current one is
// scored; each tile passes through a small padded wavefront-private LDS tile
// that turns rows into the MFMA operand layout without bank conflicts.
// fp8 keys are widened to bf16 in registers (exact) and their per-token
// scale is applied to the fp32 dot before the ReLU.  The epilogue applies
// ReLU, multiplies by the head weight and sums the heads (4 rows per lane, 2
// cross-lane adds), then writes a 32-bit order key per token and counts it in
// an LDS histogram of the top 12 key bits (flushed with integer atomics, so
// results do not depend on scheduling).
//
// score_f32_kernel (fp32 keys): one thread per key, plain FMAs (fp32 inputs
// have no exact low-precision MFMA form).
//
// Keys may live in a paged cache (KeyIndex): a tile's 16 consecutive tokens
// always share a page (pages hold a multiple of 16 tokens).  The streaming
// kernel reads the page numbers of all of a wavefront's tiles with one vector
// load at the start (lane j: the j-th tile) and takes each tile's page from
// that register with readlane, so the loop itself does no lookups; candidate
// gathers look each token's page up per lane.
#include "common.hpp"
#include "kernels.hpp"
#include "route_select.hpp"

namespace misa {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMaxTpw = 16;    // tiles per wavefront at most (LDS key slots)

struct ScoreParams {
  const uint16_t* q;
  const float* w;
  const uint8_t* k;
  const float* k_scale;
  const int32_t* q_seq;
  const int32_t* q_pos;
  const int32_t* heads;
  const int32_t* cand;
  int L, H_I, nrows, ncols;
  uint32_t* u;
  int u_stride;
  uint32_t* hist0;
  int tiles_per_wave;
  KeyIndex ki;
  const float* route_partial;   // routed decode step: router partials (see ScoreArgs)
  int route_nchunks, B;
  int32_t* heads_out;
  float* head_score_out;
};

template <int KT, int D>
struct KeyLayout {
  static constexpr int EB = KT == DT_E4M3 ? 1 : 2;     // bytes per element
  static constexpr int ROW = D * EB;                   // bytes per key row
  static constexpr int NLOAD = ROW / 64;               // 16-byte pieces per lane per tile
  static constexpr int KK = D / 32;                    // MFMAs per head tile
  static constexpr int LANES_PER_ROW = ROW / 16;       // flat load: lanes covering one row
  static constexpr int ROWS_PER_LOAD = 64 / LANES_PER_ROW;
  static constexpr int LDS_STRIDE = ROW + 16;          // padded row stride of the LDS tile
  static constexpr int TILE_LDS = 16 * LDS_STRIDE;
};

// Adds a 256-thread workgroup's LDS level-0 histogram to the row's global
// one.  Each thread's 16 bin counts are read together, then added (a loop that
// waited for each count before its atomic took 16 LDS round trips at the end of
// every workgroup); the caller has synchronised the workgroup.
__device__ __forceinline__ void flush_hist(const uint32_t* lh, uint32_t* hg) {
  constexpr int kPerT = kBins0 / 256;
  uint32_t cnt[kPerT];
#pragma unroll
  for (int i = 0; i < kPerT; ++i) cnt[i] = lh[threadIdx.x + 256 * i];
#pragma unroll
  for (int i = 0; i < kPerT; ++i)
    if (cnt[i]) atomicAdd(&hg[threadIdx.x + 256 * i], cnt[i]);
}

// d-elements that lane group g (= lane / 16) feeds to MFMA kk, as the first
// of 8 consecutive elements.  Load p of a lane reads bytes [64p + 16g, +16)
// of its key row, so one load instruction covers 64 contiguous bytes of each
// of 16 rows; the query fragments use the same assignment (the contraction
// order over d is free).
template <int KT>
__device__ __forceinline__ constexpr int elem_off(int g, int kk) {
  return KT == DT_E4M3 ? 64 * (kk >> 1) + 16 * g + 8 * (kk & 1) : 32 * kk + 8 * g;
}

template <int KT, int D>
__device__ __forceinline__ void to_fragments(const u32x4_t (&raw)[KeyLayout<KT, D>::NLOAD],
                                             bf16x8_t (&b)[KeyLayout<KT, D>::KK]) {
  constexpr int KK = KeyLayout<KT, D>::KK;
  if constexpr (KT == DT_BF16) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) b[kk] = __builtin_bit_cast(bf16x8_t, raw[kk]);
  } else {
    // load p holds 16 codes: the first 8 feed MFMA 2p, the last 8 MFMA 2p+1
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const u32x4_t& r = raw[kk >> 1];
      const uint32_t w0 = (kk & 1) ? r.z : r.x;
      const uint32_t w1 = (kk & 1) ? r.w : r.y;
      u32x4_t o;
      uint32_t a0, a1, a2, a3;
      e4m3x4_to_bf16x4(w0, a0, a1);
      e4m3x4_to_bf16x4(w1, a2, a3);
      o.x = a0;
      o.y = a1;
      o.z = a2;
      o.w = a3;
      b[kk] = __builtin_bit_cast(bf16x8_t, o);
    }
  }
}

// Issues the key loads of U tiles (16 elements each) starting at element e0;
// bit t of the returned mask is set when tile t's element is a valid token.
template <int KT, int D, int U>
using RawGroup = u32x4_t[U][KeyLayout<KT, D>::NLOAD];

// Issues the key loads of U tiles (16 elements each) starting at element e0.
// Without a candidate list the key address depends only on the element index
// (and, for paged keys, on the page number held in lane ord0 + t of page_v),
// so no load waits on another load; bit t of the result is set when tile t's
// element is a valid token.  Elements past the row end read a valid row of
// the sequence and are masked.
template <int KT, int D, int U, bool CAND>
__device__ __forceinline__ uint32_t issue_group(RawGroup<KT, D, U>& raw, float* sc, int tile0,
                                                int tstride, int lane, int c, int len,
                                                const int32_t* crow, const uint8_t* kbase,
                                                const float* sbase, const KeyIndex& ki, int s,
                                                int ord0, int page_v) {
  using LY = KeyLayout<KT, D>;
  const int rsub = lane / LY::LANES_PER_ROW, q = lane % LY::LANES_PER_ROW;
  uint32_t valid = 0;
  if constexpr (CAND) {
    // candidate lists: lane c of each group of 16 reads element c of each
    // tile (unconditionally, clamped to the list; masked below) and, for
    // paged keys, that token's page; a lane loading a key row takes the row's
    // token and page from the lane of that element by a cross-lane read, so
    // a group costs two round trips (three paged) however many rows it holds
    int tokc[U], pgc[U];
#pragma unroll
    for (int t = 0; t < U; ++t) {
      const int e = (tile0 + t * tstride) * 16 + c;
      tokc[t] = crow[e < len ? e : len - 1];
      pgc[t] = 0;
    }
    if (ki.table) {
#pragma unroll
      for (int t = 0; t < U; ++t) pgc[t] = ki.page(s, tokc[t] >= 0 ? tokc[t] : 0);
    }
#pragma unroll
    for (int t = 0; t < U; ++t) {
#pragma unroll
      for (int i = 0; i < LY::NLOAD; ++i) {
        // load i of lane l reads 16 bytes of the tile's row i*ROWS_PER_LOAD + l/LANES_PER_ROW
        const int src = i * LY::ROWS_PER_LOAD + rsub;
        const int tk = __shfl(tokc[t], src, 64);
        const int tok = tk >= 0 ? tk : 0;
        const size_t row = ki.table ? ki.row_in_page(__shfl(pgc[t], src, 64), tok)
                                    : static_cast<size_t>(s) * ki.L + tok;
        raw[t][i] = *reinterpret_cast<const u32x4_t*>(kbase + row * LY::ROW + 16 * q);
      }
      const int e = (tile0 + t * tstride) * 16 + c;
      valid |= e < len && tokc[t] >= 0 ? (1u << t) : 0u;
      if constexpr (KT == DT_E4M3) {
        const int tok = tokc[t] >= 0 ? tokc[t] : 0;
        sc[t] = sbase[ki.table ? ki.row_in_page(pgc[t], tok)
                               : static_cast<size_t>(s) * ki.L + tok];
      } else {
        sc[t] = 1.f;
      }
    }
    return valid;
  }
#pragma unroll
  for (int t = 0; t < U; ++t) {
    const int te = (tile0 + t * tstride) * 16;
    size_t rb;                                         // row of the tile's first token
    const int tc = te < len ? te : len - 1;
    if (ki.table) {
      const int pg = __builtin_amdgcn_readlane(page_v, ord0 + t);
      rb = (static_cast<size_t>(pg) << ki.page_shift) + (tc & ((1 << ki.page_shift) - 1));
    } else {
      rb = static_cast<size_t>(s) * ki.L + tc;
    }
    // flat: load i of lane l reads 16 bytes of row i*ROWS_PER_LOAD + l/LANES_PER_ROW
#pragma unroll
    for (int i = 0; i < LY::NLOAD; ++i) {
      const int e = te + i * LY::ROWS_PER_LOAD + rsub;
      const size_t row = e < len ? rb + (e - te) : rb;
      raw[t][i] = *reinterpret_cast<const u32x4_t*>(kbase + row * LY::ROW + 16 * q);
    }
    const int e = te + c;
    valid |= e < len ? (1u << t) : 0u;
    if constexpr (KT == DT_E4M3)
      sc[t] = sbase[e < len ? rb + c : rb];
    else
      sc[t] = 1.f;
  }
  return valid;
}

template <int KT, int NT, int D, int U>
__device__ __forceinline__ void score_group(const RawGroup<KT, D, U>& raw, const float* sc,
                                            uint32_t valid, int tile0, int tstride, uint8_t* tile,
                                            int lane,
                                            const bf16x8_t (&a)[NT][KeyLayout<KT, D>::KK],
                                            const float (&wv)[NT][4], int g, int c, int len,
                                            uint32_t* ukw, int ord0, uint32_t* lh,
                                            bool do_hist) {
  using LY = KeyLayout<KT, D>;
  constexpr int KK = LY::KK;
  const int rsub = lane / LY::LANES_PER_ROW, q = lane % LY::LANES_PER_ROW;
#pragma unroll
  for (int t = 0; t < U; ++t) {
    // rows in through the wavefront's padded LDS tile, operand pieces out
    // (LDS operations of one wavefront execute in order)
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < LY::NLOAD; ++i)
      *reinterpret_cast<u32x4_t*>(tile + (i * LY::ROWS_PER_LOAD + rsub) * LY::LDS_STRIDE +
                                  16 * q) = raw[t][i];
    __builtin_amdgcn_wave_barrier();
    u32x4_t pieces[LY::NLOAD];
#pragma unroll
    for (int p = 0; p < LY::NLOAD; ++p)
      pieces[p] = *reinterpret_cast<const u32x4_t*>(tile + c * LY::LDS_STRIDE + 64 * p + 16 * g);
    bf16x8_t b[KK];
    to_fragments<KT, D>(pieces, b);
    float part = 0.f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[nt][kk], b[kk], acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = acc[i];
        if (KT == DT_E4M3) v *= sc[t];
        part += wv[nt][i] * fmaxf(v, 0.f);
      }
    }
    // the four lane groups' partial head sums: lanes 16 apart, then 32 apart
    // (gfx950 lane swaps; a + b is the same in either lane of a pair)
    {
      const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(part),
                                                        __float_as_uint(part), false, false);
      part = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
      const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part),
                                                        __float_as_uint(part), false, false);
      part = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
    }
    // the order key goes to the wavefront's LDS key slots (written to u in
    // one burst after the loop: a global store here would sit in the same
    // in-order memory counter as the key loads in flight)
    const int e = (tile0 + t * tstride) * 16 + c;
    if (g == 0) {
      const bool ok = ((valid >> t) & 1u) && e < len;
      const uint32_t key = ok ? order_key(part) : 0u;
      ukw[(ord0 + t) * 16 + c] = key;
      if (do_hist && ok) atomicAdd(&lh[key >> kShift0], 1u);
    }
  }
}

template <int KT, int NT, int D, int U, bool CAND, bool ROUTE>
__global__ __launch_bounds__(256) void score_mfma_kernel(ScoreParams p) {
  using LY = KeyLayout<KT, D>;
  constexpr int KK = LY::KK;
  __shared__ uint32_t lh[kBins0];
  __shared__ __align__(16) uint8_t tiles[4][LY::TILE_LDS];
  // each wavefront's order keys in tile order (at most kMaxTpw tiles of 16)
  __shared__ __align__(16) uint32_t ukeys[4][kMaxTpw * 16];
  __shared__ int32_t heads_lds[ROUTE ? 64 : 1];
  __shared__ __align__(16) uint16_t qlds[ROUTE ? 64 * D : 8];   // the row's query heads
  __shared__ float wlds[ROUTE ? 64 : 1];                          // and their weights
  __shared__ float red_lds[ROUTE ? 4 : 1][64];                    // router partial sums

  const int n = blockIdx.y;
  // the row's length and its sequence travel together (one scalar round trip)
  // the row's length and sequence, and the arguments the first loads
  // address with, are all read before the exit test (two scalar round trips
  // in all: the arguments, then the row's two words)
  const int qp = CAND ? 0 : p.q_pos[n];
  const int s = p.q_seq[n];
  asm volatile("" ::"s"(qp), "s"(s), "s"(p.q), "s"(p.k), "s"(p.ki.table), "s"(p.ki.L),
               "s"(p.H_I), "s"(p.route_partial), "s"(p.route_nchunks), "s"(gridDim.x));
  const int len = CAND ? p.ncols : qp + 1;
  // tiles of 16 elements are dealt round-robin to the row's wavefronts, so at
  // any moment the whole grid streams one compact stretch of the keys
  const int ntiles = (len + 15) / 16;
  const int tstride = gridDim.x * 4;                 // wavefronts per row
  if (static_cast<int>(blockIdx.x) * 4 >= ntiles) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int g = lane >> 4, c = lane & 15;
  const bool do_hist = p.hist0 != nullptr;

  const uint8_t* kseq = p.k;                           // rows addressed through p.ki
  uint8_t* tile = tiles[wave];
  const float* sseq = p.k_scale;
  const int32_t* crow = CAND ? p.cand + static_cast<size_t>(n) * p.ncols : nullptr;
  uint32_t* urow = p.u + static_cast<size_t>(n) * p.u_stride;
  uint32_t* ukw = ukeys[threadIdx.x >> 6];
  const int wtile = blockIdx.x * 4 + wave;            // this wavefront's first tile
  const int wtiles = wtile < ntiles ? (ntiles - wtile + tstride - 1) / tstride : 0;
  // paged keys: lane j holds the page of this wavefront's j-th tile (at most
  // 64 tiles per wavefront; tiles past the row end use the row's last token)
  int page_v = 0;
  if constexpr (!CAND) {
    if (p.ki.table) {
      const int te = (wtile + lane * tstride) * 16;
      const int tc = te < len ? te : len - 1;
      page_v = p.ki.table[static_cast<size_t>(s) * p.ki.max_pages + (tc >> p.ki.page_shift)];
    }
  }

  // routed step: the selection's inputs are loaded first (the row's query
  // heads, their weights, the router partials), so that waiting for them
  // leaves the first key group, issued right behind, in flight
  constexpr int QV = ROUTE ? 64 * D / 8 / 256 : 1;     // 16-byte query pieces per thread
  u32x4_t qv[QV];
  float pv[ROUTE ? 16 : 1];
  float wj = 0.f, tail = 0.f;
  const size_t prow = static_cast<size_t>(n) * (p.route_nchunks + 1) * p.H_I;
  const bool partial_block = ROUTE && len % p.B != 0;
  if constexpr (ROUTE) {
    // (unconditional loads, clamped to valid elements: an exact wait count)
    const int nqv = p.H_I * D / 8;
    const u32x4_t* qsrc =
        reinterpret_cast<const u32x4_t*>(p.q + static_cast<size_t>(n) * p.H_I * D);
#pragma unroll
    for (int i = 0; i < QV; ++i) {
      const int f = threadIdx.x + 256 * i;
      qv[i] = qsrc[f < nqv ? f : nqv - 1];
    }
    const int jc = static_cast<int>(threadIdx.x & 63) < p.H_I ? (threadIdx.x & 63) : p.H_I - 1;
    wj = p.w[static_cast<size_t>(n) * p.H_I + jc];
    tail = p.route_partial[prow + static_cast<size_t>(p.route_nchunks) * p.H_I + jc];
    load_chunk_partials(p.route_partial + prow, p.route_nchunks, p.H_I, pv);
  }

  // the first two key groups in flight before anything else (unconditional:
  // a wavefront without tiles reads valid rows and scores nothing)
  const int gstep = U * tstride;                       // tiles between consecutive groups
  u32x4_t ra[U][LY::NLOAD], rb[U][LY::NLOAD], rc[U][LY::NLOAD];
  float sa[U], sb[U], sc[U];
  uint32_t va = 0, vb = 0, vc = 0;
  va = issue_group<KT, D, U, CAND>(ra, sa, wtile, tstride, lane, c, len, crow, kseq, sseq,
                                   p.ki, s, 0, page_v);
  // (a candidate-list wavefront has its tiles in one group as a rule: its
  // second group, whose index reads would wait behind the first's keys, is
  // read only when it is scored)
  if (!CAND || wtiles > U)
    vb = issue_group<KT, D, U, CAND>(rb, sb, wtile + gstep, tstride, lane, c, len, crow, kseq,
                                     sseq, p.ki, s, U, page_v);

  if (do_hist) {
    for (int b = threadIdx.x; b < kBins0; b += 256) lh[b] = 0u;
  }
  if constexpr (ROUTE) {
    // the router's selection step for this row, as the selection kernel
    // forms it (same partial order, same ranking), while the first keys load
    finish_chunk_partials(p.route_partial + prow, p.route_nchunks, p.H_I, pv, red_lds);
    const int nqv = p.H_I * D / 8;
#pragma unroll
    for (int i = 0; i < QV; ++i) {
      const int f = threadIdx.x + 256 * i;
      if (f < nqv) reinterpret_cast<u32x4_t*>(qlds)[f] = qv[i];
    }
    if (threadIdx.x < 64) wlds[threadIdx.x] = static_cast<int>(threadIdx.x) < p.H_I ? wj : 0.f;
    __syncthreads();
    if (threadIdx.x < 64) {
      const int j = threadIdx.x;
      float r = -1.f;
      if (j < p.H_I) {
        float a = combine_partials(red_lds, j);
        if (partial_block) a += tail;
        r = fabsf(wj) * a;
        if (blockIdx.x == 0 && p.head_score_out)
          p.head_score_out[static_cast<size_t>(n) * p.H_I + j] = r;
      }
      rank_heads(r, p.H_I, p.nrows, heads_lds);
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      if (blockIdx.x == 0 && j < p.nrows)
        p.heads_out[static_cast<size_t>(n) * p.nrows + j] = heads_lds[j];
    }
    __syncthreads();
  }
  // A operand: head rows of this query row; W: weights of this lane's D rows.
  // (every read unconditional: rows past nrows read row nrows - 1 and are
  // zeroed; the head indices first, so the setup is two round trips)
  bf16x8_t a[NT][KK];
  float wv[NT][4];
  int ja[NT], jw[NT][4];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = nt * 16 + c;
    const int rc = r < p.nrows ? r : p.nrows - 1;
    ja[nt] = ROUTE ? heads_lds[rc] : p.heads ? p.heads[static_cast<size_t>(n) * p.nrows + rc] : rc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = nt * 16 + 4 * g + i;
      const int rrc = rr < p.nrows ? rr : p.nrows - 1;
      jw[nt][i] = ROUTE ? heads_lds[rrc]
                        : p.heads ? p.heads[static_cast<size_t>(n) * p.nrows + rrc] : rrc;
    }
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const bool rv = nt * 16 + c < p.nrows;
    const uint16_t* qrow =
        ROUTE ? qlds + ja[nt] * D : p.q + (static_cast<size_t>(n) * p.H_I + ja[nt]) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4_t x = *reinterpret_cast<const u32x4_t*>(qrow + elem_off<KT>(g, kk));
      if (!rv) x = u32x4_t{0u, 0u, 0u, 0u};
      a[nt][kk] = __builtin_bit_cast(bf16x8_t, x);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float wf = ROUTE ? wlds[jw[nt][i]] : p.w[static_cast<size_t>(n) * p.H_I + jw[nt][i]];
      wv[nt][i] = nt * 16 + 4 * g + i < p.nrows ? wf : 0.f;
    }
  }
  if (do_hist) __syncthreads();

  // three register buffers in rotation: while group i is scored, groups i+1
  // and i+2 are in flight (group i+2 is issued just before group i is
  // scored).  Every load is unconditional (groups past the wavefront's last
  // tile read valid rows and are never scored), so the compiler's wait counts
  // are exact and never drain the prefetch.
  if (wtiles > 0) {
    const int ng = (wtiles + U - 1) / U;               // groups of this wavefront
    int t0 = wtile;                                    // first tile of group i
    int o0 = 0;                                        // ordinal of group i's first tile
    int i = 0;
    for (; i + 3 <= ng; i += 3) {
      vc = issue_group<KT, D, U, CAND>(rc, sc, t0 + 2 * gstep, tstride, lane, c, len, crow, kseq,
                                       sseq, p.ki, s, o0 + 2 * U, page_v);
      score_group<KT, NT, D, U>(ra, sa, va, t0, tstride, tile, lane, a, wv, g, c, len, ukw,
                                o0, lh, do_hist);
      va = issue_group<KT, D, U, CAND>(ra, sa, t0 + 3 * gstep, tstride, lane, c, len, crow, kseq,
                                       sseq, p.ki, s, o0 + 3 * U, page_v);
      score_group<KT, NT, D, U>(rb, sb, vb, t0 + gstep, tstride, tile, lane, a, wv, g, c, len,
                                ukw, o0 + U, lh, do_hist);
      vb = issue_group<KT, D, U, CAND>(rb, sb, t0 + 4 * gstep, tstride, lane, c, len, crow, kseq,
                                       sseq, p.ki, s, o0 + 4 * U, page_v);
      score_group<KT, NT, D, U>(rc, sc, vc, t0 + 2 * gstep, tstride, tile, lane, a, wv, g, c,
                                len, ukw, o0 + 2 * U, lh, do_hist);
      t0 += 3 * gstep;
      o0 += 3 * U;
    }
    // groups i (in ra) and i+1 (in rb) are in flight; at most two remain
    if (i < ng)
      score_group<KT, NT, D, U>(ra, sa, va, t0, tstride, tile, lane, a, wv, g, c, len, ukw,
                                o0, lh, do_hist);
    if (i + 1 < ng)
      score_group<KT, NT, D, U>(rb, sb, vb, t0 + gstep, tstride, tile, lane, a, wv, g, c, len,
                                ukw, o0 + U, lh, do_hist);
    // the wavefront's order keys to u: tile j's 16 keys are 64 contiguous
    // bytes, written by 4 lanes with 16-byte stores (keys past the row end
    // are 0, inside the row's padded stride)
    __builtin_amdgcn_wave_barrier();
    for (int j0 = 0; j0 < wtiles; j0 += 16) {
      const int j = j0 + (lane >> 2), qd = lane & 3;
      if (j < wtiles) {
        const u32x4_t kv = *reinterpret_cast<const u32x4_t*>(ukw + j * 16 + 4 * qd);
        *reinterpret_cast<u32x4_t*>(urow + (wtile + j * tstride) * 16 + 4 * qd) = kv;
      }
    }
  }
  if (do_hist) {
    __syncthreads();
    flush_hist(lh, p.hist0 + static_cast<size_t>(n) * kHistWords);
  }
}

template <int D>
__global__ __launch_bounds__(256) void score_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ w, const float* __restrict__ k,
    const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ heads, const int32_t* __restrict__ cand, int L, int H_I,
    int nrows, int ncols, uint32_t* __restrict__ u, int u_stride, uint32_t* __restrict__ hist0,
    KeyIndex ki) {
  __shared__ float q_lds[64][D];
  __shared__ float w_lds[64];
  __shared__ uint32_t lh[kBins0];
  const int n = blockIdx.y;
  const int len = cand ? ncols : q_pos[n] + 1;
  const int e0 = blockIdx.x * 256;
  if (e0 >= len) return;
  for (int x = threadIdx.x; x < nrows * D; x += 256) {
    const int r = x / D, i = x % D;
    const int j = heads ? heads[static_cast<size_t>(n) * nrows + r] : r;
    q_lds[r][i] = q[(static_cast<size_t>(n) * H_I + j) * D + i];
  }
  for (int r = threadIdx.x; r < nrows; r += 256) {
    const int j = heads ? heads[static_cast<size_t>(n) * nrows + r] : r;
    w_lds[r] = w[static_cast<size_t>(n) * H_I + j];
  }
  if (hist0)
    for (int b = threadIdx.x; b < kBins0; b += 256) lh[b] = 0u;
  __syncthreads();
  const int e = e0 + threadIdx.x;
  if (e < len) {
    const int tok = cand ? cand[static_cast<size_t>(n) * ncols + e] : e;
    uint32_t key = 0u;
    if (tok >= 0) {
      float kr[D];
      const float4* kp = reinterpret_cast<const float4*>(k + ki.row(q_seq[n], tok) * D);
#pragma unroll
      for (int i = 0; i < D / 4; ++i) {
        const float4 x = kp[i];
        kr[4 * i] = x.x;
        kr[4 * i + 1] = x.y;
        kr[4 * i + 2] = x.z;
        kr[4 * i + 3] = x.w;
      }
      float acc = 0.f;
      for (int r = 0; r < nrows; ++r) {
        float dt = 0.f;
#pragma unroll
        for (int i = 0; i < D; ++i) dt += q_lds[r][i] * kr[i];
        acc += w_lds[r] * fmaxf(dt, 0.f);
      }
      key = order_key(acc);
      if (hist0) atomicAdd(&lh[key >> kShift0], 1u);
    }
    u[static_cast<size_t>(n) * u_stride + e] = key;
  }
  if (hist0) {
    __syncthreads();
    flush_hist(lh, hist0 + static_cast<size_t>(n) * kHistWords);
  }
}

template <int KT, int NT, int D>
hipError_t launch_mfma(const ScoreArgs& a, hipStream_t st, int tiles_per_wave) {
  constexpr int U = 2;                                 // tiles per group (two groups in flight)
  ScoreParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.w = a.w;
  p.k = static_cast<const uint8_t*>(a.k);
  p.k_scale = a.k_scale;
  p.q_seq = a.q_seq;
  p.q_pos = a.q_pos;
  p.heads = a.heads;
  p.cand = a.cand;
  p.L = a.L;
  p.H_I = a.H_I;
  p.nrows = a.heads ? a.h : a.H_I;
  p.ncols = a.ncols;
  p.u = a.u;
  p.u_stride = a.u_stride;
  p.hist0 = a.hist0;
  p.tiles_per_wave = tiles_per_wave;
  p.ki = a.kidx;
  p.route_partial = a.route_partial;
  p.route_nchunks = a.route_nchunks;
  p.B = a.B;
  p.heads_out = a.heads_out;
  p.head_score_out = a.head_score_out;
  if (a.route_partial) p.nrows = a.h;
  const int maxlen = a.cand ? a.ncols : a.L;
  const int per_wg = 4 * tiles_per_wave * 16;
  const int nchunks = (maxlen + per_wg - 1) / per_wg;
  if (a.cand)
    MISA_LAUNCH(K_SCORE_MFMA, (score_mfma_kernel<KT, NT, D, U, true, false>), dim3(nchunks, a.N),
                dim3(256), 0, st, p);
  else if (a.route_partial)
    MISA_LAUNCH(K_SCORE_MFMA, (score_mfma_kernel<KT, NT, D, U, false, true>), dim3(nchunks, a.N),
                dim3(256), 0, st, p);
  else
    MISA_LAUNCH(K_SCORE_MFMA, (score_mfma_kernel<KT, NT, D, U, false, false>),
                dim3(nchunks, a.N), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <int KT, int D>
hipError_t launch_mfma_rows(const ScoreArgs& a, hipStream_t st, int tpw) {
  const int nrows = (a.heads || a.route_partial) ? a.h : a.H_I;
  if (nrows <= 16) return launch_mfma<KT, 1, D>(a, st, tpw);
  if (nrows <= 32) return launch_mfma<KT, 2, D>(a, st, tpw);
  if (nrows <= 48) return launch_mfma<KT, 3, D>(a, st, tpw);
  return launch_mfma<KT, 4, D>(a, st, tpw);
}

}  // namespace

hipError_t launch_score(const ScoreArgs& a, hipStream_t st) {
  if (a.k_dt == DT_F32) {
    const int maxlen = a.cand ? a.ncols : a.L;
    const dim3 grid((maxlen + 255) / 256, a.N);
    const int nrows = a.heads ? a.h : a.H_I;
    if (a.d == 64)
      MISA_LAUNCH(K_SCORE_F32, score_f32_kernel<64>, grid, dim3(256), 0, st,
                  static_cast<const float*>(a.q), a.w, static_cast<const float*>(a.k), a.q_seq,
                  a.q_pos, a.heads, a.cand, a.L, a.H_I, nrows, a.ncols, a.u, a.u_stride,
                  a.hist0, a.kidx);
    else
      MISA_LAUNCH(K_SCORE_F32, score_f32_kernel<128>, grid, dim3(256), 0, st,
                  static_cast<const float*>(a.q), a.w, static_cast<const float*>(a.k), a.q_seq,
                  a.q_pos, a.heads, a.cand, a.L, a.H_I, nrows, a.ncols, a.u, a.u_stride,
                  a.hist0, a.kidx);
    return hipGetLastError();
  }
  // tiles (of 16 keys) per wavefront; short candidate lists use smaller
  // chunks so more workgroups share the gather (at most 64 tiles per
  // wavefront: the paged path keeps one page number per lane)
  const int tpw = a.cand ? 2 : kMaxTpw;
  if (a.k_dt == DT_BF16)
    return a.d == 64 ? launch_mfma_rows<DT_BF16, 64>(a, st, tpw)
                     : launch_mfma_rows<DT_BF16, 128>(a, st, tpw);
  return a.d == 64 ? launch_mfma_rows<DT_E4M3, 64>(a, st, tpw)
                   : launch_mfma_rows<DT_E4M3, 128>(a, st, tpw);
}

}  // namespace misa
