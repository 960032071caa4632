// CPU oracle of the MISA routed indexer -- TEST INFRASTRUCTURE ONLY.
// Plain loops in double precision; see misa_ref.h for what each function
// computes and which passage of the MISA pages it follows.  Library routines
// used as steps: std::sort (ordering by score then index).
#include "misa_ref.h"

#include <omp.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <limits>
#include <numeric>
#include <vector>

namespace {

constexpr int DT_F32 = 0, DT_BF16 = 1, DT_E4M3 = 2;
constexpr double NEG_INF = -std::numeric_limits<double>::infinity();

double bf16_value(uint16_t bits) {
  uint32_t u = static_cast<uint32_t>(bits) << 16;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return f;
}

// OCP 8-bit floating point, E4M3 ("fn") encoding: sign bit, 4 exponent bits
// (bias 7), 3 mantissa bits; exponent field 0 holds subnormals m/8 * 2^-6;
// S.1111.111 is NaN; there are no infinities.
double e4m3_value(uint8_t code) {
  const int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
  double mag;
  if (e == 15 && m == 7) return std::numeric_limits<double>::quiet_NaN();
  if (e == 0)
    mag = std::ldexp(m / 8.0, -6);
  else
    mag = std::ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

double stored_value(const void* base, int dt, int64_t i) {
  switch (dt) {
    case DT_F32: return static_cast<const float*>(base)[i];
    case DT_BF16: return bf16_value(static_cast<const uint16_t*>(base)[i]);
    default: return e4m3_value(static_cast<const uint8_t*>(base)[i]);
  }
}

// Decoded key row t of sequence s (scale applied for e4m3).
void key_row(const void* k, const float* k_scale, int k_dt, int L, int d, int s, int64_t t,
             double* out) {
  const int64_t row = static_cast<int64_t>(s) * L + t;
  const double sc = (k_dt == DT_E4M3) ? static_cast<double>(k_scale[row]) : 1.0;
  for (int i = 0; i < d; ++i) out[i] = stored_value(k, k_dt, row * d + i) * sc;
}

// Decoded query heads of row n: [H_I][d] (e4m3: head j's codes times
// q_scale[n, j]).
std::vector<double> query_heads(const void* q, int q_dt, const float* q_scale, int n, int H_I,
                                int d) {
  std::vector<double> out(static_cast<size_t>(H_I) * d);
  const int64_t base = static_cast<int64_t>(n) * H_I * d;
  for (int j = 0; j < H_I; ++j) {
    const double sc =
        (q_dt == DT_E4M3) ? static_cast<double>(q_scale[static_cast<int64_t>(n) * H_I + j]) : 1.0;
    for (int i = 0; i < d; ++i) {
      const int64_t e = static_cast<int64_t>(j) * d + i;
      out[e] = stored_value(q, q_dt, base + e) * sc;
    }
  }
  return out;
}

double dot(const double* a, const double* b, int d) {
  double acc = 0.0;
  for (int i = 0; i < d; ++i) acc += a[i] * b[i];
  return acc;
}

double relu(double x) { return x > 0.0 ? x : 0.0; }

int check_common(const void* q, int q_dt, const float* q_scale, const float* w, const void* k,
                 const float* k_scale, int k_dt, const int32_t* q_seq, const int32_t* q_pos,
                 int N, int S, int L, int d, int H_I) {
  if (!q || !w || !k || !q_seq || !q_pos) return 1;
  if (k_dt == DT_E4M3 && !k_scale) return 1;
  if (q_dt == DT_E4M3 && !q_scale) return 1;
  if (q_dt != DT_F32 && q_dt != DT_BF16 && q_dt != DT_E4M3) return 3;
  if (k_dt != DT_F32 && k_dt != DT_BF16 && k_dt != DT_E4M3) return 3;
  if (N < 0 || S < 1 || L < 1 || d < 1 || H_I < 1) return 2;
  for (int n = 0; n < N; ++n) {
    if (q_seq[n] < 0 || q_seq[n] >= S) return 2;
    if (q_pos[n] < 0 || q_pos[n] >= L) return 2;
  }
  return 0;
}

// Order (score desc, index asc) and keep the first topk; pads -1 / -inf.
void select_topk(const std::vector<double>& sc, const std::vector<int32_t>& tok, int topk,
                 int32_t* idx, double* score, double* kth) {
  std::vector<size_t> order(sc.size());
  std::iota(order.begin(), order.end(), size_t{0});
  std::sort(order.begin(), order.end(), [&](size_t a, size_t b) {
    if (sc[a] != sc[b]) return sc[a] > sc[b];
    return tok[a] < tok[b];
  });
  const size_t take = std::min(order.size(), static_cast<size_t>(topk));
  for (size_t i = 0; i < static_cast<size_t>(topk); ++i) {
    if (i < take) {
      idx[i] = tok[order[i]];
      if (score) score[i] = sc[order[i]];
    } else {
      idx[i] = -1;
      if (score) score[i] = NEG_INF;
    }
  }
  if (kth) *kth = take ? sc[order[take - 1]] : NEG_INF;
}

// Routed or dense scores of query n over its visible prefix.
std::vector<double> query_scores(const void* q, int q_dt, const float* q_scale, const float* w,
                                 const void* k, const float* k_scale, int k_dt, int n, int s,
                                 int Ln, int L, int d, int H_I, const std::vector<int>& heads) {
  const std::vector<double> qh = query_heads(q, q_dt, q_scale, n, H_I, d);
  std::vector<double> out(Ln);
#pragma omp parallel
  {
    std::vector<double> kr(d);
#pragma omp for schedule(static)
    for (int t = 0; t < Ln; ++t) {
      key_row(k, k_scale, k_dt, L, d, s, t, kr.data());
      double acc = 0.0;
      for (int j : heads)
        acc += static_cast<double>(w[static_cast<int64_t>(n) * H_I + j]) *
               relu(dot(&qh[static_cast<size_t>(j) * d], kr.data(), d));
      out[t] = acc;
    }
  }
  return out;
}

std::vector<int> heads_of(const int32_t* heads, int n, int h, int H_I) {
  std::vector<int> hs;
  if (heads) {
    for (int i = 0; i < h; ++i) hs.push_back(heads[static_cast<int64_t>(n) * h + i]);
    std::sort(hs.begin(), hs.end());       // summation order: ascending head index
  } else {
    for (int j = 0; j < H_I; ++j) hs.push_back(j);
  }
  return hs;
}

}  // namespace

extern "C" {

int misa_ref_max_threads(void) { return omp_get_max_threads(); }

void misa_ref_set_threads(int n) {
  if (n > 0) omp_set_num_threads(n);
}

int misa_ref_decode(const void* src, const float* scale, int dt, int64_t rows, int d,
                    double* out) {
  if (!src || !out || (dt == DT_E4M3 && !scale)) return 1;
  if (dt < DT_F32 || dt > DT_E4M3) return 3;
  for (int64_t r = 0; r < rows; ++r) {
    const double sc = (dt == DT_E4M3) ? static_cast<double>(scale[r]) : 1.0;
    for (int i = 0; i < d; ++i) out[r * d + i] = stored_value(src, dt, r * d + i) * sc;
  }
  return 0;
}

int misa_ref_pool_keys(const void* k, const float* k_scale, int k_dt, int S, int L, int d,
                       int B, double* kbar, uint64_t* mac) {
  if (!k || !kbar || (k_dt == DT_E4M3 && !k_scale)) return 1;
  if (k_dt < DT_F32 || k_dt > DT_E4M3) return 3;
  if (S < 1 || L < 1 || d < 1 || B < 1) return 2;
  const int M = (L + B - 1) / B;
  uint64_t adds = 0;
#pragma omp parallel for collapse(2) reduction(+ : adds) schedule(static)
  for (int s = 0; s < S; ++s) {
    for (int b = 0; b < M; ++b) {
      std::vector<double> kr(d), sum(d, 0.0);
      const int t0 = b * B, t1 = std::min(t0 + B, L);
      for (int t = t0; t < t1; ++t) {
        key_row(k, k_scale, k_dt, L, d, s, t, kr.data());
        for (int i = 0; i < d; ++i) sum[i] += kr[i];
      }
      adds += static_cast<uint64_t>(t1 - t0) * d;
      double* dst = kbar + (static_cast<int64_t>(s) * M + b) * d;
      for (int i = 0; i < d; ++i) dst[i] = sum[i] / (t1 - t0);
    }
  }
  if (mac) mac[3] += adds;
  return 0;
}

int misa_ref_route_heads(const void* q, int q_dt, const float* q_scale, const float* w, const void* k,
                         const float* k_scale, int k_dt, const int32_t* q_seq,
                         const int32_t* q_pos, int N, int S, int L, int d, int B, int H_I,
                         int h, int32_t* heads, double* head_score, uint64_t* mac) {
  int rc = check_common(q, q_dt, q_scale, w, k, k_scale, k_dt, q_seq, q_pos, N, S, L, d, H_I);
  if (rc) return rc;
  if (!heads) return 1;
  if (B < 1 || h < 1 || h > H_I) return 2;
  uint64_t router_macs = 0, pool_adds = 0;
#pragma omp parallel for reduction(+ : router_macs, pool_adds) schedule(dynamic, 1)
  for (int n = 0; n < N; ++n) {
    const int s = q_seq[n], Ln = q_pos[n] + 1;
    const int Mn = (Ln + B - 1) / B;
    const std::vector<double> qh = query_heads(q, q_dt, q_scale, n, H_I, d);
    std::vector<double> affinity(H_I, 0.0), kr(d), mean(d);
    for (int b = 0; b < Mn; ++b) {
      const int t0 = b * B, t1 = std::min(t0 + B, Ln);       // visible part of block b
      std::fill(mean.begin(), mean.end(), 0.0);
      for (int t = t0; t < t1; ++t) {
        key_row(k, k_scale, k_dt, L, d, s, t, kr.data());
        for (int i = 0; i < d; ++i) mean[i] += kr[i];
      }
      for (int i = 0; i < d; ++i) mean[i] /= (t1 - t0);
      pool_adds += static_cast<uint64_t>(t1 - t0) * d;
      for (int j = 0; j < H_I; ++j) affinity[j] += relu(dot(&qh[static_cast<size_t>(j) * d], mean.data(), d));
      router_macs += static_cast<uint64_t>(H_I) * d;
    }
    std::vector<double> r(H_I);
    for (int j = 0; j < H_I; ++j)
      r[j] = std::fabs(static_cast<double>(w[static_cast<int64_t>(n) * H_I + j])) * affinity[j];
    std::vector<int> order(H_I);
    std::iota(order.begin(), order.end(), 0);
    std::sort(order.begin(), order.end(), [&](int a, int b) {
      if (r[a] != r[b]) return r[a] > r[b];
      return a < b;
    });
    std::vector<int> chosen(order.begin(), order.begin() + h);
    std::sort(chosen.begin(), chosen.end());
    for (int i = 0; i < h; ++i) heads[static_cast<int64_t>(n) * h + i] = chosen[i];
    if (head_score)
      for (int j = 0; j < H_I; ++j) head_score[static_cast<int64_t>(n) * H_I + j] = r[j];
  }
  if (mac) {
    mac[0] += router_macs;
    mac[3] += pool_adds;
  }
  return 0;
}

int misa_ref_scores(const void* q, int q_dt, const float* q_scale, const float* w, const void* k,
                    const float* k_scale, int k_dt, const int32_t* q_seq, const int32_t* q_pos,
                    const int32_t* heads, int N, int S, int L, int d, int H_I, int h,
                    double* scores, uint64_t* mac) {
  int rc = check_common(q, q_dt, q_scale, w, k, k_scale, k_dt, q_seq, q_pos, N, S, L, d, H_I);
  if (rc) return rc;
  if (!scores) return 1;
  if (heads && (h < 1 || h > H_I)) return 2;
  uint64_t score_macs = 0;
  for (int n = 0; n < N; ++n) {
    const std::vector<int> hs = heads_of(heads, n, h, H_I);
    for (int j : hs)
      if (j < 0 || j >= H_I) return 2;
    const int Ln = q_pos[n] + 1;
    const std::vector<double> sc =
        query_scores(q, q_dt, q_scale, w, k, k_scale, k_dt, n, q_seq[n], Ln, L, d, H_I, hs);
    double* row = scores + static_cast<int64_t>(n) * L;
    for (int t = 0; t < L; ++t) row[t] = t < Ln ? sc[t] : NEG_INF;
    score_macs += static_cast<uint64_t>(hs.size()) * Ln * d;
  }
  if (mac) mac[1] += score_macs;
  return 0;
}

int misa_ref_score_topk(const void* q, int q_dt, const float* q_scale, const float* w, const void* k,
                        const float* k_scale, int k_dt, const int32_t* q_seq,
                        const int32_t* q_pos, const int32_t* heads, int N, int S, int L, int d,
                        int H_I, int h, int topk, int32_t* idx, double* score, double* kth,
                        uint64_t* mac) {
  int rc = check_common(q, q_dt, q_scale, w, k, k_scale, k_dt, q_seq, q_pos, N, S, L, d, H_I);
  if (rc) return rc;
  if (!idx) return 1;
  if (topk < 1 || (heads && (h < 1 || h > H_I))) return 2;
  uint64_t score_macs = 0;
  for (int n = 0; n < N; ++n) {
    const std::vector<int> hs = heads_of(heads, n, h, H_I);
    for (int j : hs)
      if (j < 0 || j >= H_I) return 2;
    const int Ln = q_pos[n] + 1;
    const std::vector<double> sc =
        query_scores(q, q_dt, q_scale, w, k, k_scale, k_dt, n, q_seq[n], Ln, L, d, H_I, hs);
    std::vector<int32_t> tok(Ln);
    std::iota(tok.begin(), tok.end(), 0);
    select_topk(sc, tok, topk, idx + static_cast<int64_t>(n) * topk,
                score ? score + static_cast<int64_t>(n) * topk : nullptr, kth ? kth + n : nullptr);
    score_macs += static_cast<uint64_t>(hs.size()) * Ln * d;
  }
  if (mac) mac[1] += score_macs;
  return 0;
}

int dsa_ref_score_topk(const void* q, int q_dt, const float* q_scale, const float* w, const void* k,
                       const float* k_scale, int k_dt, const int32_t* q_seq,
                       const int32_t* q_pos, int N, int S, int L, int d, int H_I, int topk,
                       int32_t* idx, double* score, double* kth, uint64_t* mac) {
  return misa_ref_score_topk(q, q_dt, q_scale, w, k, k_scale, k_dt, q_seq, q_pos, nullptr, N, S, L, d,
                             H_I, H_I, topk, idx, score, kth, mac);
}

int misa_ref_rerank(const void* q, int q_dt, const float* q_scale, const float* w, const void* k,
                    const float* k_scale, int k_dt, const int32_t* q_seq, const int32_t* q_pos,
                    const int32_t* cand, int N, int S, int L, int d, int H_I, int k_prime,
                    int topk, int32_t* idx, double* score, double* kth, uint64_t* mac) {
  int rc = check_common(q, q_dt, q_scale, w, k, k_scale, k_dt, q_seq, q_pos, N, S, L, d, H_I);
  if (rc) return rc;
  if (!cand || !idx) return 1;
  if (topk < 1 || k_prime < topk) return 2;
  uint64_t rerank_macs = 0;
  for (int n = 0; n < N; ++n) {
    const int Ln = q_pos[n] + 1, s = q_seq[n];
    std::vector<int32_t> tok;
    for (int c = 0; c < k_prime; ++c) {
      const int32_t t = cand[static_cast<int64_t>(n) * k_prime + c];
      if (t < 0) continue;
      if (t >= Ln) return 2;
      tok.push_back(t);
    }
    std::vector<int32_t> sorted_tok(tok);
    std::sort(sorted_tok.begin(), sorted_tok.end());
    if (std::adjacent_find(sorted_tok.begin(), sorted_tok.end()) != sorted_tok.end()) return 2;
    const std::vector<double> qh = query_heads(q, q_dt, q_scale, n, H_I, d);
    std::vector<double> sc(tok.size());
#pragma omp parallel
    {
      std::vector<double> kr(d);
#pragma omp for schedule(static)
      for (int64_t c = 0; c < static_cast<int64_t>(tok.size()); ++c) {
        key_row(k, k_scale, k_dt, L, d, s, tok[c], kr.data());
        double acc = 0.0;
        for (int j = 0; j < H_I; ++j)
          acc += static_cast<double>(w[static_cast<int64_t>(n) * H_I + j]) *
                 relu(dot(&qh[static_cast<size_t>(j) * d], kr.data(), d));
        sc[c] = acc;
      }
    }
    select_topk(sc, tok, topk, idx + static_cast<int64_t>(n) * topk,
                score ? score + static_cast<int64_t>(n) * topk : nullptr, kth ? kth + n : nullptr);
    rerank_macs += static_cast<uint64_t>(H_I) * tok.size() * d;
  }
  if (mac) mac[2] += rerank_macs;
  return 0;
}

int misa_ref_score_topk_blocks(const void* q, int q_dt, const float* q_scale, const float* w,
                               const void* k, const float* k_scale, int k_dt,
                               const int32_t* q_seq, const int32_t* q_pos, const int32_t* heads,
                               int N, int S, int L, int d, int B, int H_I, int h, int m_blocks,
                               int topk, int32_t* blocks, int32_t* idx, double* score) {
  int rc = check_common(q, q_dt, q_scale, w, k, k_scale, k_dt, q_seq, q_pos, N, S, L, d, H_I);
  if (rc) return rc;
  if (!heads || !blocks || !idx) return 1;
  if (B < 1 || h < 1 || h > H_I || m_blocks < 1 || topk < 1) return 2;
  for (int n = 0; n < N; ++n) {
    const int Ln = q_pos[n] + 1, s = q_seq[n];
    const int Mn = (Ln + B - 1) / B;
    const std::vector<int> hs = heads_of(heads, n, h, H_I);
    const std::vector<double> qh = query_heads(q, q_dt, q_scale, n, H_I, d);
    // block keys: means of the row's visible keys of each block
    std::vector<double> bsc(Mn);
    std::vector<int32_t> bid(Mn);
    std::vector<double> mean(d), kr(d);
    for (int b = 0; b < Mn; ++b) {
      const int t0 = b * B, t1 = std::min((b + 1) * B, Ln);
      std::fill(mean.begin(), mean.end(), 0.0);
      for (int t = t0; t < t1; ++t) {
        key_row(k, k_scale, k_dt, L, d, s, t, kr.data());
        for (int i = 0; i < d; ++i) mean[i] += kr[i];
      }
      for (int i = 0; i < d; ++i) mean[i] /= (t1 - t0);
      double acc = 0.0;
      for (int j : hs)
        acc += static_cast<double>(w[static_cast<int64_t>(n) * H_I + j]) *
               relu(dot(&qh[static_cast<size_t>(j) * d], mean.data(), d));
      bsc[b] = acc;
      bid[b] = b;
    }
    // the m highest block scores (ties: lower block), listed ascending
    std::vector<int32_t> kept(m_blocks);
    select_topk(bsc, bid, m_blocks, kept.data(), nullptr, nullptr);
    std::vector<int32_t> kb;
    for (int32_t b : kept)
      if (b >= 0) kb.push_back(b);
    std::sort(kb.begin(), kb.end());
    for (int i = 0; i < m_blocks; ++i)
      blocks[static_cast<int64_t>(n) * m_blocks + i] = i < static_cast<int>(kb.size()) ? kb[i] : -1;
    // token scores over the kept blocks' visible tokens, then the top-k
    std::vector<int32_t> tok;
    for (int32_t b : kb)
      for (int t = b * B; t < std::min((b + 1) * B, Ln); ++t) tok.push_back(t);
    std::vector<double> sc(tok.size());
#pragma omp parallel
    {
      std::vector<double> kt(d);
#pragma omp for schedule(static)
      for (int64_t c = 0; c < static_cast<int64_t>(tok.size()); ++c) {
        key_row(k, k_scale, k_dt, L, d, s, tok[c], kt.data());
        double acc = 0.0;
        for (int j : hs)
          acc += static_cast<double>(w[static_cast<int64_t>(n) * H_I + j]) *
                 relu(dot(&qh[static_cast<size_t>(j) * d], kt.data(), d));
        sc[c] = acc;
      }
    }
    select_topk(sc, tok, topk, idx + static_cast<int64_t>(n) * topk,
                score ? score + static_cast<int64_t>(n) * topk : nullptr, nullptr);
  }
  return 0;
}

int misa_ref_sparse_attention(const void* q, int q_dt, const void* kv, int kv_dt,
                              const int32_t* q_seq, const int32_t* idx, int N, int S, int L,
                              int H, int d_qk, int d_v, int topk, double scale, double* out,
                              double* lse) {
  if (!q || !kv || !q_seq || !idx || !out || !lse) return 1;
  if ((q_dt != DT_F32 && q_dt != DT_BF16) || (kv_dt != DT_F32 && kv_dt != DT_BF16)) return 3;
  if (N < 0 || S < 1 || L < 1 || H < 1 || d_qk < 1 || d_v < 1 || d_v > d_qk || topk < 1) return 2;
  for (int n = 0; n < N; ++n) {
    if (q_seq[n] < 0 || q_seq[n] >= S) return 2;
    std::vector<int32_t> tok;
    for (int i = 0; i < topk; ++i) {
      const int32_t t = idx[static_cast<int64_t>(n) * topk + i];
      if (t < 0) continue;
      if (t >= L) return 2;
      tok.push_back(t);
    }
    std::vector<int32_t> sorted_tok(tok);
    std::sort(sorted_tok.begin(), sorted_tok.end());
    if (std::adjacent_find(sorted_tok.begin(), sorted_tok.end()) != sorted_tok.end()) return 2;
    // selected cache rows, decoded once
    std::vector<double> rows(tok.size() * static_cast<size_t>(d_qk));
    const int64_t seq0 = static_cast<int64_t>(q_seq[n]) * L;
    for (size_t c = 0; c < tok.size(); ++c)
      for (int i = 0; i < d_qk; ++i)
        rows[c * d_qk + i] = stored_value(kv, kv_dt, (seq0 + tok[c]) * d_qk + i);
#pragma omp parallel for schedule(static)
    for (int h = 0; h < H; ++h) {
      const int64_t qrow = (static_cast<int64_t>(n) * H + h) * d_qk;
      std::vector<double> qh(d_qk);
      for (int i = 0; i < d_qk; ++i) qh[i] = stored_value(q, q_dt, qrow + i);
      double* o = out + (static_cast<int64_t>(n) * H + h) * d_v;
      for (int i = 0; i < d_v; ++i) o[i] = 0.0;
      if (tok.empty()) {
        lse[static_cast<int64_t>(n) * H + h] = NEG_INF;
        continue;
      }
      std::vector<double> sc(tok.size());
      double m = NEG_INF;
      for (size_t c = 0; c < tok.size(); ++c) {
        sc[c] = scale * dot(qh.data(), &rows[c * d_qk], d_qk);
        m = std::max(m, sc[c]);
      }
      double z = 0.0;
      for (size_t c = 0; c < tok.size(); ++c) {
        const double pc = std::exp(sc[c] - m);
        z += pc;
        for (int i = 0; i < d_v; ++i) o[i] += pc * rows[c * d_qk + i];
      }
      for (int i = 0; i < d_v; ++i) o[i] /= z;
      lse[static_cast<int64_t>(n) * H + h] = m + std::log(z);
    }
  }
  return 0;
}

}  // extern "C"
