"""Seeded synthetic inputs for the MISA routed indexer.

This module only draws random numbers and stores them in the byte formats the
indexer consumes (fp32, bf16, OCP fp8 e4m3 + per-token fp32 scale).  It holds
none of the indexer's arithmetic (no pooling, routing, scoring or selection);
both the GPU library and the CPU oracle receive exactly the arrays built here.

Shapes follow the DSA indexer of DeepSeek-V3.2 as described on the MISA pages
(H_I = 64 indexer heads with h = 8 routed heads; MISA technical summary,
"Experimental results"), with the index keys shared by all heads.  Keys come
from a Gaussian-cluster mixture; queries are N(0, 1/d); head weights N(0, 1).

Storage conventions (all C-contiguous numpy arrays):
  q       [N, H_I, d]  float32, uint16 holding bf16 bit patterns, or uint8 (e4m3 codes)
  q_scale [N, H_I]     float32 (fp8 queries only, else None: one scale per head vector)
  w       [N, H_I]     float32
  k       [S, L, d]    float32, uint16 (bf16 bits), or uint8 (e4m3 codes)
  k_scale [S, L]       float32 (fp8 keys only, else None)
  q_seq   [N]          int32   key sequence read by each query row
  q_pos   [N]          int32   position of the query row; it sees keys 0..q_pos
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

F32, BF16, FP8 = 0, 1, 2          # dtype codes shared with the C ABI
DTYPE_NAMES = {F32: "f32", BF16: "bf16", FP8: "e4m3"}


# --------------------------------------------------------------------------
# storage-format conversions (input preparation only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return
    the 16-bit patterns.  Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _e4m3_positive_table() -> np.ndarray:
    """Values of the finite non-negative OCP e4m3 ("fn") codes 0x00..0x7E,
    from the format's definition: 4 exponent bits with bias 7, 3 mantissa
    bits, subnormals at exponent field 0, no infinities, 0x7F is NaN."""
    vals = np.empty(127, dtype=np.float64)
    for code in range(127):
        e, m = code >> 3, code & 7
        vals[code] = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3_POS = _e4m3_positive_table()
E4M3_MAX = 448.0


def f64_to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """Round values to OCP e4m3 codes: nearest representable value, ties to
    the code with an even mantissa, magnitudes above 448 saturate to 448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, a, side="left")          # first value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((hi & 1) == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    sign = np.signbit(x).astype(np.uint8) << 7
    return code | sign


def quantize_e4m3(x32: np.ndarray):
    """fp8 storage of vectors along the last axis (a key token, or one query
    head): scale = absmax/448 (fp32), codes = e4m3(x/scale).  An all-zero
    vector gets scale 1 and zero codes."""
    absmax = np.abs(x32).max(axis=-1).astype(np.float32)
    scale = np.where(absmax > 0, absmax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    codes = f64_to_e4m3_codes(x32.astype(np.float64) / scale[..., None].astype(np.float64))
    return codes, scale


def e4m3_codes_to_f32(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Stored value of fp8 vectors: scale * code value (fp32 product)."""
    c = np.asarray(codes, dtype=np.uint8)
    mag = _E4M3_POS[np.minimum(c & 0x7F, 126)]
    v = np.where(c & 0x80, -mag, mag).astype(np.float32)
    return (v * np.asarray(scale, np.float32)[..., None]).astype(np.float32)


def to_pages(k: np.ndarray, k_scale: Optional[np.ndarray], page_size: int, seed: int,
             spare: int = 3):
    """Paged storage of keys [S, L, d] (and fp8 scales [S, L]): a pool of
    pages [P, page_size, d] holding the sequences' logical pages in a seeded
    random order, `spare` unused pages, and the block table
    [S, ceil(L / page_size)] of physical page numbers."""
    S, L = k.shape[:2]
    mp = -(-L // page_size)
    P = S * mp + spare
    rng = np.random.default_rng(seed)
    perm = rng.permutation(P)[:S * mp].reshape(S, mp).astype(np.int32)
    # unused rows hold NaN patterns (e4m3 0x7F, bf16 0x7FC0, fp32 NaN): a read
    # of the wrong page shows up in every result
    poison = {np.dtype(np.uint8): 0x7F, np.dtype(np.uint16): 0x7FC0}.get(k.dtype, np.nan)
    pages = np.empty((P, page_size) + k.shape[2:], dtype=k.dtype)
    pages[...] = np.array(poison).astype(k.dtype)
    spages = None
    if k_scale is not None:
        spages = np.full((P, page_size), np.float32(1.0), dtype=np.float32)
    for s in range(S):
        for j in range(mp):
            t0, t1 = j * page_size, min(L, (j + 1) * page_size)
            pages[perm[s, j], :t1 - t0] = k[s, t0:t1]
            if spages is not None:
                spages[perm[s, j], :t1 - t0] = k_scale[s, t0:t1]
    return pages, spages, perm


# --------------------------------------------------------------------------
# problem container
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Problem:
    name: str
    q: np.ndarray
    q_dt: int
    w: np.ndarray
    k: np.ndarray
    k_dt: int
    k_scale: Optional[np.ndarray]
    q_seq: np.ndarray
    q_pos: np.ndarray
    B: int
    h: int
    topk: int
    k_prime: int = 0
    needles: Optional[np.ndarray] = None      # [N, n_needle, 2] (position, head)
    q_scale: Optional[np.ndarray] = None      # [N, H_I] float32 (fp8 queries only)

    @property
    def N(self): return self.q.shape[0]
    @property
    def H_I(self): return self.q.shape[1]
    @property
    def d(self): return self.q.shape[2]
    @property
    def S(self): return self.k.shape[0]
    @property
    def L(self): return self.k.shape[1]

    def visible(self) -> np.ndarray:
        return self.q_pos.astype(np.int64) + 1

    def tokens_indexed(self) -> int:
        return int(self.visible().sum())


def _mixture_keys(rng, L, d, n_clusters, sigma):
    centers = rng.standard_normal((n_clusters, d))
    assign = rng.integers(0, n_clusters, size=L)
    noise = rng.standard_normal((L, d))
    return (centers[assign] + sigma * noise).astype(np.float32)


def _store(x32: np.ndarray, dt: int):
    if dt == F32:
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dt == BF16:
        return f32_to_bf16_bits(x32)
    raise ValueError(dt)


def mixture_problem(name, *, seed, N, S, L, d, H_I, h, B, topk, q_dt, k_dt,
                    n_clusters, sigma, q_pos=None, q_seq=None, k_prime=0,
                    n_needles=0, alpha=3.0):
    """Draw centers -> assignments -> noise per sequence, then q, then w,
    then needles.  q ~ N(0, 1/d), w ~ N(0, 1)."""
    rng = np.random.default_rng(seed)
    keys32 = np.empty((S, L, d), dtype=np.float32)
    for s in range(S):
        keys32[s] = _mixture_keys(rng, L, d, n_clusters, sigma)
    q32 = (rng.standard_normal((N, H_I, d)) / np.sqrt(d)).astype(np.float32)
    w = rng.standard_normal((N, H_I)).astype(np.float32)
    q_scale = None
    if q_dt == FP8:
        q, q_scale = quantize_e4m3(q32)
    else:
        q = _store(q32, q_dt)
    if q_seq is None:
        q_seq = np.arange(N, dtype=np.int32) % S
    if q_pos is None:
        q_pos = np.full(N, L - 1, dtype=np.int32)
    q_seq = np.ascontiguousarray(q_seq, dtype=np.int32)
    q_pos = np.ascontiguousarray(q_pos, dtype=np.int32)

    needles = None
    if n_needles:
        qv = (bf16_bits_to_f32(q) if q_dt == BF16 else
              e4m3_codes_to_f32(q, q_scale) if q_dt == FP8 else q)
        needles = np.empty((N, n_needles, 2), dtype=np.int64)
        for n in range(N):
            pos = rng.choice(int(q_pos[n]) + 1, size=n_needles, replace=False)
            heads = rng.integers(0, H_I, size=n_needles)
            needles[n, :, 0] = pos
            needles[n, :, 1] = heads
            keys32[q_seq[n], pos] = (np.float32(alpha) * qv[n, heads]).astype(np.float32)

    k_scale = None
    if k_dt == FP8:
        k, k_scale = quantize_e4m3(keys32)
    else:
        k = _store(keys32, k_dt)
    return Problem(name, q, q_dt, w, k, k_dt, k_scale, q_seq, q_pos, B, h, topk,
                   k_prime, needles, q_scale)


# --------------------------------------------------------------------------
# the named workloads
# --------------------------------------------------------------------------
CONFIG_SEEDS = {"c1": 1001, "c2": 1002, "c3": 1003, "c3x": 1013, "c3f8": 1003, "c4": 1004,
                "c5": 1005}


def make(name: str, seed: Optional[int] = None, **over) -> Problem:
    """Named workloads (DeepSeek-V3.2-like indexer shapes):
      c1  tiny fp32 decode: 1 query, L=4096, d=64, H_I=16, h=4, B=64, k=256, 8 clusters (sigma 0.3)
      c2  bf16 decode batch: 8 queries each over its own L=32768, d=128, H_I=64, h=8, B=128, k=2048,
          64 clusters (sigma 0.5)
      c3  bf16 prefill chunk: 4096 rows at positions 61440..65535 over one causal L=65536 prefix
      c3x the same prefill chunk at L=131072 (positions 126976..131071)
      c3f8 the c3 chunk (same seed, same fp32 draws) stored in fp8: q per head and k per token
          as e4m3 codes with an absmax/448 scale
      c4  bf16 long decode: 4 queries each over its own L=131072 with 32 planted needles (alpha=3)
      c5  fp8-key long decode for MISA-dagger: as c4 without needles, k'=8192 -> k=2048
    """
    seed = CONFIG_SEEDS[name] if seed is None else seed
    if name == "c1":
        kw = dict(N=1, S=1, L=4096, d=64, H_I=16, h=4, B=64, topk=256, q_dt=F32, k_dt=F32,
                  n_clusters=8, sigma=0.3)
    elif name == "c2":
        kw = dict(N=8, S=8, L=32768, d=128, H_I=64, h=8, B=128, topk=2048, q_dt=BF16, k_dt=BF16,
                  n_clusters=64, sigma=0.5)
    elif name in ("c3", "c3x", "c3f8"):
        L = 131072 if name == "c3x" else 65536
        T = 4096
        dt = FP8 if name == "c3f8" else BF16
        kw = dict(N=T, S=1, L=L, d=128, H_I=64, h=8, B=128, topk=2048, q_dt=dt, k_dt=dt,
                  n_clusters=64, sigma=0.5, q_seq=np.zeros(T, np.int32),
                  q_pos=np.arange(L - T, L, dtype=np.int32))
    elif name == "c4":
        kw = dict(N=4, S=4, L=131072, d=128, H_I=64, h=8, B=128, topk=2048, q_dt=BF16, k_dt=BF16,
                  n_clusters=64, sigma=0.5, n_needles=32, alpha=3.0)
    elif name == "c5":
        kw = dict(N=4, S=4, L=131072, d=128, H_I=64, h=8, B=128, topk=2048, q_dt=BF16, k_dt=FP8,
                  n_clusters=64, sigma=0.5, k_prime=8192)
    else:
        raise KeyError(name)
    kw.update(over)
    return mixture_problem(name, seed=seed, **kw)


def small(name: str, seed: int, *, N=2, S=2, L=1000, d=128, H_I=16, h=4, B=64, topk=100,
          q_dt=BF16, k_dt=BF16, k_prime=0, q_pos=None, q_seq=None, n_clusters=8, sigma=0.5,
          n_needles=0) -> Problem:
    """A small mixture problem of any shape (tests)."""
    return mixture_problem(name, seed=seed, N=N, S=S, L=L, d=d, H_I=H_I, h=h, B=B, topk=topk,
                           q_dt=q_dt, k_dt=k_dt, n_clusters=n_clusters, sigma=sigma,
                           q_pos=q_pos, q_seq=q_seq, k_prime=k_prime, n_needles=n_needles)


def integer_problem(name: str, seed: int, *, N=2, S=2, L=300, d=64, H_I=8, h=3, B=32, topk=40,
                    q_dt=BF16, k_dt=BF16, k_prime=0, q_pos=None, q_seq=None, qmax=3, kmax=3,
                    wmax=4) -> Problem:
    """Small-integer q, k, w (exact in bf16, fp32 and e4m3): every dot product
    and every weighted head sum is an exact small integer in any precision,
    so exact ties occur and every implementation must agree bit for bit.
    fp8 queries get power-of-two head scales, so their sums stay exact
    (multiples of 1/4)."""
    rng = np.random.default_rng(seed)
    k32 = rng.integers(-kmax, kmax + 1, size=(S, L, d)).astype(np.float32)
    q32 = rng.integers(-qmax, qmax + 1, size=(N, H_I, d)).astype(np.float32)
    w = rng.integers(-wmax, wmax + 1, size=(N, H_I)).astype(np.float32)
    q_scale = None
    if q_dt == FP8:
        # power-of-two head scales 1/4 .. 4: scaled products and sums stay exact
        q_scale = np.ldexp(np.float32(1.0), rng.integers(-2, 3, size=(N, H_I))).astype(np.float32)
    if q_seq is None:
        q_seq = np.arange(N, dtype=np.int32) % S
    if q_pos is None:
        q_pos = np.full(N, L - 1, dtype=np.int32)
    k_scale = None
    if k_dt == FP8:
        k = f64_to_e4m3_codes(k32.astype(np.float64))        # integers |v|<=3 are exact codes
        k_scale = np.ones((S, L), dtype=np.float32)
    else:
        k = _store(k32, k_dt)
    q = f64_to_e4m3_codes(q32.astype(np.float64)) if q_dt == FP8 else _store(q32, q_dt)
    return Problem(name, q, q_dt, w, k, k_dt, k_scale,
                   np.ascontiguousarray(q_seq, np.int32), np.ascontiguousarray(q_pos, np.int32),
                   B, h, topk, k_prime, q_scale=q_scale)


# --------------------------------------------------------------------------
# sparse attention over the selected tokens (the consumer of the top-k)
# --------------------------------------------------------------------------
@dataclasses.dataclass
class AttentionProblem:
    """q [N, H, d_qk] and the latent key/value cache kv [S, L, d_qk] as bf16
    bits; value rows are kv[..., :d_v].  idx [N, topk] holds each row's
    selected tokens (distinct, ascending, -1 padding at the end)."""
    name: str
    q: np.ndarray
    kv: np.ndarray
    q_seq: np.ndarray
    idx: np.ndarray
    d_v: int
    scale: float

    @property
    def N(self): return self.q.shape[0]
    @property
    def H(self): return self.q.shape[1]
    @property
    def d_qk(self): return self.q.shape[2]
    @property
    def S(self): return self.kv.shape[0]
    @property
    def L(self): return self.kv.shape[1]
    @property
    def topk(self): return self.idx.shape[1]


def attention_problem(name, seed, *, N, S, L, H, d_qk, d_v, topk, n_valid=None, q_seq=None,
                      scale=None, q_sigma=1.0):
    """Cache rows ~ N(0, 1), queries ~ N(0, q_sigma^2), each row selecting
    n_valid[n] (default min(topk, L)) distinct tokens uniformly at random,
    listed ascending then padded with -1.  scale defaults to 1/sqrt(d_qk)."""
    rng = np.random.default_rng(seed)
    kv32 = rng.standard_normal((S, L, d_qk)).astype(np.float32)
    q32 = (q_sigma * rng.standard_normal((N, H, d_qk))).astype(np.float32)
    if q_seq is None:
        q_seq = np.arange(N, dtype=np.int32) % S
    if n_valid is None:
        n_valid = np.full(N, min(topk, L), dtype=np.int64)
    idx = np.full((N, topk), -1, dtype=np.int32)
    for n in range(N):
        sel = np.sort(rng.choice(L, size=int(n_valid[n]), replace=False))
        idx[n, :len(sel)] = sel
    scale = float(1.0 / np.sqrt(d_qk)) if scale is None else float(scale)
    return AttentionProblem(name, f32_to_bf16_bits(q32), f32_to_bf16_bits(kv32),
                            np.ascontiguousarray(q_seq, dtype=np.int32), idx, d_v, scale)
