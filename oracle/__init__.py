"""CPU oracle of the MISA routed indexer -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this package.  The GPU library never imports, links or calls it,
and it shares no code with the GPU library.  The arithmetic lives in
misa_ref.cpp (plain C++ loops in double precision); this file only passes
numpy arrays to it.

Every function takes a synth.Problem-like object (or explicit arrays) and
returns numpy arrays.  Output idx rows are in (score desc, index asc) order,
padded with -1.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libmisa_ref.so")
_SRC = os.path.join(_HERE, "misa_ref.cpp")

GXX_CMD = ["g++", "-O2", "-std=c++17", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           _SRC, "-o", _SO]


def build() -> str:
    subprocess.run(GXX_CMD, check=True)
    return _SO


def _load():
    if not os.path.exists(_SO):
        build()
    lib = ctypes.CDLL(_SO)
    P = ctypes.c_void_p
    I = ctypes.c_int
    I64 = ctypes.c_int64
    common = [P, I, P, P, P, P, I, P, P]   # q q_dt q_scale w k k_scale k_dt q_seq q_pos
    lib.misa_ref_decode.argtypes = [P, P, I, I64, I, P]
    lib.misa_ref_pool_keys.argtypes = [P, P, I, I, I, I, I, P, P]
    lib.misa_ref_route_heads.argtypes = common + [I] * 7 + [P, P, P]
    lib.misa_ref_scores.argtypes = common + [P] + [I] * 6 + [P, P]
    lib.misa_ref_score_topk.argtypes = common + [P] + [I] * 7 + [P, P, P, P]
    lib.dsa_ref_score_topk.argtypes = common + [I] * 6 + [P, P, P, P]
    lib.misa_ref_rerank.argtypes = common + [P] + [I] * 7 + [P, P, P, P]
    lib.misa_ref_score_topk_blocks.argtypes = common + [P] + [I] * 9 + [P, P, P]
    lib.misa_ref_sparse_attention.argtypes = [P, I, P, I, P, P] + [I] * 7 + [ctypes.c_double,
                                                                              P, P]
    lib.misa_ref_max_threads.argtypes = []
    lib.misa_ref_set_threads.argtypes = [I]
    lib.misa_ref_set_threads.restype = None
    for f in ("misa_ref_decode", "misa_ref_pool_keys", "misa_ref_route_heads",
              "misa_ref_scores", "misa_ref_score_topk", "dsa_ref_score_topk",
              "misa_ref_rerank", "misa_ref_sparse_attention", "misa_ref_score_topk_blocks",
              "misa_ref_max_threads"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


class OracleError(RuntimeError):
    pass


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what} failed with code {rc}")


def _args(p):
    """(q, q_scale, w, k, k_scale, q_seq, q_pos) as contiguous arrays (scales may be None)."""
    q = np.ascontiguousarray(p.q)
    k = np.ascontiguousarray(p.k)
    return (q, _c(getattr(p, "q_scale", None), np.float32), _c(p.w, np.float32), k,
            _c(p.k_scale, np.float32), _c(p.q_seq, np.int32), _c(p.q_pos, np.int32))


def max_threads() -> int:
    return lib().misa_ref_max_threads()


def set_threads(n: int) -> None:
    """Threads of the caller's later oracle calls (OpenMP)."""
    lib().misa_ref_set_threads(int(n))


def decode(src: np.ndarray, dt: int, scale=None) -> np.ndarray:
    src = np.ascontiguousarray(src)
    d = src.shape[-1] if src.ndim else 1
    rows = src.size // d
    out = np.empty(src.shape, dtype=np.float64)
    sc = _c(scale, np.float32)
    _check(lib().misa_ref_decode(_p(src), _p(sc), dt, rows, d, _p(out)), "decode")
    return out


def pool_keys(p, mac=None):
    S, L, d = p.k.shape
    M = (L + p.B - 1) // p.B
    kbar = np.empty((S, M, d), dtype=np.float64)
    k = np.ascontiguousarray(p.k)
    _check(lib().misa_ref_pool_keys(_p(k), _p(_c(p.k_scale, np.float32)), p.k_dt, S, L, d, p.B,
                                    _p(kbar), _p(mac)), "pool_keys")
    return kbar


def route_heads(p, h=None, mac=None):
    h = p.h if h is None else h
    q, qsc, w, k, ks, sq, qp = _args(p)
    N, H_I, d = q.shape
    heads = np.empty((N, h), dtype=np.int32)
    r = np.empty((N, H_I), dtype=np.float64)
    _check(lib().misa_ref_route_heads(_p(q), p.q_dt, _p(qsc), _p(w), _p(k), _p(ks), p.k_dt, _p(sq), _p(qp),
                                      N, p.k.shape[0], p.k.shape[1], d, p.B, H_I, h,
                                      _p(heads), _p(r), _p(mac)), "route_heads")
    return heads, r


def scores(p, heads=None, mac=None):
    """Full score rows [N, L] (-inf past each row's visible prefix); heads None = all heads."""
    q, qsc, w, k, ks, sq, qp = _args(p)
    N, H_I, d = q.shape
    hd = _c(heads, np.int32)
    h = H_I if hd is None else hd.shape[1]
    out = np.empty((N, p.k.shape[1]), dtype=np.float64)
    _check(lib().misa_ref_scores(_p(q), p.q_dt, _p(qsc), _p(w), _p(k), _p(ks), p.k_dt, _p(sq), _p(qp),
                                 _p(hd), N, p.k.shape[0], p.k.shape[1], d, H_I, h, _p(out),
                                 _p(mac)), "scores")
    return out


def score_topk(p, heads, topk=None, mac=None):
    topk = p.topk if topk is None else topk
    q, qsc, w, k, ks, sq, qp = _args(p)
    N, H_I, d = q.shape
    hd = _c(heads, np.int32)
    idx = np.empty((N, topk), dtype=np.int32)
    sc = np.empty((N, topk), dtype=np.float64)
    kth = np.empty(N, dtype=np.float64)
    _check(lib().misa_ref_score_topk(_p(q), p.q_dt, _p(qsc), _p(w), _p(k), _p(ks), p.k_dt, _p(sq), _p(qp),
                                     _p(hd), N, p.k.shape[0], p.k.shape[1], d, H_I, hd.shape[1],
                                     topk, _p(idx), _p(sc), _p(kth), _p(mac)), "score_topk")
    return idx, sc, kth


def dsa_score_topk(p, topk=None, mac=None):
    topk = p.topk if topk is None else topk
    q, qsc, w, k, ks, sq, qp = _args(p)
    N, H_I, d = q.shape
    idx = np.empty((N, topk), dtype=np.int32)
    sc = np.empty((N, topk), dtype=np.float64)
    kth = np.empty(N, dtype=np.float64)
    _check(lib().dsa_ref_score_topk(_p(q), p.q_dt, _p(qsc), _p(w), _p(k), _p(ks), p.k_dt, _p(sq), _p(qp),
                                    N, p.k.shape[0], p.k.shape[1], d, H_I, topk,
                                    _p(idx), _p(sc), _p(kth), _p(mac)), "dsa_score_topk")
    return idx, sc, kth


def rerank(p, cand, topk=None, mac=None):
    topk = p.topk if topk is None else topk
    q, qsc, w, k, ks, sq, qp = _args(p)
    N, H_I, d = q.shape
    cd = _c(cand, np.int32)
    idx = np.empty((N, topk), dtype=np.int32)
    sc = np.empty((N, topk), dtype=np.float64)
    kth = np.empty(N, dtype=np.float64)
    _check(lib().misa_ref_rerank(_p(q), p.q_dt, _p(qsc), _p(w), _p(k), _p(ks), p.k_dt, _p(sq), _p(qp),
                                 _p(cd), N, p.k.shape[0], p.k.shape[1], d, H_I, cd.shape[1], topk,
                                 _p(idx), _p(sc), _p(kth), _p(mac)), "rerank")
    return idx, sc, kth


def score_topk_blocks(p, heads, m_blocks, topk=None):
    """Routed scoring over the m_blocks best blocks (see misa_ref.h).  Returns
    (blocks [N, m_blocks] ascending, idx [N, topk] in (score desc, index asc)
    order, score [N, topk])."""
    topk = p.topk if topk is None else topk
    q, qsc, w, k, ks, sq, qp = _args(p)
    N, H_I, d = q.shape
    hd = _c(heads, np.int32)
    blocks = np.empty((N, m_blocks), dtype=np.int32)
    idx = np.empty((N, topk), dtype=np.int32)
    sc = np.empty((N, topk), dtype=np.float64)
    _check(lib().misa_ref_score_topk_blocks(_p(q), p.q_dt, _p(qsc), _p(w), _p(k), _p(ks), p.k_dt,
                                            _p(sq), _p(qp), _p(hd), N, p.k.shape[0], p.k.shape[1],
                                            d, p.B, H_I, hd.shape[1], m_blocks, topk,
                                            _p(blocks), _p(idx), _p(sc)), "score_topk_blocks")
    return blocks, idx, sc


def misa(p, h=None, topk=None, mac=None):
    """Full MISA: route, then routed score + top-k.  Returns (heads, r, idx, score, kth)."""
    heads, r = route_heads(p, h, mac)
    idx, sc, kth = score_topk(p, heads, topk, mac)
    return heads, r, idx, sc, kth


def misa_dagger(p, h=None, k_prime=None, topk=None, mac=None):
    """MISA-dagger: route, routed top-k', full-head rerank to top-k."""
    k_prime = p.k_prime if k_prime is None else k_prime
    heads, r = route_heads(p, h, mac)
    cand, _, _ = score_topk(p, heads, k_prime, mac)
    idx, sc, kth = rerank(p, cand, topk, mac)
    return heads, cand, idx, sc, kth


def sparse_attention(q, q_dt, kv, kv_dt, q_seq, idx, scale, d_v):
    """Softmax attention of every head of every row over the row's selected
    tokens (see misa_ref.h).  Returns (out [N, H, d_v], lse [N, H]) in float64."""
    q = np.ascontiguousarray(q)
    kv = np.ascontiguousarray(kv)
    N, H, d_qk = q.shape
    S, L = kv.shape[:2]
    sq = _c(q_seq, np.int32)
    ix = _c(idx, np.int32)
    out = np.empty((N, H, d_v), dtype=np.float64)
    lse = np.empty((N, H), dtype=np.float64)
    _check(lib().misa_ref_sparse_attention(_p(q), q_dt, _p(kv), kv_dt, _p(sq), _p(ix), N, S, L, H,
                                           d_qk, d_v, ix.shape[1], float(scale), _p(out),
                                           _p(lse)), "sparse_attention")
    return out, lse
