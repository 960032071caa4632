"""Python binding of libmisa.so (include/misa.h): argument marshalling only.

Each function has the name of the C entry point it calls.  Arguments are
torch tensors on the GPU; sizes are read from their shapes, outputs are
allocated with torch when not given, and the call is enqueued on torch's
current HIP stream of the tensors' device.  Every step of the computation
runs in the library's HIP kernels.  A missing library raises
MisaLibraryMissing: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

from . import synth

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmisa.so")

MISA_F32, MISA_BF16, MISA_FP8_E4M3 = 0, 1, 2
MISA_OP_ROUTE, MISA_OP_SCORE_TOPK, MISA_OP_RERANK, MISA_OP_ATTENTION, MISA_OP_BLOCKS = 0, 1, 2, 3, 4
MISA_OP_ROUTE_SCORE_TOPK = 5
MISA_OK = 0

EXPORTED = ("misa_pool_keys", "misa_pool_update", "misa_route_heads", "misa_score_topk",
            "misa_route_score_topk", "misa_pool_route_score_topk",
            "misa_pool_route_score_topk_scratch", "dsa_score_topk",
            "misa_rerank", "misa_score_topk_blocks", "misa_sparse_attention",
            "misa_workspace_bytes", "misa_candidate_flags_offset", "misa_status_string",
            "misa_last_hip_error", "misa_profile_begin", "misa_profile_end", "misa_kernel_name")


class MisaLibraryMissing(ImportError):
    pass


class MisaError(RuntimeError):
    def __init__(self, fn, status):
        msg = lib().misa_status_string(status).decode()
        if status == 5:
            msg += f" (hipError {lib().misa_last_hip_error()})"
        super().__init__(f"{fn}: {msg} [status {status}]")
        self.status = status


_lib = None


def lib():
    """The loaded libmisa.so (raises MisaLibraryMissing if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise MisaLibraryMissing(
            f"{LIB_PATH} is not built; run `python -m long_context_mean_amd.build_lib`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    # k k_scale k_dt block_table page_size
    KEYS = [P, P, I32, P, I32]
    L.misa_pool_keys.argtypes = KEYS + [I32] * 4 + [P, P]
    L.misa_pool_update.argtypes = KEYS + [I32] * 4 + [P, P, I32, P, P]
    # q q_dt q_scale w [kbar] <keys> q_seq q_pos [heads | cand] sizes... outputs ws ws_bytes stream
    L.misa_route_heads.argtypes = [P, I32, P, P, P] + KEYS + [P, P] + [I32] * 7 + [P, P, P, SZ, P]
    L.misa_score_topk.argtypes = [P, I32, P, P] + KEYS + [P, P, P] + [I32] * 7 + [P, P, P, SZ, P]
    L.misa_route_score_topk.argtypes = ([P, I32, P, P, P] + KEYS + [P, P] + [I32] * 8 +
                                        [P, P, P, P, P, SZ, P])
    # ... kbar <keys> q_seq q_pos len_old len_new max_new N S L d B H_I h topk ...
    L.misa_pool_route_score_topk.argtypes = ([P, I32, P, P, P] + KEYS + [P, P, P, P] +
                                             [I32] * 9 + [P, P, P, P, P, SZ, P])
    L.misa_pool_route_score_topk_scratch.argtypes = ([P, I32, P, P, P] + KEYS + [P, P, P, P] +
                                                     [I32] * 9 + [P, P, P, P, P])
    L.dsa_score_topk.argtypes = [P, I32, P, P] + KEYS + [P, P] + [I32] * 6 + [P, P, P, SZ, P]
    L.misa_rerank.argtypes = [P, I32, P, P] + KEYS + [P, P, P] + [I32] * 7 + [P, P, P, SZ, P]
    L.misa_score_topk_blocks.argtypes = [P, I32, P, P, P] + KEYS + [P, P, P] + [I32] * 9 + \
        [P, P, P, P, SZ, P]
    L.misa_sparse_attention.argtypes = [P, I32, P, I32, P, I32, P, P] + [I32] * 7 + \
        [ctypes.c_float, P, P, P, SZ, P]
    L.misa_workspace_bytes.argtypes = [I32] * 9
    L.misa_workspace_bytes.restype = ctypes.c_size_t
    L.misa_candidate_flags_offset.argtypes = [I32] * 3
    L.misa_candidate_flags_offset.restype = ctypes.c_int64
    L.misa_status_string.argtypes = [I32]
    L.misa_status_string.restype = ctypes.c_char_p
    L.misa_last_hip_error.argtypes = []
    L.misa_profile_begin.argtypes = [I32]
    L.misa_profile_end.argtypes = [P, P, I32]
    L.misa_kernel_name.argtypes = [I32]
    L.misa_kernel_name.restype = ctypes.c_char_p
    for f in ("misa_score_topk_blocks", "misa_sparse_attention", "misa_pool_keys", "misa_pool_update", "misa_route_heads", "misa_score_topk", "misa_route_score_topk", "misa_pool_route_score_topk", "misa_pool_route_score_topk_scratch", "dsa_score_topk",
              "misa_rerank", "misa_last_hip_error", "misa_profile_begin", "misa_profile_end"):
        getattr(L, f).restype = ctypes.c_int32
    _lib = L
    return L


# ---------------------------------------------------------------- marshalling helpers
def _ptr(t: Optional[torch.Tensor], name: str = "tensor", dtypes=None, shape=None):
    """Device pointer of a contiguous GPU tensor (None passes through).  The
    library reads and writes raw memory, so layout mistakes are caught here."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


_F32 = (torch.float32,)
_I32 = (torch.int32,)
_KEYS = (torch.float32, torch.bfloat16, torch.int16, torch.uint8, torch.float8_e4m3fn)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MISA_F32
    if t.dtype in (torch.bfloat16, torch.int16):
        return MISA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return MISA_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check(fn, status):
    if status != MISA_OK:
        raise MisaError(fn, status)


def _keys(k, k_scale, block_table, page_size, L=None, d_q=None):
    """(S, L, d) of the key storage and its pointer arguments (k, k_scale,
    k_dt, block_table, page_size).  Contiguous keys are [S, L, d]; paged keys
    are a page pool [P, page_size, d] with block_table [S, pages per sequence]
    (L defaults to pages per sequence * page_size)."""
    if d_q is not None and k.shape[-1] != d_q:
        raise ValueError(f"q has d={d_q} but k has d={k.shape[-1]}")
    if block_table is None:
        if page_size:
            raise ValueError("page_size given without a block table")
        S, L, d = k.shape
        return S, L, d, [_ptr(k, "k", _KEYS), _ptr(k_scale, "k_scale", _F32, (S, L)),
                         _dtype_code(k), None, 0]
    P, ps, d = k.shape
    if ps != page_size:
        raise ValueError(f"k pages hold {ps} tokens, page_size is {page_size}")
    S, mp = block_table.shape
    L = mp * page_size if L is None else L
    if -(-L // page_size) != mp:
        raise ValueError(f"block table has {mp} pages per sequence, L={L} needs {-(-L // page_size)}")
    return S, L, d, [_ptr(k, "k", _KEYS), _ptr(k_scale, "k_scale", _F32, (P, page_size)),
                     _dtype_code(k), _ptr(block_table, "block_table", _I32, (S, mp)), page_size]


def workspace(op: int, N: int, L: int, d: int, H_I: int, B: int = 1, topk: int = 1,
              k_prime: int = 0, q_dt: int = MISA_BF16, device="cuda") -> torch.Tensor:
    n = misa_workspace_bytes(op, q_dt, N, L, d, H_I, B, topk, k_prime)
    if n == 0:
        raise ValueError(f"no workspace size for op {op} at N={N} L={L} d={d} H_I={H_I} "
                         f"B={B} topk={topk} k_prime={k_prime} q_dt={q_dt}")
    return torch.empty(n, dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- the C entry points
def misa_workspace_bytes(op, q_dt, N, L, d, H_I, B=1, topk=1, k_prime=0) -> int:
    return int(lib().misa_workspace_bytes(op, q_dt, N, L, d, H_I, B, topk, k_prime))


def misa_candidate_flags_offset(N, L, topk) -> int:
    """Byte offset of the candidate path's per-row fallback flags in a score
    workspace, or -1 when calls at these sizes do not take that path."""
    return int(lib().misa_candidate_flags_offset(N, L, topk))


def misa_pool_keys(k: torch.Tensor, B: int, k_scale: Optional[torch.Tensor] = None,
                   kbar: Optional[torch.Tensor] = None, block_table=None, page_size=0,
                   L=None) -> torch.Tensor:
    S, L, d, kargs = _keys(k, k_scale, block_table, page_size, L)
    M = -(-L // B)
    if kbar is None:
        kbar = torch.empty((S, M, d), dtype=torch.float32, device=k.device)
    _check("misa_pool_keys", lib().misa_pool_keys(
        *kargs, S, L, d, B, _ptr(kbar, "kbar", _F32, (S, M, d)), _stream(k)))
    return kbar


def misa_pool_update(k: torch.Tensor, B: int, len_old: torch.Tensor, len_new: torch.Tensor,
                     max_new: int, kbar: torch.Tensor, k_scale=None, block_table=None,
                     page_size=0, L=None) -> torch.Tensor:
    S, L, d, kargs = _keys(k, k_scale, block_table, page_size, L)
    M = -(-L // B)
    _check("misa_pool_update", lib().misa_pool_update(
        *kargs, S, L, d, B, _ptr(len_old, "len_old", _I32, (S,)),
        _ptr(len_new, "len_new", _I32, (S,)), max_new, _ptr(kbar, "kbar", _F32, (S, M, d)),
        _stream(k)))
    return kbar


def misa_route_heads(q, w, kbar, k, q_seq, q_pos, B: int, h: int, k_scale=None, heads=None,
                     head_score=None, ws=None, want_scores=True, q_scale=None, block_table=None,
                     page_size=0, L=None):
    N, H_I, d = q.shape
    S, L, _, kargs = _keys(k, k_scale, block_table, page_size, L, d_q=d)
    if heads is None:
        heads = torch.empty((N, h), dtype=torch.int32, device=q.device)
    if head_score is None and want_scores:
        head_score = torch.empty((N, H_I), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = workspace(MISA_OP_ROUTE, N, L, d, H_I, B, q_dt=_dtype_code(q), device=q.device)
    _check("misa_route_heads", lib().misa_route_heads(
        _ptr(q, "q", _KEYS), _dtype_code(q), _ptr(q_scale, "q_scale", _F32, (N, H_I)),
        _ptr(w, "w", _F32, (N, H_I)), _ptr(kbar, "kbar", _F32, (S, -(-L // B), d)), *kargs,
        _ptr(q_seq, "q_seq", _I32, (N,)), _ptr(q_pos, "q_pos", _I32, (N,)), N, S, L, d, B, H_I, h,
        _ptr(heads, "heads", _I32, (N, h)), _ptr(head_score, "head_score", _F32, (N, H_I)),
        _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(q)))
    return heads, head_score


def misa_score_topk(q, w, k, q_seq, q_pos, heads, topk: int, k_scale=None, idx=None, score=None,
                    ws=None, want_score=True, q_scale=None, block_table=None, page_size=0,
                    L=None):
    N, H_I, d = q.shape
    S, L, _, kargs = _keys(k, k_scale, block_table, page_size, L, d_q=d)
    h = heads.shape[1]
    if idx is None:
        idx = torch.empty((N, topk), dtype=torch.int32, device=q.device)
    if score is None and want_score:
        score = torch.empty((N, topk), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = workspace(MISA_OP_SCORE_TOPK, N, L, d, H_I, topk=topk, q_dt=_dtype_code(q),
                       device=q.device)
    _check("misa_score_topk", lib().misa_score_topk(
        _ptr(q, "q", _KEYS), _dtype_code(q), _ptr(q_scale, "q_scale", _F32, (N, H_I)),
        _ptr(w, "w", _F32, (N, H_I)), *kargs, _ptr(q_seq, "q_seq", _I32, (N,)),
        _ptr(q_pos, "q_pos", _I32, (N,)), _ptr(heads, "heads", _I32, (N, h)), N, S, L, d, H_I, h,
        topk, _ptr(idx, "idx", _I32, (N, topk)), _ptr(score, "score", _F32, (N, topk)),
        _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(q)))
    return idx, score


def misa_route_score_topk(q, w, kbar, k, q_seq, q_pos, B: int, h: int, topk: int,
                          k_scale=None, heads=None, head_score=None, idx=None, score=None,
                          ws=None, want_scores=True, want_score=True, q_scale=None,
                          block_table=None, page_size=0, L=None):
    N, H_I, d = q.shape
    S, L, _, kargs = _keys(k, k_scale, block_table, page_size, L, d_q=d)
    if heads is None:
        heads = torch.empty((N, h), dtype=torch.int32, device=q.device)
    if head_score is None and want_scores:
        head_score = torch.empty((N, H_I), dtype=torch.float32, device=q.device)
    if idx is None:
        idx = torch.empty((N, topk), dtype=torch.int32, device=q.device)
    if score is None and want_score:
        score = torch.empty((N, topk), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = workspace(MISA_OP_ROUTE_SCORE_TOPK, N, L, d, H_I, B, topk=topk,
                       q_dt=_dtype_code(q), device=q.device)
    _check("misa_route_score_topk", lib().misa_route_score_topk(
        _ptr(q, "q", _KEYS), _dtype_code(q), _ptr(q_scale, "q_scale", _F32, (N, H_I)),
        _ptr(w, "w", _F32, (N, H_I)), _ptr(kbar, "kbar", _F32, (S, -(-L // B), d)), *kargs,
        _ptr(q_seq, "q_seq", _I32, (N,)), _ptr(q_pos, "q_pos", _I32, (N,)), N, S, L, d, B, H_I, h,
        topk, _ptr(heads, "heads", _I32, (N, h)), _ptr(head_score, "head_score", _F32, (N, H_I)),
        _ptr(idx, "idx", _I32, (N, topk)), _ptr(score, "score", _F32, (N, topk)),
        _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(q)))
    return heads, head_score, idx, score


def misa_pool_route_score_topk(q, w, kbar, k, q_seq, q_pos, len_old, len_new, max_new: int,
                               B: int, h: int, topk: int, k_scale=None, heads=None,
                               head_score=None, idx=None, score=None, ws=None, want_scores=True,
                               want_score=True, q_scale=None, block_table=None, page_size=0,
                               L=None):
    N, H_I, d = q.shape
    S, L, _, kargs = _keys(k, k_scale, block_table, page_size, L, d_q=d)
    if heads is None:
        heads = torch.empty((N, h), dtype=torch.int32, device=q.device)
    if head_score is None and want_scores:
        head_score = torch.empty((N, H_I), dtype=torch.float32, device=q.device)
    if idx is None:
        idx = torch.empty((N, topk), dtype=torch.int32, device=q.device)
    if score is None and want_score:
        score = torch.empty((N, topk), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = workspace(MISA_OP_ROUTE_SCORE_TOPK, N, L, d, H_I, B, topk=topk,
                       q_dt=_dtype_code(q), device=q.device)
    _check("misa_pool_route_score_topk", lib().misa_pool_route_score_topk(
        _ptr(q, "q", _KEYS), _dtype_code(q), _ptr(q_scale, "q_scale", _F32, (N, H_I)),
        _ptr(w, "w", _F32, (N, H_I)), _ptr(kbar, "kbar", _F32, (S, -(-L // B), d)), *kargs,
        _ptr(q_seq, "q_seq", _I32, (N,)), _ptr(q_pos, "q_pos", _I32, (N,)),
        _ptr(len_old, "len_old", _I32, (S,)), _ptr(len_new, "len_new", _I32, (S,)), max_new,
        N, S, L, d, B, H_I, h, topk, _ptr(heads, "heads", _I32, (N, h)),
        _ptr(head_score, "head_score", _F32, (N, H_I)), _ptr(idx, "idx", _I32, (N, topk)),
        _ptr(score, "score", _F32, (N, topk)), _ptr(ws, "ws"), ws.numel() * ws.element_size(),
        _stream(q)))
    return kbar, heads, head_score, idx, score


def misa_pool_route_score_topk_scratch(q, w, kbar, k, q_seq, q_pos, len_old, len_new,
                                       max_new: int, B: int, h: int, topk: int, k_scale=None,
                                       heads=None, head_score=None, idx=None, score=None,
                                       want_scores=True, want_score=True, q_scale=None,
                                       block_table=None, page_size=0, L=None):
    """misa_pool_route_score_topk on the library's static device scratch (no
    workspace argument).  Returns (kbar, heads, head_score, idx, score)."""
    N, H_I, d = q.shape
    S, L, _, kargs = _keys(k, k_scale, block_table, page_size, L, d_q=d)
    if heads is None:
        heads = torch.empty((N, h), dtype=torch.int32, device=q.device)
    if head_score is None and want_scores:
        head_score = torch.empty((N, H_I), dtype=torch.float32, device=q.device)
    if idx is None:
        idx = torch.empty((N, topk), dtype=torch.int32, device=q.device)
    if score is None and want_score:
        score = torch.empty((N, topk), dtype=torch.float32, device=q.device)
    _check("misa_pool_route_score_topk_scratch", lib().misa_pool_route_score_topk_scratch(
        _ptr(q, "q", _KEYS), _dtype_code(q), _ptr(q_scale, "q_scale", _F32, (N, H_I)),
        _ptr(w, "w", _F32, (N, H_I)), _ptr(kbar, "kbar", _F32, (S, -(-L // B), d)), *kargs,
        _ptr(q_seq, "q_seq", _I32, (N,)), _ptr(q_pos, "q_pos", _I32, (N,)),
        _ptr(len_old, "len_old", _I32, (S,)), _ptr(len_new, "len_new", _I32, (S,)), max_new,
        N, S, L, d, B, H_I, h, topk, _ptr(heads, "heads", _I32, (N, h)),
        _ptr(head_score, "head_score", _F32, (N, H_I)), _ptr(idx, "idx", _I32, (N, topk)),
        _ptr(score, "score", _F32, (N, topk)), _stream(q)))
    return kbar, heads, head_score, idx, score


def dsa_score_topk(q, w, k, q_seq, q_pos, topk: int, k_scale=None, idx=None, score=None,
                   ws=None, want_score=True, q_scale=None, block_table=None, page_size=0,
                   L=None):
    N, H_I, d = q.shape
    S, L, _, kargs = _keys(k, k_scale, block_table, page_size, L, d_q=d)
    if idx is None:
        idx = torch.empty((N, topk), dtype=torch.int32, device=q.device)
    if score is None and want_score:
        score = torch.empty((N, topk), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = workspace(MISA_OP_SCORE_TOPK, N, L, d, H_I, topk=topk, q_dt=_dtype_code(q),
                       device=q.device)
    _check("dsa_score_topk", lib().dsa_score_topk(
        _ptr(q, "q", _KEYS), _dtype_code(q), _ptr(q_scale, "q_scale", _F32, (N, H_I)),
        _ptr(w, "w", _F32, (N, H_I)), *kargs, _ptr(q_seq, "q_seq", _I32, (N,)),
        _ptr(q_pos, "q_pos", _I32, (N,)), N, S, L, d, H_I, topk,
        _ptr(idx, "idx", _I32, (N, topk)), _ptr(score, "score", _F32, (N, topk)), _ptr(ws, "ws"),
        ws.numel() * ws.element_size(),
        _stream(q)))
    return idx, score


def misa_rerank(q, w, k, q_seq, q_pos, cand, topk: int, k_scale=None, idx=None, score=None,
                ws=None, want_score=True, q_scale=None, block_table=None, page_size=0, L=None):
    N, H_I, d = q.shape
    S, L, _, kargs = _keys(k, k_scale, block_table, page_size, L, d_q=d)
    k_prime = cand.shape[1]
    if idx is None:
        idx = torch.empty((N, topk), dtype=torch.int32, device=q.device)
    if score is None and want_score:
        score = torch.empty((N, topk), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = workspace(MISA_OP_RERANK, N, L, d, H_I, topk=topk, k_prime=k_prime,
                       q_dt=_dtype_code(q), device=q.device)
    _check("misa_rerank", lib().misa_rerank(
        _ptr(q, "q", _KEYS), _dtype_code(q), _ptr(q_scale, "q_scale", _F32, (N, H_I)),
        _ptr(w, "w", _F32, (N, H_I)), *kargs, _ptr(q_seq, "q_seq", _I32, (N,)),
        _ptr(q_pos, "q_pos", _I32, (N,)), _ptr(cand, "cand", _I32, (N, k_prime)), N, S, L, d,
        H_I, k_prime, topk, _ptr(idx, "idx", _I32, (N, topk)),
        _ptr(score, "score", _F32, (N, topk)), _ptr(ws, "ws"), ws.numel() * ws.element_size(),
        _stream(q)))
    return idx, score


def misa_score_topk_blocks(q, w, kbar, k, q_seq, q_pos, heads, B: int, m_blocks: int, topk: int,
                           k_scale=None, blocks=None, idx=None, score=None, ws=None,
                           want_score=True, q_scale=None, block_table=None, page_size=0, L=None):
    """Routed top-k over each row's m_blocks best blocks.  Returns (blocks, idx, score)."""
    N, H_I, d = q.shape
    S, L, _, kargs = _keys(k, k_scale, block_table, page_size, L, d_q=d)
    h = heads.shape[1]
    if blocks is None:
        blocks = torch.empty((N, m_blocks), dtype=torch.int32, device=q.device)
    if idx is None:
        idx = torch.empty((N, topk), dtype=torch.int32, device=q.device)
    if score is None and want_score:
        score = torch.empty((N, topk), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = workspace(MISA_OP_BLOCKS, N, L, d, H_I, B, topk=topk, k_prime=m_blocks,
                       q_dt=_dtype_code(q), device=q.device)
    _check("misa_score_topk_blocks", lib().misa_score_topk_blocks(
        _ptr(q, "q", _KEYS), _dtype_code(q), _ptr(q_scale, "q_scale", _F32, (N, H_I)),
        _ptr(w, "w", _F32, (N, H_I)), _ptr(kbar, "kbar", _F32, (S, -(-L // B), d)), *kargs,
        _ptr(q_seq, "q_seq", _I32, (N,)), _ptr(q_pos, "q_pos", _I32, (N,)),
        _ptr(heads, "heads", _I32, (N, h)), N, S, L, d, B, H_I, h, m_blocks, topk,
        _ptr(blocks, "blocks", _I32, (N, m_blocks)), _ptr(idx, "idx", _I32, (N, topk)),
        _ptr(score, "score", _F32, (N, topk)), _ptr(ws, "ws"), ws.numel() * ws.element_size(),
        _stream(q)))
    return blocks, idx, score


def misa_sparse_attention(q, kv, q_seq, idx, scale: float, d_v: int, out=None, lse=None, ws=None,
                          block_table=None, page_size=0, L=None):
    """Softmax attention of every head over each row's selected tokens
    (idx [N, topk], -1 = empty); values are kv[..., :d_v].  Returns (out, lse)."""
    N, H, d_qk = q.shape
    S, L, _, kargs = _keys(kv, None, block_table, page_size, L, d_q=d_qk)
    topk = idx.shape[1]
    if out is None:
        out = torch.empty((N, H, d_v), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((N, H), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = workspace(MISA_OP_ATTENTION, N, L, d_v, H, topk=topk, device=q.device)
    _check("misa_sparse_attention", lib().misa_sparse_attention(
        _ptr(q, "q", _KEYS), _dtype_code(q), kargs[0], kargs[2], kargs[3], kargs[4],
        _ptr(q_seq, "q_seq", _I32, (N,)), _ptr(idx, "idx", _I32, (N, topk)), N, S, L, H, d_qk,
        d_v, topk, float(scale), _ptr(out, "out", _F32, (N, H, d_v)),
        _ptr(lse, "lse", _F32, (N, H)), _ptr(ws, "ws"), ws.numel() * ws.element_size(),
        _stream(q)))
    return out, lse


class DeviceAttention:
    """A synth.AttentionProblem on the device (bf16 tensors); page_size > 0
    stores the cache rows as a paged cache (synth.to_pages)."""

    def __init__(self, p, device="cuda", page_size: int = 0, page_seed: int = 0):
        self.p = p

        def up(a, dtype=None):
            t = torch.from_numpy(np.ascontiguousarray(a))
            return (t.view(dtype) if dtype is not None else t).to(device)

        self.q = up(p.q.view(np.int16), torch.bfloat16)
        kv = p.kv
        self.kw = dict(L=None)
        if page_size:
            pages, _, table = synth.to_pages(kv, None, page_size, page_seed)
            kv = pages
            self.kw = dict(block_table=up(table), page_size=page_size, L=p.L)
        self.kv = up(kv.view(np.int16), torch.bfloat16)
        self.q_seq = up(p.q_seq)
        self.idx = up(p.idx)

    def run(self, idx=None, **kw):
        return misa_sparse_attention(self.q, self.kv, self.q_seq,
                                     self.idx if idx is None else idx, self.p.scale, self.p.d_v,
                                     **self.kw, **kw)


def misa_profile_begin(capacity: int):
    _check("misa_profile_begin", lib().misa_profile_begin(capacity))


def misa_profile_end(max_records: int):
    """Returns a list of (kernel_name, ms) records."""
    ids = (ctypes.c_int32 * max_records)()
    ms = (ctypes.c_float * max_records)()
    n = lib().misa_profile_end(ids, ms, max_records)
    if n < 0:
        raise MisaError("misa_profile_end", -n)
    return [(lib().misa_kernel_name(ids[i]).decode(), float(ms[i])) for i in range(n)]


# ---------------------------------------------------------------- problems on the device
class DeviceProblem:
    """A synth.Problem's arrays as device tensors (q/k bf16 as torch.bfloat16,
    e4m3 codes as torch.uint8).  With page_size > 0 the keys are stored as a
    paged cache (synth.to_pages: seeded page order, spare pages) and every
    call passes the block table."""

    def __init__(self, p: synth.Problem, device="cuda", page_size: int = 0, page_seed: int = 0):
        self.p = p

        def up(a, dtype=None):
            t = torch.from_numpy(np.ascontiguousarray(a))
            if dtype is not None:
                t = t.view(dtype)
            return t.to(device)

        def keys(a):
            return up(a.view(np.int16), torch.bfloat16) if p.k_dt == synth.BF16 else up(a)

        self.q = up(p.q.view(np.int16), torch.bfloat16) if p.q_dt == synth.BF16 else up(p.q)
        self.block_table, self.page_size = None, 0
        if page_size:
            pages, spages, table = synth.to_pages(p.k, p.k_scale, page_size, page_seed)
            self.k = keys(pages)
            self.k_scale = up(spages) if spages is not None else None
            self.block_table, self.page_size = up(table), page_size
        else:
            self.k = keys(p.k)
            self.k_scale = up(p.k_scale) if p.k_scale is not None else None
        self.kv = dict(k_scale=self.k_scale, block_table=self.block_table,
                       page_size=self.page_size, L=p.L if page_size else None)
        self.w = up(p.w)
        self.q_scale = up(p.q_scale) if p.q_scale is not None else None
        self.q_seq = up(p.q_seq)
        self.q_pos = up(p.q_pos)

    def pool(self, B=None):
        return misa_pool_keys(self.k, self.p.B if B is None else B, **self.kv)

    def pool_update(self, len_old, len_new, max_new, kbar, B=None):
        return misa_pool_update(self.k, self.p.B if B is None else B, len_old, len_new, max_new,
                                kbar, **self.kv)

    def route(self, kbar, h=None, **kw):
        return misa_route_heads(self.q, self.w, kbar, self.k, self.q_seq, self.q_pos, self.p.B,
                                self.p.h if h is None else h, q_scale=self.q_scale,
                                **self.kv, **kw)

    def score_topk(self, heads, topk=None, **kw):
        return misa_score_topk(self.q, self.w, self.k, self.q_seq, self.q_pos, heads,
                               self.p.topk if topk is None else topk, q_scale=self.q_scale,
                               **self.kv, **kw)

    def route_score_topk(self, kbar, h=None, topk=None, **kw):
        return misa_route_score_topk(self.q, self.w, kbar, self.k, self.q_seq, self.q_pos,
                                     self.p.B, self.p.h if h is None else h,
                                     self.p.topk if topk is None else topk,
                                     q_scale=self.q_scale, **self.kv, **kw)

    def pool_route_score_topk(self, kbar, len_old, len_new, max_new, h=None, topk=None, **kw):
        return misa_pool_route_score_topk(self.q, self.w, kbar, self.k, self.q_seq, self.q_pos,
                                          len_old, len_new, max_new, self.p.B,
                                          self.p.h if h is None else h,
                                          self.p.topk if topk is None else topk,
                                          q_scale=self.q_scale, **self.kv, **kw)

    def pool_route_score_topk_scratch(self, kbar, len_old, len_new, max_new, h=None, topk=None,
                                      **kw):
        return misa_pool_route_score_topk_scratch(self.q, self.w, kbar, self.k, self.q_seq,
                                                  self.q_pos, len_old, len_new, max_new,
                                                  self.p.B, self.p.h if h is None else h,
                                                  self.p.topk if topk is None else topk,
                                                  q_scale=self.q_scale, **self.kv, **kw)

    def score_topk_blocks(self, kbar, heads, m_blocks, topk=None, **kw):
        return misa_score_topk_blocks(self.q, self.w, kbar, self.k, self.q_seq, self.q_pos, heads,
                                      self.p.B, m_blocks, self.p.topk if topk is None else topk,
                                      q_scale=self.q_scale, **self.kv, **kw)

    def dsa(self, topk=None, **kw):
        return dsa_score_topk(self.q, self.w, self.k, self.q_seq, self.q_pos,
                              self.p.topk if topk is None else topk, q_scale=self.q_scale,
                              **self.kv, **kw)

    def rerank(self, cand, topk=None, **kw):
        return misa_rerank(self.q, self.w, self.k, self.q_seq, self.q_pos, cand,
                           self.p.topk if topk is None else topk, q_scale=self.q_scale,
                           **self.kv, **kw)
