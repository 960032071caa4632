"""CPU-side checks of the C ABI: the library loads, exports every entry point
declared in include/misa.h, and rejects invalid arguments before touching the
GPU (every call here returns at validation, so no device is needed)."""
import ctypes
import os
import re

import pytest

from long_context_mean_amd import binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "misa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for f in ("misa_pool_keys", "misa_route_heads", "misa_score_topk", "misa_rerank",
              "dsa_score_topk", "misa_workspace_bytes", "misa_status_string"):
        assert f in names


def test_library_exports_every_declared_symbol():
    lib = b.lib()
    for f in declared_functions():
        assert hasattr(lib, f), f"{f} not exported"
    assert set(b.EXPORTED) <= set(declared_functions())


def test_status_strings():
    lib = b.lib()
    for s in range(6):
        assert lib.misa_status_string(s)
    assert lib.misa_status_string(99) == b"unknown status"


def test_workspace_sizes():
    lib = b.lib()
    ws = lambda *a: lib.misa_workspace_bytes(*a)
    BF, F8 = b.MISA_BF16, b.MISA_FP8_E4M3
    # decode shape: order keys + 3 histogram levels + per-chunk counts
    n = ws(b.MISA_OP_SCORE_TOPK, BF, 4, 131072, 128, 64, 128, 2048, 0)
    assert n >= 4 * 131072 * 4
    assert ws(b.MISA_OP_SCORE_TOPK, BF, 4096, 65536, 128, 64, 128, 2048, 0) >= 4096 * 65536 * 4
    assert ws(b.MISA_OP_RERANK, BF, 4, 131072, 128, 64, 128, 2048, 8192) >= 4 * 8192 * 4
    assert ws(b.MISA_OP_ROUTE, BF, 4, 131072, 128, 64, 128, 2048, 0) >= 4 * 32 * 64 * 4
    assert ws(b.MISA_OP_SCORE_TOPK, BF, 0, 100, 128, 64, 128, 10, 0) == 0
    assert ws(b.MISA_OP_ROUTE, BF, 1, 100, 128, 64, 0, 10, 0) == 0
    assert ws(7, BF, 1, 100, 128, 64, 1, 10, 0) == 0
    assert ws(b.MISA_OP_SCORE_TOPK, 3, 4, 100, 128, 64, 1, 10, 0) == 0       # unknown q dtype
    assert ws(b.MISA_OP_SCORE_TOPK, BF, 4, 100, 96, 64, 1, 10, 0) == 0       # d
    # fp8 queries: + bf16 copies (2d bytes) and folded weights (4 bytes) per head row
    for op in (b.MISA_OP_ROUTE, b.MISA_OP_SCORE_TOPK, b.MISA_OP_RERANK):
        for N, L in ((4, 131072), (4096, 65536)):
            extra = ws(op, F8, N, L, 128, 64, 128, 2048, 8192) - ws(op, BF, N, L, 128, 64, 128,
                                                                    2048, 8192)
            assert N * 64 * (2 * 128 + 4) <= extra < N * 64 * (2 * 128 + 4) + 512


FAKE = ctypes.c_void_p(0x100000)        # aligned, never dereferenced: validation fails first


def _score(**over):
    a = dict(q=FAKE, q_dt=1, qsc=None, w=FAKE, k=FAKE, ks=None, k_dt=1, bt=None, ps=0, qs=FAKE,
             qp=FAKE, heads=FAKE, N=4, S=4, L=1000, d=128, H_I=64, h=8, topk=100, idx=FAKE,
             score=None, ws=FAKE, ws_bytes=1 << 30)
    a.update(over)
    return b.lib().misa_score_topk(a["q"], a["q_dt"], a["qsc"], a["w"], a["k"], a["ks"], a["k_dt"],
                                   a["bt"], a["ps"],
                                   a["qs"], a["qp"], a["heads"], a["N"], a["S"], a["L"], a["d"],
                                   a["H_I"], a["h"], a["topk"], a["idx"], a["score"], a["ws"],
                                   a["ws_bytes"], None)


@pytest.mark.parametrize("over,status", [
    (dict(q=None), 1), (dict(heads=None), 1), (dict(idx=None), 1), (dict(ws=None), 1),
    (dict(k_dt=2), 1),                                   # fp8 keys without scale
    (dict(q_dt=0), 3), (dict(d=96), 3),
    (dict(q_dt=2, k_dt=1), 3),                           # fp8 queries need fp8 keys
    (dict(q_dt=2, k_dt=2, ks=FAKE), 1),                  # fp8 queries without scale
    (dict(q_dt=2, k_dt=2, ks=FAKE, qsc=FAKE, ws_bytes=4 * 1000 * 4 + 4096), 4),
    (dict(h=0), 2), (dict(h=65), 2), (dict(H_I=65, h=8), 2), (dict(topk=0), 2),
    (dict(N=0), 2), (dict(L=0), 2), (dict(S=0), 2), (dict(N=70000), 2),
    (dict(q=ctypes.c_void_p(0x100004)), 2),              # misaligned
    (dict(ws_bytes=16), 4),
    (dict(ps=64), 1),                                    # paged keys without a block table
    (dict(bt=FAKE), 2),                                  # block table with page_size 0
    (dict(bt=FAKE, ps=48), 2), (dict(bt=FAKE, ps=8), 2), (dict(bt=FAKE, ps=1 << 17), 2),
])
def test_score_topk_rejects(over, status):
    assert _score(**over) == status


def test_rerank_and_route_and_pool_reject():
    lib = b.lib()
    # k_prime < topk
    KV = (FAKE, None, 1, None, 0)            # contiguous bf16 keys
    assert lib.misa_rerank(FAKE, 1, None, FAKE, *KV, FAKE, FAKE, FAKE, 4, 4, 1000, 128,
                           64, 100, 200, FAKE, None, FAKE, 1 << 30, None) == 2
    # fp8 queries without their scale
    KV8 = (FAKE, FAKE, 2, None, 0)
    assert lib.misa_rerank(FAKE, 2, None, FAKE, *KV8, FAKE, FAKE, FAKE, 4, 4, 1000, 128,
                           64, 200, 100, FAKE, None, FAKE, 1 << 30, None) == 1
    # fp8 queries: the bf16 copies need room past the rerank's own workspace
    own = lib.misa_workspace_bytes(b.MISA_OP_RERANK, 1, 4, 1000, 128, 64, 1, 100, 200)
    assert lib.misa_rerank(FAKE, 2, FAKE, FAKE, *KV8, FAKE, FAKE, FAKE, 4, 4, 1000, 128,
                           64, 200, 100, FAKE, None, FAKE, own, None) == 4
    # paged keys: page size not a power of two
    assert lib.misa_rerank(FAKE, 1, None, FAKE, FAKE, None, 1, FAKE, 100, FAKE, FAKE, FAKE, 4, 4,
                           1000, 128, 64, 200, 100, FAKE, None, FAKE, 1 << 30, None) == 2
    # B out of range
    assert lib.misa_route_heads(FAKE, 1, None, FAKE, FAKE, *KV, FAKE, FAKE, 4, 4, 1000,
                                128, 2048, 64, 8, FAKE, None, FAKE, 1 << 30, None) == 2
    # workspace too small
    assert lib.misa_route_heads(FAKE, 1, None, FAKE, FAKE, *KV, FAKE, FAKE, 4, 4,
                                100000, 128, 128, 64, 8, FAKE, None, FAKE, 8, None) == 4
    own = lib.misa_workspace_bytes(b.MISA_OP_ROUTE, 1, 4, 100000, 128, 64, 128, 1, 0)
    assert lib.misa_route_heads(FAKE, 2, FAKE, FAKE, FAKE, *KV8, FAKE, FAKE, 4, 4,
                                100000, 128, 128, 64, 8, FAKE, None, FAKE, own, None) == 4
    # paged route without a block table
    assert lib.misa_route_heads(FAKE, 1, None, FAKE, FAKE, FAKE, None, 1, None, 64, FAKE, FAKE, 4,
                                4, 1000, 128, 128, 64, 8, FAKE, None, FAKE, 1 << 30, None) == 1
    assert lib.misa_pool_keys(None, None, 1, None, 0, 1, 100, 128, 16, FAKE, None) == 1
    assert lib.misa_pool_keys(FAKE, None, 2, None, 0, 1, 100, 128, 16, FAKE, None) == 1
    assert lib.misa_pool_keys(FAKE, None, 5, None, 0, 1, 100, 128, 16, FAKE, None) == 3
    assert lib.misa_pool_keys(FAKE, None, 1, None, 0, 1, 100, 128, 0, FAKE, None) == 2
    assert lib.misa_pool_keys(FAKE, None, 1, FAKE, 24, 1, 100, 128, 16, FAKE, None) == 2
    # incremental pooling: length arrays required, 0 <= max_new <= L
    upd = lib.misa_pool_update
    assert upd(FAKE, None, 1, None, 0, 2, 100, 128, 16, None, FAKE, 1, FAKE, None) == 1
    assert upd(FAKE, None, 1, None, 0, 2, 100, 128, 16, FAKE, FAKE, -1, FAKE, None) == 2
    assert upd(FAKE, None, 1, None, 0, 2, 100, 128, 16, FAKE, FAKE, 101, FAKE, None) == 2
    assert upd(FAKE, None, 1, FAKE, 0, 2, 100, 128, 16, FAKE, FAKE, 1, FAKE, None) == 2
    assert upd(FAKE, None, 1, None, 0, 2, 100, 128, 16, FAKE, FAKE, 0, FAKE, None) == 0  # no-op


def _route_score(**over):
    a = dict(q=FAKE, q_dt=1, qsc=None, w=FAKE, kbar=FAKE, k=FAKE, ks=None, k_dt=1, bt=None, ps=0,
             qs=FAKE, qp=FAKE, N=4, S=4, L=1000, d=128, B=128, H_I=64, h=8, topk=100,
             heads=FAKE, hs=None, idx=FAKE, score=None, ws=FAKE, ws_bytes=1 << 30)
    a.update(over)
    return b.lib().misa_route_score_topk(
        a["q"], a["q_dt"], a["qsc"], a["w"], a["kbar"], a["k"], a["ks"], a["k_dt"], a["bt"],
        a["ps"], a["qs"], a["qp"], a["N"], a["S"], a["L"], a["d"], a["B"], a["H_I"], a["h"],
        a["topk"], a["heads"], a["hs"], a["idx"], a["score"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("over,status", [
    (dict(q=None), 1), (dict(kbar=None), 1), (dict(heads=None), 1), (dict(idx=None), 1),
    (dict(ws=None), 1), (dict(k_dt=2), 1), (dict(q_dt=0), 3), (dict(d=96), 3),
    (dict(B=0), 2), (dict(B=2048), 2), (dict(h=0), 2), (dict(h=65), 2), (dict(topk=0), 2),
    (dict(N=0), 2), (dict(q=ctypes.c_void_p(0x100004)), 2), (dict(ps=64), 1),
    (dict(ws_bytes=16), 4),
])
def test_route_score_topk_rejects(over, status):
    assert _route_score(**over) == status


def test_route_score_topk_workspace_covers_both_steps():
    lib = b.lib()
    for q_dt, k_dt in ((1, 1), (2, 2)):
        for N, L in ((4, 131072), (4096, 65536), (3, 1000)):
            both = lib.misa_workspace_bytes(b.MISA_OP_ROUTE_SCORE_TOPK, q_dt, N, L, 128, 64, 128,
                                            2048, 0)
            route = lib.misa_workspace_bytes(b.MISA_OP_ROUTE, q_dt, N, L, 128, 64, 128, 2048, 0)
            score = lib.misa_workspace_bytes(b.MISA_OP_SCORE_TOPK, q_dt, N, L, 128, 64, 128,
                                             2048, 0)
            assert both >= route + score
            # one byte short of the size is rejected before any launch
            ks = FAKE if k_dt == 2 else None
            qsc = FAKE if q_dt == 2 else None
            assert _route_score(q_dt=q_dt, k_dt=k_dt, ks=ks, qsc=qsc, N=N, S=N, L=L,
                                topk=min(2048, L), ws_bytes=both - 1) == 4


def _pool_route_score(**over):
    a = dict(q=FAKE, q_dt=1, qsc=None, w=FAKE, kbar=FAKE, k=FAKE, ks=None, k_dt=1, bt=None, ps=0,
             qs=FAKE, qp=FAKE, lo=FAKE, hi=FAKE, max_new=1, N=4, S=4, L=1000, d=128, B=128,
             H_I=64, h=8, topk=100, heads=FAKE, hs=None, idx=FAKE, score=None, ws=FAKE,
             ws_bytes=1 << 30)
    a.update(over)
    return b.lib().misa_pool_route_score_topk(
        a["q"], a["q_dt"], a["qsc"], a["w"], a["kbar"], a["k"], a["ks"], a["k_dt"], a["bt"],
        a["ps"], a["qs"], a["qp"], a["lo"], a["hi"], a["max_new"], a["N"], a["S"], a["L"], a["d"],
        a["B"], a["H_I"], a["h"], a["topk"], a["heads"], a["hs"], a["idx"], a["score"], a["ws"],
        a["ws_bytes"], None)


# every check of both calls runs before anything is enqueued (a failing
# route/score check must not leave the table half updated)
@pytest.mark.parametrize("over,status", [
    (dict(q=None), 1), (dict(kbar=None), 1), (dict(k=None), 1), (dict(lo=None), 1),
    (dict(hi=None), 1), (dict(heads=None), 1), (dict(idx=None), 1), (dict(ws=None), 1),
    (dict(k_dt=2), 1), (dict(q_dt=0), 3), (dict(d=96), 3), (dict(B=0), 2), (dict(B=2048), 2),
    (dict(max_new=-1), 2), (dict(max_new=1001), 2), (dict(h=0), 2), (dict(h=65), 2),
    (dict(topk=0), 2), (dict(N=0), 2), (dict(q=ctypes.c_void_p(0x100004)), 2),
    (dict(ps=64), 1), (dict(ws_bytes=16), 4),
])
def test_pool_route_score_topk_rejects(over, status):
    assert _pool_route_score(**over) == status


def test_pool_route_score_topk_workspace_is_the_fused_calls():
    lib = b.lib()
    both = lib.misa_workspace_bytes(b.MISA_OP_ROUTE_SCORE_TOPK, 1, 4, 131072, 128, 64, 128, 2048,
                                    0)
    assert _pool_route_score(L=131072, topk=2048, ws_bytes=both - 1) == 4


def _param_counts():
    text = open(os.path.join(ROOT, "include", "misa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    out = {}
    for m in re.finditer(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(([^)]*)\)\s*;", text, flags=re.M):
        args = [a for a in m.group(2).split(",") if a.strip() and a.strip() != "void"]
        out[m.group(1)] = len(args)
    return out


def test_binding_argument_counts_match_header():
    lib = b.lib()
    counts = _param_counts()
    for name, n in counts.items():
        fn = getattr(lib, name)
        assert fn.argtypes is not None and len(fn.argtypes) == n, name


def test_binding_rejects_host_and_strided_tensors():
    """The binding hands raw pointers to the library: host tensors, strided
    views and wrong dtypes are refused before any call."""
    import torch
    k = torch.zeros((1, 256, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        b.misa_pool_keys(k, 128)
    q = torch.zeros((2, 4, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        b.misa_score_topk(q, torch.zeros((2, 4)), k, torch.zeros(2, dtype=torch.int32),
                          torch.zeros(2, dtype=torch.int32), torch.zeros((2, 1), dtype=torch.int32),
                          8, ws=torch.zeros(256, dtype=torch.uint8))
    with pytest.raises(ValueError, match="d="):
        b.misa_score_topk(q, torch.zeros((2, 4)), torch.zeros((1, 256, 64), dtype=torch.bfloat16),
                          torch.zeros(2, dtype=torch.int32), torch.zeros(2, dtype=torch.int32),
                          torch.zeros((2, 1), dtype=torch.int32), 8)


def test_binding_pointer_checks():
    import torch
    with pytest.raises(ValueError, match="GPU tensor"):
        b._ptr(torch.zeros((4, 4)), "t")
    with pytest.raises(ValueError, match="GPU tensor"):
        b._ptr(object(), "t")
    assert b._ptr(None, "t") is None


def test_candidate_flags_offset():
    """The prefill candidate path's row flags lie inside the score workspace
    at the sizes that take the path; other sizes report -1."""
    BF = b.MISA_BF16
    for N, L in ((4096, 65536), (4096, 131072), (128, 32768)):
        off = b.misa_candidate_flags_offset(N, L, 2048)
        ws = b.misa_workspace_bytes(b.MISA_OP_SCORE_TOPK, BF, N, L, 128, 64, 128, 2048, 0)
        assert 0 <= off and off + 4 * N <= ws and off % 256 == 0
    assert b.misa_candidate_flags_offset(4, 131072, 2048) == -1      # decode rows
    assert b.misa_candidate_flags_offset(4096, 20000, 2048) == -1    # short prefix
    assert b.misa_candidate_flags_offset(4096, 65536, 4096) == -1    # large k
    assert b.misa_candidate_flags_offset(0, 65536, 2048) == -1


def _scratch_step(**over):
    a = dict(q=FAKE, q_dt=1, qsc=None, w=FAKE, kbar=FAKE, k=FAKE, ks=None, k_dt=1, bt=None, ps=0,
             qs=FAKE, qp=FAKE, lo=FAKE, hi=FAKE, max_new=1, N=4, S=4, L=1000, d=128, B=128,
             H_I=64, h=8, topk=100, heads=FAKE, hs=None, idx=FAKE, score=None)
    a.update(over)
    return b.lib().misa_pool_route_score_topk_scratch(
        a["q"], a["q_dt"], a["qsc"], a["w"], a["kbar"], a["k"], a["ks"], a["k_dt"], a["bt"],
        a["ps"], a["qs"], a["qp"], a["lo"], a["hi"], a["max_new"], a["N"], a["S"], a["L"], a["d"],
        a["B"], a["H_I"], a["h"], a["topk"], a["heads"], a["hs"], a["idx"], a["score"], None)


# the static-scratch serving step: the same checks, before the GPU is touched
@pytest.mark.parametrize("over,status", [
    (dict(q=None), 1), (dict(kbar=None), 1), (dict(k=None), 1), (dict(lo=None), 1),
    (dict(hi=None), 1), (dict(heads=None), 1), (dict(idx=None), 1), (dict(k_dt=2), 1),
    (dict(q_dt=0), 3), (dict(d=96), 3), (dict(B=0), 2), (dict(max_new=-1), 2), (dict(h=65), 2),
    (dict(topk=0), 2), (dict(N=0), 2), (dict(q=ctypes.c_void_p(0x100004)), 2), (dict(ps=64), 1),
])
def test_scratch_serving_step_rejects(over, status):
    assert _scratch_step(**over) == status


def test_scratch_serving_step_size_limit():
    """Workspaces above the 32 MiB scratch are refused (4 rows of 2^21 keys
    need 32 MiB of order keys alone)."""
    need = b.misa_workspace_bytes(b.MISA_OP_ROUTE_SCORE_TOPK, 1, 4, 1 << 21, 128, 64, 128, 2048)
    assert need > 32 << 20
    assert _scratch_step(L=1 << 21, topk=2048, max_new=1) == 4
