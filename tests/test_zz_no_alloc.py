"""misa_pool_route_score_topk_scratch (the serving step on the library's
static device scratch, for callers that cannot allocate) against
misa_pool_route_score_topk with a caller workspace: every output bit for bit,
over two calls in a row, the second on a smaller problem (the scratch keeps
the first call's contents)."""
import numpy as np
import pytest
import torch

from long_context_mean_amd import synth
from long_context_mean_amd.binding import DeviceProblem

pytestmark = pytest.mark.gpu


def _np(t):
    torch.cuda.synchronize()
    return None if t is None else t.cpu().numpy()


def _stale_table(dp, len_old, len_new):
    p = dp.p
    table = dp.pool()
    for s in range(p.S):
        table[s, len_old[s] // p.B:len_new[s] // p.B] = 0.0
    return table


@pytest.mark.parametrize("k_dt", [synth.BF16, synth.FP8])
def test_scratch_step_matches_workspace_step(k_dt):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    problems = [
        synth.make("c4") if k_dt == synth.BF16 else synth.make("c5"),
        synth.small("scratch2", 130, N=3, S=3, L=20000, d=128, H_I=64, h=8, B=64, topk=1000,
                    k_dt=k_dt, q_pos=np.array([19999, 19000, 700], np.int32)),
    ]
    for p in problems:
        print(f"[scratch] N={p.N} L={p.L} B={p.B} k_dt={synth.DTYPE_NAMES[k_dt]}", flush=True)
        dp = DeviceProblem(p)
        len_new = (p.q_pos[p.q_seq] + 1).astype(np.int32)
        len_old = len_new - 1
        lo = torch.from_numpy(len_old).cuda()
        hi = torch.from_numpy(len_new).cuda()
        ta = _stale_table(dp, len_old, len_new)
        tb = ta.clone()
        ref = dp.pool_route_score_topk(ta, lo, hi, 1)
        got = dp.pool_route_score_topk_scratch(tb, lo, hi, 1)
        for name, a, b in zip(("table", "heads", "router scores", "idx", "score"), ref, got):
            a, b = _np(a), _np(b)
            if a.dtype == np.float32:
                a, b = a.view(np.uint32), b.view(np.uint32)
            assert np.array_equal(a, b), name


def test_scratch_step_replayed_from_a_graph():
    """The scratch serving step captured once in a HIP graph (it allocates
    nothing, so capture needs no workspace) and replayed three times, with new
    queries, weights and a reset table written eagerly between the replays:
    every replay's outputs equal an eager workspace call's bit for bit."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    p = synth.small("graph", 131, N=4, S=4, L=20000, d=128, H_I=64, h=8, B=128, topk=1000,
                    q_pos=np.array([19999, 12799, 9000, 255], np.int32))
    print(f"[graph] N={p.N} L={p.L} B={p.B}", flush=True)
    dp = DeviceProblem(p)
    len_new = (p.q_pos[p.q_seq] + 1).astype(np.int32)
    len_old = len_new - 1
    lo = torch.from_numpy(len_old).cuda()
    hi = torch.from_numpy(len_new).cuda()
    base = _stale_table(dp, len_old, len_new)
    table = base.clone()
    out = dict(heads=torch.empty((p.N, p.h), dtype=torch.int32, device="cuda"),
               head_score=torch.empty((p.N, p.H_I), dtype=torch.float32, device="cuda"),
               idx=torch.empty((p.N, p.topk), dtype=torch.int32, device="cuda"),
               score=torch.empty((p.N, p.topk), dtype=torch.float32, device="cuda"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                    # first call outside the capture
        dp.pool_route_score_topk_scratch(table, lo, hi, 1, **out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dp.pool_route_score_topk_scratch(table, lo, hi, 1, **out)
    gen = torch.Generator(device="cpu").manual_seed(131)
    for r in range(3):
        dp.q.copy_(torch.randn(dp.q.shape, generator=gen).to(torch.bfloat16))
        dp.w.copy_(torch.randn(dp.w.shape, generator=gen))
        table.copy_(base)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [_np(t) for t in (table, out["heads"], out["head_score"], out["idx"], out["score"])]
        ref = [_np(t) for t in dp.pool_route_score_topk(base.clone(), lo, hi, 1)]
        for name, a, b in zip(("table", "heads", "router scores", "idx", "score"), ref, got):
            if a.dtype == np.float32:
                a, b = a.view(np.uint32), b.view(np.uint32)
            assert np.array_equal(a, b), f"replay {r}: {name}"
        print(f"[graph] replay {r} equal to the eager call", flush=True)
