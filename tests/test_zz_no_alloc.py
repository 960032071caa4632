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
