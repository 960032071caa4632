"""Comparison rules between the GPU library and the CPU oracle.

Tolerances (fp32-accumulated GPU scores vs the double-precision oracle):
  |gpu - ref| <= ATOL + RTOL * |ref|,  RTOL = 1e-3, ATOL = 1e-4.
Selections (heads, top-k sets) must be identical, except that an element may
be swapped only if its oracle value lies within that tolerance of the
boundary value (the h-th router score, the k-th token score): there the two
precisions can legitimately order near-equal values differently.  Exact
ties are not exempt: integer inputs must match bit for bit.
"""
import numpy as np

RTOL, ATOL = 1e-3, 1e-4


def tol(x):
    return ATOL + RTOL * np.abs(x)


def check_heads(gpu_heads, ref_r, h):
    """GPU head sets vs oracle router scores r [N, H_I].  Returns the number of
    rows whose sets differ (all differences near-tied)."""
    N, H_I = ref_r.shape
    differing = 0
    for n in range(N):
        g = np.asarray(gpu_heads[n])
        assert len(set(g.tolist())) == h and np.all(np.diff(g) > 0), f"row {n}: heads {g}"
        assert g.min() >= 0 and g.max() < H_I
        order = np.lexsort((np.arange(H_I), -ref_r[n]))
        ref = set(order[:h].tolist())
        if set(g.tolist()) != ref:
            differing += 1
            boundary = ref_r[n, order[h - 1]]
            for j in set(g.tolist()) ^ ref:
                assert abs(ref_r[n, j] - boundary) <= tol(boundary), (
                    f"row {n}: head {j} r={ref_r[n, j]} vs h-th {boundary}")
    return differing


def check_topk(gpu_idx, gpu_score, ref_scores, topk, lengths, exact=False, cand=None):
    """GPU top-k (ascending index order, -1 padding) vs oracle score rows.

    ref_scores [N, L] holds the oracle score of every token (-inf where not a
    candidate).  `lengths[n]` = number of eligible tokens.  With exact=True
    the set must be identical and scores bit-equal to the oracle value."""
    N = gpu_idx.shape[0]
    swapped = 0
    for n in range(N):
        K = min(topk, int(lengths[n]))
        gi = np.asarray(gpu_idx[n])
        assert np.all(gi[K:] == -1), f"row {n}: padding {gi[K:][:8]}"
        if gpu_score is not None:
            assert np.all(np.isneginf(gpu_score[n][K:]))
        sel = gi[:K]
        assert np.all(sel >= 0), f"row {n}: fewer than {K} selected"
        assert np.all(np.diff(sel) > 0), f"row {n}: not strictly ascending"
        sc = ref_scores[n]
        elig = np.nonzero(~np.isneginf(sc))[0] if cand is None else np.asarray(cand[n])
        elig = elig[elig >= 0]
        assert np.all(np.isin(sel, elig)), f"row {n}: selected non-eligible token"
        order = elig[np.lexsort((elig, -sc[elig]))]
        ref = order[:K]
        kth = sc[ref[-1]]
        if exact:
            assert np.array_equal(np.sort(ref), sel), f"row {n}: set differs"
        else:
            diff = set(sel.tolist()) ^ set(ref.tolist())
            for t in diff:
                assert abs(sc[t] - kth) <= tol(kth), (
                    f"row {n}: token {t} score {sc[t]} vs k-th {kth}")
            swapped += len(diff) // 2
        if gpu_score is not None:
            gs = np.asarray(gpu_score[n][:K], dtype=np.float64)
            if exact:
                assert np.array_equal(gs, sc[sel]), f"row {n}: scores differ"
            else:
                err = np.abs(gs - sc[sel])
                bad = err > tol(sc[sel])
                assert not bad.any(), (
                    f"row {n}: score {gs[bad][:4]} vs {sc[sel][bad][:4]}")
    return swapped


def recall(a_idx, b_idx):
    """Mean fraction of b's selected tokens that a selects (rows, -1 ignored)."""
    rs = []
    for a, b in zip(a_idx, b_idx):
        b = set(int(x) for x in b if x >= 0)
        a = set(int(x) for x in a if x >= 0)
        rs.append(len(a & b) / max(1, len(b)))
    return float(np.mean(rs))
