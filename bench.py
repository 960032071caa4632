"""Benchmark of the MISA routed indexer on one MI355X.

Workload (DeepSeek-V3.2-like long-context decode): 4 queries, each over its
own prefix of L = 131072 bf16 index keys (d = 128), H_I = 64 indexer heads,
h = 8 routed heads, B = 128 (M = 1024 pooled blocks), top-k = 2048, with 32
planted needle keys per query.

One step = the indexer hot path of one decode step for the batch, as a
serving loop runs it: the newest token of each sequence completes its last
pooling block, which is pooled into the cached table (incremental block
pooling), then head routing, then routed scoring + exact top-k over the whole
prefix.  Inputs are resident in HBM before timing; the timed steps rotate over
4 replicas of the keys (512 MiB in all, twice the 256 MB last-level Infinity
Cache), so every step reads keys that are not cache resident.  Timed beside
it with the same protocol: the step with a full pooling pass instead of the
incremental update (its scoring then reads keys the pooling pass has just
brought into the Infinity Cache), the same serving step on a paged key cache,
the dense 64-head DSA indexer, and MISA-dagger (coarse top-8192 + all-head
rerank) on bf16 and fp8 keys, both with a full pooling pass and in serving
form (the single call at top-8192, then the rerank call).

Prints ONE JSON line.  `value` = prefix tokens indexed per second (sum of
the visible prefix lengths per step / time per step).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefix tokens indexed/sec (L=128K, h=8 of 64) + % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
REPLICAS = 4


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--h", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--workload", default="c4", choices=["c4", "c3", "c3x", "c3f8"],
                    help="c4: the long-context decode indexer (the headline line); "
                         "c3 / c3x: the prefill chunk at L=64K / 128K; c3f8: the L=64K "
                         "chunk with e4m3 queries and keys")
    # profiling helpers (no benchmark line)
    ap.add_argument("--copy-probe", action="store_true",
                    help="run plain 256 MiB device copies (scale reference for HBM counters)")
    ap.add_argument("--summarize", metavar="DB",
                    help="print a markdown kernel table of a rocprofv3 --kernel-trace database")
    ap.add_argument("--traffic", nargs=4, metavar=("FETCH_DB", "WRITE_DB", "COPY_FETCH_DB",
                                                   "COPY_WRITE_DB"),
                    help="print the per-launch HBM traffic record of --kernel from rocprofv3 "
                         "--pmc FETCH_SIZE / WRITE_SIZE databases, scaled by the copy probe's")
    ap.add_argument("--counters", metavar="DB",
                    help="print the per-launch matrix-core counter summary of --match dispatches "
                         "from a rocprofv3 --pmc database (SQ_INSTS_MFMA, "
                         "SQ_VALU_MFMA_BUSY_CYCLES, SQ_VALU_MFMA_COEXEC_CYCLES, SQ_INSTS_VALU, "
                         "SQ_BUSY_CYCLES, SQ_WAVE_CYCLES, GRBM_GUI_ACTIVE)")
    ap.add_argument("--flop", type=float, default=None,
                    help="algorithmic flop per launch (for --counters)")
    ap.add_argument("--kernel", default="score_mfma_kernel")
    ap.add_argument("--match", default=None,
                    help="kernel-name substring selecting the dispatches (default: --kernel)")
    ap.add_argument("--title", default="")
    ap.add_argument("--cmd", default="")
    return ap.parse_args()


COPY_BYTES = 256 << 20


def copy_probe():
    import torch
    x = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "copies": 5}), flush=True)


def summarize(db, title, cmd):
    import sqlite3
    c = sqlite3.connect(db)
    rows = list(c.execute("select name, count(*), avg(end-start), min(end-start), max(end-start), "
                          "sum(end-start) from kernels group by name order by sum(end-start) desc"))
    tot = sum(r[5] for r in rows)
    out = [f"# {title}", "", "Command (from the repository root, on one MI355X):", "", "```", cmd,
           "```", "", "| kernel | calls | avg us | min us | max us | share |",
           "|---|---|---|---|---|---|"]
    for name, n, avg, mn, mx, sm in rows:
        short = name.replace("misa::(anonymous namespace)::", "").split("(")[0]
        out.append(f"| `{short}` | {n} | {avg / 1000:.2f} | {mn / 1000:.2f} | {mx / 1000:.2f} "
                   f"| {100 * sm / tot:.1f}% |")
    print("\n".join(out))


def _counter_per_dispatch(db, counter, name_part):
    """Mean value of `counter` per dispatch of kernels whose name contains name_part."""
    import sqlite3
    c = sqlite3.connect(db)
    rows = c.execute("select dispatch_id, kernel_name, value from counters_collection "
                     "where counter_name = ?", (counter,)).fetchall()
    per = {}
    for did, kn, v in rows:
        if name_part in kn:
            per[did] = per.get(did, 0.0) + v
    return sum(per.values()) / len(per) if per else None


# source files whose text defines each measured kernel
KERNEL_SOURCES = {
    "score_mfma_kernel": ["score.hip", "route_select.hpp", "partial_block.hpp"],
    "pool_kernel": ["pool.hip", "pool_block.hpp"],
    "score_prefill_kernel": ["prefill.hip"],
}


def kernel_source_sha(kernel):
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "long_context_mean_amd", "csrc")
    for f in KERNEL_SOURCES.get(kernel, []) + ["common.hpp"]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_record(fetch_db, write_db, copy_fetch_db, copy_write_db, kernel, match, cmd):
    copy_name = "copyBuffer"
    kf = _counter_per_dispatch(fetch_db, "FETCH_SIZE", match)
    kw = _counter_per_dispatch(write_db, "WRITE_SIZE", match)
    cf = _counter_per_dispatch(copy_fetch_db, "FETCH_SIZE", copy_name)
    cw = _counter_per_dispatch(copy_write_db, "WRITE_SIZE", copy_name)
    # counters read KiB; the copy moves COPY_BYTES each way
    sf = COPY_BYTES / (cf * 1024.0)
    sw = COPY_BYTES / (cw * 1024.0)
    return {"kernel": kernel, "dispatches": match, "source_sha256": kernel_source_sha(kernel),
            "fetch_kib_per_launch": kf, "write_kib_per_launch": kw,
            "copy_fetch_kib": cf, "copy_write_kib": cw, "scale_fetch": sf, "scale_write": sw,
            "fetch_bytes_per_launch": kf * 1024.0 * sf, "write_bytes_per_launch": kw * 1024.0 * sw,
            "traffic_bytes_per_launch": (kf * 1024.0 * sf + kw * 1024.0 * sw), "command": cmd}


def counter_record(db, match, flop, cmd, mfma_flop=16384, simds=1024, xcds=8):
    """Matrix-core counters per launch of the dispatches whose kernel name
    contains `match`: the rocprofv3 values are sums over the chip (per-SE or
    per-SIMD counters added up; GRBM_GUI_ACTIVE once per XCD), averaged over
    the dispatches."""
    import sqlite3
    c = sqlite3.connect(db)
    rows = c.execute("select dispatch_id, kernel_name, counter_name, value, duration "
                     "from counters_collection").fetchall()
    per, dur, name = {}, {}, None
    for did, kn, cn, v, d in rows:
        if match in kn:
            per.setdefault(did, {})
            per[did][cn] = per[did].get(cn, 0.0) + v
            dur[did] = d
            name = kn
    if not per:
        return None
    keys = sorted({k for v in per.values() for k in v})
    mean = {k: sum(v.get(k, 0.0) for v in per.values()) / len(per) for k in keys}
    rec = {"kernel": name.replace("misa::(anonymous namespace)::", "").split("(")[0],
           "dispatches": len(per), "command": cmd,
           "counters_per_launch": {k: round(v) for k, v in mean.items()},
           "profiled_duration_us": round(sum(dur.values()) / len(dur) / 1e3, 2)}
    gui = mean.get("GRBM_GUI_ACTIVE", 0.0) / xcds          # cycles the chip was busy
    mf = mean.get("SQ_INSTS_MFMA", 0.0)
    busy = mean.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
    if gui and busy:
        rec["mfma_busy_frac_of_simd_cycles"] = round(busy / (gui * simds), 4)
        rec["clock_ghz_under_load"] = round(gui / (rec["profiled_duration_us"] * 1e3), 3)
    if busy and "SQ_VALU_MFMA_COEXEC_CYCLES" in mean:
        rec["coexec_frac_of_mfma_busy"] = round(mean["SQ_VALU_MFMA_COEXEC_CYCLES"] / busy, 4)
    if mf:
        rec["mfma_busy_cycles_per_mfma"] = round(busy / mf, 2)
        rec["non_mfma_valu_per_mfma"] = round((mean.get("SQ_INSTS_VALU", 0.0) - mf) / mf, 3)
        rec["flop_from_counters"] = mf * mfma_flop
        if flop:
            rec["algorithmic_flop"] = flop
            rec["counter_flop_over_algorithmic"] = round(mf * mfma_flop / flop, 4)
    wave = mean.get("SQ_WAVE_CYCLES", 0.0)
    if wave and "SQ_WAIT_INST_ANY" in mean:
        # wave-time shares: SQ_WAVE_CYCLES, SQ_WAIT_INST_* and SQ_ACTIVE_INST_*
        # are quad-cycles summed over the wavefronts
        rec["wave_time_waiting_on_dependencies"] = round(mean["SQ_WAIT_INST_ANY"] / wave, 4)
        if "SQ_WAIT_INST_LDS" in mean:
            rec["wave_time_waiting_on_lds"] = round(mean["SQ_WAIT_INST_LDS"] / wave, 4)
        if "SQ_ACTIVE_INST_VALU" in mean:
            rec["wave_time_issuing_vector_or_matrix"] = round(mean["SQ_ACTIVE_INST_VALU"] / wave, 4)
        if mean.get("SQ_INSTS_LDS"):
            rec["lds_bank_conflict_cycles_per_lds_instruction"] = round(
                mean.get("SQ_LDS_BANK_CONFLICT", 0.0) / mean["SQ_INSTS_LDS"], 4)
    return rec


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter record, if the kernel's
    source is unchanged since the counters were taken (else None)."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    try:
        with open(path) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_sha(kernel):
        return None
    return round(rec["traffic_bytes_per_launch"])


class Replicas:
    """Device copies of one problem's keys plus preallocated outputs."""

    def __init__(self, p, torch, binding, h, k_prime):
        from long_context_mean_amd.binding import DeviceProblem
        self.p = p
        self.dp = DeviceProblem(p)
        self.k = [self.dp.k] + [self.dp.k.clone() for _ in range(REPLICAS - 1)]
        self.ks = [self.dp.k_scale] * REPLICAS if self.dp.k_scale is None else \
            [self.dp.k_scale] + [self.dp.k_scale.clone() for _ in range(REPLICAS - 1)]
        dev = self.dp.q.device
        N, H_I, d, L, B = p.N, p.H_I, p.d, p.L, p.B
        M = -(-L // B)
        self.h = h
        self.kbar = [torch.empty((p.S, M, d), dtype=torch.float32, device=dev)
                     for _ in range(REPLICAS)]
        self.heads = torch.empty((N, h), dtype=torch.int32, device=dev)
        self.r = torch.empty((N, H_I), dtype=torch.float32, device=dev)
        self.idx = torch.empty((N, p.topk), dtype=torch.int32, device=dev)
        self.sc = torch.empty((N, p.topk), dtype=torch.float32, device=dev)
        self.k_prime = k_prime
        self.cand = torch.empty((N, max(k_prime, 1)), dtype=torch.int32, device=dev)
        self.ws_route = binding.workspace(binding.MISA_OP_ROUTE, N, L, d, H_I, B, q_dt=p.q_dt,
                                          device=dev)
        self.ws_score = binding.workspace(binding.MISA_OP_SCORE_TOPK, N, L, d, H_I,
                                          topk=max(p.topk, k_prime), q_dt=p.q_dt, device=dev)
        self.ws_rerank = binding.workspace(binding.MISA_OP_RERANK, N, L, d, H_I, topk=p.topk,
                                           k_prime=max(k_prime, p.topk), q_dt=p.q_dt, device=dev)
        self.b = binding

    def pool(self, i):
        self.b.misa_pool_keys(self.k[i], self.p.B, self.ks[i], kbar=self.kbar[i])

    def route(self, i):
        d = self.dp
        self.b.misa_route_heads(d.q, d.w, self.kbar[i], self.k[i], d.q_seq, d.q_pos, self.p.B,
                                self.h, k_scale=self.ks[i], q_scale=d.q_scale, heads=self.heads,
                                head_score=self.r, ws=self.ws_route)

    def score(self, i, topk=None, out=None):
        d = self.dp
        self.b.misa_score_topk(d.q, d.w, self.k[i], d.q_seq, d.q_pos, self.heads,
                               self.p.topk if topk is None else topk, k_scale=self.ks[i],
                               q_scale=d.q_scale, idx=self.idx if out is None else out, score=None,
                               ws=self.ws_score, want_score=False)

    def dense(self, i):
        d = self.dp
        self.b.dsa_score_topk(d.q, d.w, self.k[i], d.q_seq, d.q_pos, self.p.topk,
                              k_scale=self.ks[i], q_scale=d.q_scale, idx=self.idx, score=self.sc,
                              ws=self.ws_score)

    def rerank(self, i):
        d = self.dp
        self.b.misa_rerank(d.q, d.w, self.k[i], d.q_seq, d.q_pos, self.cand, self.p.topk,
                           k_scale=self.ks[i], q_scale=d.q_scale, idx=self.idx, score=self.sc,
                           ws=self.ws_rerank)

    # step variants -------------------------------------------------------
    def step_misa(self, i):
        self.pool(i)
        self.route(i)
        self.score(i)

    def step_dense(self, i):
        self.dense(i)

    def step_dagger(self, i):
        self.pool(i)
        self.route(i)
        self.score(i, topk=self.k_prime, out=self.cand)
        self.rerank(i)


class Serving:
    """The decode serving step on a key cache (contiguous, or paged with
    page_size tokens per page): the newest token of every sequence completes
    its last block, so the step pools that one block into the cached table,
    routes and scores in one call (misa_pool_route_score_topk: the pooling
    runs in the router's launch, the head selection in the scoring kernel);
    step_pool_then_fused makes the pooling a call of its own
    (misa_pool_update + misa_route_score_topk), step_two_calls also splits
    the routing from the scoring (misa_route_heads + misa_score_topk).
    REPLICAS copies of the keys rotate like Replicas."""

    def __init__(self, p, torch, binding, h, page_size=0):
        from long_context_mean_amd.binding import DeviceProblem
        self.p, self.b, self.h = p, binding, h
        self.dps = [DeviceProblem(p, page_size=page_size, page_seed=i) for i in range(REPLICAS)]
        if not page_size:                    # distinct contiguous copies of the keys
            for dp in self.dps[1:]:
                dp.k = dp.k.clone()
        self.kbar = [dp.pool() for dp in self.dps]
        dev = self.dps[0].q.device
        self.len_old = torch.full((p.S,), p.L - 1, dtype=torch.int32, device=dev)
        self.len_new = torch.full((p.S,), p.L, dtype=torch.int32, device=dev)
        self.heads = torch.empty((p.N, h), dtype=torch.int32, device=dev)
        self.r = torch.empty((p.N, p.H_I), dtype=torch.float32, device=dev)
        self.idx = torch.empty((p.N, p.topk), dtype=torch.int32, device=dev)
        self.ws_route = binding.workspace(binding.MISA_OP_ROUTE, p.N, p.L, p.d, p.H_I, p.B,
                                          device=dev)
        self.ws_score = binding.workspace(binding.MISA_OP_SCORE_TOPK, p.N, p.L, p.d, p.H_I,
                                          topk=p.topk, device=dev)
        self.ws_fused = binding.workspace(binding.MISA_OP_ROUTE_SCORE_TOPK, p.N, p.L, p.d,
                                          p.H_I, p.B, topk=p.topk, device=dev)

    def step(self, i):
        dp = self.dps[i]
        dp.pool_route_score_topk(self.kbar[i], self.len_old, self.len_new, 1, self.h,
                                 heads=self.heads, head_score=self.r, idx=self.idx, score=None,
                                 ws=self.ws_fused, want_score=False)

    def step_pool_then_fused(self, i):
        dp = self.dps[i]
        dp.pool_update(self.len_old, self.len_new, 1, self.kbar[i])
        dp.route_score_topk(self.kbar[i], self.h, heads=self.heads, head_score=self.r,
                            idx=self.idx, score=None, ws=self.ws_fused, want_score=False)

    def step_two_calls(self, i):
        dp = self.dps[i]
        dp.pool_update(self.len_old, self.len_new, 1, self.kbar[i])
        dp.route(self.kbar[i], self.h, heads=self.heads, head_score=self.r, ws=self.ws_route)
        dp.score_topk(self.heads, idx=self.idx, score=None, ws=self.ws_score, want_score=False)

    def use_dagger(self, k_prime):
        """MISA-dagger in serving form: the single call selects the top k_prime
        tokens under the routed heads, then misa_rerank re-scores them with
        every head and keeps the top k."""
        p, b = self.p, self.b
        dev = self.heads.device
        self.k_prime = k_prime
        self.cand = self.heads.new_empty((p.N, k_prime))
        self.sc = self.r.new_empty((p.N, p.topk))
        self.ws_dag = b.workspace(b.MISA_OP_ROUTE_SCORE_TOPK, p.N, p.L, p.d, p.H_I, p.B,
                                  topk=k_prime, device=dev)
        self.ws_rerank = b.workspace(b.MISA_OP_RERANK, p.N, p.L, p.d, p.H_I, topk=p.topk,
                                     k_prime=k_prime, q_dt=p.q_dt, device=dev)

    def step_dagger(self, i):
        dp = self.dps[i]
        dp.pool_route_score_topk(self.kbar[i], self.len_old, self.len_new, 1, self.h,
                                 topk=self.k_prime, heads=self.heads, head_score=self.r,
                                 idx=self.cand, score=None, ws=self.ws_dag, want_score=False)
        dp.rerank(self.cand, idx=self.idx, score=self.sc, ws=self.ws_rerank)

    def use_blocks(self, m_blocks):
        """Switch the step's scoring to the block prefilter (m_blocks blocks)."""
        p = self.p
        self.m = m_blocks
        self.blocks = self.b.workspace(self.b.MISA_OP_BLOCKS, p.N, p.L, p.d, p.H_I, p.B,
                                       topk=p.topk, k_prime=m_blocks,
                                       device=self.heads.device)
        self.kept = self.heads.new_empty((p.N, m_blocks))

    def step_blocks(self, i):
        dp = self.dps[i]
        dp.pool_update(self.len_old, self.len_new, 1, self.kbar[i])
        dp.route(self.kbar[i], self.h, heads=self.heads, head_score=self.r, ws=self.ws_route)
        dp.score_topk_blocks(self.kbar[i], self.heads, self.m, blocks=self.kept, idx=self.idx,
                             score=None, ws=self.blocks, want_score=False)


def attention_extra(torch, binding, synth, idx, p, steps):
    """Sparse attention of DeepSeek-V3.2-like decode rows (H = 128 heads,
    576-element latent rows, values = their first 512 elements) over the
    indexer's 2048 selected tokens per row; REPLICAS copies of the latent
    cache rotate so the gathers are cold."""
    import numpy as np

    from long_context_mean_amd.binding import DeviceAttention
    H, dqk, dv = 128, 576, 512
    ap = synth.attention_problem("attn", 2001, N=p.N, S=p.S, L=p.L, H=H, d_qk=dqk, d_v=dv,
                                 topk=p.topk, n_valid=np.zeros(p.N, np.int64))
    da = DeviceAttention(ap)
    kvs = [da.kv] + [da.kv.clone() for _ in range(REPLICAS - 1)]
    sel = idx.clone()
    out = torch.empty((p.N, H, dv), dtype=torch.float32, device="cuda")
    lse = torch.empty((p.N, H), dtype=torch.float32, device="cuda")
    ws = binding.workspace(binding.MISA_OP_ATTENTION, p.N, p.L, dv, H, topk=p.topk)

    def step(i):
        binding.misa_sparse_attention(da.q, kvs[i], da.q_seq, sel, ap.scale, dv, out=out,
                                      lse=lse, ws=ws)
    ms = timed(torch, step, steps, 5)
    _, kt, _ = kernel_times(torch, binding, step, max(3, steps // 2), 1, 4)
    nsel = int((sel >= 0).sum().item())
    gathered = nsel * dqk * 2                                  # cache bytes read
    flops = 2.0 * H * nsel * (dqk + dv)
    sk = kt.get("attn_split_kernel")
    del kvs, da
    torch.cuda.empty_cache()
    return {"sparse_attention_ms": round(ms, 4),
            "sparse_attention_kernel_ms": {k: round(v, 5) for k, v in kt.items()},
            "sparse_attention_shape": f"{p.N} rows x {H} heads x {nsel // p.N} selected tokens, "
                                      f"d_qk={dqk}, d_v={dv}",
            "sparse_attention_split_kernel_gbs": round(gathered / (sk * 1e-3) / 1e9, 1)
            if sk else None,
            "sparse_attention_split_kernel_tflops": round(flops / (sk * 1e-3) / 1e12, 1)
            if sk else None}


def timed(torch, fn, steps, warmup):
    for s in range(warmup):
        fn(s % REPLICAS)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        fn(s % REPLICAS)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def kernel_times(torch, binding, fn, steps, warmup, per_step):
    """Per-kernel HIP-event durations (ms) over `steps` steps of fn."""
    for s in range(warmup):
        fn(s % REPLICAS)
    torch.cuda.synchronize()
    binding.misa_profile_begin(steps * per_step + 16)
    t0 = time.perf_counter()
    for s in range(steps):
        fn(s % REPLICAS)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    recs = binding.misa_profile_end(steps * per_step + 16)
    by = {}
    for name, ms in recs:
        by.setdefault(name, []).append(ms)
    return ms_step, {k: sum(v) / len(v) for k, v in by.items()}, \
        {k: len(v) / steps for k, v in by.items()}


def step_percentiles(torch, fn, reps=100, warmup=5):
    """Per-step latency (us) from a torch event pair around each step: p10/p50/p90."""
    import numpy as np
    for s in range(warmup):
        fn(s % REPLICAS)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for s, (a, b) in enumerate(ev):
        a.record()
        fn(s % REPLICAS)
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    return {"p10": round(float(np.percentile(t, 10)), 2), "p50": round(float(np.median(t)), 2),
            "p90": round(float(np.percentile(t, 90)), 2)}


def measured_read_gbs(torch):
    """In-run streaming-read reference: row sums of a [4096, 32768] fp32 tensor
    (512 MiB read, 16 KiB written) with torch, not the library: what a plain
    HBM-bound kernel reaches on this GPU."""
    x = torch.ones((4096, 32768), dtype=torch.float32, device="cuda")
    for _ in range(3):
        x.sum(dim=1)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(10):
        x.sum(dim=1)
    b.record()
    torch.cuda.synchronize()
    gbs = 10 * x.numel() * 4 / (a.elapsed_time(b) * 1e-3) / 1e9
    del x
    return round(gbs, 1)


def measured_mfma_tflops(torch, fp8=False):
    """In-run matrix-core reference: an 8192^3 bf16 torch.matmul, or for fp8
    an e4m3 x e4m3 torch._scaled_mm (both hipBLASLt); None if unavailable."""
    n = 8192
    x = torch.randn((n, n), dtype=torch.bfloat16, device="cuda")
    y = torch.randn((n, n), dtype=torch.bfloat16, device="cuda")
    if fp8:
        x = x.to(torch.float8_e4m3fn)
        y = y.to(torch.float8_e4m3fn).t().contiguous().t()      # column-major right operand
        one = torch.ones((), dtype=torch.float32, device="cuda")

        def mm():
            return torch._scaled_mm(x, y, scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
    else:
        def mm():
            return torch.matmul(x, y)
    try:
        for _ in range(3):
            mm()
        torch.cuda.synchronize()
    except RuntimeError as e:
        log(f"[bench] matrix-core reference unavailable: {e}")
        return None
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(10):
        mm()
    b.record()
    torch.cuda.synchronize()
    tf = 10 * 2.0 * n ** 3 / (a.elapsed_time(b) * 1e-3) / 1e12
    del x, y
    return round(tf, 1)


def cpu_baseline(p, h, min_seconds=10.0, max_passes=200):
    """The oracle on the host cores over the whole workload, repeated until
    about min_seconds of CPU work have run (one pass is well under a second);
    beside it, one-thread oracle times of the two small decode workloads."""
    import oracle
    from long_context_mean_amd import synth
    passes, t0 = 0, time.perf_counter()
    while True:
        oracle.misa(p, h=h)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or passes >= max_passes:
            break
    threads = oracle.max_threads()
    one = {}
    oracle.set_threads(1)
    try:
        for name in ("c1", "c2"):
            pc = synth.make(name)
            t1 = time.perf_counter()
            oracle.misa(pc)
            one[f"{name}_ms"] = round((time.perf_counter() - t1) * 1e3, 1)
            one[f"{name}_tokens_per_s"] = round(pc.tokens_indexed() /
                                                (time.perf_counter() - t1), 1)
    finally:
        oracle.set_threads(threads)
    return {"value": passes * p.tokens_indexed() / dt, "unit": "tokens/s",
            "cores": threads, "kind": "oracle",
            "sample": f"the full workload ({p.N} queries x {p.L} keys, pooling+routing+scoring+"
                      f"top-k in double precision), {passes} passes in {dt:.1f} s",
            "cores_available": len(os.sched_getaffinity(0)),
            "one_thread": one}


def prefill_measure(torch, workload, h, steps, warmup):
    """Prefill chunk `workload` (4096 consecutive query rows over one causal
    prefix): the routed step (pool -> route -> score + top-k), the dense
    64-head step, kernel times and the scoring GEMM against the MFMA peak."""
    from long_context_mean_amd import binding, synth
    from long_context_mean_amd.binding import DeviceProblem
    p = synth.make(workload, h=h)
    dp = DeviceProblem(p)
    N, L, d, H_I, B = p.N, p.L, p.d, p.H_I, p.B
    fp8 = p.q_dt == synth.FP8
    M = -(-L // B)
    dev = dp.q.device
    kbar = torch.empty((1, M, d), dtype=torch.float32, device=dev)
    heads = torch.empty((N, h), dtype=torch.int32, device=dev)
    r = torch.empty((N, H_I), dtype=torch.float32, device=dev)
    idx = torch.empty((N, p.topk), dtype=torch.int32, device=dev)
    ws_r = binding.workspace(binding.MISA_OP_ROUTE, N, L, d, H_I, B, q_dt=p.q_dt, device=dev)
    ws_s = binding.workspace(binding.MISA_OP_SCORE_TOPK, N, L, d, H_I, topk=p.topk, q_dt=p.q_dt,
                             device=dev)
    ks, qs = dp.k_scale, dp.q_scale

    def step(_):
        binding.misa_pool_keys(dp.k, B, ks, kbar=kbar)
        binding.misa_route_heads(dp.q, dp.w, kbar, dp.k, dp.q_seq, dp.q_pos, B, h,
                                 k_scale=ks, q_scale=qs, heads=heads, head_score=r, ws=ws_r)
        binding.misa_score_topk(dp.q, dp.w, dp.k, dp.q_seq, dp.q_pos, heads, p.topk, k_scale=ks,
                                q_scale=qs, idx=idx, ws=ws_s, want_score=False)

    def dense(_):
        binding.dsa_score_topk(dp.q, dp.w, dp.k, dp.q_seq, dp.q_pos, p.topk, k_scale=ks,
                               q_scale=qs, idx=idx, ws=ws_s, want_score=False)

    ms = timed(torch, step, steps, warmup)
    pct = step_percentiles(torch, step, reps=max(20, steps), warmup=2)
    ms_e, kt, per = kernel_times(torch, binding, step, max(3, steps // 4), 1, 16)
    ms_d = timed(torch, dense, max(3, steps // 4), 1)
    _, ktd, _ = kernel_times(torch, binding, dense, 3, 1, 8)
    pairs = p.tokens_indexed()
    flops = 2.0 * h * d * pairs
    sc_ms = kt.get("score_prefill_kernel")
    tflops = flops / (sc_ms * 1e-3) / 1e12 if sc_ms else None
    dflops = 2.0 * H_I * d * pairs
    dsc = ktd.get("score_prefill_kernel")
    peak = 5000.0 if fp8 else 2500.0              # dense MFMA: e4m3 5.0, bf16 2.5 PFLOP/s
    line = {
        "metric": "prefix tokens indexed/sec (prefill chunk)", "value": pairs / (ms * 1e-3),
        "unit": "(query, prefix token) pairs/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "dtype": "e4m3" if fp8 else "bf16", "data": "synthetic",
        "config": {"workload": f"prefill chunk: {N} rows at positions {int(p.q_pos[0])}.."
                               f"{int(p.q_pos[-1])} over L={L}, H_I={H_I}, d={d}, h={h}, "
                               f"B={B}, top-k={p.topk}" +
                               (", e4m3 q (per-head scale) and k (per-token scale)" if fp8
                                else "")},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1) if tflops else None,
                     "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4) if tflops else None,
                     "traffic": measured_traffic("score_prefill_kernel", workload),
                     "kernel": "score_prefill_kernel", "kernel_ms": sc_ms,
                     "algorithmic_flop_per_launch": flops},
        "extra": {"kernel_ms": {k: round(v, 4) for k, v in kt.items()},
                  "step_us_percentiles": pct,
                  "dense_ms": round(ms_d, 4), "speedup_vs_dense": round(ms_d / ms, 3),
                  "dense_kernel_ms": {k: round(v, 4) for k, v in ktd.items()},
                  "dense_score_tflops": round(dflops / (dsc * 1e-3) / 1e12, 1) if dsc else None,
                  "routed_score_vs_dense_score": round(dsc / sc_ms, 3) if dsc and sc_ms else None},
    }
    del dp, ws_s, ws_r
    torch.cuda.empty_cache()
    return line


def prefill_main(args):
    import torch
    line = prefill_measure(torch, args.workload, args.h, args.steps, args.warmup)
    mtf = measured_mfma_tflops(torch, line["dtype"] == "e4m3")
    tflops = line["roofline"]["achieved"]
    line["roofline"]["measured_peak"] = mtf
    line["roofline"]["frac_vs_measured_peak"] = round(tflops / mtf, 4) if tflops and mtf else None
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize, args.title, args.cmd)
        return
    if args.traffic:
        print(json.dumps(traffic_record(*args.traffic, args.kernel, args.match or args.kernel,
                                        args.cmd), indent=1))
        return
    if args.counters:
        print(json.dumps(counter_record(args.counters, args.match or args.kernel, args.flop,
                                        args.cmd), indent=1))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the indexer's queries shard across GPUs without any exchange)",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return
    if args.workload != "c4":
        prefill_main(args)
        return
    import numpy as np
    import torch

    from long_context_mean_amd import binding, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    binding.lib()
    h = args.h
    log("[bench] generating c4 workload")
    p = synth.make("c4", h=h)
    rep = Replicas(p, torch, binding, h, k_prime=8192)
    tokens = p.tokens_indexed()
    key_bytes = p.N * p.L * p.d * 2

    srv = Serving(p, torch, binding, h)
    log("[bench] timing the serving step (incremental pool + route + score/top-k in one call)")
    ms = timed(torch, srv.step, args.steps, args.warmup)
    value = tokens / (ms * 1e-3)
    pct = step_percentiles(torch, srv.step, reps=max(100, args.steps), warmup=5)
    log(f"[bench] misa {ms:.4f} ms/step -> {value:.4e} tokens/s")

    log("[bench] per-kernel HIP events over the timed steps")
    ms_ev, kt, per = kernel_times(torch, binding, srv.step, args.steps, 2, 16)
    dominant = max(kt, key=lambda k: kt[k] * per[k])
    bytes_per_launch = {"pool_kernel": key_bytes, "score_mfma_kernel": key_bytes}
    alg = bytes_per_launch.get(dominant, key_bytes)
    achieved = alg / (kt[dominant] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(dominant, "c4"),
                "kernel": dominant, "kernel_ms": round(kt[dominant], 5),
                "algorithmic_bytes_per_launch": alg,
                "frac_is": f"{dominant} alone: its algorithmic bytes over its own duration"}
    # the whole step against the same roofline: the step's algorithmic bytes
    # (every key once, plus the pooled table the router reads) over ms_per_step
    step_bytes = key_bytes + p.S * (p.L // p.B) * p.d * 4
    roofline["step_algorithmic_bytes"] = step_bytes
    roofline["step_achieved"] = round(step_bytes / (ms * 1e-3) / 1e9, 1)
    roofline["step_frac"] = round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)

    extra = {"kernel_ms": {k: round(v, 5) for k, v in kt.items()},
             "step_ms_with_kernel_events": round(ms_ev, 4), "step_us_percentiles": pct}
    mgbs = measured_read_gbs(torch)
    roofline["measured_peak"] = mgbs
    roofline["frac_vs_measured_peak"] = round(achieved / mgbs, 4)
    sc_ms = kt.get("score_mfma_kernel")
    if sc_ms:
        extra["score_kernel_hbm_gbs"] = round(key_bytes / (sc_ms * 1e-3) / 1e9, 1)
    pl_ms = kt.get("pool_kernel")
    if pl_ms:
        extra["pool_kernel_hbm_gbs"] = round(key_bytes / (pl_ms * 1e-3) / 1e9, 1)

    if not args.no_extras:
        ms_2 = timed(torch, srv.step_two_calls, args.steps, args.warmup)
        _, kt2, _ = kernel_times(torch, binding, srv.step_two_calls, max(3, args.steps // 2), 1,
                                 16)
        extra["serving_step_two_calls_ms"] = round(ms_2, 4)
        extra["serving_step_two_calls_kernel_ms"] = {k: round(v, 5) for k, v in kt2.items()}
        extra["serving_step_pool_then_fused_ms"] = round(
            timed(torch, srv.step_pool_then_fused, args.steps, args.warmup), 4)
        ms_f = timed(torch, rep.step_misa, args.steps, args.warmup)
        _, ktf, _ = kernel_times(torch, binding, rep.step_misa, max(3, args.steps // 2), 1, 16)
        ms_d = timed(torch, rep.step_dense, args.steps, args.warmup)
        ms_g = timed(torch, rep.step_dagger, args.steps, args.warmup)
        srv.use_dagger(8192)
        ms_gs = timed(torch, srv.step_dagger, args.steps, args.warmup)
        _, ktg, _ = kernel_times(torch, binding, srv.step_dagger, max(3, args.steps // 2), 1, 16)
        extra.update({
            "full_pool_step_ms": round(ms_f, 4),
            "full_pool_step_tokens_per_s": tokens / (ms_f * 1e-3),
            "full_pool_step_kernel_ms": {k: round(v, 5) for k, v in ktf.items()},
            "dense_dsa_ms": round(ms_d, 4),
            "speedup_vs_dense": round(ms_d / ms, 3),
            "misa_dagger_ms": round(ms_g, 4),
            "misa_dagger_serving_ms": round(ms_gs, 4),
            "misa_dagger_serving_kernel_ms": {k: round(v, 5) for k, v in ktg.items()},
        })
        # recall of the dense top-k set (outside timing)
        srv.step(0)
        torch.cuda.synchronize()
        misa_idx = srv.idx.cpu().numpy()
        rep.step_dense(0)
        torch.cuda.synchronize()
        dense_idx = rep.idx.cpu().numpy()
        rep.step_dagger(0)
        torch.cuda.synchronize()
        dag_idx = rep.idx.cpu().numpy()

        def rec(a, b):
            return float(np.mean([len(set(x[x >= 0]) & set(y[y >= 0])) / max(1, (y >= 0).sum())
                                  for x, y in zip(a, b)]))
        def iou(a, b):
            return float(np.mean([len(set(x[x >= 0]) & set(y[y >= 0])) /
                                  max(1, len(set(x[x >= 0]) | set(y[y >= 0])))
                                  for x, y in zip(a, b)]))
        extra["recall_vs_dense"] = round(rec(misa_idx, dense_idx), 4)
        extra["iou_vs_dense"] = round(iou(misa_idx, dense_idx), 4)
        extra["misa_dagger_recall_vs_dense"] = round(rec(dag_idx, dense_idx), 4)
        extra["misa_dagger_iou_vs_dense"] = round(iou(dag_idx, dense_idx), 4)
        extra["needle_recall"] = round(float(np.mean(
            [np.isin(p.needles[n, :, 0], misa_idx[n]).mean() for n in range(p.N)])), 4)
        extra["needle_recall_dense"] = round(float(np.mean(
            [np.isin(p.needles[n, :, 0], dense_idx[n]).mean() for n in range(p.N)])), 4)
        del rep
        torch.cuda.empty_cache()
        log("[bench] serving step with a block prefilter (routing x token hierarchy)")
        for m_blocks in (64, 16):
            srv.use_blocks(m_blocks)
            ms_b = timed(torch, srv.step_blocks, args.steps, args.warmup)
            srv.step_blocks(0)
            torch.cuda.synchronize()
            bidx = srv.idx.cpu().numpy()
            extra[f"blocks{m_blocks}_step_ms"] = round(ms_b, 4)
            extra[f"blocks{m_blocks}_tokens_per_s"] = tokens / (ms_b * 1e-3)
            extra[f"blocks{m_blocks}_recall_vs_misa"] = round(rec(bidx, misa_idx), 4)
            extra[f"blocks{m_blocks}_recall_vs_dense"] = round(rec(bidx, dense_idx), 4)
        srv.step(0)
        torch.cuda.synchronize()
        log("[bench] sparse attention over the selected tokens (128 heads, 576/512 latent rows)")
        extra.update(attention_extra(torch, binding, synth, srv.idx, p, args.steps))
        log("[bench] the serving step on a paged key cache (pages of 64 tokens)")
        del srv
        pg = Serving(p, torch, binding, h, page_size=64)
        ms_s = timed(torch, pg.step, args.steps, args.warmup)
        _, kts, _ = kernel_times(torch, binding, pg.step, max(3, args.steps // 2), 1, 16)
        pg.step(0)
        torch.cuda.synchronize()
        extra["paged_serving_step_ms"] = round(ms_s, 4)
        extra["paged_serving_tokens_per_s"] = tokens / (ms_s * 1e-3)
        extra["paged_serving_kernel_ms"] = {k: round(v, 5) for k, v in kts.items()}
        extra["paged_recall_vs_dense"] = round(rec(pg.idx.cpu().numpy(), dense_idx), 4)
        del pg
        torch.cuda.empty_cache()
        log("[bench] the serving step at h = 4 and 16")
        for hh in (4, 16):
            sv = Serving(p, torch, binding, hh)
            ms_h = timed(torch, sv.step, args.steps, args.warmup)
            sv.step(0)
            torch.cuda.synchronize()
            hidx = sv.idx.cpu().numpy()
            extra[f"serving_step_ms_h{hh}"] = round(ms_h, 4)
            extra[f"serving_tokens_per_s_h{hh}"] = tokens / (ms_h * 1e-3)
            extra[f"recall_vs_dense_h{hh}"] = round(rec(hidx, dense_idx), 4)
            extra[f"needle_recall_h{hh}"] = round(float(np.mean(
                [np.isin(p.needles[n, :, 0], hidx[n]).mean() for n in range(p.N)])), 4)
            del sv
            torch.cuda.empty_cache()
        log("[bench] the serving step at 32 queries, each over its own 131072 keys")
        p32 = synth.small("c4x32", 1104, N=32, S=32, L=p.L, d=p.d, H_I=p.H_I, h=h, B=p.B,
                          topk=p.topk, n_clusters=64, sigma=0.5)
        s32 = Serving(p32, torch, binding, h)
        ms32 = timed(torch, s32.step, args.steps, args.warmup)
        _, kt32, _ = kernel_times(torch, binding, s32.step, max(3, args.steps // 2), 1, 8)
        keys32 = p32.S * p32.L * p32.d * 2
        bytes32 = keys32 + p32.S * (p32.L // p32.B) * p32.d * 4
        extra["serving_step_n32"] = {
            "workload": "32 queries x L=131072 bf16 keys (32 sequences), H_I=64, d=128, h=8, "
                        "B=128, top-k=2048, the c4 mixture recipe without needles",
            "ms_per_step": round(ms32, 4),
            "tokens_per_s": p32.tokens_indexed() / (ms32 * 1e-3),
            "kernel_ms": {k: round(v, 5) for k, v in kt32.items()},
            "score_kernel_hbm_gbs": round(keys32 / (kt32["score_mfma_kernel"] * 1e-3) / 1e9, 1)
            if kt32.get("score_mfma_kernel") else None,
            "step_frac": round(bytes32 / (ms32 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del s32, p32
        torch.cuda.empty_cache()
        log("[bench] fp8-key MISA-dagger (c5 shape)")
        p5 = synth.make("c5")
        r5 = Replicas(p5, torch, binding, p5.h, k_prime=p5.k_prime)
        ms5 = timed(torch, r5.step_dagger, args.steps, args.warmup)
        s5 = Serving(p5, torch, binding, p5.h)
        s5.use_dagger(p5.k_prime)
        ms5s = timed(torch, s5.step_dagger, args.steps, args.warmup)
        s5.step_dagger(0)
        r5.step_dagger(0)
        torch.cuda.synchronize()
        same5 = bool(torch.equal(s5.idx, r5.idx))
        del s5
        ms5d = timed(torch, r5.step_dense, args.steps, args.warmup)
        extra["fp8_misa_dagger_ms"] = round(ms5, 4)
        extra["fp8_misa_dagger_serving_ms"] = round(ms5s, 4)
        extra["fp8_misa_dagger_serving_same_idx"] = same5
        extra["fp8_misa_dagger_tokens_per_s"] = p5.tokens_indexed() / (ms5 * 1e-3)
        extra["fp8_misa_dagger_serving_tokens_per_s"] = p5.tokens_indexed() / (ms5s * 1e-3)
        extra["fp8_dense_dsa_ms"] = round(ms5d, 4)
        del r5
        torch.cuda.empty_cache()
        log("[bench] prefill chunk at L=128K (4096 rows): routed and dense 64-head steps")
        pl = prefill_measure(torch, "c3x", h, 30, 3)
        extra["prefill_c3x"] = {
            "workload": pl["config"]["workload"], "ms_per_step": pl["ms_per_step"],
            "step_us_percentiles": pl["extra"]["step_us_percentiles"],
            "pairs_per_s": pl["value"], "dense_ms": pl["extra"]["dense_ms"],
            "speedup_vs_dense": pl["extra"]["speedup_vs_dense"],
            "kernel_ms": pl["extra"]["kernel_ms"],
            "score_prefill_kernel_tflops": pl["roofline"]["achieved"],
            "score_prefill_kernel_mfma_frac": pl["roofline"]["frac"],
            "mfma_peak_tflops": pl["roofline"]["peak"],
            "dense_score_tflops": pl["extra"]["dense_score_tflops"]}

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline")
        cpu = cpu_baseline(p, h)

    line = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded 64-cluster Gaussian-mixture keys + planted needles)",
        "config": {"workload": "long-context decode indexer: 4 queries x L=131072 bf16 keys, "
                               "H_I=64, d=128, h=8, B=128, top-k=2048",
                   "N": p.N, "L": p.L, "H_I": p.H_I, "h": h, "d": p.d, "B": p.B,
                   "topk": p.topk,
                   "step": "incremental block pooling (the appended token completes each "
                           "sequence's last block) + route + routed score/top-k in one "
                           "call (misa_pool_route_score_topk)",
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
