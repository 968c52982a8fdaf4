"""Benchmark of the proportional-sampling hot path on one MI355X.

A step is one pass of the PER-mid workload: B = 262144 float priorities
(Exp(1) + 1e-6, alpha 0.6, beta 0.4) and 32 minibatch updates, each one
rebuilding the CDF (p^alpha + inclusive scan), drawing 8192 stratified
indices, computing their IS weights and rewriting those 8192 priorities with
new values.  All inputs are resident in HBM before timing starts.  `value` is
sampled indices per second over the timed steps.

The JSON line also carries:
  roofline      the kernel of the step (the fused update, the only kernel in
                the timed region): algorithmic bytes per launch / its average
                launch duration (HIP events around the timed region, on the
                launch stream, over the number of launches); `traffic` comes
                from the committed rocprofv3 counter summary in profiles/ when
                the kernel's sources still hash to the profiled ones;
  cpu_baseline  the CPU oracle (single-threaded, as it stands) running the
                same 32-update chain on a bounded number of steps;
  extra         the CDF-scan bandwidth sweep (2^22..2^26, the Infinity Cache
                flushed before every timed call), the sum-tree workload
                (1024 updates + 1024 draws on 2^19 leaves), particle
                resampling (1024 x 4096) and PER large (2^24 / 2^20).

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "CDF-scan HBM GB/s (% of peak) + sampled indices/sec at B=262144, 8192 draws"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=8.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="launch every kernel from Python instead of replaying a HIP graph")
    ap.add_argument("--only", default="",
                    help="profiling helper: per_mid | scan:<n> | ceiling:<n> | copy:<MiB> | "
                         "pf | per_large | rows | sample_large")
    return ap.parse_args()


# ----------------------------------------------------------------- GPU side
class PerMid:
    """The PER-mid chain with every input resident on the GPU."""

    def __init__(self, ps, torch):
        import synthetic_inputs as si
        d = si.per_mid()
        self.ps, self.torch = ps, torch
        self.n, self.k, self.rounds = d["p0"].size, d["U"].shape[1], d["U"].shape[0]
        self.alpha, self.beta = d["alpha"], d["beta"]
        dev = lambda a: torch.from_numpy(a).cuda()
        self.p = dev(d["p0"].copy())
        self.U = dev(d["U"])
        self.v = dev(d["v"])
        self.cdf = torch.empty(self.n, dtype=torch.float64, device="cuda")
        self.tot = torch.empty(1, dtype=torch.float64, device="cuda")
        self.idx = torch.empty(self.k, dtype=torch.int32, device="cuda")
        self.w = torch.empty(self.k, dtype=torch.float32, device="cuda")
        self.ws = ps.Workspace(ps.build_cdf_workspace_size(self.n))
        self.rws = ps.Workspace(ps.per_round_workspace_size(self.n, self.k))
        self.iws = ps.Workspace(ps.is_weights_workspace_size(self.k))

    def step_fused(self):
        """One step through the fused update entry point (one kernel per
        minibatch update when the grid fits on the GPU at once)."""
        ps = self.ps
        for r in range(self.rounds):
            ps.per_round(self.p, self.U[r], self.alpha, self.beta, self.v[r], out_idx=self.idx,
                         out_w=self.w, cdf=self.cdf, total=self.tot, ws=self.rws)

    def step(self):
        """The same step as four separate calls per update."""
        ps = self.ps
        for r in range(self.rounds):
            ps.build_cdf(self.p, self.alpha, cdf=self.cdf, total=self.tot, ws=self.ws)
            ps.sample(self.cdf, self.tot, self.U[r], stratified=True, out=self.idx)
            ps.is_weights(self.p, self.idx, self.alpha, self.beta, out=self.w, ws=self.iws)
            ps.scatter_lww(self.p, self.idx, self.v[r], grouped=True)

    def per_call_us(self, reps=200):
        """Each of the four calls alone, back to back, on the chain's current
        priorities (the CDF built from them first); the sample call's draws
        per second is the sample-only rate."""
        ps, torch = self.ps, self.torch
        ps.build_cdf(self.p, self.alpha, cdf=self.cdf, total=self.tot, ws=self.ws)
        ps.sample(self.cdf, self.tot, self.U[0], stratified=True, out=self.idx)
        calls = {
            "build_cdf": lambda: ps.build_cdf(self.p, self.alpha, cdf=self.cdf, total=self.tot,
                                              ws=self.ws),
            "sample": lambda: ps.sample(self.cdf, self.tot, self.U[0], stratified=True,
                                        out=self.idx),
            "is_weights": lambda: ps.is_weights(self.p, self.idx, self.alpha, self.beta,
                                                out=self.w, ws=self.iws),
            # rewrites the drawn priorities with the same values every time
            "scatter_lww": lambda: ps.scatter_lww(self.p, self.idx, self.v[0], grouped=True),
        }
        out = {k: round(graph_us(torch, fn, reps), 3) for k, fn in calls.items()}
        out["sample_only_indices_per_s"] = round(self.k / (out["sample"] * 1e-6), 1)
        return out

    def algo_bytes(self, name):
        """Algorithmic bytes per launch, by the per-unit table of the scope
        contract: scan 12 B per element (f32 in, f64 out); stratified sample
        + IS 12 B per draw (U in, index and weight out) plus the touched CDF
        lines min(8 n, 64 k) and the gathered priority lines min(4 n, 64 k).
        The fused update is the scan plus the sample + IS row (its rewrite of
        the drawn priorities, 8 B per draw, is in no row of that table and is
        left out); `per_round_own` is the fused kernel's own count, which
        reads no CDF line back and gathers no priority line twice."""
        n, k = self.n, self.k
        return {
            "build_cdf": 12 * n,                                   # f32 in, f64 out
            "sample": 8 * k + min(8 * n, 64 * k),                  # U in, idx out, CDF lines
            "is_weights": 8 * k + min(4 * n, 64 * k),              # idx in, w out, p lines
            "scatter_lww": 8 * k + 4 * k,                          # idx, vals in; prio out
            "per_round": 12 * n + 12 * k + min(8 * n, 64 * k) + min(4 * n, 64 * k),
            # fused, its own bytes: p in, CDF out, U in, idx + w out, new p in, p rewrites
            "per_round_own": 12 * n + 4 * k + 8 * k + 4 * k + 4 * k,
        }[name]


KERNEL_NAMES = {
    "build_cdf": "k_build_cdf<4, true, float, double, false, false, false, false>",
    "sample": "k_sample_strat_fp<4, true, double>",
    "is_weights": "k_isw_exch<float, 1, 1>",
    "scatter_lww": "k_scatter_grouped",
    "per_round": "k_per_round<1, true, true, false>",
}


def profiled_traffic(name):
    """HBM bytes per launch from a committed rocprofv3 summary, or None when
    the kernel's sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith((" ", "|", "#")):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    try:
        h = hashlib.sha256()
        for f in kv["source_files"].split():
            h.update(open(os.path.join(ROOT, "proportional_sampling_amd", "csrc", f), "rb").read())
        if h.hexdigest() != kv["source_sha256"]:
            return None
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, OSError, ValueError):
        return None


def capture(torch, fn):
    """fn's launches as a HIP graph (captured on a side stream after one
    eager run there, as torch requires)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def graph_us(torch, fn, reps=200, per=32):
    """Average time of one call of fn, from a HIP graph of `per` calls
    replayed back to back (host launches do not bound short calls)."""
    g = capture(torch, lambda: [fn() for _ in range(per)])
    return loop_us(torch, g.replay, max(1, reps // per)) / per


def small_bench(ps, torch):
    """The scan at the two sizes the PR page times it (B = 8192 and 262144:
    7.5 and 7.2 us there, on a GPU it does not name -- context, not a
    target), and the PER-small update (B = 8192, 1024 stratified draws, IS
    weights) as one fused call."""
    import synthetic_inputs as si
    out = {}
    for n in (8192, 262144):
        p = torch.from_numpy(si.generic_f32(n, n + 5, "exp")).cuda()
        cdf = torch.empty(n, dtype=torch.float64, device="cuda")
        tot = torch.empty(1, dtype=torch.float64, device="cuda")
        ws = ps.Workspace(ps.build_cdf_workspace_size(n))
        out[f"build_cdf_{n}_us"] = round(graph_us(torch, lambda: ps.build_cdf(
            p, 0.6, cdf=cdf, total=tot, ws=ws)), 3)
    d = si.per_small()
    P = torch.from_numpy(d["p"]).cuda()
    U = torch.from_numpy(d["U"]).cuda()
    n, k = P.numel(), U.numel()
    idx = torch.empty(k, dtype=torch.int32, device="cuda")
    w = torch.empty(k, dtype=torch.float32, device="cuda")
    cdf = torch.empty(n, dtype=torch.float64, device="cuda")
    tot = torch.empty(1, dtype=torch.float64, device="cuda")
    rws = ps.Workspace(ps.per_round_workspace_size(n, k))
    us = graph_us(torch, lambda: ps.per_round(P, U, d["alpha"], d["beta"], None, out_idx=idx,
                                              out_w=w, cdf=cdf, total=tot, ws=rws))
    out["per_small_update_us"] = round(us, 3)
    out["per_small_indices_per_s"] = round(k / (us * 1e-6), 1)
    return out


def timed_steps(torch, fn, steps):
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / 1000.0, wall


class CacheFlush:
    """Evicts the 256 MB Infinity Cache before a cold-cache timing: a 512 MiB
    read-modify-write pushes everything out, then a 512 MiB read replaces the
    dirty lines it leaves with clean ones (otherwise the timed kernel would
    also pay for writing the flush buffer back)."""

    def __init__(self, torch):
        self.w = torch.zeros(128 * 1024 * 1024, dtype=torch.float32, device="cuda")
        self.r = torch.ones(128 * 1024 * 1024, dtype=torch.float32, device="cuda")
        self.sink = torch.empty((), dtype=torch.float32, device="cuda")
        self.torch = torch

    def __call__(self):
        self.w.add_(1)
        self.torch.sum(self.r, dim=0, out=self.sink)


def flush_cache(torch, flush):
    flush()


def scan_sweep(ps, torch, sizes, reps=8, copy=True):
    """Median launch time of psamp_build_cdf per size, cache flushed, next to
    the copy ceiling: psamp_ceiling_copy (the scan's bytes in its access
    pattern, no arithmetic, no exchange) in the scan's tile geometry (8 rows)
    and in the smaller one (4 rows), timed the same way."""
    out = []
    flush = CacheFlush(torch)
    for n in sizes:
        ceil = {}
        if copy:
            src = torch.rand(n, device="cuda")
            dst = torch.empty(n, dtype=torch.float64, device="cuda")
            for rows, nt in ((8, True), (2, False)):
                ps.ceiling_copy(src, dst, rows, nt)
                ts = []
                for _ in range(reps):
                    flush_cache(torch, flush)
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record()
                    ps.ceiling_copy(src, dst, rows, nt)
                    e1.record()
                    torch.cuda.synchronize()
                    ts.append(e0.elapsed_time(e1) * 1e3)
                ceil[rows] = statistics.median(ts)
            log(f"copy ceiling n=2^{n.bit_length() - 1}: {ceil[8]:.1f} us (scan's tile: 8 rows, "
                f"non-temporal), {ceil[2]:.1f} us (best copy: 2 rows, plain stores)")
            del src, dst
        g = torch.Generator(device="cuda").manual_seed(n)
        p = torch.exp(2.0 * torch.randn(n, device="cuda", generator=g)).float()
        q = torch.randint(1, (1 << 20) + 1, (n,), device="cuda", generator=g,
                          dtype=torch.int64).to(torch.int32).view(torch.uint32)
        for mode, prio, cdt, alpha in (("fp64", p, torch.float64, 0.7),
                                       ("int", q, torch.uint64, 1.0)):
            cdf = torch.empty(n, dtype=cdt, device="cuda")
            tot = torch.empty(1, dtype=cdt, device="cuda")
            ws = ps.Workspace(ps.build_cdf_workspace_size(n))
            ps.build_cdf(prio, alpha, cdf=cdf, total=tot, ws=ws)
            ts = []
            for _ in range(reps):
                flush_cache(torch, flush)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                ps.build_cdf(prio, alpha, cdf=cdf, total=tot, ws=ws)
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3)
            us = statistics.median(ts)
            gbs = 12.0 * n / (us * 1e-6) / 1e9
            row = {"n": n, "mode": mode, "us": round(us, 2), "GB/s": round(gbs, 1),
                   "frac_peak": round(gbs / HBM_PEAK_GBS, 4)}
            if ceil:
                row["copy_ceiling_us"] = {"scan_tile_nt": round(ceil[8], 2),
                                          "best_rows2_plain": round(ceil[2], 2)}
                row["copy_ceiling_frac_peak"] = round(12.0 * n / (min(ceil.values()) * 1e-6)
                                                      / 1e9 / HBM_PEAK_GBS, 4)
                row["scan_frac_of_best_copy"] = round(min(ceil.values()) / us, 3)
            out.append(row)
            log(f"scan {mode} n=2^{n.bit_length() - 1}: {us:.1f} us {gbs:.0f} GB/s")
            del cdf, ws
        del p, q
    del flush
    torch.cuda.empty_cache()
    return out


def loop_us(torch, fn, reps):
    """Average time of `reps` back-to-back calls (one event pair around the
    loop, on the launch stream)."""
    fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return 1e3 * e0.elapsed_time(e1) / reps


def sumtree_bench(ps, torch, rounds=200):
    """Sum tree: 2^19 leaves (500000 valid), rounds of a 1024-entry update
    then 1024 iid draws."""
    import synthetic_inputs as si
    d = si.sumtree(rounds=rounds)
    cap, nv = 1 << 19, 500000
    tree = torch.zeros(2 * cap, dtype=torch.float32, device="cuda")
    ps.segtree_build(tree, torch.from_numpy(d["p0"]).cuda(), d["alpha"])
    idx = torch.from_numpy(d["idx"]).cuda()
    v = torch.from_numpy(d["v"]).cuda()
    U = torch.from_numpy(d["U"]).cuda()
    out = torch.empty(d["U"].shape[1], dtype=torch.int32, device="cuda")
    uws = ps.Workspace(ps.segtree_update_workspace_size(cap, 1024))
    it = {"r": 0}

    def one_round():
        r = it["r"] % rounds
        it["r"] += 1
        ps.segtree_update(tree, idx[r], v[r], d["alpha"], ws=uws)
        ps.segtree_sample(tree, nv, U[r], out=out)

    # each from a HIP graph of 32 calls (rounds r .. r + 31 for the round),
    # so that Python launches do not bound these short calls
    res = {"round_us": round(graph_us(torch, one_round, rounds), 2),
           "update_us": round(graph_us(torch, lambda: ps.segtree_update(tree, idx[0], v[0],
                                                                         d["alpha"], ws=uws),
                                       rounds), 2),
           "sample_us": round(graph_us(torch, lambda: ps.segtree_sample(tree, nv, U[0], out=out),
                                       rounds), 2)}
    res["samples_per_s"] = round(1024 / (res["sample_us"] * 1e-6))
    log(f"sum tree: {res}")
    return res


def replay_bench(ps, torch, rounds=200):
    """Replay priorities at capacity 500000 (a full ring): per round, insert
    1024 new items, update the priorities of 1024 sampled slots, sample 1024
    stratified slots with IS weights."""
    import synthetic_inputs as si
    d = si.sumtree(rounds=rounds)
    rb = ps.ReplayPriorities(500000, d["alpha"], max_batch=1024)
    p0 = torch.from_numpy(d["p0"]).cuda()
    for j in range(0, p0.numel(), 1024):
        rb.insert(p0[j:j + 1024])
    v = torch.from_numpy(d["v"]).cuda()
    U = torch.from_numpy(d["U"]).cuda()
    slots_in = torch.empty(1024, dtype=torch.int32, device="cuda")
    slots = torch.empty(1024, dtype=torch.int32, device="cuda")
    w = torch.empty(1024, dtype=torch.float32, device="cuda")
    it = {"r": 0}

    def one_round():
        r = it["r"] % rounds
        it["r"] += 1
        rb.insert(v[r], out=slots_in)
        rb.sample(U[r], 0.4, out=slots, out_w=w)
        rb.update(slots, v[(r + 1) % rounds])

    res = {"round_us": round(loop_us(torch, one_round, rounds), 2)}
    log(f"replay: {res}")
    return res


def cold_us(torch, fn, flush, reps):
    """Median of single calls, each after a write that evicts the Infinity
    Cache (inputs come from HBM)."""
    ts = []
    for _ in range(reps):
        flush_cache(torch, flush)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(1e3 * e0.elapsed_time(e1))
    return statistics.median(ts)


def resample_bench(ps, torch, reps=50):
    """Row resampling at 1024 x 4096: one call after a cache-evicting write
    (median), and back-to-back calls (the input then comes from the Infinity
    Cache).  HBM bytes: 4 B log-weight in, 4 B ancestor out per particle."""
    import synthetic_inputs as si
    d = si.resample()
    lw = torch.from_numpy(d["lw"]).cuda()
    u = torch.from_numpy(d["u_row"]).cuda()
    out = torch.empty_like(lw, dtype=torch.int32)
    fn = lambda: ps.resample_rows(lw, u, out=out)
    warm = graph_us(torch, fn, 128)           # back to back, launched from a graph
    flush = CacheFlush(torch)
    us = cold_us(torch, fn, flush, max(5, reps // 4))
    del flush
    gbs = (8 * lw.numel() + 4 * u.numel()) / (us * 1e-6) / 1e9
    log(f"resample 1024x4096: {us:.1f} us cold, {warm:.1f} us back-to-back, {gbs:.0f} GB/s")
    return {"us": round(us, 2), "us_back_to_back": round(warm, 2), "GB/s": round(gbs, 1),
            "frac_peak": round(gbs / HBM_PEAK_GBS, 4)}


def pf_bench(ps, torch, reps=50):
    """The fused particle-filter step at 1024 filters x 4096 particles (D = 4,
    O = 2) and at 16 x 1024; HBM bytes per particle: x, eps, x_out (3 D
    floats), lw in and out, the ancestor out (4 + 4 + 4)."""
    import synthetic_inputs as si
    res = {}
    flush = CacheFlush(torch)
    for name, d in (("1024x4096", si.pf_step()), ("16x1024", si.pf_small())):
        t = {k: torch.from_numpy(d[k]).cuda() for k in ("x", "lw", "obs", "A", "C", "eps",
                                                         "u_row")}
        rows, P, D = d["x"].shape
        xo = torch.empty_like(t["x"])
        lo = torch.empty_like(t["lw"])
        an = torch.empty(rows, P, dtype=torch.int32, device="cuda")
        fn = lambda: ps.pf_step(t["x"], t["lw"], t["obs"], t["A"], t["C"], t["eps"],
                                d["sigma_p"], d["sigma_o"], t["u_row"], x_out=xo, logw_out=lo,
                                anc_out=an)
        warm = graph_us(torch, fn, 128)       # back to back, launched from a graph
        us = cold_us(torch, fn, flush, max(5, reps // 4))
        nbytes = rows * P * (3 * 4 * D + 12) + rows * 4 * (1 + d["obs"].shape[1])
        gbs = nbytes / (us * 1e-6) / 1e9
        log(f"pf_step {name}: {us:.1f} us cold, {warm:.1f} us back-to-back, {gbs:.0f} GB/s")
        res[name] = {"us": round(us, 2), "us_back_to_back": round(warm, 2),
                     "GB/s": round(gbs, 1), "frac_peak": round(gbs / HBM_PEAK_GBS, 4),
                     "particles_per_s": round(rows * P / (us * 1e-6), 1)}
    return res


def per_large_bench(ps, torch, reps=10):
    """PER large: B = 2^24, 2^20 stratified draws, CDF path and tree path, and
    the whole update through psamp_per_round."""
    import synthetic_inputs as si
    d = si.per_large()
    p = torch.from_numpy(d["p"]).cuda()
    U = torch.from_numpy(d["U"]).cuda()
    cdf, tot = ps.build_cdf(p, d["alpha"])
    idx = ps.sample(cdf, tot, U)
    w = ps.is_weights(p, idx, d["alpha"], d["beta"])
    tree = torch.zeros(2 * p.numel(), dtype=torch.float32, device="cuda")
    ws = ps.Workspace(ps.build_cdf_workspace_size(p.numel()))
    iws = ps.Workspace(ps.is_weights_workspace_size(U.numel()))
    # the whole update (CDF, draws, IS, rewrite) on a copy that it rewrites
    p_pr = p.clone()
    newp = torch.from_numpy(si.generic_f32(U.numel(), 77, "lognormal")).cuda()
    pws = ps.Workspace(ps.per_round_workspace_size(p.numel(), U.numel()))
    calls = {
        "build_cdf": lambda: ps.build_cdf(p, d["alpha"], cdf=cdf, total=tot, ws=ws),
        "sample": lambda: ps.sample(cdf, tot, U, out=idx),
        "build_cdf_sample_fused": lambda: ps.build_cdf_sample(p, U, d["alpha"], cdf=cdf, total=tot,
                                                              out=idx, ws=ws),
        "is_weights": lambda: ps.is_weights(p, idx, d["alpha"], d["beta"], out=w, ws=iws),
        "per_round": lambda: ps.per_round(p_pr, U, d["alpha"], d["beta"], newp, out_idx=idx,
                                          out_w=w, cdf=cdf, total=tot, ws=pws),
        "tree_build": lambda: ps.segtree_build(tree, p, d["alpha"]),
        "tree_sample": lambda: ps.segtree_sample(tree, p.numel(), U, stratified=True, out=idx),
    }
    res = {k: round(loop_us(torch, fn, reps), 2) for k, fn in calls.items()}
    res["draws_per_s"] = round(U.numel() / ((res["sample"] + res["is_weights"]) * 1e-6))
    log(f"per large: {res}")
    return res


# ----------------------------------------------------------------- CPU side
def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _median_s(fn, runs):
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return statistics.median(ts)


def cpu_functions(gpu_us):
    """The oracle's steps one by one at their workloads (median of 3 runs; one
    run for the 2^24-leaf pointer tree), each next to the GPU's time of the
    same step (from this run's measurements, when taken) and the ratio."""
    import oracle
    import synthetic_inputs as si
    rows = {}

    def put(name, secs, what, gpu_key):
        us = secs * 1e6
        g = gpu_us.get(gpu_key)
        rows[name] = {"oracle_us": round(us, 1), "gpu_us": g, "workload": what,
                      "oracle_over_gpu": round(us / g, 1) if g else None}

    d = si.per_mid()
    p, U, a, b = d["p0"], d["U"][0], d["alpha"], d["beta"]
    C, T = oracle.build_cdf(p, a)
    t = oracle.thresholds(U, T, True)
    idx = oracle.search(C, t)
    put("scan", _median_s(lambda: oracle.build_cdf(p, a), 3), "PER mid: 262144 priorities",
        "build_cdf_per_mid")
    put("search", _median_s(lambda: oracle.search(C, oracle.thresholds(U, T, True)), 3),
        "PER mid: 8192 stratified draws", "sample_per_mid")
    put("is_weights", _median_s(lambda: oracle.is_weights(p, a, T, idx, b), 3),
        "PER mid: 8192 draws", "is_weights_per_mid")
    d = si.per_large()
    p, U, a, b = d["p"], d["U"], d["alpha"], d["beta"]
    C, T = oracle.build_cdf(p, a)
    t = oracle.thresholds(U, T, True)
    idx = oracle.search(C, t)
    put("scan_large", _median_s(lambda: oracle.build_cdf(p, a), 3), "PER large: 2^24 priorities",
        "build_cdf_per_large")
    put("search_large", _median_s(lambda: oracle.search(C, oracle.thresholds(U, T, True)), 3),
        "PER large: 2^20 stratified draws", "sample_per_large")
    put("is_weights_large", _median_s(lambda: oracle.is_weights(p, a, T, idx, b), 3),
        "PER large: 2^20 draws", "is_weights_per_large")
    del C, t, idx
    big = oracle.Tree("f32", 1 << 24)
    put("tree_build_large", _median_s(lambda: big.build(p, p.size, a), 1),
        "PER large: 2^24-leaf tree build", "tree_build_per_large")
    put("tree_sample_large", _median_s(lambda: big.sample(U, p.size, stratified=True), 1),
        "PER large: 2^20 stratified descents", "tree_sample_per_large")
    del big
    d = si.sumtree(rounds=3)
    tr = oracle.Tree("f32", 1 << 19).build(d["p0"], 500000, d["alpha"])
    it = iter(range(3))
    put("tree_update", _median_s(lambda: tr.update(d["idx"][next(it)], d["v"][0], d["alpha"]), 3),
        "sum tree: 1024 updates on 2^19 leaves", "tree_update_sumtree")
    put("tree_sample", _median_s(lambda: tr.sample(d["U"][0], 500000), 3),
        "sum tree: 1024 iid descents", "tree_sample_sumtree")
    d = si.resample()
    put("resample_rows", _median_s(lambda: oracle.resample_rows(d["lw"], d["u_row"]), 3),
        "particle resampling: 1024 rows x 4096", "resample_rows")
    return rows


def cpu_baseline(seconds, gpu_us):
    import oracle
    import synthetic_inputs as si
    d = si.per_mid()
    p = d["p0"].copy()
    steps = 0
    t0 = time.perf_counter()
    while True:
        for r in range(d["U"].shape[0]):
            C, T, t, idx = oracle.sample(p, d["alpha"], d["U"][r], True)
            oracle.is_weights(p, d["alpha"], T, idx, d["beta"])
            p = oracle.scatter_lww(p, idx, d["v"][r])
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    k, rounds = d["U"].shape[1], d["U"].shape[0]
    val = steps * rounds * k / el
    log(f"cpu oracle: {steps} steps in {el:.1f} s -> {val:.0f} indices/s")
    t1 = time.perf_counter()
    funcs = cpu_functions(gpu_us)
    log(f"cpu oracle functions ({time.perf_counter() - t1:.1f} s): {json.dumps(funcs)}")
    return {"value": round(val, 1), "unit": "sampled indices/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} full steps (32 updates of B=262144 / 8192 draws each) of the "
                      f"same seeded workload, {el:.1f} s, single thread",
            "cpu_model": cpu_model(), "host_threads": os.cpu_count(),
            "functions": funcs}


# ----------------------------------------------------------------- main
def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported "
              "(the library runs on a single MI355X; a sharded run would use these "
              "kernels per shard, with an all-gather of the shard totals)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import proportional_sampling_amd as ps
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    ps.lib()

    if args.only.startswith("scan:"):
        n = int(args.only.split(":")[1])
        scan_sweep(ps, torch, [n], reps=20)
        return
    if args.only == "pf":
        log(json.dumps(pf_bench(ps, torch, reps=20)))
        return
    if args.only == "per_large":
        log(json.dumps(per_large_bench(ps, torch)))
        return
    if args.only in ("rows", "sample_large"):
        # five calls of one kernel (row resampling at 1024 x 4096, or the
        # stratified sample of 2^20 draws over the PER-large CDF), nothing
        # else timed: for counter runs
        import synthetic_inputs as si
        if args.only == "rows":
            d = si.resample()
            lw = torch.from_numpy(d["lw"]).cuda()
            u = torch.from_numpy(d["u_row"]).cuda()
            out = torch.empty_like(lw, dtype=torch.int32)
            fn = lambda: ps.resample_rows(lw, u, out=out)
        else:
            d = si.per_large()
            cdf, tot = ps.build_cdf(torch.from_numpy(d["p"]).cuda(), d["alpha"])
            U = torch.from_numpy(d["U"]).cuda()
            idx = torch.empty(U.numel(), dtype=torch.int32, device="cuda")
            fn = lambda: ps.sample(cdf, tot, U, out=idx)
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        log(f"{args.only}: 5 calls")
        return
    if args.only.startswith("ceiling:"):
        n = int(args.only.split(":")[1])
        src = torch.rand(n, device="cuda")
        dst = torch.empty(n, dtype=torch.float64, device="cuda")
        flush = CacheFlush(torch)
        for rows, nt in ((8, True), (2, False)):
            for _ in range(10):
                flush()
                ps.ceiling_copy(src, dst, rows, nt)
        torch.cuda.synchronize()
        log(f"ceiling copy n={n}: 10 calls per geometry, each after a cache flush")
        return
    if args.only.startswith("copy:"):
        mib = int(args.only.split(":")[1])
        a = torch.ones(mib * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"copied {mib} MiB x5")
        return

    work = PerMid(ps, torch)
    if args.only == "per_mid":
        # profiling helper: only the timed region of the headline (the step
        # replayed from its HIP graph), nothing else
        for _ in range(args.warmup):
            work.step_fused()
        g = capture(torch, work.step_fused)
        gpu_s, _ = timed_steps(torch, g.replay, args.steps)
        log(f"PER mid graph: {1e3 * gpu_s / args.steps:.4f} ms/step over {args.steps} steps")
        return
    log(f"PER mid: warmup {args.warmup} steps")
    for _ in range(args.warmup):
        work.step_fused()
        work.step()
    # A step is 32 launches, each a few microseconds of GPU work: issued one
    # by one from Python the host cannot keep up, so the step is captured
    # once as a HIP graph and replayed (the kernels keep their state on the
    # device, so every replay is a fresh step).  The eager rate is reported
    # next to it.
    fused = capture(torch, work.step_fused) if not args.eager else work.step_fused
    gpu_s, wall_s = timed_steps(torch, fused if args.eager else fused.replay, args.steps)
    ms_per_step = 1e3 * gpu_s / args.steps
    draws = work.rounds * work.k * args.steps
    value = draws / gpu_s
    log(f"PER mid (fused update{'' if args.eager else ', graph'}): {ms_per_step:.3f} ms/step, "
        f"{value:.4g} indices/s (wall {wall_s:.3f} s)")
    eager_s, _ = timed_steps(torch, work.step_fused, args.steps)
    log(f"PER mid (fused update, eager launches): {1e3 * eager_s / args.steps:.3f} ms/step")
    sep = capture(torch, work.step) if not args.eager else work.step
    sep_s, _ = timed_steps(torch, work.step if args.eager else sep.replay, args.steps)
    log(f"PER mid (four separate calls): {1e3 * sep_s / args.steps:.3f} ms/step, "
        f"{draws / sep_s:.4g} indices/s")

    # The timed region holds only launches of the fused update kernel (one
    # per minibatch update, all on this stream), so its average launch
    # duration is the timed region over the number of launches.
    launches = work.rounds * args.steps
    avg_us = 1e6 * gpu_s / launches
    dom = "per_round"
    ab = work.algo_bytes(dom)
    ab_own = work.algo_bytes("per_round_own")
    achieved = ab / (avg_us * 1e-6) / 1e9
    traffic = profiled_traffic("per_round_per_mid.md")
    roofline = {"bound": "hbm", "kernel": KERNEL_NAMES[dom], "achieved": round(achieved, 2),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 5),
                "traffic": traffic, "algo_bytes_per_launch": ab,
                "own_bytes_per_launch": ab_own,
                "own_frac": round(ab_own / (avg_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 5),
                "avg_launch_us": round(avg_us, 3), "launches_timed": launches}
    log(f"k_per_round: {avg_us:.2f} us/launch, {achieved:.0f} GB/s algorithmic, traffic {traffic}")

    extra = {"launch": "eager" if args.eager else "hip graph of one step",
             "fused_eager": {"ms_per_step": round(1e3 * eager_s / args.steps, 4),
                             "indices_per_s": round(draws / eager_s, 1)},
             "separate_calls": {"ms_per_step": round(1e3 * sep_s / args.steps, 4),
                                "indices_per_s": round(draws / sep_s, 1)}}
    extra["separate_calls"]["per_call_us"] = work.per_call_us()
    extra["small"] = small_bench(ps, torch)
    if not args.no_extra:
        extra["scan_sweep"] = scan_sweep(ps, torch, [1 << 22, 1 << 23, 1 << 24, 1 << 25, 1 << 26])
        extra["sumtree"] = sumtree_bench(ps, torch)
        extra["replay"] = replay_bench(ps, torch)
        extra["resample_rows"] = resample_bench(ps, torch)
        extra["pf_step"] = pf_bench(ps, torch)
        extra["per_large"] = per_large_bench(ps, torch)

    cpu = None
    if not args.no_cpu:
        pc = extra["separate_calls"]["per_call_us"]
        gpu_us = {"build_cdf_per_mid": pc["build_cdf"], "sample_per_mid": pc["sample"],
                  "is_weights_per_mid": pc["is_weights"]}
        if "per_large" in extra:
            pl = extra["per_large"]
            gpu_us.update({"build_cdf_per_large": pl["build_cdf"],
                           "sample_per_large": pl["sample"],
                           "is_weights_per_large": pl["is_weights"],
                           "tree_build_per_large": pl["tree_build"],
                           "tree_sample_per_large": pl["tree_sample"],
                           "tree_update_sumtree": extra["sumtree"]["update_us"],
                           "tree_sample_sumtree": extra["sumtree"]["sample_us"],
                           "resample_rows": extra["resample_rows"]["us"]})
        cpu = cpu_baseline(args.cpu_seconds, gpu_us)
        extra["gpu_over_cpu"] = round(value / cpu["value"], 1)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "sampled indices/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f64", "data": "synthetic",
        "config": {"workload": "PER mid: B=262144 fp32 priorities ~ Exp(1)+1e-6, alpha=0.6, "
                               "beta=0.4; 32 minibatch updates per step, each rebuilding the "
                               "CDF, drawing 8192 stratified samples (+ IS weights) and "
                               "rewriting those 8192 priorities",
                   "B": work.n, "draws": work.k, "updates_per_step": work.rounds,
                   "parallelism": "single GPU"},
        "roofline": roofline, "cpu_baseline": cpu, "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
