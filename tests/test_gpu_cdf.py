"""GPU parity of the CDF path (scan, search, IS weights, rewrite) against
the CPU oracle, through the C ABI (proportional_sampling_amd binding)."""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from parity_util import assert_indices, rel_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ps():
    import proportional_sampling_amd as ps
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ps.lib()
    return ps


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def check_is_weights(w_g, p, alpha, T_o, idx_g, idx_o, beta, what, int_mode=False):
    """IS weights against the oracle, always: on the GPU's index array (which
    assert_indices has already matched to the oracle's own draws, up to
    excused boundary ties), so that an excused index flip cannot move the
    normaliser and skip the comparison; and, where the two index arrays are
    the same, also against the oracle's own chain of draws."""
    isw = oracle.is_weights_int if int_mode else oracle.is_weights
    args = (p, T_o) if int_mode else (p, alpha, T_o)
    w_v = isw(*args, np.asarray(idx_g, np.int32), beta)
    e = rel_err(w_g, w_v)
    say(f"  {what}: IS max rel err {e:.3e} (on the GPU's indices)")
    assert e <= 1e-6, what
    if np.array_equal(idx_g, idx_o):
        assert rel_err(w_g, isw(*args, idx_o, beta)) <= 1e-6, what
    assert w_g.max() == 1.0 and np.all(w_g > 0), what


SIZES = [1, 2, 63, 64, 1023, 1024, 1025, 4095, 4096, 4097, 65536 + 3, 100003,
         (1 << 20), (1 << 20) + 1, (1 << 22) + 17]


@pytest.mark.parametrize("n", SIZES)
def test_scan_int_bit_exact(ps, n):
    say(f"scan int n={n}")
    q = si.sweep_u32(n)
    C_o, T_o = oracle.build_cdf_int(q)
    cdf, tot = ps.build_cdf(dev(q))
    C_g = host(cdf)
    assert C_g.dtype == np.uint64
    assert np.array_equal(C_g, C_o)
    assert int(host(tot)[0]) == T_o


@pytest.mark.parametrize("n", SIZES)
def test_scan_fp(ps, n):
    say(f"scan fp n={n}")
    p = si.sweep_f32(n)
    C_o, T_o = oracle.build_cdf(p, 0.7)
    ws = ps.Workspace(ps.build_cdf_workspace_size(n))
    cdf, tot = ps.build_cdf(dev(p), 0.7, ws=ws)
    C_g = host(cdf)
    e = rel_err(C_g, C_o)
    say(f"  max rel CDF err {e:.3e}")
    assert e <= 1e-6
    assert e <= 1e-12            # what fp64 weights and sums actually give
    assert host(tot)[0] == C_g[-1]
    # deterministic: the same bits on a second run with the same workspace
    cdf2, _ = ps.build_cdf(dev(p), 0.7, ws=ws)
    assert np.array_equal(host(cdf2), C_g)
    assert ws.errors() == 0


def test_scan_many_groups(ps):
    """2^27 + 12345 elements: 16386 tiles in 257 groups of 64, more than one
    lookback round (128 group totals per round) -- integer mode bit for bit,
    fp within the tolerance, T = C_{n-1}."""
    n = (1 << 27) + 12345
    say(f"scan int+fp n={n}")
    q = si.sweep_u32(n)
    C_o, T_o = oracle.build_cdf_int(q)
    cdf, tot = ps.build_cdf(dev(q))
    assert np.array_equal(host(cdf), C_o)
    assert int(host(tot)[0]) == T_o
    del cdf, C_o, q
    p = si.sweep_f32(n)
    C_o, T_o = oracle.build_cdf(p, 0.7)
    cdf, tot = ps.build_cdf(dev(p), 0.7)
    C_g = host(cdf)
    e = rel_err(C_g, C_o)
    say(f"  max rel CDF err {e:.3e}")
    assert e <= 1e-12
    assert np.all(np.diff(C_g) >= 0)
    assert host(tot)[0] == C_g[-1]


@pytest.mark.parametrize("n", [(1 << 20) + 1000, 8000])
@pytest.mark.parametrize("alpha", [0.05, 0.6, 1.0, 2.0, 7.5, 16.0, 17.0])
def test_scan_pow_extremes_large_tiles(ps, alpha, n):
    """8-row tiles (n > 2^20) and small inputs (n <= 8192), where p^alpha
    comes from per-workgroup tables for alpha <= 16 (17 takes the general
    pow): subnormal, tiny, huge, zero and unit priorities.  The first 4096
    elements are all tiny, so the CDF there checks the relative accuracy of
    small weights; the rest spans the whole float range alpha allows without
    overflow.  The fused update on the same input gives the same CDF."""
    rng = np.random.default_rng(int(alpha * 100))
    hi = min(38.0, 300.0 / alpha)
    lo = max(-44.5, -300.0 / alpha)
    e = rng.uniform(lo, hi, n)
    e[:4096] = rng.uniform(lo, min(lo + 4.0, hi), 4096)
    p = (10.0 ** e).astype(np.float32)
    p[5000::97] = 0.0
    p[6001::89] = 1.0
    p[7002::83] = np.float32(1.4e-45)              # the smallest subnormal
    C_o, T_o = oracle.build_cdf(p, alpha)
    cdf, tot = ps.build_cdf(dev(p), alpha)
    C_g = host(cdf)
    pos = C_o > 0
    e_rel = float(np.max(np.abs(C_g[pos] - C_o[pos]) / C_o[pos]))
    say(f"pow extremes alpha={alpha} n={n}: max rel CDF err {e_rel:.3e}")
    assert np.all(C_g[~pos] == 0)
    assert e_rel <= 1e-12
    assert np.all(np.diff(C_g) >= 0)
    if n <= 8192:
        U = si.uniform_f32(np.random.default_rng(n), 1000)
        _, _, cdf_r, _ = ps.per_round(dev(p), dev(U), alpha, 0.5)
        assert np.array_equal(host(cdf_r), C_g)


@pytest.mark.parametrize("alpha", [12.5, 15.97, 16.0])
def test_scan_pow_table_range_ends(ps, alpha):
    """The table pow of 8-row tiles at both ends of the double range.  (1)
    One weight at a time from 0.95 DBL_MAX to just below it, 200 priorities
    (its factor 2^(alpha e) times c_k^(-alpha) alone may pass DBL_MAX while
    the weight does not): the CDF's last value, that weight, within 1e-12
    of the oracle's and never NaN.  (2) 64 weights just above DBL_MIN (where
    2^(alpha e) alone is subnormal): the CDF within 1e-12 of the oracle's.
    (3) A weight that overflows: 0 before it, +inf from it on, no NaN."""
    n = (1 << 20) + 4096 + 3
    buf = torch.zeros(n, dtype=torch.float32, device="cuda")
    cand = np.exp2((1024.0 + np.log2(np.linspace(0.95, 0.9999, 200))) / alpha).astype(np.float32)
    w_o = oracle.weights(cand, alpha)
    assert np.all(np.isfinite(w_o))
    got = np.empty(cand.size)
    for i, pv in enumerate(cand):
        buf[123] = float(pv)
        got[i] = host(ps.build_cdf(buf, alpha)[0][-1:])[0]
    assert not np.any(np.isnan(got))
    e_rel = float(np.max(np.abs(got - w_o) / w_o))
    say(f"alpha={alpha}: weights near DBL_MAX, max rel err {e_rel:.3e}")
    assert e_rel <= 1e-12
    # weights just above DBL_MIN
    q = np.zeros(n, np.float32)
    q[200000:200064] = (np.float32(np.exp2(-1021.5 / alpha))
                        * np.float32(1.0 + np.arange(64) / 128.0))
    C_o, _ = oracle.build_cdf(q, alpha)
    C_g = host(ps.build_cdf(dev(q), alpha)[0])
    pos = C_o > 0
    assert C_o[200000] >= 2.2250738585072014e-308
    assert np.all(C_g[~pos] == 0)
    assert float(np.max(np.abs(C_g[pos] - C_o[pos]) / C_o[pos])) <= 1e-12
    # an overflowing weight
    q[:] = 0
    q[77] = np.float32(np.exp2(1025.0 / alpha))
    q[5000] = 1.0
    C_g = host(ps.build_cdf(dev(q), alpha)[0])
    assert np.all(C_g[:77] == 0) and np.all(np.isposinf(C_g[77:]))


# Large-tile sizes (8192-element tiles) past what one round of workgroups
# covers on 256 CUs: a one-element tail, whole tiles only, a ragged tail,
# several rounds.
LARGE_SIZES = [512 * 8192 + 1, 1 << 23, 513 * 8192 + 4, 3 * (1 << 22) + 4100, (1 << 24) + 12]


@pytest.mark.parametrize("n", LARGE_SIZES)
def test_scan_large_sizes(ps, n):
    """Integer mode bit for bit against the oracle; fp mode within 1e-12 of
    the oracle and bit for bit equal to the CDF of the fused scan + sample
    (a different pair of kernels over the same tiles); T = C_{n-1}; one
    workspace shared with a small scan in between."""
    say(f"scan large n={n}")
    ws = ps.Workspace(ps.build_cdf_workspace_size(n))
    q = si.sweep_u32(n)
    C_o, T_o = oracle.build_cdf_int(q)
    cdf, tot = ps.build_cdf(dev(q), ws=ws)
    assert np.array_equal(host(cdf), C_o)
    assert int(host(tot)[0]) == T_o
    del cdf, C_o
    small, _ = ps.build_cdf(dev(q[:5000]), ws=ws)
    assert np.array_equal(host(small), np.cumsum(q[:5000].astype(np.uint64)))
    p = si.sweep_f32(n)
    C_o, T_o = oracle.build_cdf(p, 0.7)
    P = dev(p)
    cdf, tot = ps.build_cdf(P, 0.7, ws=ws)
    C_g = host(cdf)
    e = rel_err(C_g, C_o)
    say(f"  max rel CDF err {e:.3e}")
    assert e <= 1e-12
    assert host(tot)[0] == C_g[-1]
    _, cdf_f, tot_f = ps.build_cdf_sample(P, dev(si.uniform_f32(np.random.default_rng(n), 64)),
                                          0.7, ws=ws)
    assert np.array_equal(host(cdf_f), C_g)
    assert np.array_equal(host(tot_f), host(tot))
    assert ws.errors() == 0


def test_scan_all_ones_exact(ps):
    n = (1 << 21) + 5
    cdf, tot = ps.build_cdf(torch.ones(n, dtype=torch.float32, device="cuda"), 0.6)
    assert np.array_equal(host(cdf), np.arange(1, n + 1, dtype=np.float64))
    assert host(tot)[0] == float(n)


def test_scan_f32_cdf_variant(ps):
    p = si.sweep_f32(300007)
    C_o, T_o = oracle.build_cdf(p, 0.7)
    cdf, tot = ps.build_cdf(dev(p), 0.7, cdf_dtype=torch.float32)
    C_g = host(cdf)
    assert C_g.dtype == np.float32
    assert rel_err(C_g, C_o) <= 1e-6
    assert host(tot)[0] == C_g[-1]


def test_scan_workspace_reuse_across_sizes(ps):
    # alternate parities and sizes on one workspace; zeros and a tail
    ws = ps.Workspace(ps.build_cdf_workspace_size(1 << 21))
    for n in [(1 << 21), 7, 5000, (1 << 21) - 3, 1, 300000, 4096]:
        q = si.sweep_u32(n)
        q[::7] = 0
        C_o, T_o = oracle.build_cdf_int(q)
        cdf, tot = ps.build_cdf(dev(q), ws=ws)
        assert np.array_equal(host(cdf), C_o), n
    assert ws.errors() == 0


def test_scan_unaligned_views(ps):
    q = si.sweep_u32(100001)
    t = dev(q)
    sub = t[3:]                      # 12-byte offset: scalar path
    C_o, _ = oracle.build_cdf_int(q[3:])
    cdf = torch.empty(sub.numel() + 1, dtype=torch.uint64, device="cuda")[1:]
    ps.build_cdf(sub, cdf=cdf)
    assert np.array_equal(host(cdf), C_o)


def _per_round(ps, p, U, alpha, beta, ws=None):
    Pd = dev(p)
    cdf, tot = ps.build_cdf(Pd, alpha, ws=ws)
    idx = ps.sample(cdf, tot, dev(U), stratified=True)
    w = ps.is_weights(Pd, idx, alpha, beta)
    return host(cdf), host(tot)[0], host(idx), host(w)


def test_per_small_cfg(ps):
    d = si.per_small()
    say("PER small: B=8192 k=1024")
    C_o, T_o, t_o, idx_o = oracle.sample(d["p"], d["alpha"], d["U"], True)
    C_g, T_g, idx_g, w_g = _per_round(ps, d["p"], d["U"], d["alpha"], d["beta"])
    assert rel_err(C_g, C_o) <= 1e-6
    assert_indices(idx_g, idx_o, t_o, C_o, T_o, "per_small")
    assert np.all(np.diff(idx_g) >= 0)
    check_is_weights(w_g, d["p"], d["alpha"], T_o, idx_g, idx_o, d["beta"], "per_small")


@pytest.mark.parametrize("k,strat", [(1, True), (7, True), (1000, True), (1024, False),
                                     (5000, True), (8192, True), (8193, True), (100000, False),
                                     (1 << 18, True)])
def test_sample_and_weights_shapes(ps, k, strat):
    say(f"sample k={k} stratified={strat}")
    p = si.generic_f32(262144, 77 + k, "exp")
    U = si.uniform_f32(np.random.default_rng(k), k)
    C_o, T_o, t_o, idx_o = oracle.sample(p, 0.6, U, strat)
    Pd = dev(p)
    cdf, tot = ps.build_cdf(Pd, 0.6)
    idx = host(ps.sample(cdf, tot, dev(U), stratified=strat))
    assert_indices(idx, idx_o, t_o, C_o, T_o, f"k={k}")
    w_g = host(ps.is_weights(Pd, dev(idx), 0.6, 0.4))
    check_is_weights(w_g, p, 0.6, T_o, idx, idx_o, 0.4, f"k={k}")


def test_sample_edges(ps):
    # zero-weight items, ties, t = 0 (U = 0 at i = 0), and the clamp
    p = np.array([0.0, 2.0, 0.0, 0.0, 1.0, 0.0], np.float32)
    U = np.array([0.0, 0.5, 0.999999, 0.0], np.float32)
    for strat in (True, False):
        C_o, T_o, t_o, idx_o = oracle.sample(p, 1.0, U, strat)
        cdf, tot = ps.build_cdf(dev(p), 1.0)
        idx = host(ps.sample(cdf, tot, dev(U), stratified=strat))
        assert_indices(idx, idx_o, t_o, C_o, T_o, f"edges strat={strat}")
    # a single item
    cdf, tot = ps.build_cdf(dev(np.array([3.0], np.float32)), 0.5)
    assert list(host(ps.sample(cdf, tot, dev(np.array([0.0, 0.7], np.float32))))) == [0, 0]


def _host_search(C, t):
    """min(first j with C_j >= t, n - 1) -- numpy's left searchsorted."""
    return np.searchsorted(C, t, side="left").clip(0, C.size - 1).astype(np.int32)


# (n, k, CDF dtype, weights): the draws placed from the CDF's side (small
# CDFs, dense draws) and by binary search (otherwise) must both be the
# lower bound of the definition on the same CDF, bit for bit.  The CDF is
# built on the host (a plain cumulative sum), so only the search runs on the
# GPU; the thresholds are the same IEEE double operations on both sides.
SEARCH_CASES = [(1000, 100000, "f64", "exp"), (262147, 8191, "f64", "exp"),
                (65539, 1 << 16, "f32", "exp"), (10000, 8192, "f64", "heavy"),
                (4096, 4096, "f64", "ones"), (300000, 5000, "f64", "zeros"),
                (1 << 20, 1 << 14, "f64", "exp"), (3, 7, "f64", "exp"), (1, 5, "f32", "exp"),
                ((1 << 20) + 4, 1 << 15, "f64", "exp"), (5000, 10, "f64", "exp")]


@pytest.mark.parametrize("n,k,dt,kind", SEARCH_CASES)
def test_stratified_search_host_cdf(ps, n, k, dt, kind):
    say(f"stratified search n={n} k={k} {dt} {kind}")
    rng = np.random.default_rng(n + k)
    if kind == "ones":
        w = np.ones(n)
    elif kind == "heavy":
        w = np.full(n, 1e-3)
        w[n // 3] = 1e6                         # most draws land on one element
    elif kind == "zeros":
        w = rng.exponential(1.0, n)
        w[rng.random(n) < 0.7] = 0.0            # long runs of equal CDF values
    else:
        w = rng.exponential(1.0, n)
    C = np.cumsum(w)
    if dt == "f32":
        C = C.astype(np.float32)
    U = si.uniform_f32(rng, k)
    U[0] = 0.0
    T = float(C[-1])
    t = oracle.thresholds(U, T, True)
    expect = oracle.search_f32cdf(C, t) if dt == "f32" else oracle.search(C, t)
    assert np.array_equal(expect, _host_search(C.astype(np.float64), t))
    cdf = dev(C)
    idx = host(ps.sample(cdf, cdf[-1:].clone(), dev(U), stratified=True))
    assert np.array_equal(idx, expect)


@pytest.mark.parametrize("case", ["one_half", "four_quarters", "all_on_one", "int_one_half"])
def test_stratified_sample_heavy_elements(ps, case):
    """Elements that receive a large share of the draws (one with half the
    mass, four with a quarter each, one with all of it; 2^22 priorities,
    2^18 draws): indices against the oracle under the excuse rule and
    exactly the lower bounds on the GPU's own CDF; every call well inside a
    bound that a single lane writing a heavy element's draws alone (tens of
    milliseconds here) would break."""
    import time
    n, k = 1 << 22, 1 << 18
    rng = np.random.default_rng(321)
    if case == "int_one_half":
        q = rng.integers(1, 1 << 10, n, dtype=np.uint32)
        q[123457] = np.uint32(min(int(q.astype(np.int64).sum()), (1 << 32) - 1))
        r = si.uniform_u32(rng, k)
        Q, R = dev(q), dev(r)
        cdf, tot = ps.build_cdf(Q)
        idx = ps.sample(cdf, tot, R, stratified=True)
        _, _, _, idx_o = oracle.sample_int(q, r, True)
        assert np.array_equal(host(idx), idx_o)
        calls = lambda: ps.sample(cdf, tot, R, stratified=True, out=idx)
    else:
        p = (rng.random(n, dtype=np.float32) + np.float32(0.01))
        total = float(p.astype(np.float64).sum())
        if case == "one_half":
            p[123457] = np.float32(total)
        elif case == "four_quarters":
            p[[0, 1_000_003, 2_500_000, n - 1]] = np.float32(total / 4)
        else:
            p[:] = 0.0
            p[777777] = 1.0
        U = si.uniform_f32(rng, k)
        P, Ud = dev(p), dev(U)
        cdf, tot = ps.build_cdf(P, 1.0)
        idx = ps.sample(cdf, tot, Ud, stratified=True)
        C_o, T_o, t_o, idx_o = oracle.sample(p, 1.0, U, True)
        assert_indices(host(idx), idx_o, t_o, C_o, T_o, f"heavy {case}")
        C_g, T_g = host(cdf), float(host(tot)[0])
        t_g = ((np.arange(k) + U.astype(np.float64)) / k) * T_g
        assert np.array_equal(host(idx), np.minimum(np.searchsorted(C_g, t_g, side="left"), n - 1))
        calls = lambda: ps.sample(cdf, tot, Ud, stratified=True, out=idx)
    calls()
    torch.cuda.synchronize()
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        calls()
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
    say(f"heavy {case}: {1e6 * min(times):.0f} us per call")
    assert min(times) < 5e-3, times


def test_stratified_search_int_host_cdf(ps):
    """Integer mode: exact thresholds from Python integers, host CDF."""
    for n, k in [(4097, 5000), (300007, 1 << 16), (17, 64), (1 << 20, 1 << 14)]:
        rng = np.random.default_rng(n)
        q = rng.integers(0, 1 << 20, n, dtype=np.uint64)
        q[0] = max(int(q[0]), 1)
        C = np.cumsum(q, dtype=np.uint64)
        r = rng.integers(0, 1 << 32, k, dtype=np.uint64).astype(np.uint32)
        T = int(C[-1])
        t = np.array([(((i << 32) + int(r[i])) * T) // (k << 32) + 1 for i in range(k)],
                     dtype=np.uint64)
        expect = _host_search(C, t)
        cdf = dev(C)
        idx = host(ps.sample(cdf, cdf[-1:].clone(), dev(r), stratified=True))
        assert np.array_equal(idx, expect), (n, k)


@pytest.mark.parametrize("k,strat", [(1, True), (1000, True), (1 << 16, True), (1000, False),
                                     (4099, False)])
def test_sample_int_bit_exact(ps, k, strat):
    say(f"sample int k={k} stratified={strat}")
    d = si.per_large_int(n=300007, k=k)
    C_o, T_o, t_o, idx_o = oracle.sample_int(d["q"], d["r"], strat)
    Q = dev(d["q"])
    cdf, tot = ps.build_cdf(Q)
    idx = host(ps.sample(cdf, tot, dev(d["r"]), stratified=strat))
    assert np.array_equal(idx, idx_o)
    w_g = host(ps.is_weights(Q, dev(idx), 1.0, d["beta"]))
    w_o = oracle.is_weights_int(d["q"], T_o, idx_o, d["beta"])
    assert rel_err(w_g, w_o) <= 1e-6


def test_is_weights_workspace_reuse(ps):
    """One workspace across batch sizes on all three paths (blocks of 1024
    samples up to 8192; blocks of 4096 exchanging minima while they can all
    be resident; two kernels beyond 1024 such blocks), each call against the
    oracle's closed form; a block counter of the two-kernel path left at a
    stray value is back in step after one call."""
    n = 262144
    p = si.generic_f32(n, 91, "exp")
    Pd = dev(p)
    big = (4 << 20) + 5
    ws = ps.Workspace(ps.is_weights_workspace_size(big))
    rng = np.random.default_rng(4)
    # ((1 << 20) + 1: 257 blocks of 4096, more than one per CU can be
    # resident on 256 CUs, so the occupancy check sends it to two kernels)
    for step, k in enumerate([8192, 1000, 5000, 1 << 16, big, 1024, 8193, 3, 8192, 70001,
                              big, 1 << 20, 4097, (1 << 20) + 1, 1 << 20]):
        if step == 10:
            ws.buf.view(torch.int32)[0] = 5         # stray counter: this call is not checked
            ps.is_weights(Pd, dev(rng.integers(0, n, big).astype(np.int32)), 0.6, 0.4, ws=ws)
        idx = np.sort(rng.integers(0, n, k)).astype(np.int32)
        w_g = host(ps.is_weights(Pd, dev(idx), 0.6, 0.4, ws=ws))
        w_o = oracle.is_weights(p, 0.6, 1.0, idx, 0.4)
        assert rel_err(w_g, w_o) <= 1e-6, (step, k)
        assert w_g.max() == 1.0
    assert ws.errors() == 0


def test_per_mid_cfg_32_rounds(ps):
    """PER mid: B=262144, 32 updates of (CDF rebuild, 8192 stratified draws,
    IS weights, rewrite of the drawn priorities).  The oracle runs its own
    chain; both must agree on every index of every round."""
    d = si.per_mid()
    n, k = d["p0"].size, d["U"].shape[1]
    p_o = d["p0"].copy()
    Pd = dev(d["p0"])
    ws = ps.Workspace(ps.build_cdf_workspace_size(n))
    exc_total = 0
    for r in range(d["U"].shape[0]):
        C_o, T_o, t_o, idx_o = oracle.sample(p_o, d["alpha"], d["U"][r], True)
        cdf, tot = ps.build_cdf(Pd, d["alpha"], ws=ws)
        idx = ps.sample(cdf, tot, dev(d["U"][r]), stratified=True)
        w = ps.is_weights(Pd, idx, d["alpha"], d["beta"])
        # stratified indices are non-decreasing: the grouped rewrite applies
        ps.scatter_lww(Pd, idx, dev(d["v"][r]), grouped=True)
        idx_g = host(idx)
        exc = assert_indices(idx_g, idx_o, t_o, C_o, T_o, f"per_mid round {r}")
        exc_total += exc
        assert exc == 0, "chains would fork; the oracle never takes GPU data"
        w_o = oracle.is_weights(p_o, d["alpha"], T_o, idx_o, d["beta"])
        assert rel_err(host(w), w_o) <= 1e-6
        p_o = oracle.scatter_lww(p_o, idx_o, d["v"][r])
        assert np.array_equal(host(Pd), p_o)
    assert exc_total < 1e-4 * k * d["U"].shape[0]


def test_scatter_lww(ps):
    n = 10000
    rng = np.random.default_rng(5)
    p = si.generic_f32(n, 6)
    Pd = dev(p)
    ws = ps.Workspace(ps.scatter_workspace_size(n, 1))
    for m in (1, 100, 5000, 30000):
        idx = rng.integers(-3, n + 3, m).astype(np.int32)     # some out of range
        v = si.generic_f32(m, m)
        ok = (idx >= 0) & (idx < n)
        p = oracle.scatter_lww(p, idx[ok], v[ok])
        ps.scatter_lww(Pd, dev(idx), dev(v), ws)
        assert np.array_equal(host(Pd), p), m
    # the owner words are all zero again after each call
    assert int(host(ws.buf).astype(np.int64).sum()) == 0
    # grouped indices (sorted, with runs): one kernel, no workspace
    for m in (1, 7, 8192, 20000):
        idx = np.sort(rng.integers(-2, n + 2, m)).astype(np.int32)
        v = si.generic_f32(m, m + 1)
        ok = (idx >= 0) & (idx < n)
        p = oracle.scatter_lww(p, idx[ok], v[ok])
        ps.scatter_lww(Pd, dev(idx), dev(v), grouped=True)
        assert np.array_equal(host(Pd), p), ("grouped", m)


def test_per_large_cfg(ps):
    """PER large: B=2^24 LogNormal(0,2), alpha=0.7, beta=0.5, 2^20 draws."""
    d = si.per_large()
    say("PER large: oracle (serial) ...")
    C_o, T_o, t_o, idx_o = oracle.sample(d["p"], d["alpha"], d["U"], True)
    say("PER large: GPU ...")
    C_g, T_g, idx_g, w_g = _per_round(ps, d["p"], d["U"], d["alpha"], d["beta"])
    e = rel_err(C_g, C_o)
    say(f"  max rel CDF err {e:.3e}; T gpu {T_g!r} oracle {T_o!r}")
    assert e <= 1e-6
    assert_indices(idx_g, idx_o, t_o, C_o, T_o, "per_large")
    check_is_weights(w_g, d["p"], d["alpha"], T_o, idx_g, idx_o, d["beta"], "per_large")


def test_per_large_int_cfg(ps):
    d = si.per_large_int()
    C_o, T_o, t_o, idx_o = oracle.sample_int(d["q"], d["r"], True)
    Q = dev(d["q"])
    cdf, tot = ps.build_cdf(Q)
    assert np.array_equal(host(cdf), C_o)
    assert int(host(tot)[0]) == T_o
    idx = host(ps.sample(cdf, tot, dev(d["r"]), stratified=True))
    assert np.array_equal(idx, idx_o)
    w_g = host(ps.is_weights(Q, dev(idx), 1.0, d["beta"]))
    w_o = oracle.is_weights_int(d["q"], T_o, idx_o, d["beta"])
    assert rel_err(w_g, w_o) <= 1e-6


@pytest.mark.timeout(400)
def test_max_n_int(ps):
    """The largest n the ABI takes, 2^31 - 1 (int32 indices; 262144 tiles in
    4096 lookback groups, a ragged last tile, element-wise loads since n is
    odd), integer mode so that every check is exact: the CDF and T bit for
    bit; stratified draws through the binary search (k = 2^20 < n/64) and
    from the CDF's side (k = 2^25 >= n/64), each equal to the oracle's
    merge search over the oracle's thresholds; IS weights of the first."""
    n = (1 << 31) - 1
    say(f"max n int: n={n} generating")
    q = si.sweep_u32(n)
    C_o, T_o = oracle.build_cdf_int(q)
    say("  oracle CDF done; GPU scan")
    Q = dev(q)
    cdf, tot = ps.build_cdf(Q)
    C_g = host(cdf)
    assert int(host(tot)[0]) == T_o
    assert np.array_equal(C_g, C_o)
    del C_g
    say("  CDF bit-exact; searches")
    rng = np.random.default_rng(31)
    for k in (1 << 20, 1 << 25):
        r = si.uniform_u32(rng, k)
        t_o = oracle.thresholds_int(r, T_o, True)
        idx_o = oracle.search_int(C_o, t_o)
        idx = host(ps.sample(cdf, tot, dev(r), stratified=True))
        say(f"  k={k}: {int(np.sum(idx != idx_o))} index mismatches")
        assert np.array_equal(idx, idx_o)
        if k == 1 << 20:
            w_g = host(ps.is_weights(Q, dev(idx), 1.0, 0.5))
            w_o = oracle.is_weights_int(q, T_o, idx_o, 0.5)
            assert rel_err(w_g, w_o) <= 1e-6
        del r, t_o, idx_o, idx
    del cdf, tot, Q, C_o, q
    torch.cuda.empty_cache()


# ------------------------------------------------------------ fused update
def check_round_vs_oracle(p, U, newp, alpha, beta, C_g, T_g, idx_g, w_g, p_g, what):
    """One PER update (CDF, stratified draws, IS weights, rewrite) against
    the oracle's own steps on the same inputs.  Returns the number of
    excused index mismatches (boundary ties) and the oracle's rewritten
    priorities (its own draws)."""
    C_o, T_o, t_o, idx_o = oracle.sample(p, alpha, U, True)
    e = rel_err(C_g, C_o)
    assert e <= 1e-12, f"{what}: CDF rel err {e:.3e}"
    assert abs(float(T_g) - T_o) <= 1e-12 * T_o, what
    exc = assert_indices(idx_g, idx_o, t_o, C_o, T_o, what)
    check_is_weights(w_g, p, alpha, T_o, idx_g, idx_o, beta, what)
    p_next = p
    if newp is not None:
        # rewritten priorities: the oracle's last-write-wins scatter of the
        # new values at the draws (at the GPU's draws when an excused tie
        # moved one: the rest of the rewrite must still be exact)
        p_next = oracle.scatter_lww(p, idx_o, newp)
        p_chk = p_next if exc == 0 else oracle.scatter_lww(p, idx_g, newp)
        assert np.array_equal(p_g, p_chk), f"{what}: rewritten priorities"
    return exc, p_next


def _separate_round(ps, p, U, newp, alpha, beta):
    """The four separate calls, for comparison with the fused update."""
    Pd = dev(p)
    cdf, tot = ps.build_cdf(Pd, alpha)
    idx = ps.sample(cdf, tot, dev(U), stratified=True)
    w = ps.is_weights(Pd, idx, alpha, beta)
    if newp is not None:
        ps.scatter_lww(Pd, idx, dev(newp), grouped=True)
    return host(cdf), host(tot), host(idx), host(w), host(Pd)


@pytest.mark.parametrize("n,k", [(1, 1), (1000, 7), (1024, 1024), (5000, 300), (8192, 1024),
                                 (262144, 8192), (262147, 8191), (100000, 100000),
                                 (1 << 20, 4096), (1500001, 8192), (1 << 21, 20000),
                                 ((1 << 22) + 5, 1 << 16), (3 * (1 << 21) + 7, 8192),
                                 ((1 << 23) + 1, 1 << 18)])
def test_per_round_equals_separate_calls(ps, n, k):
    say(f"per_round n={n} k={k}")
    p = si.generic_f32(n, n + 13, "exp")
    p[::17] = 0.0                          # zero-weight items too
    p[0] = max(p[0], np.float32(1e-3))
    U = si.uniform_f32(np.random.default_rng(k + 1), k)
    newp = si.generic_f32(k, k + 2, "exp")
    C_s, T_s, idx_s, w_s, p_s = _separate_round(ps, p, U, newp, 0.6, 0.4)
    Pd = dev(p)
    idx, w, cdf, tot = ps.per_round(Pd, dev(U), 0.6, 0.4, dev(newp))
    assert np.array_equal(host(cdf), C_s)
    assert np.array_equal(host(tot), T_s)
    assert np.array_equal(host(idx), idx_s)
    assert np.array_equal(host(w), w_s)
    assert np.array_equal(host(Pd), p_s)
    # the CDF is exactly monotone and ends at T
    assert np.all(np.diff(C_s) >= 0) and C_s[-1] == T_s[0]
    # and the fused update meets the oracle directly
    check_round_vs_oracle(p, U, newp, 0.6, 0.4, C_s, T_s[0], idx_s, w_s, p_s,
                          f"per_round n={n} k={k}")


def test_per_round_chain_vs_oracle(ps):
    """PER mid through the fused update: 32 chained updates against the
    oracle's own chain."""
    d = si.per_mid()
    n, k = d["p0"].size, d["U"].shape[1]
    p_o = d["p0"].copy()
    Pd = dev(d["p0"])
    ws = ps.Workspace(ps.per_round_workspace_size(n, k))
    for r in range(d["U"].shape[0]):
        C_o, T_o, t_o, idx_o = oracle.sample(p_o, d["alpha"], d["U"][r], True)
        idx, w, cdf, tot = ps.per_round(Pd, dev(d["U"][r]), d["alpha"], d["beta"],
                                        dev(d["v"][r]), ws=ws)
        exc = assert_indices(host(idx), idx_o, t_o, C_o, T_o, f"per_round chain {r}")
        assert exc == 0
        assert rel_err(host(cdf), C_o) <= 1e-12
        w_o = oracle.is_weights(p_o, d["alpha"], T_o, idx_o, d["beta"])
        assert rel_err(host(w), w_o) <= 1e-6
        p_o = oracle.scatter_lww(p_o, idx_o, d["v"][r])
        assert np.array_equal(host(Pd), p_o)
    assert ws.errors() == 0


def test_per_round_graph_replays(ps):
    """The fused update captured in a HIP graph (as bench.py runs it): every
    replay, with eager work and synchronisations in between, gives the same
    bits as the same updates launched one by one."""
    d = si.per_mid()
    rounds = 4
    n, k = d["p0"].size, d["U"].shape[1]
    a, b = d["alpha"], d["beta"]
    U = [dev(d["U"][r]) for r in range(rounds)]
    V = [dev(d["v"][r]) for r in range(rounds)]
    p_g, p_e = dev(d["p0"]), dev(d["p0"])
    ws_g = ps.Workspace(ps.per_round_workspace_size(n, k))
    ws_e = ps.Workspace(ps.per_round_workspace_size(n, k))
    out_g = [(torch.empty(k, dtype=torch.int32, device="cuda"),
              torch.empty(k, dtype=torch.float32, device="cuda")) for _ in range(rounds)]
    cdf_g = torch.empty(n, dtype=torch.float64, device="cuda")
    tot_g = torch.empty(1, dtype=torch.float64, device="cuda")

    def graph_rounds():
        for r in range(rounds):
            ps.per_round(p_g, U[r], a, b, V[r], out_idx=out_g[r][0], out_w=out_g[r][1],
                         cdf=cdf_g, total=tot_g, ws=ws_g)

    def check(tag):
        for r in range(rounds):
            idx, w, cdf, tot = ps.per_round(p_e, U[r], a, b, V[r], ws=ws_e)
            assert torch.equal(out_g[r][0], idx), f"{tag} round {r}: indices"
            assert torch.equal(out_g[r][1], w), f"{tag} round {r}: weights"
        assert torch.equal(cdf_g, cdf) and torch.equal(tot_g, tot), f"{tag}: cdf"
        assert torch.equal(p_g, p_e), f"{tag}: priorities"

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        graph_rounds()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    check("warm-up")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graph_rounds()
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        check(f"replay {rep}")
        x = torch.randn(1 << 16, device="cuda").sum().item()   # eager work in between
        assert x == x
    assert ws_g.errors() == 0 and ws_e.errors() == 0


# ------------------------------------------------- fused scan + sample
@pytest.mark.parametrize("n,k", [(1, 1), (1000, 7), (8192, 1024), (262144, 8192), (262147, 8191),
                                 (1 << 20, 4096), ((1 << 20) + 12, 1 << 16),
                                 ((1 << 22) + 5, 1 << 16), (1 << 22, 1 << 22), (5000, 20000)])
@pytest.mark.parametrize("mode", ["fp", "int"])
def test_build_cdf_sample_equals_separate(ps, n, k, mode):
    """psamp_build_cdf_sample gives the bits of psamp_build_cdf followed by
    psamp_sample(stratified), on both tilings, ragged sizes and k > n; three
    calls in a row on one workspace (its parities alternate)."""
    say(f"build_cdf_sample {mode} n={n} k={k}")
    ws = ps.Workspace(ps.build_cdf_workspace_size(n))
    ws2 = ps.Workspace(ps.build_cdf_workspace_size(n))
    for rep in range(3):
        rng = np.random.default_rng(n + 7 * k + rep)
        if mode == "fp":
            p = si.generic_f32(n, n + rep, "lognormal")
            p[::13] = 0.0
            p[0] = max(p[0], np.float32(1e-3))
            u = si.uniform_f32(rng, k)
            alpha = 0.7
        else:
            p = rng.integers(0, 1 << 20, n, dtype=np.uint32)
            p[0] = 1
            u = si.uniform_u32(rng, k)
            alpha = 1.0
        P, Ud = dev(p), dev(u)
        idx, cdf, tot = ps.build_cdf_sample(P, Ud, alpha, ws=ws)
        c_s, t_s = ps.build_cdf(P, alpha, ws=ws2)
        i_s = ps.sample(c_s, t_s, Ud, stratified=True)
        assert torch.equal(cdf, c_s), f"rep {rep}: cdf"
        assert torch.equal(tot, t_s), f"rep {rep}: total"
        assert torch.equal(idx, i_s), f"rep {rep}: indices"
        # the fused call against the oracle directly
        what = f"build_cdf_sample {mode} n={n} k={k} rep {rep}"
        if mode == "fp":
            C_o, T_o, t_o, idx_o = oracle.sample(p, alpha, u, True)
            assert rel_err(host(cdf), C_o) <= 1e-12, what
            assert abs(float(host(tot)[0]) - T_o) <= 1e-12 * T_o, what
            assert_indices(host(idx), idx_o, t_o, C_o, T_o, what)
        else:
            C_o, T_o, t_o, idx_o = oracle.sample_int(p, u, True)
            assert np.array_equal(host(cdf), C_o), what
            assert int(host(tot)[0]) == T_o, what
            assert np.array_equal(host(idx), idx_o), what
    assert ws.errors() == 0


def test_build_cdf_sample_per_large(ps):
    """PER large (2^24 priorities, 2^20 stratified draws), fp and integer:
    the fused call equals the two calls, and its integer indices equal the
    oracle's."""
    d = si.per_large()
    P, Ud = dev(d["p"]), dev(d["U"])
    idx, cdf, tot = ps.build_cdf_sample(P, Ud, d["alpha"])
    c_s, t_s = ps.build_cdf(P, d["alpha"])
    assert torch.equal(cdf, c_s) and torch.equal(tot, t_s)
    assert torch.equal(idx, ps.sample(c_s, t_s, Ud, stratified=True))
    say("PER large fused fp: oracle ...")
    C_o, T_o, t_o, idx_o = oracle.sample(d["p"], d["alpha"], d["U"], True)
    e = rel_err(host(cdf), C_o)
    say(f"  max rel CDF err {e:.3e}")
    assert e <= 1e-12
    assert abs(float(host(tot)[0]) - T_o) <= 1e-12 * T_o
    assert_indices(host(idx), idx_o, t_o, C_o, T_o, "per_large fused fp")
    di = si.per_large_int()
    Q, R = dev(di["q"]), dev(di["r"])
    idx_i, _, _ = ps.build_cdf_sample(Q, R)
    _, _, _, idx_o = oracle.sample_int(di["q"], di["r"], True)
    assert np.array_equal(host(idx_i), idx_o)


@pytest.mark.parametrize("n,k", [((1 << 20) - 3, 1 << 18), ((1 << 22) + 5, 1 << 16),
                                 (1 << 23, 1 << 20)])
@pytest.mark.parametrize("case", ["one_half", "all_on_one", "int_one_half"])
def test_build_cdf_sample_heavy_elements(ps, n, k, case):
    """The fused call where one element takes a large share of the draws
    (half the mass, or all of it), on both tilings: the bits of the two
    calls, the oracle's integer indices, and a time bound that one lane
    placing the heavy element's draws alone would break."""
    import time
    say(f"build_cdf_sample heavy {case} n={n} k={k}")
    rng = np.random.default_rng(n + k)
    if case == "int_one_half":
        q = rng.integers(1, 1 << 10, n, dtype=np.uint32)
        q[n // 3] = np.uint32(min(int(q.astype(np.int64).sum()), (1 << 32) - 1))
        P, Ud, alpha = dev(q), dev(si.uniform_u32(rng, k)), 1.0
    else:
        p = rng.random(n, dtype=np.float32) + np.float32(0.01)
        if case == "one_half":
            p[n // 3] = np.float32(p.astype(np.float64).sum())
        else:
            p[:] = 0.0
            p[n // 3] = 1.0
        P, Ud, alpha = dev(p), dev(si.uniform_f32(rng, k)), 1.0
    ws = ps.Workspace(ps.build_cdf_workspace_size(n))
    idx, cdf, tot = ps.build_cdf_sample(P, Ud, alpha, ws=ws)
    c_s, t_s = ps.build_cdf(P, alpha)
    assert torch.equal(cdf, c_s) and torch.equal(tot, t_s)
    assert torch.equal(idx, ps.sample(c_s, t_s, Ud, stratified=True))
    if case == "int_one_half":
        _, _, _, idx_o = oracle.sample_int(q, host(Ud), True)
        assert np.array_equal(host(idx), idx_o)
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        ps.build_cdf_sample(P, Ud, alpha, cdf=cdf, total=tot, out=idx, ws=ws)
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
    say(f"  {1e6 * min(times):.0f} us per call")
    assert min(times) < 5e-3, times
    assert ws.errors() == 0


@pytest.mark.parametrize("mode", ["fp", "int"])
def test_build_cdf_sample_mixed_calls_one_workspace(ps, mode):
    """The fused call and the plain scan alternate on one workspace at 2^24
    (2048 tiles: more workgroups than fit at once), six calls: the parity
    stays in step (each result equals a fresh-workspace reference and no
    bounded wait runs out).  A regression test: the second pass must not
    advance the call counter itself, since its last tile can finish before
    other workgroups have started."""
    n, k = 1 << 24, 1 << 16
    rng = np.random.default_rng(11)
    if mode == "fp":
        p, u, alpha = si.generic_f32(n, 12, "lognormal"), si.uniform_f32(rng, k), 0.7
    else:
        p = rng.integers(1, 1 << 20, n, dtype=np.uint32)
        u, alpha = si.uniform_u32(rng, k), 1.0
    P, Ud = dev(p), dev(u)
    c_ref, t_ref = ps.build_cdf(P, alpha)
    i_ref = ps.sample(c_ref, t_ref, Ud, stratified=True)
    ws = ps.Workspace(ps.build_cdf_workspace_size(n))
    for rep in range(6):
        if rep % 2 == 0:
            idx, cdf, tot = ps.build_cdf_sample(P, Ud, alpha, ws=ws)
            assert torch.equal(idx, i_ref), f"rep {rep}: indices"
        else:
            cdf, tot = ps.build_cdf(P, alpha, ws=ws)
        assert torch.equal(cdf, c_ref) and torch.equal(tot, t_ref), f"rep {rep}"
    assert ws.errors() == 0


def test_per_round_large_chain(ps):
    """Beyond a resident grid (2^23 priorities, three kernels per update):
    four chained updates on one workspace, each equal to the separate calls
    on the previous update's rewritten priorities."""
    n, k = 1 << 23, 1 << 16
    p = si.generic_f32(n, 21, "lognormal")
    Pd = dev(p)
    ws = ps.Workspace(ps.per_round_workspace_size(n, k))
    p_ref = p.copy()
    for r in range(4):
        U = si.uniform_f32(np.random.default_rng(100 + r), k)
        newp = si.generic_f32(k, 200 + r, "exp")
        C_s, T_s, idx_s, w_s, p_ref = _separate_round(ps, p_ref, U, newp, 0.7, 0.5)
        idx, w, cdf, tot = ps.per_round(Pd, dev(U), 0.7, 0.5, dev(newp), ws=ws)
        assert np.array_equal(host(cdf), C_s), f"update {r}: cdf"
        assert np.array_equal(host(idx), idx_s), f"update {r}: indices"
        assert np.array_equal(host(w), w_s), f"update {r}: weights"
        assert np.array_equal(host(Pd), p_ref), f"update {r}: rewritten priorities"
    assert ws.errors() == 0


def test_per_round_large_chain_vs_oracle(ps):
    """Beyond a resident grid (2^23 + 1 priorities: 1025 tiles, three
    kernels per update), 2^18 stratified draws, four chained updates on one
    workspace, against the oracle's own chain: CDF within 1e-12, indices
    under the boundary rule (none observed; the chains would fork on one),
    IS weights within 1e-6, rewritten priorities bit for bit."""
    n, k = (1 << 23) + 1, 1 << 18
    p_o = si.generic_f32(n, 23, "lognormal")
    Pd = dev(p_o)
    ws = ps.Workspace(ps.per_round_workspace_size(n, k))
    for r in range(4):
        U = si.uniform_f32(np.random.default_rng(300 + r), k)
        newp = si.generic_f32(k, 400 + r, "exp")
        idx, w, cdf, tot = ps.per_round(Pd, dev(U), 0.7, 0.5, dev(newp), ws=ws)
        what = f"per_round large chain update {r}"
        say(what)
        exc, p_o = check_round_vs_oracle(p_o, U, newp, 0.7, 0.5, host(cdf), host(tot)[0],
                                         host(idx), host(w), host(Pd), what)
        assert exc == 0, "chains would fork; the oracle never takes GPU data"
    assert ws.errors() == 0


def test_per_round_one_workspace_shrinking_then_growing(ps):
    """One workspace for fused updates whose tile counts shrink and then grow
    again (1025 tiles on the three-kernel path, 256 and 8 on the one-kernel
    path, then 2048): every update's status words must be clean, i.e. each
    call clears the other parity up to the largest tile count the workspace
    has seen, not only up to its own.  A regression test: the clearing was
    bounded by the capacity the current n needs, which left stale tile sums
    of an earlier, larger update for a later one to read."""
    sizes = [((1 << 23) + 1, 1 << 16), (262144, 8192), (8192, 1024), (1 << 24, 1 << 18),
             (300000, 5000), ((1 << 23) + 1, 1 << 16)]
    ws = ps.Workspace(ps.per_round_workspace_size(1 << 24, 1 << 18))
    for call, (n, k) in enumerate(sizes):
        say(f"shared workspace call {call}: n={n} k={k}")
        p = si.generic_f32(n, 600 + call, "lognormal")
        U = dev(si.uniform_f32(np.random.default_rng(700 + call), k))
        newp = dev(si.generic_f32(k, 800 + call, "exp"))
        P_ref, P_sh = dev(p), dev(p)
        ref = ps.per_round(P_ref, U, 0.7, 0.5, newp,
                           ws=ps.Workspace(ps.per_round_workspace_size(n, k)))
        got = ps.per_round(P_sh, U, 0.7, 0.5, newp, ws=ws)
        for name, r, g in zip(("indices", "weights", "cdf", "total"), ref, got):
            assert torch.equal(r, g), f"call {call}: {name}"
        assert torch.equal(P_ref, P_sh), f"call {call}: rewritten priorities"
    assert ws.errors() == 0


@pytest.mark.parametrize("n,k,rewrite", [(262144, 8192, True), (8192, 8192, True),
                                         (300001, 5000, False), (1 << 20, 4096, True),
                                         (5000, 300, True), (1000, 7, True)])
def test_per_round_chain_on_one_workspace(ps, n, k, rewrite):
    """Chained fused updates on one workspace: every update equals the four
    separate calls bit for bit, also with work between updates -- a priority
    written outside the updates, the same value written again, a scan on the
    same workspace (the call parity moves), another alpha -- with and without
    the rewrite, and with more draws in a tile than it has threads (8192
    priorities, 8192 draws)."""
    rounds = 8
    p = si.generic_f32(n, n + 3, "lognormal")
    p[::29] = 0.0
    p[0] = max(p[0], np.float32(1e-3))
    ws = ps.Workspace(ps.per_round_workspace_size(n, k))
    Pd = dev(p)
    p_ref = p.copy()
    alpha, beta = 0.7, 0.5
    for r in range(rounds):
        say(f"chain n={n} k={k} rewrite={rewrite} update {r}")
        U = si.uniform_f32(np.random.default_rng(900 + r), k)
        newp = si.generic_f32(k, 950 + r, "exp") if rewrite else None
        if r == 2:                      # a write between updates
            j = n // 2
            p_ref[j] = np.float32(2.5) if p_ref[j] != np.float32(2.5) else np.float32(3.5)
            Pd[j] = float(p_ref[j])
        if r == 3:                      # the same value written again: nothing changes
            Pd[n // 3] = float(p_ref[n // 3])
        if r == 4:                      # a scan on the same workspace in between
            ps.build_cdf(Pd, 0.3, ws=ws)
        if r == 6:                      # another alpha
            alpha = 0.9
        C_s, T_s, idx_s, w_s, p_s = _separate_round(ps, p_ref, U, newp, alpha, beta)
        idx, w, cdf, tot = ps.per_round(Pd, dev(U), alpha, beta,
                                        dev(newp) if rewrite else None, ws=ws)
        assert np.array_equal(host(cdf), C_s), f"update {r}: cdf"
        assert np.array_equal(host(tot), T_s), f"update {r}: total"
        assert np.array_equal(host(idx), idx_s), f"update {r}: indices"
        assert np.array_equal(host(w), w_s), f"update {r}: weights"
        assert np.array_equal(host(Pd), p_s), f"update {r}: priorities"
        p_ref = p_s
    assert ws.errors() == 0


@pytest.mark.parametrize("n,rows,nt", [(4, 8, True), (1 << 20, 8, True), ((1 << 22) + 12, 4, False),
                                       (8200, 8, False), (4100, 2, False), ((1 << 20) + 4, 2, True)])
def test_ceiling_copy(ps, n, rows, nt):
    """The measurement aid copies every float to a double, tail included."""
    src = torch.rand(n, device="cuda")
    dst = torch.full((n,), -1.0, dtype=torch.float64, device="cuda")
    ps.ceiling_copy(src, dst, rows, nt)
    assert torch.equal(dst, src.double())
