"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a closed
form, a library routine (numpy / scipy), brute force over tiny inputs, an
invariant, or a fixture under tests/golden/ that cites the page it comes
from.  They are chosen so that a dropped term, a wrong sign, an off-by-one
or a transposed operand in the oracle fails at least one of them.
"""
import json
import os

import numpy as np
import pytest
from scipy import special, stats

import synthetic_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ weights
def test_weights_alpha_one_is_identity(orc):
    p = si.generic_f32(5000, 11, "lognormal")
    assert np.array_equal(orc.weights(p, 1.0), p.astype(np.float64))


def test_weights_alpha_two_is_exact_square(orc):
    # p is float32, so p*p is exact in double: a faithful pow must return it.
    p = si.generic_f32(5000, 12, "exp")
    pd = p.astype(np.float64)
    assert np.array_equal(orc.weights(p, 2.0), pd * pd)


def test_weights_alpha_half_is_sqrt(orc):
    p = si.generic_f32(20000, 13, "lognormal")
    w = orc.weights(p, 0.5)
    ref = np.sqrt(p.astype(np.float64))
    ulps = np.abs(w.view(np.int64) - ref.view(np.int64))
    assert ulps.max() <= 1


def test_weights_inverse_power_roundtrip(orc):
    # Leaves of the sum-tree workload are U^(1/alpha): raising them to alpha
    # must give U back (catches an inverted or mis-scaled exponent).
    rng = np.random.default_rng(3)
    U = rng.uniform(0.01, 1.0, 10000)
    p = (U ** (1 / 0.6)).astype(np.float32)
    w = orc.weights(p, 0.6)
    back = p.astype(np.float64) ** 0.6
    assert np.allclose(w, back, rtol=1e-14, atol=0)
    assert np.allclose(w, U, rtol=1e-6)


# ---------------------------------------------------------------------- CDF
def test_cdf_all_ones_closed_form(orc):
    n = 100003
    Cc, T = orc.build_cdf(np.ones(n, np.float32), 0.6)
    assert np.array_equal(Cc, np.arange(1, n + 1, dtype=np.float64))
    assert T == float(n)


def test_cdf_matches_sequential_numpy_accumulate(orc):
    p = si.generic_f32(300001, 21, "lognormal")
    Cc, T = orc.build_cdf(p, 0.7)
    w = p.astype(np.float64) ** 0.7
    # numpy's add.accumulate is a sequential left-to-right sum.
    ref = np.add.accumulate(orc.weights(p, 0.7))
    assert np.array_equal(Cc, ref)
    assert np.allclose(Cc, np.cumsum(w), rtol=1e-12)
    assert Cc[-1] == T
    assert np.all(np.diff(Cc) >= 0)


def test_cdf_int_exact(orc):
    q = si.sweep_u32(200003)
    Cc, T = orc.build_cdf_int(q)
    assert T == sum(int(x) for x in q)
    assert np.array_equal(Cc, np.cumsum(q.astype(np.uint64)))
    assert int(Cc[-1]) == T


def test_cdf_inclusive_not_exclusive(orc):
    Cc, T = orc.build_cdf(np.array([3.0, 1.0, 4.0], np.float32), 1.0)
    assert list(Cc) == [3.0, 4.0, 8.0] and T == 8.0


# --------------------------------------------------------------- thresholds
def test_thresholds_stratified_in_strata(orc):
    k = 1024
    U = si.uniform_f32(np.random.default_rng(5), k)
    T = 12345.678
    t = orc.thresholds(U, T, True)
    i = np.arange(k)
    lo = i / k * T
    hi = (i + 1) / k * T
    assert np.all(t >= lo * (1 - 1e-15)) and np.all(t <= hi * (1 + 1e-15))
    assert np.all(np.diff(t) >= 0)
    t0 = orc.thresholds(np.zeros(k, np.float32), T, True)
    assert np.array_equal(t0, i / k * T)


def test_thresholds_iid(orc):
    U = si.uniform_f32(np.random.default_rng(6), 1000)
    t = orc.thresholds(U, 3.5, False)
    assert np.array_equal(t, U.astype(np.float64) * 3.5)


def test_thresholds_int_range_and_order(orc):
    rng = np.random.default_rng(7)
    r = si.uniform_u32(rng, 4096)
    T = (1 << 44) + 12345
    t = orc.thresholds_int(r, T, True)
    assert t.min() >= 1 and t.max() <= T
    assert np.all(np.diff(t.astype(np.int64)) >= 0)
    # extremes: r = 0 at i = 0 gives 1; r = 2^32-1 at i = k-1 gives T.
    r2 = np.zeros(4, np.uint32)
    r2[-1] = 0xFFFFFFFF
    t2 = orc.thresholds_int(r2, 1000, True)
    assert t2[0] == 1 and t2[-1] == 1000


# ------------------------------------------------------------------- search
def test_search_golden_rule(orc):
    g = json.load(open(os.path.join(GOLDEN, "searchsorted_rule.json")))
    Cc = np.array(g["cumsum"], np.float64)
    t = np.array(g["u"], np.float64)
    assert list(orc.search(Cc, t)) == g["expected"]


def test_search_matches_numpy_searchsorted(orc):
    p = si.generic_f32(50000, 31, "lognormal")
    U = si.uniform_f32(np.random.default_rng(32), 7000)
    for strat in (True, False):
        Cc, T, t, idx = orc.sample(p, 0.7, U, strat)
        ref = np.searchsorted(Cc, t, side="left").clip(0, Cc.size - 1)
        assert np.array_equal(idx, ref)


def test_search_ties_and_clamp(orc):
    Cc = np.array([1.0, 1.0, 2.0, 5.0])   # a zero weight at index 1
    t = np.array([0.0, 1.0, 1.5, 2.0, 5.0, 6.0, -1.0])
    assert list(orc.search(Cc, t)) == [0, 0, 2, 2, 3, 3, 0]


def test_search_f32cdf_matches_numpy_and_brute_force(orc):
    """The search over a float32 CDF with double thresholds: equal to numpy's
    left searchsorted on the CDF widened to double (exact, every float is a
    double), clamped; and, on a tiny CDF with ties and rounding collisions,
    to a brute-force scan for the first entry >= t."""
    rng = np.random.default_rng(44)
    w = rng.exponential(1.0, 40000)
    w[rng.random(w.size) < 0.3] = 0.0
    Cf = np.cumsum(w).astype(np.float32)
    U = si.uniform_f32(rng, 5000)
    for strat in (True, False):
        t = orc.thresholds(U, float(Cf[-1]), strat)
        ref = np.searchsorted(Cf.astype(np.float64), t, side="left").clip(0, Cf.size - 1)
        assert np.array_equal(orc.search_f32cdf(Cf, t), ref)
    Cs = np.array([0.5, 0.5, 1.0, np.float32(1.0) + np.float32(2**-23), 3.0], np.float32)
    t = np.array([-1.0, 0.0, 0.5, 0.5 + 1e-12, 1.0, 1.0 + 1e-9, 1.0 + 2**-23, 2.9, 3.0, 3.5])
    brute = []
    for x in t:
        hits = [j for j in range(Cs.size) if float(Cs[j]) >= x]
        brute.append(hits[0] if hits else Cs.size - 1)
    assert list(orc.search_f32cdf(Cs, t)) == brute == [0, 0, 0, 2, 2, 3, 3, 4, 4, 4]


def test_search_int_brute_force_counts(orc):
    rng = np.random.default_rng(41)
    for n in (1, 2, 3, 5, 8):
        q = rng.integers(1, 9, n).astype(np.uint32)
        Cc, T = orc.build_cdf_int(q)
        t = np.arange(1, T + 1, dtype=np.uint64)
        idx = orc.search_int(Cc, t)
        counts = np.bincount(idx, minlength=n)
        assert np.array_equal(counts, q.astype(np.int64))


def test_search_int_closed_form_unit_weights(orc):
    # All q = 1 gives C_j = j+1, so the stratified integer sample i lands on
    # floor((i + r_i / 2^32) * n / k).
    n, k = 1000, 256
    r = si.uniform_u32(np.random.default_rng(42), k)
    _, _, _, idx = orc.sample_int(np.ones(n, np.uint32), r, True)
    expect = [((i * 2**32 + int(r[i])) * n) // (k * 2**32) for i in range(k)]
    assert list(idx) == expect


def test_search_int_matches_numpy(orc):
    d = si.per_large_int(n=100000, k=20000)
    Cc, T, t, idx = orc.sample_int(d["q"], d["r"], True)
    ref = np.searchsorted(Cc, t, side="left").clip(0, Cc.size - 1)
    assert np.array_equal(idx, ref)
    assert np.all(np.diff(idx) >= 0)


def test_iid_chi_square(orc):
    rng = np.random.default_rng(51)
    for n, alpha in ((8, 0.6), (16, 0.7)):
        p = rng.uniform(0.05, 3.0, n).astype(np.float32)
        U = si.uniform_f32(rng, 1_000_000)
        _, T, _, idx = orc.sample(p, alpha, U, stratified=False)
        counts = np.bincount(idx, minlength=n)
        P = p.astype(np.float64) ** alpha
        P /= P.sum()
        chi2, pv = stats.chisquare(counts, P * U.size)
        assert pv > 1e-3, (n, chi2, pv)


def test_stratified_counts_within_two(orc):
    rng = np.random.default_rng(52)
    p = rng.uniform(0.05, 3.0, 300).astype(np.float32)
    k = 4096
    U = si.uniform_f32(rng, k)
    _, _, _, idx = orc.sample(p, 0.6, U, True)
    P = p.astype(np.float64) ** 0.6
    P /= P.sum()
    counts = np.bincount(idx, minlength=p.size)
    assert np.all(np.abs(counts - k * P) < 2)


# ---------------------------------------------------------------- IS weights
def test_is_weights_closed_form(orc):
    d = si.per_small()
    Cc, T, t, idx = orc.sample(d["p"], d["alpha"], d["U"], True)
    w = orc.is_weights(d["p"], d["alpha"], T, idx, d["beta"])
    pw = d["p"].astype(np.float64)[idx] ** d["alpha"]
    closed = (pw.min() / pw) ** d["beta"]            # N and T cancel
    assert np.allclose(w, closed, rtol=1e-6, atol=0)
    assert w.max() == 1.0
    assert np.all(w > 0) and np.all(w <= 1.0)
    # depends on beta with the right sign: larger beta -> smaller weights
    w2 = orc.is_weights(d["p"], d["alpha"], T, idx, 0.8)
    assert np.all(w2 <= w + 1e-7)


def test_is_weights_constant_priorities(orc):
    p = np.full(1000, 2.5, np.float32)
    idx = np.arange(0, 1000, 7, dtype=np.int32)
    assert np.all(orc.is_weights(p, 0.6, 1000 * 2.5 ** 0.6, idx, 0.4) == 1.0)


def test_is_weights_int_closed_form(orc):
    d = si.per_large_int(n=50000, k=4096)
    Cc, T, t, idx = orc.sample_int(d["q"], d["r"], True)
    w = orc.is_weights_int(d["q"], T, idx, d["beta"])
    qq = d["q"].astype(np.float64)[idx]
    assert np.allclose(w, (qq.min() / qq) ** d["beta"], rtol=1e-6, atol=0)
    assert w.max() == 1.0


# -------------------------------------------------------------- LWW scatter
def test_scatter_lww_dict_replay():
    import oracle
    rng = np.random.default_rng(61)
    p = si.generic_f32(1000, 62)
    idx = rng.integers(0, 1000, 3000).astype(np.int32)
    v = si.generic_f32(3000, 63)
    out = oracle.scatter_lww(p, idx, v)
    last = {}
    for j, i in enumerate(idx):
        last[int(i)] = v[j]
    ref = p.copy()
    for i, val in last.items():
        ref[i] = val
    assert np.array_equal(out, ref)


# ------------------------------------------------------------------ sum tree
def test_tree_layout_golden(orc):
    g = json.load(open(os.path.join(GOLDEN, "segtree_layout.json")))
    cap = g["diagram_capacity"]
    leaves = np.arange(1, cap + 1, dtype=np.uint32)       # distinct leaves
    t = orc.Tree("u64", cap).build(leaves)
    flat = t.flat().astype(np.int64)
    assert flat.size == 2 * cap and flat[0] == 0
    assert flat[g["root_index"]] == leaves.sum()
    # leaf i sits at capacity + i; parent of j is j // 2; children 2j, 2j+1
    assert list(flat[g["diagram_levels"][-1]]) == list(leaves)
    for level in g["diagram_levels"][:-1]:
        for j in level:
            assert flat[j] == flat[2 * j] + flat[2 * j + 1]
    for row in g["memory_table"]:
        c2 = orc.cap_pow2(row["capacity"])
        assert c2 == row["capacity_pow2"]
        assert 2 * c2 * g["node_bytes"] == row["bytes"]   # 2*cap_pow2*sizeof(f32): 4 MB / 1 MB as printed
    assert orc.cap_pow2(1) == 1 and orc.cap_pow2(2) == 2 and orc.cap_pow2(3) == 4


def test_tree_int_root_and_descent_brute_force(orc):
    rng = np.random.default_rng(71)
    for n_valid, cap in ((1, 1), (3, 4), (5, 8), (8, 8), (11, 16)):
        q = rng.integers(1, 7, n_valid).astype(np.uint32)
        t = orc.Tree("u64", cap).build(q, n_valid)
        T = int(q.sum())
        assert t.root() == T
        Cc, _ = orc.build_cdf_int(q)
        # every integer threshold in [1, T] via the iid integer map with r
        # chosen so that floor(r*T/2^32)+1 sweeps 1..T
        thr = np.arange(1, T + 1, dtype=np.uint64)
        r = np.array([((int(x) - 1) * 2**32 + T - 1) // T for x in thr], dtype=np.uint64)
        assert np.array_equal(orc.thresholds_int(r.astype(np.uint32), T, False), thr)
        idx = t.sample(r.astype(np.uint32), n_valid, stratified=False)
        assert np.array_equal(idx, orc.search_int(Cc, thr))
        assert np.array_equal(np.bincount(idx, minlength=n_valid), q.astype(np.int64))


def test_tree_int_equals_cdf_path_large(orc):
    d = si.per_large_int(n=200000, k=50000)
    cap = orc.cap_pow2(200000)
    t = orc.Tree("u64", cap).build(d["q"], 200000)
    _, T, _, idx_cdf = orc.sample_int(d["q"], d["r"], True)
    assert t.root() == T
    assert np.array_equal(t.sample(d["r"], 200000, True), idx_cdf)


def test_tree_f64_vs_searchsorted(orc):
    p = si.generic_f32(3000, 72, "exp")
    cap = orc.cap_pow2(3000)
    t = orc.Tree("f64", cap).build(p, 3000, 0.6)
    U = si.uniform_f32(np.random.default_rng(73), 100000)
    a = t.sample(U, 3000, False)
    Cc, T = orc.build_cdf(p, 0.6)
    b = np.searchsorted(Cc, orc.thresholds(U, t.root(), False), "left").clip(0, 2999)
    assert np.count_nonzero(a != b) <= 2      # fp64 boundary ties only


def test_tree_f32_integer_leaves_match_exact_lower_bound(orc):
    # Small integer leaves keep every f32 sum exact, so the f32 descent must
    # equal lower_bound on the exact CDF.
    rng = np.random.default_rng(74)
    q = rng.integers(0, 50, 1000).astype(np.float32)
    q[0] = 1
    cap = 1024
    t = orc.Tree("f32", cap).build(q, 1000, 1.0)
    U = si.uniform_f32(rng, 20000)
    root = np.float32(t.root())
    thr = (U * root).astype(np.float32)          # float32 product, as the tree does
    Cc = np.cumsum(q.astype(np.float64))
    ref = np.searchsorted(Cc, thr.astype(np.float64), "left").clip(0, 999)
    assert np.array_equal(t.sample(U, 1000, False), ref)


def test_tree_update_lww_and_rebuild_invariant(orc):
    d = si.sumtree(n_valid=5000, m=256, k=256, rounds=5)
    cap = orc.cap_pow2(5000)
    t = orc.Tree("f32", cap).build(d["p0"], 5000, d["alpha"])
    leaves = np.array([orc.leaf_f32(x, d["alpha"]) for x in d["p0"]], np.float32)
    for r in range(5):
        t.update(d["idx"][r], d["v"][r], d["alpha"])
        for j, i in enumerate(d["idx"][r]):
            leaves[i] = orc.leaf_f32(d["v"][r][j], d["alpha"])
        flat = t.flat()
        assert np.array_equal(flat[cap:cap + 5000], leaves)
        fresh = orc.Tree("f32", cap).build(np.zeros(0, np.float32), 0, 1.0)
        # rebuild from the same leaves (alpha = 1 keeps them as they are)
        pad = np.zeros(cap, np.float32)
        pad[:5000] = leaves
        fresh = orc.Tree("f32", cap).build(pad, cap, 1.0)
        assert np.array_equal(fresh.flat(), flat)
        # every internal node is the float sum of its children
        j = np.arange(1, cap)
        assert np.array_equal(flat[j], (flat[2 * j] + flat[2 * j + 1]).astype(np.float32))


def test_leaf_f32_correct_rounding(orc):
    p = si.generic_f32(3000, 75, "lognormal")
    for x in p[:1000]:
        assert orc.leaf_f32(x, 0.5) == np.sqrt(np.float32(x))       # CR sqrt
        assert orc.leaf_f32(x, 1.0) == np.float32(x)
        assert orc.leaf_f32(x, 2.0) == np.float32(np.float64(x) ** 2)
    # general alpha: equals float(pow in double) except at rare near-ties
    a = np.array([orc.leaf_f32(x, 0.6) for x in p], np.float32)
    b = (p.astype(np.float64) ** 0.6).astype(np.float32)
    assert np.count_nonzero(a != b) <= 1


# --------------------------------------------------------------- resampling
def test_row_cdf_vs_softmax(orc):
    x = si.resample(rows=1, P=4096)["lw"][0]
    W, Cc = orc.row_cdf(x)
    ref = special.softmax(x.astype(np.float64))
    assert np.allclose(W, ref, rtol=1e-13, atol=0)
    assert np.array_equal(Cc, np.add.accumulate(W))
    assert abs(Cc[-1] - 1.0) < 1e-12


def test_resample_matches_searchsorted_of_float32_thresholds(orc):
    d = si.resample(rows=64, P=4096)
    anc = orc.resample_rows(d["lw"], d["u_row"])
    P = 4096
    for b in range(64):
        _, Cc = orc.row_cdf(d["lw"][b])
        uk = (np.arange(P, dtype=np.float32) + d["u_row"][b]) / np.float32(P)
        assert uk.dtype == np.float32
        ref = np.searchsorted(Cc, uk.astype(np.float64), "left").clip(0, P - 1)
        assert np.array_equal(anc[b], ref)
        assert np.all(np.diff(anc[b]) >= 0)


def test_resample_uniform_rows_identity(orc):
    P = 4096
    lw = np.zeros((8, P), np.float32)
    lw[1] = 3.25     # any constant row is uniform
    u = np.linspace(0.01, 0.99, 8).astype(np.float32)
    anc = orc.resample_rows(lw, u)
    assert np.array_equal(anc, np.tile(np.arange(P, dtype=np.int32), (8, 1)))


def test_resample_offspring_counts(orc):
    d = si.resample(rows=32, P=1024, sigma=1.0)
    anc = orc.resample_rows(d["lw"], d["u_row"])
    for b in range(32):
        W, _ = orc.row_cdf(d["lw"][b])
        cnt = np.bincount(anc[b], minlength=1024)
        assert np.all(np.abs(cnt - 1024 * W) < 1 + 1e-9)


# ------------------------------------------------------ particle-filter step
def _pf_golden():
    with open(os.path.join(os.path.dirname(__file__), "golden", "pf_step_worked.json")) as f:
        return json.load(f)


def test_pf_step_worked_example(orc):
    g = _pf_golden()
    f = lambda k, dt=np.float32: np.array(g[k], dt)
    x_out, lw_out, anc, pred, lwn = orc.pf_step(f("x"), f("lw"), f("obs"), f("A"), f("C"),
                                               f("eps"), g["sigma_p"], g["sigma_o"], f("u_row"))
    assert np.array_equal(pred, f("pred"))
    assert np.array_equal(lwn, f("lw_new"))
    assert np.array_equal(anc, f("anc", np.int32))
    assert np.array_equal(x_out, f("x_out"))
    assert np.all(lw_out == np.float32(-np.log(4.0)))


def test_pf_step_vs_library_gaussian(orc):
    """pred against a float64 matmul, the log-likelihood against scipy's
    multivariate normal density (its normalising constant is the same for
    every particle and is added back here)."""
    d = si.pf_step(rows=3, P=64, D=4, O=2)
    A = np.array([[0.9, 0.1, 0.0, -0.2], [0.0, 0.8, 0.3, 0.0], [0.1, 0.0, 0.7, 0.0],
                  [0.0, -0.4, 0.0, 1.1]], np.float32)          # not symmetric
    _, _, _, pred, lwn = orc.pf_step(d["x"], d["lw"], d["obs"], A, d["C"], d["eps"],
                                     d["sigma_p"], d["sigma_o"], d["u_row"])
    x64, e64 = d["x"].astype(np.float64), d["eps"].astype(np.float64)
    ref = x64 @ A.astype(np.float64).T + d["sigma_p"] * e64
    assert np.allclose(pred, ref, rtol=1e-5, atol=1e-6)
    so = d["sigma_o"]
    const = -0.5 * 2 * np.log(2 * np.pi * so * so)
    for b in range(3):
        mean = pred[b].astype(np.float64) @ d["C"].astype(np.float64).T
        ll = np.array([stats.multivariate_normal(mean=m, cov=so * so * np.eye(2))
                       .logpdf(d["obs"][b].astype(np.float64)) for m in mean]) - const
        assert np.allclose(lwn[b], d["lw"][b] + ll, rtol=1e-5, atol=1e-4)


def test_pf_step_reduces_to_resampling(orc):
    """A = I, no process noise, C = 0, obs = 0: pred = x and lw' = lw
    exactly, so the step is the resampler followed by a gather."""
    d = si.pf_step(rows=8, P=1024, D=4, O=2)
    A = np.eye(4, dtype=np.float32)
    Cm = np.zeros((2, 4), np.float32)
    obs = np.zeros((8, 2), np.float32)
    x_out, lw_out, anc, pred, lwn = orc.pf_step(d["x"], d["lw"], obs, A, Cm, d["eps"], 0.0,
                                               d["sigma_o"], d["u_row"])
    assert np.array_equal(pred, d["x"])
    assert np.array_equal(lwn, d["lw"])
    assert np.array_equal(anc, orc.resample_rows(d["lw"], d["u_row"]))
    assert np.array_equal(x_out, np.take_along_axis(d["x"], anc[:, :, None].astype(np.int64),
                                                    axis=1))
    assert np.all(lw_out == np.float32(-np.log(1024.0)))


def test_pf_step_offspring_counts(orc):
    """Systematic resampling gives particle j floor or ceil of P W_j
    offspring, W = softmax of the updated log-weights (scipy)."""
    d = si.pf_step(rows=16, P=1024, D=4, O=2)
    x_out, _, anc, pred, lwn = orc.pf_step(d["x"], d["lw"], d["obs"], d["A"], d["C"], d["eps"],
                                          d["sigma_p"], d["sigma_o"], d["u_row"])
    for b in range(16):
        W = special.softmax(lwn[b].astype(np.float64))
        cnt = np.bincount(anc[b], minlength=1024)
        assert np.all(np.abs(cnt - 1024 * W) < 1 + 1e-6)
        assert np.all(np.diff(anc[b]) >= 0)
        assert np.array_equal(x_out[b], pred[b][anc[b]])


# ------------------------------------------------------ replay priorities
def test_replay_ring_slots_and_leaves_dict_replay(orc):
    """Inserting 2.5 rings' worth in uneven batches: the slots walk the ring
    in order and every leaf is the correctly rounded p^alpha of the last item
    written to that slot (a dict replay of the same writes)."""
    cap, alpha = 1000, 0.6
    rb = orc.Replay(cap, alpha)
    rng = np.random.default_rng(5)
    last = {}
    n = 0
    for m in (1, 7, 300, 999, 1000, 193):
        p = (rng.random(m) + 0.01).astype(np.float32)
        slots = rb.insert(p)
        assert np.array_equal(slots, (n + np.arange(m)) % cap)
        for s_, v in zip(slots, p):
            last[int(s_)] = v
        n += m
    assert rb.cursor == n % cap and rb.size == cap
    leaves = rb.tree.flat()[orc.cap_pow2(cap):]
    for s_, v in last.items():
        assert leaves[s_] == orc.leaf_f32(float(v), alpha)
    assert np.all(leaves[cap:] == 0)


def test_replay_total_and_descent_integer_leaves(orc):
    """alpha = 1 and integer priorities: leaves and sums are exact, so the
    root is the integer sum and each descent is the exact lower bound of its
    threshold over the integer CDF of the filled slots (brute force)."""
    cap = 300
    rb = orc.Replay(cap, 1.0)
    rng = np.random.default_rng(6)
    p = rng.integers(0, 50, 200).astype(np.float32)
    rb.insert(p)
    upd = rng.integers(0, 200, 40).astype(np.int32)
    val = rng.integers(1, 50, 40).astype(np.float32)
    rb.update(upd, val)
    cur = p.copy()
    for i, v in zip(upd, val):
        cur[i] = v
    assert rb.total() == float(cur.sum())
    U = (np.arange(64, dtype=np.float32) + 0.5) / np.float32(64)
    idx, w = rb.sample(U, 0.4, stratified=False)
    Cc = np.cumsum(cur.astype(np.float64))
    t = (U * np.float32(rb.total())).astype(np.float64)     # iid: t = U * root in float
    ref = np.minimum(np.searchsorted(Cc, t, "left"), 199)
    assert np.array_equal(idx, ref)
    # IS: (N P_i)^-beta / max equals (L_min / L_i)^beta
    L = cur[idx].astype(np.float64)
    assert np.allclose(w, (L.min() / L) ** 0.4, rtol=1e-6)


def test_replay_partial_ring_samples_only_filled_slots(orc):
    rb = orc.Replay(4096, 0.6)
    rb.insert(np.full(100, 2.0, np.float32))
    U = np.random.default_rng(7).random(4096, dtype=np.float32)
    idx, w = rb.sample(U, 0.4, stratified=True)
    assert idx.min() >= 0 and idx.max() <= 99
    assert np.all(w == 1.0)                 # equal priorities
    counts = np.bincount(idx, minlength=100)
    assert np.all(np.abs(counts - 4096 / 100) <= 2)
