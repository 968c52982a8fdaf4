"""GPU parity of the sum tree and of row resampling against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from parity_util import assert_indices, say, ulp_diff_f32

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


def check_f32_tree(flat_g, otree, cap, what):
    """Leaves equal bit for bit (they are p^alpha rounded to float on both
    sides), then every node equal to the oracle's."""
    flat_o = otree.flat()
    lg, lo = flat_g[cap:], flat_o[cap:]
    if not np.array_equal(lg, lo):
        d = ulp_diff_f32(lg, lo)
        raise AssertionError(f"{what}: {np.count_nonzero(d)} leaves differ (max {d.max()} ulp)")
    assert np.array_equal(flat_g[1:], flat_o[1:]), what


@pytest.mark.parametrize("cap,n_valid", [(1, 1), (2, 1), (8, 5), (1024, 1000), (4096, 4096),
                                         (1 << 19, 500000), (1 << 22, (1 << 22) - 9)])
def test_tree_build(ps, cap, n_valid):
    say(f"tree build cap={cap} n_valid={n_valid}")
    p = si.generic_f32(n_valid, cap + 3, "uniform")
    tree = torch.zeros(2 * cap, dtype=torch.float32, device="cuda")
    ps.segtree_build(tree, dev(p), 0.6)
    ot = oracle.Tree("f32", cap).build(p, n_valid, 0.6)
    check_f32_tree(host(tree), ot, cap, "build f32")
    q = si.sweep_u32(n_valid)
    treeq = torch.zeros(2 * cap, dtype=torch.uint64, device="cuda")
    ps.segtree_build(treeq, dev(q))
    otq = oracle.Tree("u64", cap).build(q, n_valid)
    assert np.array_equal(host(treeq)[1:], otq.flat()[1:])


def test_sumtree_cfg_rounds(ps):
    """Sum tree: cap 2^19 (500000 valid), 1000 rounds of a 1024-entry batch
    update (duplicates kept, last write wins) then 1024 iid descents."""
    d = si.sumtree()
    cap, nv, a = 1 << 19, 500000, d["alpha"]
    tree = torch.zeros(2 * cap, dtype=torch.float32, device="cuda")
    ps.segtree_build(tree, dev(d["p0"]), a)
    ot = oracle.Tree("f32", cap).build(d["p0"], nv, a)
    check_f32_tree(host(tree), ot, cap, "initial build")
    rounds = d["idx"].shape[0]
    for r in range(rounds):
        ps.segtree_update(tree, dev(d["idx"][r]), dev(d["v"][r]), a)
        idx_g = host(ps.segtree_sample(tree, nv, dev(d["U"][r])))
        ot.update(d["idx"][r], d["v"][r], a)
        idx_o = ot.sample(d["U"][r], nv, stratified=False)
        if r % 100 == 0 or r == rounds - 1:
            say(f"sumtree round {r}")
            check_f32_tree(host(tree), ot, cap, f"round {r}")
        assert np.array_equal(idx_g, idx_o), f"round {r}"
    check_f32_tree(host(tree), ot, cap, "final")


def _stress_batches(cap, rng):
    m = 1024
    yield "one leaf", np.full(m, 17, np.int32)
    yield "sibling pairs", ((np.arange(m) % 64) ^ (np.arange(m) % 2)).astype(np.int32)
    yield "one subtree", rng.integers(4096, 4096 + 256, m).astype(np.int32)
    yield "ascending", np.arange(m, dtype=np.int32) * (cap // m)
    yield "descending dup", np.repeat(np.arange(m // 4, dtype=np.int32)[::-1] * 3, 4)
    yield "random", rng.integers(0, cap, m).astype(np.int32)
    yield "small batch", rng.integers(0, cap, 3).astype(np.int32)
    yield "with out-of-range", np.where(rng.random(m) < 0.1, -1,
                                        rng.integers(0, cap, m)).astype(np.int32)
    yield "two chunks", rng.integers(0, 64, 2500).astype(np.int32)


@pytest.mark.parametrize("kind", ["f32", "u64"])
def test_tree_update_stress(ps, kind):
    cap = 1 << 16
    rng = np.random.default_rng(9)
    if kind == "f32":
        p0 = si.generic_f32(cap, 1, "uniform")
        tree = torch.zeros(2 * cap, dtype=torch.float32, device="cuda")
        ps.segtree_build(tree, dev(p0), 0.6)
        ot = oracle.Tree("f32", cap).build(p0, cap, 0.6)
    else:
        p0 = si.sweep_u32(cap)
        tree = torch.zeros(2 * cap, dtype=torch.uint64, device="cuda")
        ps.segtree_build(tree, dev(p0))
        ot = oracle.Tree("u64", cap).build(p0, cap)
    for name, idx in _stress_batches(cap, rng):
        say(f"stress {kind}: {name}")
        m = idx.size
        if kind == "f32":
            v = si.generic_f32(m, m + 11, "uniform")
            ps.segtree_update(tree, dev(idx), dev(v), 0.6)
            ok = (idx >= 0) & (idx < cap)
            ot.update(idx[ok], v[ok], 0.6)
            check_f32_tree(host(tree), ot, cap, name)
        else:
            v = si.sweep_u32(m)
            ps.segtree_update(tree, dev(idx), dev(v))
            ok = (idx >= 0) & (idx < cap)
            ot.update(idx[ok], v[ok])
            assert np.array_equal(host(tree)[1:], ot.flat()[1:]), name
        # the tree equals a fresh build of its own leaves
        flat = host(tree)
        j = np.arange(1, cap)
        s = (flat[2 * j] + flat[2 * j + 1]).astype(flat.dtype)
        assert np.array_equal(flat[1:cap], s), name


@pytest.mark.parametrize("k,strat", [(1, False), (1024, False), (1000, True), (1 << 16, True)])
def test_tree_sample_int_matches_cdf_path(ps, k, strat):
    d = si.per_large_int(n=300000, k=k)
    cap = ps.segtree_cap_pow2(300000)
    tree = torch.zeros(2 * cap, dtype=torch.uint64, device="cuda")
    Q = dev(d["q"])
    ps.segtree_build(tree, Q)
    idx_t = host(ps.segtree_sample(tree, 300000, dev(d["r"]), stratified=strat))
    _, _, _, idx_o = oracle.sample_int(d["q"], d["r"], strat)
    assert np.array_equal(idx_t, idx_o)


def test_per_large_tree_path(ps):
    """PER large, the same 2^20 draws through a 2^24-leaf sum tree: F32 tree
    bit-exact against the oracle's pointer tree; U64 tree identical to the
    integer CDF path."""
    d = si.per_large()
    n = d["p"].size
    cap = n
    say("PER large tree: oracle build (2^24 pointer tree) ...")
    ot = oracle.Tree("f32", cap).build(d["p"], n, d["alpha"])
    tree = torch.zeros(2 * cap, dtype=torch.float32, device="cuda")
    ps.segtree_build(tree, dev(d["p"]), d["alpha"])
    check_f32_tree(host(tree), ot, cap, "per_large f32 tree")
    idx_g = host(ps.segtree_sample(tree, n, dev(d["U"]), stratified=True))
    idx_o = ot.sample(d["U"], n, stratified=True)
    assert np.array_equal(idx_g, idx_o)
    del ot
    di = si.per_large_int()
    treeq = torch.zeros(2 * cap, dtype=torch.uint64, device="cuda")
    ps.segtree_build(treeq, dev(di["q"]))
    idx_t = host(ps.segtree_sample(treeq, n, dev(di["r"]), stratified=True))
    _, _, _, idx_c = oracle.sample_int(di["q"], di["r"], True)
    assert np.array_equal(idx_t, idx_c)


@pytest.mark.timeout(400)
def test_tree_max_cap_int(ps):
    """The largest tree the ABI takes: 2^30 leaves (2^31 uint64 nodes,
    16 GiB) with n_valid = 2^30 - 3.  Root = the exact sum of the leaves;
    stratified and iid descents equal to the oracle's integer CDF path (the
    descent of an exact tree is the lower bound on the CDF); then 4096
    updates of distinct leaves, the first and last valid ones among them,
    and the same checks on the updated priorities."""
    cap = 1 << 30
    n = cap - 3
    assert ps.segtree_cap_pow2(n) == cap
    say(f"max tree int: cap={cap} n_valid={n}")
    q = si.sweep_u32(n, seed=77)
    tree = torch.zeros(2 * cap, dtype=torch.uint64, device="cuda")
    ps.segtree_build(tree, dev(q))
    rng = np.random.default_rng(30)
    r = si.uniform_u32(rng, 1 << 16)

    def check(what):
        assert int(host(tree[1:2])[0]) == int(q.sum(dtype=np.uint64)), what
        for strat in (True, False):
            idx_t = host(ps.segtree_sample(tree, n, dev(r), stratified=strat))
            _, _, _, idx_o = oracle.sample_int(q, r, strat)
            say(f"  {what} strat={strat}: {int(np.sum(idx_t != idx_o))} mismatches")
            assert np.array_equal(idx_t, idx_o), what

    check("built")
    m = 4096
    upd = np.concatenate([[0, n - 1], 1 + rng.choice(n - 2, size=m - 2, replace=False)])
    upd = upd.astype(np.int32)
    v = rng.integers(1, 1 << 20, size=m, dtype=np.int64).astype(np.uint32)
    v[:2] = [1 << 20, 1]
    ps.segtree_update(tree, dev(upd), dev(v))
    q[upd] = v
    check("updated")
    del tree
    torch.cuda.empty_cache()


# ------------------------------------------------------------ resampling
def _row_check(lw, u_row, anc_g, what):
    anc_o = oracle.resample_rows(lw, u_row)
    if np.array_equal(anc_g, anc_o):
        say(f"{what}: identical")
        return
    P = lw.shape[1]
    unexc = exc = 0
    for b in np.nonzero(np.any(anc_g != anc_o, axis=1))[0]:
        _, Cc = oracle.row_cdf(lw[b])
        uk = ((np.arange(P, dtype=np.float32) + u_row[b]) / np.float32(P)).astype(np.float64)
        from parity_util import excuse_counts
        a, e = excuse_counts(anc_g[b], anc_o[b], uk, Cc, 1.0)
        unexc += a
        exc += e
    say(f"{what}: unexcused={unexc} excused={exc}")
    assert unexc == 0 and exc < 1e-4 * anc_g.size


def test_resample_cfg(ps):
    """Particle resampling: 1024 rows x 4096 particles, log-weights N(0, 3^2)."""
    d = si.resample()
    anc = host(ps.resample_rows(dev(d["lw"]), dev(d["u_row"])))
    _row_check(d["lw"], d["u_row"], anc, "resample cfg")
    assert np.all(np.diff(anc, axis=1) >= 0)


@pytest.mark.parametrize("rows,P", [(3, 1), (5, 7), (16, 1000), (16, 1024), (8, 1025),
                                    (8, 3000), (4, 8192), (2, 8191)])
def test_resample_shapes(ps, rows, P):
    d = si.resample(seed=P, rows=rows, P=P, sigma=2.0)
    anc = host(ps.resample_rows(dev(d["lw"]), dev(d["u_row"])))
    _row_check(d["lw"], d["u_row"], anc, f"resample {rows}x{P}")


def test_resample_edges(ps):
    """Rows whose CDF is exact (zero-weight particles, one or two carrying
    all the mass) and extreme offsets: every ancestor equals the oracle's,
    including particles with hundreds or thousands of offspring and the k
    whose threshold is 0."""
    ninf = np.float32(-np.inf)
    for P in (4096, 3000):
        lw = np.full((6, P), ninf, np.float32)
        lw[0, 123] = 0.0                       # one particle takes every k
        lw[1, 10] = 0.0
        lw[1, P - 96] = 0.0                    # two halves
        lw[2, :] = 0.0                         # uniform, u = 0: t_0 = 0
        lw[3, :] = 0.0                         # uniform, u just below 1
        lw[4, 0] = 0.0                         # all mass on the first particle
        lw[5, P - 1] = 0.0                     # all mass on the last particle
        u = np.array([0.5, 0.25, 0.0, np.nextafter(np.float32(1), np.float32(0)), 0.75, 0.1],
                     np.float32)
        anc = host(ps.resample_rows(dev(lw), dev(u)))
        anc_o = oracle.resample_rows(lw, u)
        # rows whose CDF is exact in binary: 0, 1, 4, 5 always; the uniform
        # rows only when 1/P is (P a power of two) -- otherwise every
        # threshold sits within rounding of a CDF boundary, and the excuse
        # rule applies
        exact = [0, 1, 4, 5] + ([2, 3] if P & (P - 1) == 0 else [])
        assert np.array_equal(anc[exact], anc_o[exact]), f"P={P}"
        from parity_util import excuse_counts
        for b in (2, 3):
            _, Cc = oracle.row_cdf(lw[b])
            uk = ((np.arange(P, dtype=np.float32) + u[b]) / np.float32(P)).astype(np.float64)
            unexc, _ = excuse_counts(anc[b], anc_o[b], uk, Cc, 1.0)
            assert unexc == 0, f"P={P} row {b}"
        assert np.all(anc[0] == 123) and np.all(anc[4] == 0) and np.all(anc[5] == P - 1)


def test_resample_uniform_identity(ps):
    P = 4096
    lw = np.zeros((8, P), np.float32)
    lw[3] = -7.5
    u = np.linspace(0.01, 0.99, 8).astype(np.float32)
    anc = host(ps.resample_rows(dev(lw), dev(u)))
    assert np.array_equal(anc, np.tile(np.arange(P, dtype=np.int32), (8, 1)))


@pytest.mark.parametrize("rows,P,pad_in,pad_out", [(37, 1024, 64, 8), (37, 1024, 3, 1),
                                                   (9, 1000, 3, 5), (5, 8192, 4, 4),
                                                   (6, 4097, 1, 7)])
def test_resample_strided_rows(ps, rows, P, pad_in, pad_out):
    """Row-strided input and output (ld_in = P + pad_in, ld_out = P + pad_out;
    a stride that is a multiple of 4 keeps the 16-byte path, others take the
    element-wise one): the ancestors of every row as the oracle's, and the
    padding of the output untouched."""
    d = si.resample(seed=rows * P + pad_in, rows=rows, P=P)
    big = np.full((rows, P + pad_in), np.float32(7.0))
    big[:, :P] = d["lw"]
    lw_t = dev(big)[:, :P]
    out_big = torch.full((rows, P + pad_out), -7, dtype=torch.int32, device="cuda")
    ps.resample_rows(lw_t, dev(d["u_row"]), out=out_big[:, :P])
    o = host(out_big)
    assert np.all(o[:, P:] == -7)
    _row_check(d["lw"], d["u_row"], o[:, :P], f"strided {rows}x{P} +{pad_in}/+{pad_out}")


@pytest.mark.timeout(400)
def test_resample_rows_beyond_2p31_elements(ps):
    """524291 rows x 4096 particles (2^31 + 12288 log-weights, 8 GiB in and
    8 GiB out, so row offsets need 64 bits): the first and last 32 rows and
    64 others as the oracle's; every row's ancestors non-decreasing and in
    [0, P)."""
    rows, P = (1 << 19) + 3, 4096
    say(f"resample {rows}x{P}: generating")
    d = si.resample(seed=2031, rows=rows, P=P)
    anc = ps.resample_rows(dev(d["lw"]), dev(d["u_row"]))
    rng = np.random.default_rng(5)
    sel = np.concatenate([np.arange(32), np.arange(rows - 32, rows),
                          rng.choice(rows - 64, size=64, replace=False) + 32])
    a_sel = host(anc[torch.from_numpy(sel).cuda()])
    _row_check(d["lw"][sel], d["u_row"][sel], a_sel, f"resample {rows}x{P} sampled rows")
    assert bool((anc[:, 1:] >= anc[:, :-1]).all())
    assert bool((anc >= 0).all()) and bool((anc < P).all())
    del anc
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cap", [1, 2, 4, 8, 64, 128, 256, 4096])
def test_tree_update_small_trees(ps, cap):
    """Trees with fewer levels than the update's split (1 to 64 subtree
    workgroups): random batches with repeats, f32 against the pointer tree
    bit for bit, u64 exactly; one update workspace for all calls."""
    rng = np.random.default_rng(cap)
    p0 = si.generic_f32(cap, cap + 1, "uniform")
    tree = torch.zeros(2 * cap, dtype=torch.float32, device="cuda")
    ps.segtree_build(tree, dev(p0), 0.6)
    ot = oracle.Tree("f32", cap).build(p0, cap, 0.6)
    q0 = si.sweep_u32(cap)
    treeq = torch.zeros(2 * cap, dtype=torch.uint64, device="cuda")
    ps.segtree_build(treeq, dev(q0))
    otq = oracle.Tree("u64", cap).build(q0, cap)
    ws = ps.Workspace(ps.segtree_update_workspace_size(cap, 1024))
    for m in (1, 3, 100, 1024, 3000):
        idx = rng.integers(0, cap, m).astype(np.int32)
        v = si.generic_f32(m, m + cap, "uniform")
        ps.segtree_update(tree, dev(idx), dev(v), 0.6, ws=ws)
        ot.update(idx, v, 0.6)
        check_f32_tree(host(tree), ot, cap, f"cap {cap} m {m}")
        q = si.sweep_u32(m)
        ps.segtree_update(treeq, dev(idx), dev(q), ws=ws)
        otq.update(idx, q)
        assert np.array_equal(host(treeq)[1:], otq.flat()[1:]), (cap, m)
    assert int(host(ws.buf).astype(np.int64).sum()) == 0     # the counter is back at 0


@pytest.mark.parametrize("per_sub", [63, 64, 65, 200])
def test_tree_update_crowded_subtree(ps, per_sub):
    """A subtree that receives per_sub entries of the batch (ranked in one
    wave up to 64, radix-sorted above), with repeats, next to sparsely
    updated subtrees."""
    cap = 1 << 19
    rng = np.random.default_rng(per_sub)
    p0 = si.generic_f32(cap, 5, "uniform")
    tree = torch.zeros(2 * cap, dtype=torch.float32, device="cuda")
    ps.segtree_build(tree, dev(p0), 0.6)
    ot = oracle.Tree("f32", cap).build(p0, cap, 0.6)
    sub = cap // 64
    crowd = rng.integers(5 * sub, 5 * sub + per_sub // 2 + 1, per_sub)   # repeats too
    rest = rng.integers(0, cap, 1024 - per_sub)
    idx = np.concatenate([crowd, rest]).astype(np.int32)
    rng.shuffle(idx)
    v = si.generic_f32(1024, per_sub + 7, "uniform")
    ps.segtree_update(tree, dev(idx), dev(v), 0.6)
    ot.update(idx, v, 0.6)
    check_f32_tree(host(tree), ot, cap, f"crowded {per_sub}")
