"""Every path twice on the same inputs (sharing one workspace, whose parity
and call numbers advance in between): the same bits each time -- fp mode
included, since every sum has a fixed association and no result depends on
timing."""
import numpy as np
import pytest
import torch

import synthetic_inputs as si
from parity_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ps():
    import proportional_sampling_amd as ps
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ps.lib()
    return ps


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _twice(fn):
    a = fn()
    b = fn()
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert x.dtype == y.dtype and torch.equal(x, y)


@pytest.mark.parametrize("n,k", [(262144, 8192), ((1 << 23) + 1, 1 << 18)])
def test_per_round_twice(ps, n, k):
    """The fused update on a resident grid and, at 2^23 + 1, in three kernels:
    indices, weights, CDF, total and the rewritten priorities."""
    say(f"per_round twice n={n} k={k}")
    p0 = dev(si.generic_f32(n, 17, "exp"))
    U = dev(si.uniform_f32(np.random.default_rng(18), k))
    newp = dev(si.generic_f32(k, 19, "exp"))
    ws = ps.Workspace(ps.per_round_workspace_size(n, k))

    def run():
        P = p0.clone()
        idx, w, cdf, tot = ps.per_round(P, U, 0.6, 0.4, newp, ws=ws)
        return idx, w, cdf, tot, P
    _twice(run)


def test_build_cdf_sample_twice(ps):
    n, k = (1 << 22) + 9, 1 << 16
    P = dev(si.generic_f32(n, 23, "lognormal"))
    U = dev(si.uniform_f32(np.random.default_rng(24), k))
    ws = ps.Workspace(ps.build_cdf_workspace_size(n))
    _twice(lambda: ps.build_cdf_sample(P, U, 0.7, ws=ws))


def test_is_weights_twice(ps):
    d = si.per_large(n=1 << 22, k=1 << 20)
    P = dev(d["p"])
    idx = dev(np.sort(np.random.default_rng(25).integers(0, 1 << 22, 1 << 20)).astype(np.int32))
    ws = ps.Workspace(ps.is_weights_workspace_size(1 << 20))
    _twice(lambda: (ps.is_weights(P, idx, d["alpha"], d["beta"], ws=ws),))


@pytest.mark.parametrize("kind", [torch.float32, torch.uint64])
def test_tree_update_twice(ps, kind):
    d = si.sumtree(rounds=2)
    cap = ps.segtree_cap_pow2(500000)
    base = torch.zeros(2 * cap, dtype=kind, device="cuda")
    if kind == torch.float32:
        ps.segtree_build(base, dev(d["p0"]), d["alpha"])
        vals = dev(d["v"][0])
    else:
        q = (d["p0"] * 1e6).astype(np.uint32) + 1
        ps.segtree_build(base, dev(q))
        vals = dev((d["v"][0] * 1e6).astype(np.uint32) + 1)
    idx = dev(d["idx"][0])

    def run():
        t = base.clone()
        ps.segtree_update(t, idx, vals, d["alpha"] if kind == torch.float32 else 1.0)
        return (t,)
    _twice(run)


def test_resample_and_pf_twice(ps):
    d = si.resample(rows=256)
    lw, u = dev(d["lw"]), dev(d["u_row"])
    _twice(lambda: (ps.resample_rows(lw, u),))
    f = si.pf_step(rows=64, P=4096)
    args = [dev(f[key]) for key in ("x", "lw", "obs", "A", "C", "eps")]
    ur = dev(f["u_row"])
    _twice(lambda: ps.pf_step(*args, f["sigma_p"], f["sigma_o"], ur))
