"""Device-side precondition checks: with checking on, a call given an input
that breaks a precondition sets that precondition's bit (and only then);
valid inputs set none; with checking off nothing is recorded.  Every
invalid input here goes to a kernel that stays in bounds for any value: the
scan (arithmetic only), the iid search (a branch-free binary search with a
clamped result), the tree descent (a fixed number of levels), the IS
weights (indices clamped on use) and the row resampler (counts clamped to
[0, P])."""
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
    prev = ps.check_enable(True)
    ps.check_errors(clear=True)
    yield ps
    ps.check_enable(prev)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _valid_calls(ps):
    d = si.per_small()
    p, U = dev(d["p"]), dev(d["U"])
    cdf, tot = ps.build_cdf(p, 0.6)
    idx = ps.sample(cdf, tot, U, stratified=True)
    ps.sample(cdf, tot, U, stratified=False)
    ps.is_weights(p, idx, 0.6, 0.4)
    ps.build_cdf_sample(p, U, 0.6)
    q = p.clone()
    ps.per_round(q, U, 0.6, 0.4, p[:U.numel()].clone())
    tree = torch.zeros(2 * 8192, dtype=torch.float32, device="cuda")
    ps.segtree_build(tree, p, 0.6)
    ps.segtree_update(tree, idx, p[:idx.numel()].clone(), 0.6)
    ps.segtree_sample(tree, p.numel(), U)
    rng = np.random.default_rng(3)
    lw = dev(rng.normal(0, 3, (8, 1024)).astype(np.float32))
    lw[0, 5] = float("-inf")                        # -inf is a valid log-weight
    ps.resample_rows(lw, dev(si.uniform_f32(rng, 8)))
    ps.scatter_lww(q, idx, p[:idx.numel()].clone(), grouped=True)


def test_valid_inputs_set_no_bit(ps):
    ps.check_errors(clear=True)
    _valid_calls(ps)
    assert ps.check_errors() == 0


def test_overflowing_total(ps):
    """Finite priorities whose weights pass the double range (p^alpha of
    3e38 at alpha 17): the total is +inf, flagged as not a positive finite
    total; a total just below DBL_MAX is not flagged."""
    p = si.generic_f32(5000, 4, "exp")
    p[100] = np.float32(3e38)
    ps.check_errors(clear=True)
    ps.build_cdf(dev(p), 17.0)
    assert ps.check_errors() == ps.CHECK_ZERO_TOTAL
    q = np.zeros(5000, np.float32)
    q[100] = np.float32(np.exp2(1023.5 / 16.0))        # p^16 about 0.7 DBL_MAX
    ps.check_errors(clear=True)
    ps.build_cdf(dev(q), 16.0)
    assert ps.check_errors() == 0


@pytest.mark.parametrize("case", ["nan", "neg", "inf", "zeros"])
def test_bad_priorities(ps, case):
    p = si.generic_f32(5000, 4, "exp")
    if case == "nan":
        p[17] = np.nan
    elif case == "neg":
        p[4999] = -1.0
    elif case == "inf":
        p[0] = np.inf
    else:
        p[:] = 0.0
    ps.check_errors(clear=True)
    ps.build_cdf(dev(p), 0.6)
    bits = ps.check_errors()
    say(f"priorities {case}: bits {bits}")
    if case == "zeros":
        assert bits == ps.CHECK_ZERO_TOTAL
    else:
        assert bits & ps.CHECK_PRIORITY


@pytest.mark.parametrize("bad", [1.0, -0.25, float("nan")])
def test_bad_fractions(ps, bad):
    p = dev(si.generic_f32(100000, 5, "exp"))
    cdf, tot = ps.build_cdf(p, 0.6)
    U = si.uniform_f32(np.random.default_rng(6), 100)
    U[37] = bad
    ps.check_errors(clear=True)
    ps.sample(cdf, tot, dev(U), stratified=False)          # the binary search
    assert ps.check_errors() == ps.CHECK_FRACTION
    tree = torch.zeros(2 * 131072, dtype=torch.float32, device="cuda")
    ps.segtree_build(tree, p, 0.6)
    ps.check_errors(clear=True)
    ps.segtree_sample(tree, p.numel(), dev(U))
    assert ps.check_errors() == ps.CHECK_FRACTION


def test_bad_indices(ps):
    n = 1000
    p = dev(si.generic_f32(n, 7, "exp"))
    for bad in (n, -1, 1 << 30):
        idx = np.arange(64, dtype=np.int32)
        idx[9] = bad
        ps.check_errors(clear=True)
        ps.is_weights(p, dev(idx), 0.6, 0.4)
        assert ps.check_errors() == ps.CHECK_INDEX, bad


@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_bad_log_weights(ps, bad):
    rng = np.random.default_rng(8)
    lw = rng.normal(0, 3, (4, 4096)).astype(np.float32)
    lw[2, 100] = bad
    u = si.uniform_f32(rng, 4)
    ps.check_errors(clear=True)
    anc = ps.resample_rows(dev(lw), dev(u))
    assert ps.check_errors() == ps.CHECK_LOGWEIGHT
    a = anc.cpu().numpy()
    assert a.min() >= 0 and a.max() < 4096          # still written, in range
    u[1] = 1.0
    ps.check_errors(clear=True)
    ps.resample_rows(dev(lw), dev(u))
    assert ps.check_errors() == ps.CHECK_LOGWEIGHT | ps.CHECK_FRACTION


def test_checks_off_record_nothing(ps):
    ps.check_enable(False)
    try:
        p = si.generic_f32(5000, 9, "exp")
        p[3] = np.nan
        ps.check_errors(clear=True)
        ps.build_cdf(dev(p), 0.6)
        assert ps.check_errors() == 0
    finally:
        ps.check_enable(True)
