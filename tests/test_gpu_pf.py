"""GPU parity of the fused particle-filter step against the oracle.

The predicted states and updated log-weights are float32 computations in a
fixed order on both sides, so every gathered state must equal the oracle's
prediction of the same ancestor bit for bit; the ancestors follow the
resampler's contract (identical, or excused at a CDF boundary)."""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from parity_util import excuse_counts, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ps():
    import proportional_sampling_amd as ps
    assert torch.cuda.is_available()
    return ps


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def run_gpu(ps, d, A=None, anc=True, **kw):
    A = d["A"] if A is None else A
    rows, P, _ = d["x"].shape
    a_out = torch.empty(rows, P, dtype=torch.int32, device="cuda") if anc else None
    xo, lo = ps.pf_step(dev(d["x"]), dev(d["lw"]), dev(d["obs"]), dev(A), dev(d["C"]),
                        dev(d["eps"]), d["sigma_p"], d["sigma_o"], dev(d["u_row"]),
                        anc_out=a_out, **kw)
    return host(xo), host(lo), (host(a_out) if anc else None)


def check(d, xo, lo, anc, what, A=None, rows=None):
    """Compare rows `rows` (default all) of the GPU outputs with the oracle
    run on those rows alone (filters are independent)."""
    A = d["A"] if A is None else A
    sel = np.arange(d["x"].shape[0]) if rows is None else np.asarray(rows)
    xo_o, lo_o, anc_o, pred_o, lwn_o = oracle.pf_step(
        d["x"][sel], d["lw"][sel], d["obs"][sel], A, d["C"], d["eps"][sel], d["sigma_p"],
        d["sigma_o"], d["u_row"][sel])
    xo, lo, anc = xo[sel], lo[sel], anc[sel]
    P = d["x"].shape[1]
    assert np.all(lo == np.float32(-np.log(P)))
    # every gathered state is the oracle's prediction of its ancestor, bit for bit
    got = np.take_along_axis(pred_o, anc[:, :, None].astype(np.int64), axis=1)
    assert np.array_equal(xo.view(np.int32), got.view(np.int32)), what
    unexc = exc = 0
    for i in np.nonzero(np.any(anc != anc_o, axis=1))[0]:
        _, Cc = oracle.row_cdf(lwn_o[i])
        uk = ((np.arange(P, dtype=np.float32) + d["u_row"][sel[i]]) / np.float32(P))
        a, e = excuse_counts(anc[i], anc_o[i], uk.astype(np.float64), Cc, 1.0)
        unexc += a
        exc += e
    say(f"{what}: ancestors unexcused={unexc} excused={exc}")
    assert unexc == 0 and exc < 1e-4 * anc.size
    assert np.all(np.diff(anc, axis=1) >= 0)
    if exc == 0:
        assert np.array_equal(xo, xo_o)


@pytest.mark.parametrize("rows,P,D,O", [(16, 1024, 4, 2), (7, 1000, 4, 2), (5, 4096, 4, 2),
                                        (3, 3000, 2, 3), (4, 8192, 2, 1), (6, 1, 1, 1),
                                        (5, 2048, 8, 8), (9, 777, 8, 5), (3, 5, 4, 2),
                                        (4, 5000, 1, 4), (2, 1025, 8, 2)])
def test_pf_step_shapes(ps, rows, P, D, O):
    d = si.pf_step(seed=P * 16 + D, rows=rows, P=P, D=D, O=O)
    rng = np.random.default_rng(P + D)
    A = (0.9 * np.eye(D) + 0.05 * rng.standard_normal((D, D))).astype(np.float32)
    xo, lo, anc = run_gpu(ps, d, A=A)
    check(d, xo, lo, anc, f"pf {rows}x{P} D={D} O={O}", A=A)


def test_pf_step_pages_shape(ps):
    """16 filters x 1024 particles, D = 4, O = 2, A = 0.9 I."""
    d = si.pf_small()
    xo, lo, anc = run_gpu(ps, d)
    check(d, xo, lo, anc, "pf 16x1024")


def test_pf_step_large(ps):
    """1024 filters x 4096 particles, D = 4, O = 2 (the timed shape): every
    filter checked against the oracle, and the properties that hold for any
    filter."""
    d = si.pf_step()
    xo, lo, anc = run_gpu(ps, d)
    check(d, xo, lo, anc, "pf 1024x4096")
    assert np.all(np.diff(anc, axis=1) >= 0)
    assert np.all(lo == np.float32(-np.log(4096)))
    # each output row is made of the filter's own predictions: the gathered
    # state of offspring k equals the one of every other offspring of anc_k
    same = anc[:, 1:] == anc[:, :-1]
    assert np.array_equal(xo[:, 1:][same], xo[:, :-1][same])


def test_pf_step_in_place_and_no_ancestors(ps):
    d = si.pf_step(seed=77, rows=12, P=2048, D=4, O=2)
    xo, lo, anc = run_gpu(ps, d)
    x = dev(d["x"])
    lw = dev(d["lw"])
    ps.pf_step(x, lw, dev(d["obs"]), dev(d["A"]), dev(d["C"]), dev(d["eps"]), d["sigma_p"],
               d["sigma_o"], dev(d["u_row"]), x_out=x, logw_out=lw)
    assert np.array_equal(host(x), xo)
    assert np.array_equal(host(lw), lo)
    xo2, lo2, _ = run_gpu(ps, d, anc=False)
    assert np.array_equal(xo2, xo) and np.array_equal(lo2, lo)


def test_pf_step_unaligned_logw(ps):
    """log-weights at a 4-byte (not 16-byte) offset: the scalar load path."""
    d = si.pf_step(seed=78, rows=6, P=1024, D=4, O=2)
    xo, lo, anc = run_gpu(ps, d)
    big = torch.empty(6 * 1024 + 1, dtype=torch.float32, device="cuda")
    big[1:] = dev(d["lw"]).reshape(-1)
    lw_view = big[1:].view(6, 1024)
    a2 = torch.empty(6, 1024, dtype=torch.int32, device="cuda")
    xo2, lo2 = ps.pf_step(dev(d["x"]), lw_view, dev(d["obs"]), dev(d["A"]), dev(d["C"]),
                          dev(d["eps"]), d["sigma_p"], d["sigma_o"], dev(d["u_row"]),
                          anc_out=a2)
    assert np.array_equal(host(xo2), xo) and np.array_equal(host(a2), anc)


def test_pf_step_degenerate_weights(ps):
    """All the mass on one particle (every offspring is it) and a uniform
    filter (A = I, no noise, C = 0: the state is copied unchanged)."""
    P, D = 4096, 4
    d = si.pf_step(seed=79, rows=2, P=P, D=D, O=2)
    d["lw"][0, :] = -np.inf
    d["lw"][0, 1234] = 0.0
    d["lw"][1, :] = 0.0
    A = np.eye(D, dtype=np.float32)
    d["C"] = np.zeros_like(d["C"])
    d["sigma_p"] = 0.0
    xo, lo, anc = run_gpu(ps, d, A=A)
    assert np.all(anc[0] == 1234)
    assert np.array_equal(xo[0], np.repeat(d["x"][0, 1234:1235], P, axis=0))
    assert np.array_equal(anc[1], np.arange(P))
    assert np.array_equal(xo[1], d["x"][1])
