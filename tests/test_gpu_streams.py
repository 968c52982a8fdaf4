"""Calls on a stream other than torch's current one: the binding allocates
and zero-fills its temporaries (outputs, workspaces) in that stream's order,
so the results equal those of the same calls on the default stream -- also
while the default stream is still busy with earlier work, and with the
stream given as a raw hipStream_t."""
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


def _busy_default_stream():
    """Queue ~1 ms of work on the default stream (ordinary torch ops)."""
    x = torch.ones(1 << 24, device="cuda")
    for _ in range(30):
        x = x * 1.0000001
    return x


def _calls(ps, d, p, U, tree_u, lw, u_row, mine, stream):
    """Every library call whose binding allocates something (outputs,
    workspaces), on `stream`; `mine` holds the caller-owned buffers, made
    and zeroed before the default stream was made busy."""
    a, b = d["alpha"], d["beta"]
    q, newp, tree = mine
    cdf, tot = ps.build_cdf(p, a, stream=stream)
    idx = ps.sample(cdf, tot, U, stratified=True, stream=stream)
    w = ps.is_weights(p, idx, a, b, stream=stream)
    idx_f, cdf_f, tot_f = ps.build_cdf_sample(p, U, a, stream=stream)
    idx_r, w_r, cdf_r, tot_r = ps.per_round(q, U, a, b, newp, stream=stream)
    ps.segtree_build(tree, p, a, stream=stream)
    t_idx = ps.segtree_sample(tree, p.numel(), tree_u, stream=stream)
    anc = ps.resample_rows(lw, u_row, stream=stream)
    return [cdf, tot, idx, w, idx_f, cdf_f, tot_f, q, idx_r, w_r, cdf_r, tot_r, tree, t_idx, anc]


def _mine(p, k):
    return (p.clone(), p[:k].clone(), torch.zeros(2 * 8192, dtype=torch.float32, device="cuda"))


@pytest.mark.parametrize("raw", [False, True])
def test_side_stream_equals_default_stream(ps, raw):
    say(f"side stream raw={raw}")
    d = si.per_small()
    p, U = dev(d["p"]), dev(d["U"])
    rng = np.random.default_rng(9)
    tree_u = dev(si.uniform_f32(rng, 1024))
    lw = dev(rng.normal(0, 3, (64, 4096)).astype(np.float32))
    u_row = dev(si.uniform_f32(rng, 64))
    ref = _calls(ps, d, p, U, tree_u, lw, u_row, _mine(p, U.numel()), None)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    for rep in range(3):
        mine = _mine(p, U.numel())
        torch.cuda.synchronize()
        busy = _busy_default_stream()        # default stream busy; s is not
        got = _calls(ps, d, p, U, tree_u, lw, u_row, mine, s.cuda_stream if raw else s)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        del busy
        for j, (r, g) in enumerate(zip(ref, got)):
            assert torch.equal(r, g), f"rep {rep}: output {j} differs on the side stream"
