"""psamp_per_round_noalloc (the fused update with the library's own scratch
instead of a caller's workspace) through the C ABI: the same results, bit
for bit, as psamp_per_round with a fresh workspace, on calls in a row whose
sizes shrink (the scratch keeps the previous call's state) and that take
both the one-kernel and the three-kernel path; sizes above the scratch's
limit are refused before anything is enqueued."""
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


def _case(n, k, seed):
    p = si.generic_f32(n, seed, "lognormal")
    U = si.uniform_f32(np.random.default_rng(seed + 1), k)
    newp = si.generic_f32(k, seed + 2, "exp")
    return p, U, newp


def _outs(n, k):
    return dict(out_idx=torch.empty(k, dtype=torch.int32, device="cuda"),
                out_w=torch.empty(k, dtype=torch.float32, device="cuda"),
                cdf=torch.empty(n, dtype=torch.float64, device="cuda"),
                total=torch.empty(1, dtype=torch.float64, device="cuda"))


def test_noalloc_equals_per_round(ps):
    # 2^23 + 1: beyond a resident grid (three kernels); then smaller inputs
    # on the one-kernel path; then the largest n the scratch takes
    for call, (n, k, seed) in enumerate([((1 << 23) + 1, 1 << 16, 51), (262144, 8192, 52),
                                         (8192, 1024, 53), (1 << 26, 1 << 20, 54),
                                         (5000, 700, 55)]):
        say(f"noalloc call {call}: n={n} k={k}")
        p, U, newp = _case(n, k, seed)
        P_ref, P_na = dev(p), dev(p)
        Ud, Nd = dev(U), dev(newp)
        ref = ps.per_round(P_ref, Ud, 0.7, 0.5, Nd,
                           ws=ps.Workspace(ps.per_round_workspace_size(n, k)))
        outs = _outs(n, k)
        got = ps.per_round_noalloc(P_na, Ud, 0.7, 0.5, Nd, **outs)
        torch.cuda.synchronize()
        for name, r, g in zip(("indices", "weights", "cdf", "total"), ref, got):
            assert torch.equal(r, g), f"call {call}: {name} differ"
        assert torch.equal(P_ref, P_na), f"call {call}: rewritten priorities differ"
        del P_ref, P_na, ref, got, outs
    torch.cuda.empty_cache()


def test_noalloc_refuses_sizes_beyond_the_scratch(ps):
    n = ps.NOALLOC_MAX_N + 1
    L = ps.lib()
    FAKE = 0x10000
    assert L.psamp_per_round_noalloc(FAKE, n, 0.6, 0.4, FAKE, 8, None, FAKE, FAKE, FAKE, FAKE,
                                     None) == 2        # PSAMP_E_SIZE, nothing enqueued
