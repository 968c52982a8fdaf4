"""GPU parity of the sum-tree replay priorities against the oracle's ring:
slots and the F32 tree bit for bit after every step, sampled slots equal,
IS weights within 1e-6, the total equal to the root."""
import numpy as np
import pytest
import torch

import oracle
from parity_util import say

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


def same_tree(rb, orb, what):
    g = host(rb.tree)
    o = orb.tree.flat()
    assert np.array_equal(g[1:].view(np.int32), o[1:].view(np.int32)), what
    assert host(rb.total()) == np.float32(orb.total())


@pytest.mark.parametrize("capacity,alpha", [(500000, 0.6), (1000, 0.7), (1, 1.0), (4097, 0.5)])
def test_replay_sequence(ps, capacity, alpha):
    """Inserts (batches above 1024 and above the capacity, wrapping the ring),
    updates with repeated slots, stratified and iid samples with IS weights."""
    rng = np.random.default_rng(capacity)
    rb = ps.ReplayPriorities(capacity, alpha, max_batch=8192)
    orb = oracle.Replay(capacity, alpha)
    sizes = [3, 1024, 1500, 2 * capacity + 5, 700] if capacity <= 5000 else [1024, 5000, 8192]
    for step, m in enumerate(sizes):
        p = (rng.random(m) * 2 + 0.01).astype(np.float32)
        if step == 1:
            p[:10] = 0.0                          # zero priorities are valid
        slots = host(rb.insert(dev(p)))
        assert np.array_equal(slots, orb.insert(p)), f"insert {step}"
        assert (rb.cursor, rb.size) == (orb.cursor, orb.size)
        same_tree(rb, orb, f"after insert {step}")
        # update: slots drawn from the filled ones, with repeats
        k = min(1500, 3 * orb.size)
        us = rng.integers(0, orb.size, k).astype(np.int32)
        uv = (rng.random(k) + 0.05).astype(np.float32)
        rb.update(dev(us), dev(uv))
        orb.update(us, uv)
        same_tree(rb, orb, f"after update {step}")
        for strat in (True, False):
            U = rng.random(2048, dtype=np.float32)
            idx, w = rb.sample(dev(U), 0.4, stratified=strat)
            oi, ow = orb.sample(U, 0.4, stratified=strat)
            idx, w = host(idx), host(w)
            assert np.array_equal(idx, oi), f"sample {step} strat={strat}"
            assert np.allclose(w, ow, rtol=1e-6, atol=0), f"IS {step}"
            assert idx.max() < orb.size
    say(f"replay cap={capacity}: {len(sizes)} rounds identical")


def test_replay_sample_without_weights_and_empty(ps):
    rb = ps.ReplayPriorities(64, 0.6, max_batch=64)
    U = dev(np.full(8, 0.5, np.float32))
    with pytest.raises(ps.PsampError):
        rb.sample(U, None)                      # empty ring
    rb.insert(dev(np.arange(1, 11, dtype=np.float32)))
    idx = host(rb.sample(U, None, stratified=False))
    assert idx.shape == (8,) and np.all(idx == idx[0]) and 0 <= idx[0] < 10
