"""Why "fp32 mode" sums in fp64: an all-float32 pipeline (float32 weights,
a sequential float32 prefix sum, float32 thresholds on its own total) draws
other indices than the fp64 oracle for far more than the 1e-4 of draws the
index contract allows -- at the PER-small shape already, and for nearly every
draw at the PER-large shape, where the float32 running sum has lost the
small weights' contributions.  CPU only."""
import numpy as np
import pytest

import oracle
import synthetic_inputs as si


def _fp32_pipeline(p, alpha, U):
    w = np.power(p, np.float32(alpha), dtype=np.float32)
    C = np.cumsum(w, dtype=np.float32)                  # sequential, float32
    k = np.float32(U.size)
    t = ((np.arange(U.size, dtype=np.float32) + U) / k) * C[-1]
    return np.minimum(np.searchsorted(C, t, side="left"), p.size - 1)


@pytest.mark.parametrize("shape", ["per_small", "per_large"])
def test_float32_sums_break_the_index_budget(shape):
    if shape == "per_small":
        d = si.per_small()
        p, U, alpha, lo = d["p"], d["U"], d["alpha"], 1e-4
    else:
        d = si.per_large()
        p, U, alpha, lo = d["p"], d["U"], d["alpha"], 0.5
    _, _, _, idx64 = oracle.sample(p, alpha, U, True)
    idx32 = _fp32_pipeline(p, alpha, U)
    frac = float(np.mean(idx32 != idx64))
    assert frac > lo, f"{shape}: float32 pipeline differs on {frac:.2e} of draws"
