"""The seeded input generators: the same seed gives the same bytes, and each
workload has the support and moments its recipe states.  CPU only."""
import numpy as np
import pytest

import synthetic_inputs as si


def _same(a, b):
    assert a.keys() == b.keys()
    for key in a:
        x, y = a[key], b[key]
        if isinstance(x, np.ndarray):
            assert x.dtype == y.dtype and np.array_equal(x, y), key
        else:
            assert x == y, key


@pytest.mark.parametrize("make", [si.per_small, si.per_mid, si.resample, si.pf_small,
                                  lambda: si.per_large(n=1 << 20, k=1 << 16),
                                  lambda: si.per_large_int(n=1 << 20, k=1 << 16),
                                  lambda: si.sumtree(rounds=8)])
def test_same_seed_same_bytes(make):
    _same(make(), make())


def test_fractions_in_unit_interval():
    for U in (si.per_small()["U"], si.per_mid()["U"].ravel(), si.resample()["u_row"],
              si.uniform_f32(np.random.default_rng(3), 1 << 20)):
        assert U.dtype == np.float32
        assert U.min() >= 0.0 and U.max() < 1.0
        assert abs(float(U.mean()) - 0.5) < 0.02


def test_workload_distributions():
    d = si.per_small()                                   # |N(0,1)| + 1e-6
    assert d["p"].dtype == np.float32 and d["p"].size == 8192 and d["U"].size == 1024
    assert d["p"].min() >= np.float32(1e-6)
    assert abs(float(d["p"].mean()) - np.sqrt(2 / np.pi)) < 0.03
    d = si.per_mid()                                     # Exp(1) + 1e-6, 32 rounds
    assert d["p0"].size == 262144 and d["U"].shape == (32, 8192) and d["v"].shape == (32, 8192)
    assert d["p0"].min() >= np.float32(1e-6) and abs(float(d["p0"].mean()) - 1.0) < 0.01
    d = si.sumtree(rounds=8)                             # U(0.01, 1)^(1/0.6)
    lo = 0.01 ** (1 / 0.6)
    assert d["p0"].size == 500000 and d["p0"].min() >= np.float32(lo) * 0.999
    assert d["p0"].max() <= 1.0
    assert d["idx"].min() >= 0 and d["idx"].max() < 500000 and d["idx"].dtype == np.int32
    d = si.resample()                                    # N(0, 3^2), 1024 x 4096
    assert d["lw"].shape == (1024, 4096)
    assert abs(float(d["lw"].mean())) < 0.01 and abs(float(d["lw"].std()) - 3.0) < 0.01
    d = si.per_large(n=1 << 22, k=1 << 16)               # LogNormal(0, 2)
    lp = np.log(d["p"].astype(np.float64))
    assert abs(float(np.median(lp))) < 0.01 and abs(float(lp.std()) - 2.0) < 0.01
    d = si.per_large_int(n=1 << 20, k=1 << 16)           # U{1 .. 2^20}
    assert d["q"].dtype == np.uint32 and d["q"].min() >= 1 and d["q"].max() <= 1 << 20
    assert d["r"].dtype == np.uint32
