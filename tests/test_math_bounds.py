"""Error bounds of the library's fp64 math, tested on the CPU: the functions
the kernels inline (log2, exp2, the two p^alpha paths, the row resampler's
exp) are __host__ __device__, so math_bounds.hip compiles the same source
for the host and measures each against long double over seeded samples
that cover every float exponent, the subnormals and both ends of the double
range.  The bounds asserted are the ones the source comments state; each
one sits far below the ~1e-9 on the weights that the index contract needs.
No GPU is used."""
import json
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
DBL_MIN = 2.2250738585072014e-308


@pytest.fixture(scope="module")
def bounds(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc is not installed")
    exe = str(tmp_path_factory.mktemp("math") / "math_bounds")
    # the library's own floating-point flags (no contraction beyond fma())
    subprocess.run([HIPCC, "-x", "hip", "--offload-host-only", "-O2", "-std=c++17",
                    "-ffp-contract=off", "-I", os.path.join(ROOT, "proportional_sampling_amd", "csrc"),
                    os.path.join(ROOT, "tests", "math_bounds.hip"), "-o", exe],
                   check=True, capture_output=True, text=True)
    out = subprocess.run([exe, "400000"], check=True, capture_output=True, text=True).stdout
    return json.loads(out)


@pytest.mark.parametrize("name,bound", [
    ("log2_sig32", 4e-16),                # of max(1, |log2 x|)
    ("exp2_tab_rel", 4e-16),
    ("exp2_tab_subnormal_abs", 4e-16),    # in units of DBL_MIN
    ("pow_prio_rel", 3e-13),              # about 2.6e-16 (|alpha log2 p| + 1)
    ("pow_prio_fast_rel", 4e-15),
    ("pow_prio_fast_outside_normal", 4e-15),
    ("exp_row_rel", 2e-13),
    ("exp_row_subnormal_abs", 2e-13),
])
def test_error_bound(bounds, name, bound):
    b = bounds[name]
    assert b["n"] > 1000, (name, b)
    assert b["err"] <= bound, f"{name}: {b['err']:.3e} at {b['at']!r} (alpha {b['at2']})"


def test_special_values(bounds):
    """0 -> 0, +inf -> +inf, negative or NaN -> NaN for both powers; exact
    powers of two from exp2; exp_row(0) = 1, underflow to 0, NaN through."""
    assert bounds["special"] == 1


def test_samples_reach_both_ends_of_the_range(bounds):
    """The table path was driven past DBL_MAX and below DBL_MIN (where its
    scaled exponent table matters), not only through the middle."""
    assert bounds["pow_prio_fast_outside_normal"]["n"] > 10000
    assert bounds["exp2_tab_subnormal_abs"]["n"] > 1000
    assert bounds["exp_row_subnormal_abs"]["n"] > 1000
