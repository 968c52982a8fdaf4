"""Helpers of the GPU parity tests: the boundary-excuse rule and printing.

Parity contract (floating point): an index that differs from the oracle's is
excused iff the oracle's threshold lies within 1e-6 * T of every CDF
boundary between the two picks (C_b for b in [min(g, o), max(g, o) - 1]);
no unexcused mismatch is allowed and excused ones must stay below 1e-4 of
the samples.  Integer mode is bit-exact.
"""
import sys

import numpy as np


def say(*a):
    print("[parity]", *a, flush=True)
    sys.stdout.flush()


def excuse_counts(g_idx, o_idx, t, C, T, tol=1e-6):
    """Returns (unexcused, excused) mismatch counts."""
    g_idx = np.asarray(g_idx, np.int64)
    o_idx = np.asarray(o_idx, np.int64)
    mism = np.nonzero(g_idx != o_idx)[0]
    unexc = 0
    for i in mism:
        lo, hi = sorted((int(g_idx[i]), int(o_idx[i])))
        gaps = np.abs(float(t[i]) - C[lo:hi])
        if not np.all(gaps <= tol * T):
            unexc += 1
    return unexc, int(mism.size - unexc)


def assert_indices(g_idx, o_idx, t, C, T, what=""):
    unexc, exc = excuse_counts(g_idx, o_idx, t, C, T)
    k = len(o_idx)
    say(f"{what}: k={k} mismatches unexcused={unexc} excused={exc}")
    assert unexc == 0, f"{what}: {unexc} unexcused index mismatches"
    assert exc < 1e-4 * k or exc == 0, f"{what}: {exc} excused mismatches (>= 1e-4 of {k})"
    return exc


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.maximum(np.abs(b), np.finfo(np.float64).tiny)
    return float(np.max(np.abs(a - b) / den)) if a.size else 0.0


def ulp_diff_f32(a, b):
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(a - b)
