"""Seeded synthetic workloads for proportional sampling.

This module only draws random arrays. It holds none of the sampling
arithmetic, so both the CPU oracle (``oracle/``) and the GPU library
(``proportional_sampling_amd``) can be fed from it without sharing any
computation.

Conventions
-----------
* Every array comes from ``numpy.random.default_rng(seed)`` (PCG64), drawn in
  the order written below, so a (workload, seed) pair always gives the same
  bytes.
* Threshold fractions ``U`` and ``u_row`` are drawn directly as float32 with
  ``rng.random(n, dtype=np.float32)``: that keeps them in [0, 1) with 24-bit
  resolution (a float64 uniform cast to float32 can round up to 1.0).
* Integer threshold fractions ``r`` are uniform uint32.
* All other values are drawn in float64 and cast once to the stored dtype.

The shapes and distributions are those of the five sampling workloads:
PER small / PER mid / sum tree / particle resampling / PER large, plus the
integer-priority variant of PER large and a bandwidth sweep.
"""
from __future__ import annotations

import numpy as np

# Parameters of the workloads (alpha / beta as the nearest doubles).
PER_SMALL = dict(seed=1001, n=8192, k=1024, alpha=0.6, beta=0.4)
PER_MID = dict(seed=1002, n=262144, k=8192, rounds=32, alpha=0.6, beta=0.4)
SUMTREE = dict(seed=1003, n_valid=500000, cap=1 << 19, m=1024, k=1024,
               rounds=1000, alpha=0.6)
RESAMPLE = dict(seed=1004, rows=1024, P=4096)
PF_STEP = dict(seed=1008, rows=1024, P=4096, D=4, O=2, sigma_p=0.1, sigma_o=0.5)
PF_SMALL = dict(seed=1009, rows=16, P=1024, D=4, O=2, sigma_p=0.1, sigma_o=0.5)
PER_LARGE = dict(seed=1005, n=1 << 24, k=1 << 20, alpha=0.7, beta=0.5)
PER_LARGE_INT = dict(seed=1006, n=1 << 24, k=1 << 20, qmax=1 << 20, beta=0.5)
SWEEP_SEED = 1007


def uniform_f32(rng: np.random.Generator, n) -> np.ndarray:
    """Uniform float32 in [0, 1)."""
    return rng.random(n, dtype=np.float32)


def uniform_u32(rng: np.random.Generator, n) -> np.ndarray:
    return rng.integers(0, 2**32, size=n, dtype=np.uint32)


def per_small(seed: int = PER_SMALL["seed"], n: int = PER_SMALL["n"],
              k: int = PER_SMALL["k"]):
    """p = |N(0,1)| + 1e-6 (float32), U ~ U[0,1) (float32)."""
    rng = np.random.default_rng(seed)
    p = (np.abs(rng.standard_normal(n)) + 1e-6).astype(np.float32)
    U = uniform_f32(rng, k)
    return dict(p=p, U=U, alpha=PER_SMALL["alpha"], beta=PER_SMALL["beta"])


def per_mid(seed: int = PER_MID["seed"], n: int = PER_MID["n"],
            k: int = PER_MID["k"], rounds: int = PER_MID["rounds"]):
    """p0 = Exp(1) + 1e-6; per round: U_r ~ U[0,1), v_r = Exp(1) + 1e-6."""
    rng = np.random.default_rng(seed)
    p0 = (rng.exponential(1.0, n) + 1e-6).astype(np.float32)
    U = np.empty((rounds, k), np.float32)
    v = np.empty((rounds, k), np.float32)
    for r in range(rounds):
        U[r] = uniform_f32(rng, k)
        v[r] = (rng.exponential(1.0, k) + 1e-6).astype(np.float32)
    return dict(p0=p0, U=U, v=v, alpha=PER_MID["alpha"], beta=PER_MID["beta"])


def sumtree(seed: int = SUMTREE["seed"], n_valid: int = SUMTREE["n_valid"],
            m: int = SUMTREE["m"], k: int = SUMTREE["k"],
            rounds: int = SUMTREE["rounds"], alpha: float = SUMTREE["alpha"]):
    """p0 = U(0.01,1)^(1/alpha); per round: m leaf indices (duplicates kept),
    m new priorities of the same law, k iid threshold fractions."""
    rng = np.random.default_rng(seed)
    p0 = (rng.uniform(0.01, 1.0, n_valid) ** (1.0 / alpha)).astype(np.float32)
    idx = np.empty((rounds, m), np.int32)
    v = np.empty((rounds, m), np.float32)
    U = np.empty((rounds, k), np.float32)
    for r in range(rounds):
        idx[r] = rng.integers(0, n_valid, size=m, dtype=np.int64).astype(np.int32)
        v[r] = (rng.uniform(0.01, 1.0, m) ** (1.0 / alpha)).astype(np.float32)
        U[r] = uniform_f32(rng, k)
    return dict(p0=p0, idx=idx, v=v, U=U, alpha=alpha)


def resample(seed: int = RESAMPLE["seed"], rows: int = RESAMPLE["rows"],
             P: int = RESAMPLE["P"], sigma: float = 3.0):
    """Particle log-weights ~ N(0, sigma^2) (float32), one u_row per row."""
    rng = np.random.default_rng(seed)
    lw = (rng.standard_normal((rows, P)) * sigma).astype(np.float32)
    u_row = uniform_f32(rng, rows)
    return dict(lw=lw, u_row=u_row)


def pf_step(seed: int = PF_STEP["seed"], rows: int = PF_STEP["rows"], P: int = PF_STEP["P"],
            D: int = PF_STEP["D"], O: int = PF_STEP["O"], sigma_p: float = PF_STEP["sigma_p"],
            sigma_o: float = PF_STEP["sigma_o"]):
    """One particle-filter step's inputs: states x ~ N(0, 1) (rows, P, D),
    log-weights ~ N(0, 1), observations ~ N(0, 1) (rows, O), A = 0.9 I,
    C ~ 0.5 N(0, 1) (O, D), standard normal process noise eps (rows, P, D),
    one u_row per row; all float32."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, P, D)).astype(np.float32)
    lw = rng.standard_normal((rows, P)).astype(np.float32)
    obs = rng.standard_normal((rows, O)).astype(np.float32)
    A = (0.9 * np.eye(D)).astype(np.float32)
    Cm = (0.5 * rng.standard_normal((O, D))).astype(np.float32)
    eps = rng.standard_normal((rows, P, D)).astype(np.float32)
    u_row = uniform_f32(rng, rows)
    return dict(x=x, lw=lw, obs=obs, A=A, C=Cm, eps=eps, u_row=u_row, sigma_p=sigma_p,
                sigma_o=sigma_o)


def pf_small(seed: int = PF_SMALL["seed"]):
    """The pages' filter shape: 16 filters of 1024 particles, D = 4, O = 2."""
    c = PF_SMALL
    return pf_step(seed, c["rows"], c["P"], c["D"], c["O"], c["sigma_p"], c["sigma_o"])


def per_large(seed: int = PER_LARGE["seed"], n: int = PER_LARGE["n"],
              k: int = PER_LARGE["k"]):
    """p ~ LogNormal(0, 2) (heavy tail), U ~ U[0,1)."""
    rng = np.random.default_rng(seed)
    p = rng.lognormal(0.0, 2.0, n).astype(np.float32)
    U = uniform_f32(rng, k)
    return dict(p=p, U=U, alpha=PER_LARGE["alpha"], beta=PER_LARGE["beta"])


def per_large_int(seed: int = PER_LARGE_INT["seed"], n: int = PER_LARGE_INT["n"],
                  k: int = PER_LARGE_INT["k"], qmax: int = PER_LARGE_INT["qmax"]):
    """q ~ U{1..qmax} (uint32), r ~ U{0..2^32-1} (uint32)."""
    rng = np.random.default_rng(seed)
    q = rng.integers(1, qmax + 1, size=n, dtype=np.int64).astype(np.uint32)
    r = uniform_u32(rng, k)
    return dict(q=q, r=r, beta=PER_LARGE_INT["beta"])


def sweep_f32(n: int, seed: int = SWEEP_SEED):
    """PER-large law at any size (bandwidth sweep)."""
    rng = np.random.default_rng(seed + n)
    return rng.lognormal(0.0, 2.0, n).astype(np.float32)


def sweep_u32(n: int, seed: int = SWEEP_SEED, qmax: int = 1 << 20):
    rng = np.random.default_rng(seed + 7 * n)
    return rng.integers(1, qmax + 1, size=n, dtype=np.int64).astype(np.uint32)


def generic_f32(n: int, seed: int, law: str = "exp"):
    """Priorities of a named law for ragged / edge-size tests."""
    rng = np.random.default_rng(seed)
    if law == "exp":
        return (rng.exponential(1.0, n) + 1e-6).astype(np.float32)
    if law == "lognormal":
        return rng.lognormal(0.0, 2.0, n).astype(np.float32)
    if law == "halfnormal":
        return (np.abs(rng.standard_normal(n)) + 1e-6).astype(np.float32)
    if law == "uniform":
        return rng.uniform(0.01, 1.0, n).astype(np.float32)
    raise ValueError(law)
