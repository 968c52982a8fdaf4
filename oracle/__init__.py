"""CPU oracle for proportional sampling -- TEST INFRASTRUCTURE ONLY.

A ctypes shim over ``liboracle.so`` (built from ``psamp_oracle.cpp`` with
g++).  Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this package; the GPU library never does.

All functions take and return numpy arrays.  Randomness is never drawn here:
thresholds, new priorities and indices are inputs.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "psamp_oracle.cpp")
# PSAMP_ORACLE_LIB names another build (the sanitized build of the CPU
# sanitizer test); by default the in-tree liboracle.so.
_LIB = os.environ.get("PSAMP_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

CXXFLAGS = ["-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math",
            "-Wall", "-Wextra", "-shared", "-fPIC"]


SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
            "-fno-omit-frame-pointer", "-g"]


def build(out: str | None = None, sanitize: bool = False) -> str:
    """Compile liboracle.so (always recompiles); sanitize: with ASan + UBSan,
    for the CPU sanitizer test (load it with the sanitizer runtime
    preloaded)."""
    lib = out or _LIB
    tmp = lib + ".tmp"
    subprocess.check_call(["g++", *CXXFLAGS, *(SANITIZE if sanitize else []), "-o", tmp, _SRC])
    os.replace(tmp, lib)
    return lib


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = C.CDLL(_LIB)
        _declare(_lib)
    return _lib


_i64, _f64, _i32 = C.c_int64, C.c_double, C.c_int
_p = C.c_void_p


def _declare(L):
    sig = {
        "o_weights_f32": (None, [_p, _i64, _f64, _p]),
        "o_cdf_f64": (_f64, [_p, _i64, _p]),
        "o_build_cdf_f32": (_f64, [_p, _i64, _f64, _p]),
        "o_build_cdf_u32": (C.c_uint64, [_p, _i64, _p]),
        "o_thresholds_f64": (None, [_p, _i64, _i32, _f64, _p]),
        "o_thresholds_u64": (None, [_p, _i64, _i32, C.c_uint64, _p]),
        "o_search_f64": (None, [_p, _i64, _p, _i64, _p]),
        "o_search_u64": (None, [_p, _i64, _p, _i64, _p]),
        "o_search_f32cdf": (None, [_p, _i64, _p, _i64, _p]),
        "o_is_weights_f32": (None, [_p, _i64, _f64, _f64, _p, _i64, _f64, _p]),
        "o_is_weights_u32": (None, [_p, _i64, C.c_uint64, _p, _i64, _f64, _p]),
        "o_scatter_lww_f32": (None, [_p, _i64, _p, _p, _i64]),
        "o_leaf_f32": (C.c_float, [C.c_float, _f64]),
        "o_tree_new": (_p, [_i32, _i64]),
        "o_tree_free": (None, [_i32, _p]),
        "o_tree_build_f32": (None, [_p, _p, _i64, _f64]),
        "o_tree_build_f64": (None, [_p, _p, _i64, _f64]),
        "o_tree_build_u64": (None, [_p, _p, _i64]),
        "o_tree_update_f32": (None, [_p, _p, _p, _i64, _f64]),
        "o_tree_update_f64": (None, [_p, _p, _p, _i64, _f64]),
        "o_tree_update_u64": (None, [_p, _p, _p, _i64]),
        "o_tree_sample_f32": (None, [_p, _i64, _p, _i64, _i32, _p]),
        "o_tree_sample_f64": (None, [_p, _i64, _p, _i64, _i32, _p]),
        "o_tree_sample_u64": (None, [_p, _i64, _p, _i64, _i32, _p]),
        "o_tree_export_f32": (None, [_p, _p]),
        "o_tree_export_f64": (None, [_p, _p]),
        "o_tree_export_u64": (None, [_p, _p]),
        "o_tree_root_f32": (C.c_float, [_p]),
        "o_tree_root_f64": (_f64, [_p]),
        "o_tree_root_u64": (C.c_uint64, [_p]),
        "o_resample_rows": (None, [_p, _i64, _i64, _i64, _p, _p, _i64]),
        "o_row_cdf": (None, [_p, _i64, _p, _p]),
        "o_pf_step": (None, [_p, _p, _p, _p, _p, _p, C.c_float, C.c_float, _p, _i64, _i64,
                             _i64, _i64, _p, _p, _p, _p, _p]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# --------------------------------------------------------------- CDF path
def weights(p, alpha: float) -> np.ndarray:
    p = _c(p, np.float32)
    w = np.empty(p.size, np.float64)
    lib().o_weights_f32(_ptr(p), p.size, float(alpha), _ptr(w))
    return w


def cdf_f64(w) -> tuple[np.ndarray, float]:
    w = _c(w, np.float64)
    Cc = np.empty(w.size, np.float64)
    T = lib().o_cdf_f64(_ptr(w), w.size, _ptr(Cc))
    return Cc, T


def build_cdf(p, alpha: float) -> tuple[np.ndarray, float]:
    """fp mode: C = serial fp64 prefix sum of p^alpha; returns (C, T)."""
    p = _c(p, np.float32)
    Cc = np.empty(p.size, np.float64)
    T = lib().o_build_cdf_f32(_ptr(p), p.size, float(alpha), _ptr(Cc))
    return Cc, T


def build_cdf_int(q) -> tuple[np.ndarray, int]:
    """Integer mode: exact uint64 prefix sum of uint32 priorities."""
    q = _c(q, np.uint32)
    Cc = np.empty(q.size, np.uint64)
    T = lib().o_build_cdf_u32(_ptr(q), q.size, _ptr(Cc))
    return Cc, int(T)


def thresholds(U, T: float, stratified: bool = True) -> np.ndarray:
    U = _c(U, np.float32)
    t = np.empty(U.size, np.float64)
    lib().o_thresholds_f64(_ptr(U), U.size, int(stratified), float(T), _ptr(t))
    return t


def thresholds_int(r, T: int, stratified: bool = True) -> np.ndarray:
    r = _c(r, np.uint32)
    t = np.empty(r.size, np.uint64)
    lib().o_thresholds_u64(_ptr(r), r.size, int(stratified), int(T), _ptr(t))
    return t


def search(Cc, t) -> np.ndarray:
    Cc = _c(Cc, np.float64)
    t = _c(t, np.float64)
    idx = np.empty(t.size, np.int32)
    lib().o_search_f64(_ptr(Cc), Cc.size, _ptr(t), t.size, _ptr(idx))
    return idx


def search_int(Cc, t) -> np.ndarray:
    Cc = _c(Cc, np.uint64)
    t = _c(t, np.uint64)
    idx = np.empty(t.size, np.int32)
    lib().o_search_u64(_ptr(Cc), Cc.size, _ptr(t), t.size, _ptr(idx))
    return idx


def search_f32cdf(Cf, t) -> np.ndarray:
    Cf = _c(Cf, np.float32)
    t = _c(t, np.float64)
    idx = np.empty(t.size, np.int32)
    lib().o_search_f32cdf(_ptr(Cf), Cf.size, _ptr(t), t.size, _ptr(idx))
    return idx


def sample(p, alpha: float, U, stratified: bool = True):
    """Whole CDF path: returns (C, T, t, idx)."""
    Cc, T = build_cdf(p, alpha)
    t = thresholds(U, T, stratified)
    return Cc, T, t, search(Cc, t)


def sample_int(q, r, stratified: bool = True):
    Cc, T = build_cdf_int(q)
    t = thresholds_int(r, T, stratified)
    return Cc, T, t, search_int(Cc, t)


def is_weights(p, alpha: float, T: float, idx, beta: float, N: int | None = None):
    p = _c(p, np.float32)
    idx = _c(idx, np.int32)
    out = np.empty(idx.size, np.float32)
    N = p.size if N is None else N
    lib().o_is_weights_f32(_ptr(p), int(N), float(alpha), float(T), _ptr(idx),
                           idx.size, float(beta), _ptr(out))
    return out


def is_weights_int(q, T: int, idx, beta: float, N: int | None = None):
    q = _c(q, np.uint32)
    idx = _c(idx, np.int32)
    out = np.empty(idx.size, np.float32)
    N = q.size if N is None else N
    lib().o_is_weights_u32(_ptr(q), int(N), int(T), _ptr(idx), idx.size,
                           float(beta), _ptr(out))
    return out


def scatter_lww(p, idx, v) -> np.ndarray:
    """Returns a copy of p with p[idx_j] = v_j applied in batch order."""
    p = np.array(p, dtype=np.float32, copy=True)
    idx = _c(idx, np.int32)
    v = _c(v, np.float32)
    lib().o_scatter_lww_f32(_ptr(p), p.size, _ptr(idx), _ptr(v), idx.size)
    return p


def leaf_f32(p: float, alpha: float) -> float:
    return float(lib().o_leaf_f32(float(p), float(alpha)))


# --------------------------------------------------------------- sum tree
class Tree:
    """Pointer-based sum tree.  kind: 'f32' | 'f64' | 'u64'."""

    _VT = {"f32": (0, np.float32), "f64": (1, np.float64), "u64": (2, np.uint64)}

    def __init__(self, kind: str, cap: int):
        self.kind = kind
        self.cap = int(cap)
        self._vt, self._dt = self._VT[kind]
        self._h = lib().o_tree_new(self._vt, self.cap)
        if not self._h:
            raise MemoryError("o_tree_new failed")

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            lib().o_tree_free(self._vt, h)
            self._h = None

    def build(self, prio, n_valid: int | None = None, alpha: float = 1.0):
        L = lib()
        if self.kind == "u64":
            q = _c(prio, np.uint32)
            L.o_tree_build_u64(self._h, _ptr(q), q.size if n_valid is None else n_valid)
        else:
            p = _c(prio, np.float32)
            nv = p.size if n_valid is None else n_valid
            fn = L.o_tree_build_f32 if self.kind == "f32" else L.o_tree_build_f64
            fn(self._h, _ptr(p), nv, float(alpha))
        return self

    def update(self, idx, vals, alpha: float = 1.0):
        L = lib()
        idx = _c(idx, np.int32)
        if self.kind == "u64":
            q = _c(vals, np.uint32)
            L.o_tree_update_u64(self._h, _ptr(idx), _ptr(q), idx.size)
        else:
            v = _c(vals, np.float32)
            fn = L.o_tree_update_f32 if self.kind == "f32" else L.o_tree_update_f64
            fn(self._h, _ptr(idx), _ptr(v), idx.size, float(alpha))
        return self

    def sample(self, u, n_valid: int, stratified: bool = False) -> np.ndarray:
        L = lib()
        if self.kind == "u64":
            r = _c(u, np.uint32)
            out = np.empty(r.size, np.int32)
            L.o_tree_sample_u64(self._h, int(n_valid), _ptr(r), r.size,
                                int(stratified), _ptr(out))
        else:
            U = _c(u, np.float32)
            out = np.empty(U.size, np.int32)
            fn = L.o_tree_sample_f32 if self.kind == "f32" else L.o_tree_sample_f64
            fn(self._h, int(n_valid), _ptr(U), U.size, int(stratified), _ptr(out))
        return out

    def flat(self) -> np.ndarray:
        out = np.empty(2 * self.cap, self._dt)
        fn = {"f32": lib().o_tree_export_f32, "f64": lib().o_tree_export_f64,
              "u64": lib().o_tree_export_u64}[self.kind]
        fn(self._h, _ptr(out))
        return out

    def root(self):
        fn = {"f32": lib().o_tree_root_f32, "f64": lib().o_tree_root_f64,
              "u64": lib().o_tree_root_u64}[self.kind]
        return fn(self._h)


# ------------------------------------------------------ replay priorities
class Replay:
    """[SEGT] "Integration with GpuReplayBuffer": a ring of `capacity`
    slots whose priorities live in the pointer sum tree (F32 leaves =
    p^alpha).  insert_batch writes each item at the cursor and advances it
    (mod capacity), one item after the other; update_priorities sets leaves;
    sample_proportional descends over the filled slots; IS weights take the
    textbook (N P_i)^-beta / max form with P_i = leaf_i / root, N = filled
    slots; total_priority is the root."""

    def __init__(self, capacity: int, alpha: float):
        self.capacity = int(capacity)
        self.cap = cap_pow2(self.capacity)
        self.alpha = float(alpha)
        self.tree = Tree("f32", self.cap)
        self.cursor = 0
        self.size = 0

    def insert(self, prio) -> np.ndarray:
        prio = _c(prio, np.float32)
        slots = np.empty(prio.size, np.int32)
        for i in range(prio.size):
            slots[i] = self.cursor
            self.tree.update(slots[i:i + 1], prio[i:i + 1], self.alpha)
            self.cursor = (self.cursor + 1) % self.capacity
            self.size = min(self.size + 1, self.capacity)
        return slots

    def update(self, slots, prio):
        self.tree.update(slots, prio, self.alpha)

    def sample(self, u, beta: float, stratified: bool = True):
        idx = self.tree.sample(u, self.size, stratified)
        leaves = self.tree.flat()[self.cap:self.cap + self.size]
        w = is_weights(leaves, 1.0, float(self.tree.root()), idx, beta, N=self.size)
        return idx, w

    def total(self) -> float:
        return self.tree.root()


# --------------------------------------------------------------- resampling
def resample_rows(lw, u_row) -> np.ndarray:
    lw = _c(lw, np.float32)
    u_row = _c(u_row, np.float32)
    rows, P = lw.shape
    anc = np.empty((rows, P), np.int32)
    lib().o_resample_rows(_ptr(lw), rows, P, P, _ptr(u_row), _ptr(anc), P)
    return anc


def pf_step(x, lw, obs, A, Cm, eps, sigma_p: float, sigma_o: float, u_row):
    """One particle-filter step ([PF]).  x, eps: (rows, P, D); lw: (rows, P);
    obs: (rows, O); A: (D, D); Cm: (O, D); u_row: (rows,).  Returns
    (x_out, lw_out, anc, pred, lw_new), all float32 except anc (int32)."""
    x = _c(x, np.float32)
    rows, P, D = x.shape
    lw = _c(lw, np.float32).reshape(rows, P)
    obs = _c(obs, np.float32).reshape(rows, -1)
    O = obs.shape[1]
    A = _c(A, np.float32).reshape(D, D)
    Cm = _c(Cm, np.float32).reshape(O, D)
    eps = _c(eps, np.float32).reshape(rows, P, D)
    u_row = _c(u_row, np.float32).reshape(rows)
    x_out = np.empty_like(x)
    lw_out = np.empty((rows, P), np.float32)
    anc = np.empty((rows, P), np.int32)
    pred = np.empty_like(x)
    lwn = np.empty((rows, P), np.float32)
    lib().o_pf_step(_ptr(x), _ptr(lw), _ptr(obs), _ptr(A), _ptr(Cm), _ptr(eps),
                    float(sigma_p), float(sigma_o), _ptr(u_row), rows, P, D, O,
                    _ptr(x_out), _ptr(lw_out), _ptr(anc), _ptr(pred), _ptr(lwn))
    return x_out, lw_out, anc, pred, lwn


def row_cdf(x):
    x = _c(x, np.float32)
    W = np.empty(x.size, np.float64)
    Cc = np.empty(x.size, np.float64)
    lib().o_row_cdf(_ptr(x), x.size, _ptr(W), _ptr(Cc))
    return W, Cc


def cap_pow2(capacity: int) -> int:
    """Capacity rounded up to the next power of two ([SEGT] "Tree Layout")."""
    c = 1
    while c < capacity:
        c *= 2
    return c
