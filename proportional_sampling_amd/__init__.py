"""proportional_sampling_amd -- Python binding of libpsamp (MI355X / gfx950).

Argument marshalling only: every step runs in the HIP kernels of
``libpsamp.so`` (built in-tree by ``proportional_sampling_amd.build``).
PyTorch supplies device memory (``tensor.data_ptr()``) and the stream
(``torch.cuda.current_stream().cuda_stream``).  There is no CPU fallback:
importing works anywhere, but every call needs the built library and a GPU,
and fails loudly otherwise.
"""
from __future__ import annotations

import ctypes as C
import functools
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# PSAMP_LIB names another build of the library (the host-sanitized build of
# the CPU sanitizer test); by default the in-tree libpsamp.so.
LIB_PATH = os.environ.get("PSAMP_LIB") or os.path.join(_HERE, "libpsamp.so")

F32, F64, U32, U64, I32 = 0, 1, 2, 3, 4
_DT = {torch.float32: F32, torch.float64: F64, torch.uint32: U32, torch.uint64: U64,
       torch.int32: I32}

_STATUS = {0: "ok", 1: "null pointer", 2: "size out of range", 3: "unsupported dtype",
           4: "parameter out of range", 5: "workspace missing or too small",
           6: "misaligned pointer", 7: "kernel launch failed", 8: "unsupported"}


class PsampError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn}: {_STATUS.get(code, 'unknown')} (status {code})")
        self.code = code


# Exported symbols and their C signatures (mirrors include/psamp.h).
_i64, _dbl, _int, _sz, _p = C.c_int64, C.c_double, C.c_int, C.c_size_t, C.c_void_p
SIGNATURES = {
    "psamp_status_string": (C.c_char_p, [_int]),
    "psamp_abi_version": (_int, []),
    "psamp_build_cdf_workspace_size": (_sz, [_i64]),
    "psamp_build_cdf": (_int, [_p, _int, _i64, _dbl, _p, _int, _p, _p, _sz, _p]),
    "psamp_sample": (_int, [_p, _int, _i64, _p, _p, _int, _i64, _int, _p, _p]),
    "psamp_build_cdf_sample": (_int, [_p, _int, _i64, _dbl, _p, _int, _i64, _p, _int, _p, _p, _p,
                                      _sz, _p]),
    "psamp_is_weights_workspace_size": (_sz, [_i64]),
    "psamp_is_weights": (_int, [_p, _int, _i64, _dbl, _p, _i64, _dbl, _p, _p, _sz, _p]),
    "psamp_segtree_cap_pow2": (_i64, [_i64]),
    "psamp_segtree_build": (_int, [_p, _int, _i64, _p, _int, _i64, _dbl, _p]),
    "psamp_segtree_update_workspace_size": (_sz, [_i64, _i64]),
    "psamp_segtree_update": (_int, [_p, _int, _i64, _p, _p, _int, _i64, _dbl, _p, _sz, _p]),
    "psamp_segtree_sample": (_int, [_p, _int, _i64, _i64, _p, _int, _i64, _int, _p, _p]),
    "psamp_replay_workspace_size": (_sz, [_i64, _i64]),
    "psamp_replay_init": (_int, [_p, _i64, _dbl, _p, _p, _sz]),
    "psamp_replay_insert": (_int, [_p, _p, _i64, _p, _p]),
    "psamp_replay_update": (_int, [_p, _p, _p, _i64, _p]),
    "psamp_replay_sample": (_int, [_p, _p, _i64, _int, _dbl, _p, _p, _p]),
    "psamp_replay_total": (_p, [_p]),
    "psamp_resample_rows": (_int, [_p, _i64, _i64, _i64, _p, _p, _i64, _p]),
    "psamp_pf_step": (_int, [_p, _p, _p, _p, _p, _p, C.c_float, C.c_float, _p, _i64, _i64, _i64,
                             _i64, _p, _p, _p, _p]),
    "psamp_scatter_workspace_size": (_sz, [_i64, _i64]),
    "psamp_scatter_lww": (_int, [_p, _int, _i64, _p, _p, _i64, _int, _p, _sz, _p]),
    "psamp_per_round_workspace_size": (_sz, [_i64, _i64]),
    "psamp_per_round": (_int, [_p, _i64, _dbl, _dbl, _p, _i64, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "psamp_per_round_noalloc": (_int, [_p, _i64, _dbl, _dbl, _p, _i64, _p, _p, _p, _p, _p, _p]),
    "psamp_ceiling_copy": (_int, [_p, _p, _i64, _int, _int, _p]),
    "psamp_check_enable": (_int, [_int]),
    "psamp_check_errors": (_int, [C.POINTER(C.c_uint64), _int, _p]),
    "psamp_workspace_errors": (_int, [_p, _sz, C.POINTER(C.c_uint64), _p]),
}

_lib = None


def lib() -> C.CDLL:
    """The loaded libpsamp.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m proportional_sampling_amd.build` (hipcc, gfx950)")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(fn: str, code: int):
    if code != 0:
        raise PsampError(fn, code)


def _on_stream(fn):
    """Runs fn with `stream` (a torch stream, or a raw hipStream_t as an int)
    made torch's current stream, so that every output and workspace fn
    allocates is allocated, zero-filled and later reused in that stream's
    order, the order the library's kernels run in."""
    @functools.wraps(fn)
    def run(*args, stream=None, **kw):
        if stream is None:
            return fn(*args, **kw)
        if not isinstance(stream, torch.cuda.Stream):
            stream = torch.cuda.ExternalStream(int(stream))
        with torch.cuda.stream(stream):
            return fn(*args, **kw)
    return run


def _stream(stream=None) -> int:
    """The hipStream_t to launch on: the given stream, else torch's current
    stream (read without building a Stream object: calls are launch-bound)."""
    if stream is None:
        return torch._C._cuda_getCurrentRawStream(torch.cuda.current_device())
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, name: str, dtypes=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    return t.data_ptr()


class Workspace:
    """Caller-owned scratch for calls that need one: zero-filled once, on
    allocation; the library keeps it consistent afterwards.  One workspace
    must not serve two calls that may run concurrently."""

    def __init__(self, nbytes: int, device=None):
        n = max(int(nbytes), 8)
        self.buf = torch.zeros((n + 7) // 8, dtype=torch.int64,
                               device=device if device is not None else "cuda")
        self.nbytes = self.buf.numel() * 8

    @property
    def ptr(self) -> int:
        return self.buf.data_ptr()

    @_on_stream
    def errors(self, stream=None) -> int:
        out = C.c_uint64(0)
        _check("psamp_workspace_errors",
               lib().psamp_workspace_errors(self.ptr, self.nbytes, C.byref(out), _stream(stream)))
        return int(out.value)


def abi_version() -> int:
    return lib().psamp_abi_version()


# ------------------------------------------------------------ (1) CDF
def build_cdf_workspace_size(n: int) -> int:
    return int(lib().psamp_build_cdf_workspace_size(int(n)))


@_on_stream
def build_cdf(prio: torch.Tensor, alpha: float = 1.0, *, cdf: torch.Tensor | None = None,
              total: torch.Tensor | None = None, cdf_dtype=None, ws: Workspace | None = None,
              stream=None):
    """Inclusive CDF of prio^alpha (float32 prio) or of prio (uint32 prio).
    Returns (cdf, total) -- both stay on the device."""
    n = prio.numel()
    p = _dev(prio, "prio", (torch.float32, torch.uint32))
    if cdf_dtype is None:
        cdf_dtype = torch.float64 if prio.dtype == torch.float32 else torch.uint64
    if cdf is None:
        cdf = torch.empty(n, dtype=cdf_dtype, device=prio.device)
    if total is None:
        total = torch.empty(1, dtype=cdf.dtype, device=prio.device)
    if ws is None:
        ws = Workspace(build_cdf_workspace_size(n), prio.device)
    c = _dev(cdf, "cdf")
    t = _dev(total, "total")
    _check("psamp_build_cdf", lib().psamp_build_cdf(
        p, _DT[prio.dtype], n, float(alpha), c, _DT[cdf.dtype], t, ws.ptr, ws.nbytes,
        _stream(stream)))
    return cdf, total


@_on_stream
def sample(cdf: torch.Tensor, total: torch.Tensor, u: torch.Tensor, *, stratified: bool = True,
           out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """int32 indices: first j with cdf[j] >= t_i, clamped to n-1."""
    k = u.numel()
    if out is None:
        out = torch.empty(k, dtype=torch.int32, device=cdf.device)
    c = _dev(cdf, "cdf")
    t = _dev(total, "total")
    uu = _dev(u, "u", (torch.float32, torch.uint32))
    o = _dev(out, "out", (torch.int32,))
    _check("psamp_sample", lib().psamp_sample(
        c, _DT[cdf.dtype], cdf.numel(), t, uu, _DT[u.dtype], k, int(bool(stratified)), o,
        _stream(stream)))
    return out


@_on_stream
def build_cdf_sample(prio: torch.Tensor, u: torch.Tensor, alpha: float = 1.0, *,
                     cdf: torch.Tensor | None = None, total: torch.Tensor | None = None,
                     out: torch.Tensor | None = None, cdf_dtype=None, ws: Workspace | None = None,
                     stream=None):
    """build_cdf followed by stratified sample, fused (same results).
    Returns (idx, cdf, total)."""
    n, k = prio.numel(), u.numel()
    p = _dev(prio, "prio", (torch.float32, torch.uint32))
    if cdf_dtype is None:
        cdf_dtype = torch.float64 if prio.dtype == torch.float32 else torch.uint64
    if cdf is None:
        cdf = torch.empty(n, dtype=cdf_dtype, device=prio.device)
    if total is None:
        total = torch.empty(1, dtype=cdf.dtype, device=prio.device)
    if out is None:
        out = torch.empty(k, dtype=torch.int32, device=prio.device)
    if ws is None:
        ws = Workspace(build_cdf_workspace_size(n), prio.device)
    uu = _dev(u, "u", (torch.float32, torch.uint32))
    _check("psamp_build_cdf_sample", lib().psamp_build_cdf_sample(
        p, _DT[prio.dtype], n, float(alpha), uu, _DT[u.dtype], k, _dev(cdf, "cdf"),
        _DT[cdf.dtype], _dev(total, "total"), _dev(out, "out", (torch.int32,)), ws.ptr, ws.nbytes,
        _stream(stream)))
    return out, cdf, total


def is_weights_workspace_size(k: int) -> int:
    return int(lib().psamp_is_weights_workspace_size(int(k)))


@_on_stream
def is_weights(prio: torch.Tensor, idx: torch.Tensor, alpha: float, beta: float, *,
               out: torch.Tensor | None = None, ws: Workspace | None = None,
               stream=None) -> torch.Tensor:
    """Float IS weights (w_min / w_i)^beta of the sampled entries."""
    k = idx.numel()
    if out is None:
        out = torch.empty(k, dtype=torch.float32, device=prio.device)
    need = is_weights_workspace_size(k)
    if ws is None and need > 0:
        ws = Workspace(need, prio.device)
    p = _dev(prio, "prio", (torch.float32, torch.uint32))
    i = _dev(idx, "idx", (torch.int32,))
    o = _dev(out, "out", (torch.float32,))
    _check("psamp_is_weights", lib().psamp_is_weights(
        p, _DT[prio.dtype], prio.numel(), float(alpha), i, k, float(beta), o,
        ws.ptr if ws is not None else None, ws.nbytes if ws is not None else 0,
        _stream(stream)))
    return out


# ------------------------------------------------------------ (3) sum tree
def segtree_cap_pow2(capacity: int) -> int:
    return int(lib().psamp_segtree_cap_pow2(int(capacity)))


def segtree_empty(capacity: int, kind=torch.float32, device="cuda") -> torch.Tensor:
    cap = segtree_cap_pow2(capacity)
    if cap == 0:
        raise ValueError("capacity out of range")
    return torch.zeros(2 * cap, dtype=kind, device=device)


@_on_stream
def segtree_build(tree: torch.Tensor, prio: torch.Tensor, alpha: float = 1.0,
                  n_valid: int | None = None, stream=None) -> torch.Tensor:
    cap = tree.numel() // 2
    nv = prio.numel() if n_valid is None else int(n_valid)
    t = _dev(tree, "tree", (torch.float32, torch.uint64))
    p = _dev(prio, "prio", (torch.float32, torch.uint32))
    _check("psamp_segtree_build", lib().psamp_segtree_build(
        t, _DT[tree.dtype], cap, p, _DT[prio.dtype], nv, float(alpha), _stream(stream)))
    return tree


@_on_stream
def segtree_update_workspace_size(cap_pow2: int, m: int) -> int:
    return int(lib().psamp_segtree_update_workspace_size(int(cap_pow2), int(m)))


def segtree_update(tree: torch.Tensor, idx: torch.Tensor, prio: torch.Tensor,
                   alpha: float = 1.0, *, ws: Workspace | None = None,
                   stream=None) -> torch.Tensor:
    """Batched leaf update, last write wins; ws (zeroed once) may be reused
    by every update on this stream."""
    cap = tree.numel() // 2
    m = idx.numel()
    if prio.numel() != m:
        raise ValueError("idx and prio must have the same length")
    t = _dev(tree, "tree", (torch.float32, torch.uint64))
    i = _dev(idx, "idx", (torch.int32,))
    p = _dev(prio, "prio", (torch.float32, torch.uint32))
    if ws is None:
        ws = Workspace(segtree_update_workspace_size(cap, m), tree.device)
    _check("psamp_segtree_update", lib().psamp_segtree_update(
        t, _DT[tree.dtype], cap, i, p, _DT[prio.dtype], m, float(alpha), ws.ptr, ws.nbytes,
        _stream(stream)))
    return tree


@_on_stream
def segtree_sample(tree: torch.Tensor, n_valid: int, u: torch.Tensor, *,
                   stratified: bool = False, out: torch.Tensor | None = None,
                   stream=None) -> torch.Tensor:
    cap = tree.numel() // 2
    k = u.numel()
    if out is None:
        out = torch.empty(k, dtype=torch.int32, device=tree.device)
    t = _dev(tree, "tree", (torch.float32, torch.uint64))
    uu = _dev(u, "u", (torch.float32, torch.uint32))
    o = _dev(out, "out", (torch.int32,))
    _check("psamp_segtree_sample", lib().psamp_segtree_sample(
        t, _DT[tree.dtype], cap, int(n_valid), uu, _DT[u.dtype], k, int(bool(stratified)), o,
        _stream(stream)))
    return out


# ------------------------------------------------------------ (4) rows
@_on_stream
def resample_rows(logw: torch.Tensor, u_row: torch.Tensor, *, out: torch.Tensor | None = None,
                  stream=None) -> torch.Tensor:
    """int32 ancestors per row.  logw and out may be row-strided views (unit
    column stride, row stride >= P): the row strides go to the call as
    ld_in and ld_out."""
    if logw.dim() != 2:
        raise ValueError("logw must be rows x P")
    rows, P = logw.shape
    if out is None:
        out = torch.empty(rows, P, dtype=torch.int32, device=logw.device)
    if tuple(out.shape) != (rows, P):
        raise ValueError(f"out must have shape {(rows, P)}, got {tuple(out.shape)}")
    lw, ld_in = _rows_dev(logw, "logw", torch.float32)
    ur = _dev(u_row, "u_row", (torch.float32,))
    o, ld_out = _rows_dev(out, "out", torch.int32)
    _check("psamp_resample_rows", lib().psamp_resample_rows(
        lw, rows, P, ld_in, ur, o, ld_out, _stream(stream)))
    return out


def _rows_dev(t: torch.Tensor, name: str, dtype) -> tuple[int, int]:
    """Pointer and row stride (in elements) of a rows x P GPU matrix whose
    rows are contiguous."""
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    rows, P = t.shape
    ld = t.stride(0) if rows > 1 else P
    if P > 1 and t.stride(1) != 1:
        raise ValueError(f"{name}: rows must be contiguous")
    if ld < P:
        raise ValueError(f"{name}: row stride {ld} < P = {P}")
    return t.data_ptr(), ld


class _ReplayStruct(C.Structure):
    """Mirror of psamp_replay (include/psamp.h)."""
    _fields_ = [("capacity", C.c_int64), ("cap_pow2", C.c_int64), ("cursor", C.c_int64),
                ("size", C.c_int64), ("alpha", C.c_double), ("tree", C.c_void_p),
                ("ws", C.c_void_p), ("ws_bytes", C.c_size_t)]


class ReplayPriorities:
    """Priorities of a replay ring of `capacity` slots on an F32 sum tree:
    insert (insert_batch), update (update_priorities), sample
    (sample_proportional, with IS weights) and total (total_priority).
    The tree and workspace are device tensors owned by this object."""

    def __init__(self, capacity: int, alpha: float = 0.6, max_batch: int = 8192, device=None):
        dev = device if device is not None else "cuda"
        cp = int(lib().psamp_segtree_cap_pow2(int(capacity)))
        if cp == 0:
            raise ValueError("capacity must be in [1, 2^30]")
        self.tree = torch.zeros(2 * cp, dtype=torch.float32, device=dev)
        self.max_batch = int(max_batch)
        self.ws = Workspace(lib().psamp_replay_workspace_size(int(capacity), self.max_batch),
                            device=dev)
        self._rb = _ReplayStruct()
        _check("psamp_replay_init", lib().psamp_replay_init(
            C.byref(self._rb), int(capacity), float(alpha), self.tree.data_ptr(), self.ws.ptr,
            self.ws.nbytes))

    @property
    def capacity(self) -> int:
        return int(self._rb.capacity)

    @property
    def size(self) -> int:
        return int(self._rb.size)

    @property
    def cursor(self) -> int:
        return int(self._rb.cursor)

    @_on_stream
    def insert(self, prio: torch.Tensor, *, out: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
        m = prio.numel()
        if out is None:
            out = torch.empty(m, dtype=torch.int32, device=self.tree.device)
        _check("psamp_replay_insert", lib().psamp_replay_insert(
            C.byref(self._rb), _dev(prio, "prio", (torch.float32,)), m,
            _dev(out, "out", (torch.int32,)), _stream(stream)))
        return out

    @_on_stream
    def update(self, slots: torch.Tensor, prio: torch.Tensor, stream=None):
        m = slots.numel()
        if prio.numel() != m:
            raise ValueError("slots and prio must have the same length")
        _check("psamp_replay_update", lib().psamp_replay_update(
            C.byref(self._rb), _dev(slots, "slots", (torch.int32,)),
            _dev(prio, "prio", (torch.float32,)), m, _stream(stream)))

    @_on_stream
    def sample(self, u: torch.Tensor, beta: float | None = 0.4, *, stratified: bool = True,
               out: torch.Tensor | None = None, out_w: torch.Tensor | None = None,
               stream=None):
        """Returns slots, or (slots, IS weights) when beta is not None."""
        k = u.numel()
        if out is None:
            out = torch.empty(k, dtype=torch.int32, device=self.tree.device)
        w_ptr = None
        if beta is not None:
            if out_w is None:
                out_w = torch.empty(k, dtype=torch.float32, device=self.tree.device)
            w_ptr = _dev(out_w, "out_w", (torch.float32,))
        _check("psamp_replay_sample", lib().psamp_replay_sample(
            C.byref(self._rb), _dev(u, "u", (torch.float32,)), k, int(stratified),
            float(beta or 0.0), _dev(out, "out", (torch.int32,)), w_ptr, _stream(stream)))
        return out if beta is None else (out, out_w)

    def total(self) -> torch.Tensor:
        """The root of the tree (a view: it follows later updates)."""
        addr = lib().psamp_replay_total(C.byref(self._rb))
        assert addr == self.tree.data_ptr() + 4
        return self.tree[1]


@_on_stream
def pf_step(x: torch.Tensor, logw: torch.Tensor, obs: torch.Tensor, A: torch.Tensor,
            C_obs: torch.Tensor, eps: torch.Tensor, sigma_p: float, sigma_o: float,
            u_row: torch.Tensor, *, x_out: torch.Tensor | None = None,
            logw_out: torch.Tensor | None = None, anc_out: torch.Tensor | None = None,
            stream=None):
    """One particle-filter step (predict, likelihood, resample, gather) on
    rows x P x D particles.  Returns (x_out, logw_out); x_out=x and
    logw_out=logw update in place; anc_out (rows x P int32) is optional."""
    if x.dim() != 3:
        raise ValueError("x must be rows x P x D")
    rows, P, D = x.shape
    O = C_obs.shape[0] if C_obs.dim() == 2 else 0
    if x_out is None:
        x_out = torch.empty_like(x)
    if logw_out is None:
        logw_out = torch.empty(rows, P, dtype=torch.float32, device=x.device)
    f32 = (torch.float32,)
    for t, nm, shape in ((logw, "logw", (rows, P)), (obs, "obs", (rows, O)),
                         (A, "A", (D, D)), (C_obs, "C_obs", (O, D)), (eps, "eps", (rows, P, D)),
                         (u_row, "u_row", (rows,)), (x_out, "x_out", (rows, P, D)),
                         (logw_out, "logw_out", (rows, P))):
        if tuple(t.shape) != shape:
            raise ValueError(f"{nm} must have shape {shape}, got {tuple(t.shape)}")
    a_ptr = 0
    if anc_out is not None:
        if tuple(anc_out.shape) != (rows, P):
            raise ValueError("anc_out must be rows x P")
        a_ptr = _dev(anc_out, "anc_out", (torch.int32,))
    _check("psamp_pf_step", lib().psamp_pf_step(
        _dev(x, "x", f32), _dev(logw, "logw", f32), _dev(obs, "obs", f32), _dev(A, "A", f32),
        _dev(C_obs, "C_obs", f32), _dev(eps, "eps", f32), float(sigma_p), float(sigma_o),
        _dev(u_row, "u_row", f32), rows, P, D, O, _dev(x_out, "x_out", f32),
        _dev(logw_out, "logw_out", f32), a_ptr or None, _stream(stream)))
    return x_out, logw_out


# ------------------------------------------------------------ rewrite
def scatter_workspace_size(n: int, m: int) -> int:
    return int(lib().psamp_scatter_workspace_size(int(n), int(m)))


SCATTER_GROUPED = 1


@_on_stream
def scatter_lww(prio: torch.Tensor, idx: torch.Tensor, vals: torch.Tensor,
                ws: Workspace | None = None, *, grouped: bool = False,
                stream=None) -> torch.Tensor:
    """prio[idx_j] = vals_j, last j wins.  grouped=True promises that equal
    indices are adjacent (sorted idx): one kernel, no workspace."""
    m = idx.numel()
    if vals.numel() != m or vals.dtype != prio.dtype:
        raise ValueError("vals must match idx in length and prio in dtype")
    p = _dev(prio, "prio", (torch.float32, torch.uint32))
    i = _dev(idx, "idx", (torch.int32,))
    v = _dev(vals, "vals", (torch.float32, torch.uint32))
    if ws is None and not grouped:
        ws = Workspace(scatter_workspace_size(prio.numel(), m), prio.device)
    _check("psamp_scatter_lww", lib().psamp_scatter_lww(
        p, _DT[prio.dtype], prio.numel(), i, v, m, SCATTER_GROUPED if grouped else 0,
        ws.ptr if ws is not None else None, ws.nbytes if ws is not None else 0,
        _stream(stream)))
    return prio


# ------------------------------------------------------------ fused update
def per_round_workspace_size(n: int, k: int) -> int:
    return int(lib().psamp_per_round_workspace_size(int(n), int(k)))


@_on_stream
def per_round(prio: torch.Tensor, u: torch.Tensor, alpha: float, beta: float,
              new_prio: torch.Tensor | None = None, *, out_idx: torch.Tensor | None = None,
              out_w: torch.Tensor | None = None, cdf: torch.Tensor | None = None,
              total: torch.Tensor | None = None, ws: Workspace | None = None, stream=None):
    """One fused PER minibatch update (CDF, stratified draws, IS weights,
    rewrite of the drawn priorities).  Returns (idx, w, cdf, total)."""
    n, k = prio.numel(), u.numel()
    dev_ = prio.device
    out_idx = torch.empty(k, dtype=torch.int32, device=dev_) if out_idx is None else out_idx
    out_w = torch.empty(k, dtype=torch.float32, device=dev_) if out_w is None else out_w
    cdf = torch.empty(n, dtype=torch.float64, device=dev_) if cdf is None else cdf
    total = torch.empty(1, dtype=torch.float64, device=dev_) if total is None else total
    if ws is None:
        ws = Workspace(per_round_workspace_size(n, k), dev_)
    p = _dev(prio, "prio", (torch.float32,))
    uu = _dev(u, "u", (torch.float32,))
    npp = None
    if new_prio is not None:
        if new_prio.numel() != k:
            raise ValueError("new_prio must have one value per draw")
        npp = _dev(new_prio, "new_prio", (torch.float32,))
    _check("psamp_per_round", lib().psamp_per_round(
        p, n, float(alpha), float(beta), uu, k, npp, _dev(out_idx, "out_idx", (torch.int32,)),
        _dev(out_w, "out_w", (torch.float32,)), _dev(cdf, "cdf", (torch.float64,)),
        _dev(total, "total", (torch.float64,)), ws.ptr, ws.nbytes, _stream(stream)))
    return out_idx, out_w, cdf, total


NOALLOC_MAX_N = 1 << 26      # PSAMP_NOALLOC_MAX_N


@_on_stream
def per_round_noalloc(prio: torch.Tensor, u: torch.Tensor, alpha: float, beta: float,
                      new_prio: torch.Tensor | None = None, *, out_idx: torch.Tensor,
                      out_w: torch.Tensor, cdf: torch.Tensor, total: torch.Tensor,
                      stream=None):
    """per_round with the library's own scratch instead of a workspace: the
    caller passes every output, so nothing is allocated.  Calls that overlap
    on one GPU race.  Returns (out_idx, out_w, cdf, total)."""
    n, k = prio.numel(), u.numel()
    npp = None
    if new_prio is not None:
        if new_prio.numel() != k:
            raise ValueError("new_prio must have one value per draw")
        npp = _dev(new_prio, "new_prio", (torch.float32,))
    if out_idx.numel() != k or out_w.numel() != k or cdf.numel() != n or total.numel() != 1:
        raise ValueError("outputs: k indices, k weights, n CDF values, 1 total")
    _check("psamp_per_round_noalloc", lib().psamp_per_round_noalloc(
        _dev(prio, "prio", (torch.float32,)), n, float(alpha), float(beta),
        _dev(u, "u", (torch.float32,)), k, npp, _dev(out_idx, "out_idx", (torch.int32,)),
        _dev(out_w, "out_w", (torch.float32,)), _dev(cdf, "cdf", (torch.float64,)),
        _dev(total, "total", (torch.float64,)), _stream(stream)))
    return out_idx, out_w, cdf, total


@_on_stream
def ceiling_copy(src: torch.Tensor, out: torch.Tensor, rows: int = 2, nt: bool = False,
                 stream=None):
    """out = src as float64 with the scan's bytes and access pattern (a
    measurement aid: the bandwidth ceiling of build_cdf)."""
    if src.numel() != out.numel():
        raise ValueError("src and out must have the same length")
    _check("psamp_ceiling_copy", lib().psamp_ceiling_copy(
        _dev(src, "src", (torch.float32,)), _dev(out, "out", (torch.float64,)), src.numel(),
        int(rows), int(bool(nt)), _stream(stream)))
    return out


# Device-side precondition checks (PSAMP_CHECK=1 or check_enable(True)).
CHECK_PRIORITY, CHECK_ZERO_TOTAL, CHECK_FRACTION, CHECK_INDEX, CHECK_LOGWEIGHT = 2, 4, 8, 16, 32


def check_enable(on: bool | None = True) -> bool:
    """Turns the device-side checks on or off (None: leave as is); returns
    the previous state."""
    return bool(lib().psamp_check_enable(-1 if on is None else int(bool(on))))


@_on_stream
def check_errors(clear: bool = True, stream=None) -> int:
    """The check bits set on this device so far (syncs the stream)."""
    out = C.c_uint64(0)
    _check("psamp_check_errors", lib().psamp_check_errors(C.byref(out), int(bool(clear)),
                                                            _stream(stream)))
    return int(out.value)

