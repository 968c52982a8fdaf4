"""The C-ABI library loads, exports every symbol include/psamp.h declares,
and rejects bad arguments on the host before anything is enqueued.

No call here reaches the GPU: every case fails validation first (the
pointers passed are fake and never dereferenced)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "psamp.h")

FAKE = 0x10000   # a 64 KiB-aligned non-null address that is never touched


@pytest.fixture(scope="module")
def L():
    import proportional_sampling_amd as ps
    if not os.path.exists(ps.LIB_PATH):
        from proportional_sampling_amd import build
        build.build(verbose=False)
    return ps.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(psamp_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    import proportional_sampling_amd as ps
    names = header_functions()
    assert len(names) >= 16
    for n in names:
        assert hasattr(L, n), n
    # the binding declares exactly the header's functions
    assert sorted(ps.SIGNATURES) == names


def test_status_strings_and_version(L):
    assert L.psamp_abi_version() == 1
    assert L.psamp_status_string(0) == b"ok"
    assert L.psamp_status_string(5) == b"workspace missing or too small"
    assert L.psamp_status_string(99) == b"unknown status"


def test_workspace_sizes(L):
    assert L.psamp_build_cdf_workspace_size(0) == 0
    # 256-byte header + 4 KiB per 64 tiles of 1024 elements
    assert L.psamp_build_cdf_workspace_size(1) == 256 + 4096
    assert L.psamp_build_cdf_workspace_size(64 * 1024) == 256 + 4096
    assert L.psamp_build_cdf_workspace_size(64 * 1024 + 1) == 256 + 2 * 4096
    assert L.psamp_build_cdf_workspace_size(1 << 24) == 256 + 64 * (1 << 14)
    assert L.psamp_per_round_workspace_size(262144, 8192) == 256 + 64 * 256
    assert L.psamp_per_round_workspace_size(1 << 20, 1 << 20) == 256 + 64 * 1024
    assert L.psamp_is_weights_workspace_size(8192) == 256
    assert L.psamp_is_weights_workspace_size(1) == 256
    assert L.psamp_is_weights_workspace_size(0) == 0
    assert L.psamp_is_weights_workspace_size(1 << 20) == 256 + 8 * 1024 + 4 * 256
    assert L.psamp_is_weights_workspace_size(8193) == 256 + 8 * 1024 + 4 * 3
    assert L.psamp_scatter_workspace_size(262144, 8192) == 262144 * 4
    assert L.psamp_segtree_cap_pow2(500000) == 524288
    assert L.psamp_segtree_cap_pow2(100000) == 131072
    assert L.psamp_segtree_cap_pow2(1) == 1
    assert L.psamp_segtree_cap_pow2(0) == 0
    assert L.psamp_segtree_cap_pow2((1 << 30) + 1) == 0


F32, F64, U32, U64, I32 = 0, 1, 2, 3, 4
OK, E_NULL, E_SIZE, E_DTYPE, E_PARAM, E_WS, E_ALIGN = 0, 1, 2, 3, 4, 5, 6


def test_build_cdf_validation(L):
    ws = L.psamp_build_cdf_workspace_size(1000)
    f = L.psamp_build_cdf
    assert f(None, F32, 1000, 0.6, FAKE, F64, FAKE, FAKE, ws, None) == E_NULL
    assert f(FAKE, F32, 0, 0.6, FAKE, F64, FAKE, FAKE, ws, None) == E_SIZE
    assert f(FAKE, F32, 1 << 31, 0.6, FAKE, F64, FAKE, FAKE, ws, None) == E_SIZE
    assert f(FAKE, F32, 1000, 0.6, FAKE, U64, FAKE, FAKE, ws, None) == E_DTYPE
    assert f(FAKE, U32, 1000, 0.6, FAKE, F64, FAKE, FAKE, ws, None) == E_DTYPE
    assert f(FAKE, F32, 1000, 0.0, FAKE, F64, FAKE, FAKE, ws, None) == E_PARAM
    assert f(FAKE, F32, 1000, float("nan"), FAKE, F64, FAKE, FAKE, ws, None) == E_PARAM
    assert f(FAKE, F32, 1000, float("inf"), FAKE, F64, FAKE, FAKE, ws, None) == E_PARAM
    assert f(FAKE, F32, 1000, 0.6, FAKE, F64, FAKE, None, ws, None) == E_WS
    assert f(FAKE, F32, 1000, 0.6, FAKE, F64, FAKE, FAKE, ws - 1, None) == E_WS
    assert f(FAKE + 2, F32, 1000, 0.6, FAKE, F64, FAKE, FAKE, ws, None) == E_ALIGN
    assert f(FAKE, F32, 1000, 0.6, FAKE + 4, F64, FAKE, FAKE, ws, None) == E_ALIGN


def test_sample_validation(L):
    f = L.psamp_sample
    assert f(FAKE, F64, 0, FAKE, FAKE, F32, 10, 1, FAKE, None) == E_SIZE
    assert f(FAKE, F64, 10, FAKE, FAKE, F32, -1, 1, FAKE, None) == E_SIZE
    assert f(FAKE, F64, 10, FAKE, FAKE, F32, 10, 2, FAKE, None) == E_PARAM
    assert f(FAKE, F64, 10, FAKE, FAKE, U32, 10, 1, FAKE, None) == E_DTYPE
    assert f(FAKE, U64, 10, FAKE, FAKE, F32, 10, 1, FAKE, None) == E_DTYPE
    assert f(FAKE, F64, 10, FAKE, FAKE, F32, 0, 1, None, None) == OK      # k = 0: no-op
    assert f(FAKE, F64, 10, None, FAKE, F32, 10, 1, FAKE, None) == E_NULL
    assert f(FAKE + 4, F64, 10, FAKE, FAKE, F32, 10, 1, FAKE, None) == E_ALIGN
    assert f(FAKE, F64, 10, FAKE, FAKE, F32, 10, 1, FAKE + 2, None) == E_ALIGN


def test_build_cdf_sample_validation(L):
    ws = L.psamp_build_cdf_workspace_size(1000)
    f = L.psamp_build_cdf_sample
    #       prio  pt   n     alpha u     ut   k   cdf   ct   total idx   ws    bytes
    assert f(None, F32, 1000, 0.6, FAKE, F32, 10, FAKE, F64, FAKE, FAKE, FAKE, ws, None) == E_NULL
    assert f(FAKE, F32, 0, 0.6, FAKE, F32, 10, FAKE, F64, FAKE, FAKE, FAKE, ws, None) == E_SIZE
    assert f(FAKE, F32, 1000, 0.6, FAKE, F32, -1, FAKE, F64, FAKE, FAKE, FAKE, ws, None) == E_SIZE
    assert f(FAKE, F32, 1000, 0.6, FAKE, U32, 10, FAKE, F64, FAKE, FAKE, FAKE, ws, None) == E_DTYPE
    assert f(FAKE, U32, 1000, 0.6, FAKE, U32, 10, FAKE, F64, FAKE, FAKE, FAKE, ws, None) == E_DTYPE
    assert f(FAKE, F32, 1000, 0.0, FAKE, F32, 10, FAKE, F64, FAKE, FAKE, FAKE, ws, None) == E_PARAM
    assert f(FAKE, F32, 1000, 0.6, None, F32, 10, FAKE, F64, FAKE, FAKE, FAKE, ws, None) == E_NULL
    assert f(FAKE, F32, 1000, 0.6, FAKE, F32, 10, FAKE, F64, FAKE, None, FAKE, ws, None) == E_NULL
    assert f(FAKE, F32, 1000, 0.6, FAKE, F32, 10, FAKE, F64, FAKE, FAKE, None, ws, None) == E_WS
    assert f(FAKE, F32, 1000, 0.6, FAKE, F32, 10, FAKE, F64, FAKE, FAKE, FAKE, ws - 8,
             None) == E_WS
    assert f(FAKE, F32, 1000, 0.6, FAKE + 2, F32, 10, FAKE, F64, FAKE, FAKE, FAKE, ws,
             None) == E_ALIGN
    assert f(FAKE, F32, 1000, 0.6, FAKE, F32, 10, FAKE, F64, FAKE, FAKE + 2, FAKE, ws,
             None) == E_ALIGN


def test_is_weights_validation(L):
    f = L.psamp_is_weights
    assert f(FAKE, F64, 10, 0.6, FAKE, 5, 0.4, FAKE, None, 0, None) == E_DTYPE
    assert f(FAKE, F32, 10, 0.6, FAKE, 5, -0.1, FAKE, None, 0, None) == E_PARAM
    assert f(FAKE, F32, 10, -1.0, FAKE, 5, 0.4, FAKE, None, 0, None) == E_PARAM
    assert f(FAKE, F32, 10, 0.6, FAKE, 1 << 20, 0.4, FAKE, None, 0, None) == E_WS
    assert f(FAKE, F32, 10, 0.6, FAKE, 0, 0.4, None, None, 0, None) == OK
    assert f(None, F32, 10, 0.6, FAKE, 5, 0.4, FAKE, None, 0, None) == E_NULL
    assert f(FAKE + 2, F32, 10, 0.6, FAKE, 5, 0.4, FAKE, FAKE, 256, None) == E_ALIGN
    assert f(FAKE, F32, 10, 0.6, FAKE, 5, 0.4, FAKE, FAKE + 4, 256, None) == E_ALIGN


def test_segtree_validation(L):
    b, u, s = L.psamp_segtree_build, L.psamp_segtree_update, L.psamp_segtree_sample
    assert b(FAKE, F32, 1000, FAKE, F32, 10, 0.6, None) == E_SIZE          # not a power of 2
    assert b(FAKE, F32, 1024, FAKE, F32, 1025, 0.6, None) == E_SIZE        # n_valid > cap
    assert b(FAKE, F32, 1024, FAKE, U32, 10, 0.6, None) == E_DTYPE
    assert b(FAKE, U64, 1024, FAKE, F32, 10, 0.6, None) == E_DTYPE
    assert b(FAKE, F32, 1024, FAKE, F32, 10, 0.0, None) == E_PARAM
    assert b(FAKE + 8, F32, 1024, FAKE, F32, 10, 0.6, None) == E_ALIGN
    assert b(None, F32, 1024, FAKE, F32, 10, 0.6, None) == E_NULL
    assert u(FAKE, F32, 1024, FAKE, FAKE, F32, 0, 0.6, None, 0, None) == OK
    assert u(FAKE, F32, 1024, FAKE, FAKE, F32, -1, 0.6, None, 0, None) == E_SIZE
    assert u(FAKE, F32, 1024, None, FAKE, F32, 4, 0.6, None, 0, None) == E_NULL
    assert s(FAKE, F32, 1024, 0, FAKE, F32, 4, 0, FAKE, None) == E_SIZE
    assert s(FAKE, F32, 1024, 10, FAKE, U32, 4, 0, FAKE, None) == E_DTYPE
    assert s(FAKE, F32, 1024, 10, FAKE, F32, 4, 3, FAKE, None) == E_PARAM
    assert s(FAKE + 8, F32, 1024, 10, FAKE, F32, 4, 0, FAKE, None) == E_ALIGN   # tree: 16 B
    assert u(FAKE, F32, 1024, FAKE, FAKE, F32, 4, 0.6, None, 0, None) == E_WS
    assert u(FAKE, F32, 1024, FAKE, FAKE, F32, 4, 0.6, FAKE, 511, None) == E_WS
    assert L.psamp_segtree_update_workspace_size(1024, 1024) == 512   # one word per subtree root
    assert u(FAKE + 8, F32, 1024, FAKE, FAKE, F32, 4, 0.6, FAKE, 512, None) == E_ALIGN
    assert u(FAKE, F32, 1024, FAKE + 2, FAKE, F32, 4, 0.6, FAKE, 512, None) == E_ALIGN
    assert u(FAKE, F32, 1024, FAKE, FAKE, F32, 4, 0.6, FAKE + 4, 512, None) == E_ALIGN


def test_resample_and_scatter_validation(L):
    r = L.psamp_resample_rows
    assert r(FAKE, 4, 4096, 4095, FAKE, FAKE, 4096, None) == E_SIZE
    assert r(FAKE, 4, 8193, 8193, FAKE, FAKE, 8193, None) == E_SIZE
    assert r(FAKE, 0, 4096, 4096, FAKE, FAKE, 4096, None) == E_SIZE
    assert r(None, 4, 4096, 4096, FAKE, FAKE, 4096, None) == E_NULL
    assert r(FAKE + 2, 4, 4096, 4096, FAKE, FAKE, 4096, None) == E_ALIGN
    sc = L.psamp_scatter_lww
    assert sc(FAKE, F64, 100, FAKE, FAKE, 10, 0, FAKE, 400, None) == E_DTYPE
    assert sc(FAKE, F32, 100, FAKE, FAKE, 10, 0, FAKE, 399, None) == E_WS
    assert sc(FAKE, F32, 100, FAKE, FAKE, 10, 2, FAKE, 400, None) == E_PARAM
    assert sc(FAKE, F32, 100, FAKE, FAKE, 0, 0, None, 0, None) == OK
    assert sc(FAKE + 2, F32, 100, FAKE, FAKE, 10, 0, FAKE, 400, None) == E_ALIGN
    assert L.psamp_workspace_errors(None, 256, None, None) == E_NULL
    pr = L.psamp_per_round
    wsz = L.psamp_per_round_workspace_size(1000, 10)
    assert pr(None, 1000, 0.6, 0.4, FAKE, 10, None, FAKE, FAKE, FAKE, FAKE, FAKE, wsz, None) == E_NULL
    assert pr(FAKE, 0, 0.6, 0.4, FAKE, 10, None, FAKE, FAKE, FAKE, FAKE, FAKE, wsz, None) == E_SIZE
    assert pr(FAKE, 1000, 0.0, 0.4, FAKE, 10, None, FAKE, FAKE, FAKE, FAKE, FAKE, wsz, None) == E_PARAM
    assert pr(FAKE, 1000, 0.6, -1.0, FAKE, 10, None, FAKE, FAKE, FAKE, FAKE, FAKE, wsz, None) == E_PARAM
    assert pr(FAKE, 1000, 0.6, 0.4, FAKE, 10, None, FAKE, FAKE, FAKE, FAKE, FAKE, wsz - 1, None) == E_WS
    assert pr(FAKE, 1000, 0.6, 0.4, FAKE, 10, None, FAKE, FAKE, FAKE, FAKE, FAKE + 8, wsz, None) == E_ALIGN


def test_pf_step_validation(L):
    f = L.psamp_pf_step
    ok = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, 0.5, FAKE)

    def call(*, args=ok, rows=16, P=1024, D=4, O=2, xo=FAKE, lo=FAKE, an=None):
        return f(*args, rows, P, D, O, xo, lo, an, None)

    assert call(args=(None,) + ok[1:]) == E_NULL
    assert call(lo=None) == E_NULL
    assert call(rows=0) == E_SIZE
    assert call(P=0) == E_SIZE
    assert call(P=8193, D=1) == E_SIZE
    assert call(D=3) == E_SIZE
    assert call(D=16, P=64) == E_SIZE
    assert call(P=4097, D=4) == E_SIZE          # P * D over 16384
    assert call(P=2049, D=8) == E_SIZE
    assert call(O=0) == E_SIZE
    assert call(O=9) == E_SIZE
    assert call(args=ok[:7] + (0.0, FAKE)) == E_PARAM
    assert call(args=ok[:7] + (float("inf"), FAKE)) == E_PARAM
    assert call(args=ok[:6] + (float("nan"), 0.5, FAKE)) == E_PARAM
    assert call(xo=FAKE + 8) == E_ALIGN
    assert call(args=(FAKE + 4,) + ok[1:]) == E_ALIGN
    assert call(an=FAKE + 2) == E_ALIGN


def test_replay_validation(L):
    import proportional_sampling_amd as ps
    rb = ps._ReplayStruct()
    ref = C.byref(rb)
    assert L.psamp_replay_init(None, 10, 0.6, FAKE, None, 0) == E_NULL
    assert L.psamp_replay_init(ref, 10, 0.6, None, None, 0) == E_NULL
    assert L.psamp_replay_init(ref, 0, 0.6, FAKE, None, 0) == E_SIZE
    assert L.psamp_replay_init(ref, (1 << 30) + 1, 0.6, FAKE, None, 0) == E_SIZE
    assert L.psamp_replay_init(ref, 10, 0.0, FAKE, None, 0) == E_PARAM
    assert L.psamp_replay_init(ref, 10, 0.6, FAKE + 2, None, 0) == E_ALIGN
    assert L.psamp_replay_init(ref, 1000, 0.6, FAKE, None, 0) == OK
    assert (rb.capacity, rb.cap_pow2, rb.cursor, rb.size) == (1000, 1024, 0, 0)
    assert L.psamp_replay_total(ref) == FAKE + 4
    assert L.psamp_replay_insert(ref, FAKE, 0, FAKE, None) == OK      # nothing enqueued
    assert (rb.cursor, rb.size) == (0, 0)
    assert L.psamp_replay_insert(ref, None, 5, FAKE, None) == E_NULL
    assert L.psamp_replay_insert(ref, FAKE, -1, FAKE, None) == E_SIZE
    assert L.psamp_replay_insert(ref, FAKE, 5, FAKE + 1, None) == E_ALIGN
    assert L.psamp_replay_sample(ref, FAKE, 8, 1, 0.4, FAKE, FAKE, None) == E_SIZE   # empty
    rb.size = 10
    assert L.psamp_replay_sample(ref, FAKE, 8, 2, 0.4, FAKE, FAKE, None) == E_PARAM
    assert L.psamp_replay_sample(ref, FAKE, 8, 1, -0.5, FAKE, FAKE, None) == E_PARAM
    assert L.psamp_replay_sample(ref, FAKE, 1 << 20, 1, 0.4, FAKE, FAKE, None) == E_WS
    rb.cursor = 1000                                                    # corrupted state
    assert L.psamp_replay_update(ref, FAKE, FAKE, 4, None) == E_PARAM
    assert L.psamp_replay_workspace_size(1000, 8192) == 512 + 256     # update, then IS
    assert L.psamp_replay_workspace_size(1000, 1 << 20) > 0


def test_binding_fails_loudly_without_gpu_tensors():
    import torch
    import proportional_sampling_amd as ps
    with pytest.raises(ValueError):
        ps.build_cdf(torch.ones(10, dtype=torch.float32), 0.6, ws=None)


def test_noalloc_ceiling_and_check_host_paths(L):
    """The paths of the later entry points that never reach the device:
    the no-allocation update refuses sizes beyond its scratch (and bad
    arguments) before any set-up; the copy-ceiling aid validates its
    geometry; the check switch toggles and reports its state."""
    na = L.psamp_per_round_noalloc
    assert na(FAKE, (1 << 26) + 1, 0.6, 0.4, FAKE, 8, None, FAKE, FAKE, FAKE, FAKE, None) == E_SIZE
    assert na(FAKE, 0, 0.6, 0.4, FAKE, 8, None, FAKE, FAKE, FAKE, FAKE, None) == E_SIZE
    assert na(None, 100, 0.6, 0.4, FAKE, 8, None, FAKE, FAKE, FAKE, FAKE, None) == E_NULL
    assert na(FAKE, 100, 0.0, 0.4, FAKE, 8, None, FAKE, FAKE, FAKE, FAKE, None) == E_PARAM
    assert na(FAKE, 100, 0.6, float("nan"), FAKE, 8, None, FAKE, FAKE, FAKE, FAKE, None) == E_PARAM
    cc = L.psamp_ceiling_copy
    assert cc(None, FAKE, 1024, 8, 1, None) == E_NULL
    assert cc(FAKE, FAKE, 1022, 8, 1, None) == E_SIZE
    assert cc(FAKE, FAKE, 1024, 3, 1, None) == E_PARAM
    assert cc(FAKE, FAKE, 1024, 2, 2, None) == E_PARAM
    assert cc(FAKE + 4, FAKE, 1024, 2, 0, None) == E_ALIGN
    prev = L.psamp_check_enable(-1)
    try:
        L.psamp_check_enable(1)
        assert L.psamp_check_enable(-1) == 1
        assert L.psamp_check_enable(0) == 1
        assert L.psamp_check_enable(-1) == 0
    finally:
        L.psamp_check_enable(prev)
    assert L.psamp_check_errors(None, 1, None) == E_NULL
