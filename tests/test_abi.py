"""The C-ABI library loads and exports every entry point of include/flashbob.h,
and its host-side argument checks return the documented status codes. No call
here reaches a kernel launch (there may be no GPU)."""

import ctypes
import os
import re

import pytest

import aware_flashbob_pass_amd as fb
from aware_flashbob_pass_amd.binding import FB_BF16, FB_F16, FB_F32

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashbob.h")

FB_OK, FB_ERR_NULL, FB_ERR_SHAPE, FB_ERR_DTYPE, FB_ERR_HEADDIM, FB_ERR_WORKSPACE, FB_ERR_OOM, FB_ERR_HIP, FB_ERR_ARG = (
    0, -1, -2, -3, -4, -5, -6, -7, -8)


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fb.LIB_PATH):
        pytest.fail("libflashbob.so is not built (run __graft_entry__.build())")
    return fb.load_library()


def test_header_declares_expected_entry_points():
    names = _declared_functions()
    for n in ("bob_attention", "bob_attention_ws", "bob_attention_with_stats", "bob_workspace_bytes",
              "attn_fwd", "attn_bwd", "fb_last_error", "fb_set_tuning", "fb_profile_start", "fb_profile_stop"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), f"{name} declared in flashbob.h but not exported"
        assert name in fb.SIGNATURES, f"{name} has no ctypes signature in the binding"


def test_workspace_is_linear_in_n(lib):
    fb.set_tuning(4, 4)
    try:
        ws = [lib.bob_workspace_bytes(1, 1, n, 64, FB_BF16) for n in (1 << 14, 1 << 15, 1 << 16, 1 << 18)]
        per_row = [w / n for w, n in zip(ws, (1 << 14, 1 << 15, 1 << 16, 1 << 18))]
        assert max(per_row) / min(per_row) < 1.01, per_row  # no N^2 term
        assert per_row[-1] < 64 * 1024  # bytes per query row at d=64
    finally:
        fb.set_tuning(0, 0)
    assert lib.bob_workspace_bytes(1, 1, 0, 64, FB_BF16) == 0
    assert lib.bob_workspace_bytes(1, 1, 128, 96, FB_BF16) == 0


def test_auto_splits_bounded_workspace(lib):
    # with automatic splits, the workspace of the 262,144-token endpoint stays O(N d)
    w = lib.bob_workspace_bytes(1, 1, 262144, 64, FB_BF16)
    assert 0 < w < 262144 * 64 * 2 * 4


P = 0x100000  # fake, aligned, never dereferenced: the checks fail before any launch


def _bob_ws(lib, ptrs=None, tau=0.125, causal=0, B=1, H=1, N=128, d=64, dt=FB_BF16, ws=P, ws_bytes=1 << 40):
    ptrs = ptrs or [P + 0x1000 * i for i in range(11)]
    args = [ctypes.c_void_p(p) for p in ptrs[:7]] + [tau, causal, B, H, N, d, dt] + \
           [ctypes.c_void_p(p) for p in ptrs[7:11]] + [ctypes.c_void_p(ws), ws_bytes, None]
    return lib.bob_attention_ws(*args)


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), FB_ERR_HEADDIM),
    (dict(d=32), FB_ERR_HEADDIM),
    (dict(N=0), FB_ERR_SHAPE),
    (dict(B=0), FB_ERR_SHAPE),
    (dict(H=-1), FB_ERR_SHAPE),
    (dict(B=300, H=300), FB_ERR_SHAPE),
    (dict(N=2147483647), FB_ERR_SHAPE),
    (dict(N=2147483647 - 127), FB_ERR_SHAPE),
    (dict(B=2, H=2, N=1 << 29), FB_ERR_SHAPE),
    (dict(dt=7), FB_ERR_DTYPE),
    (dict(tau=float("nan")), FB_ERR_ARG),
    (dict(tau=float("inf")), FB_ERR_ARG),
    (dict(ws=0), FB_ERR_WORKSPACE),
    (dict(ws_bytes=16), FB_ERR_WORKSPACE),
    (dict(ws=P + 16), FB_ERR_WORKSPACE),
])
def test_bob_ws_argument_checks(lib, kw, code):
    assert _bob_ws(lib, **kw) == code
    assert lib.fb_last_error().decode()


def test_null_alias_alignment_checks(lib):
    ptrs = [P + 0x1000 * i for i in range(11)]
    bad = list(ptrs)
    bad[3] = 0
    assert _bob_ws(lib, ptrs=bad) == FB_ERR_NULL
    assert b"dO" in lib.fb_last_error()
    bad = list(ptrs)
    bad[9] = ptrs[0]  # gV aliases Q
    assert _bob_ws(lib, ptrs=bad) == FB_ERR_ARG
    assert b"alias" in lib.fb_last_error()
    bad = list(ptrs)
    bad[10] = ptrs[8]  # gdO aliases gK
    assert _bob_ws(lib, ptrs=bad) == FB_ERR_ARG
    bad = list(ptrs)
    bad[2] = P + 8  # misaligned
    assert _bob_ws(lib, ptrs=bad) == FB_ERR_ARG


def test_tuning_checks(lib):
    assert lib.fb_set_tuning(-1, 0) == FB_ERR_ARG
    assert lib.fb_set_tuning(0, 65) == FB_ERR_ARG
    assert lib.fb_set_tuning(0, 0) == FB_OK


def test_other_entry_point_checks(lib):
    v = ctypes.c_void_p
    # attn_fwd with D_out but no dO
    st = lib.attn_fwd(v(P), v(P + 0x1000), v(P + 0x2000), v(0), 0.125, 0, 1, 1, 64, 64, FB_F32,
                      v(P + 0x3000), v(P + 0x4000), v(P + 0x5000), None)
    assert st == FB_ERR_NULL
    # attn_bwd with d = 80
    st = lib.attn_bwd(*[v(P + 0x1000 * i) for i in range(6)], 0.125, 0, 1, 1, 64, 80, FB_F16,
                      *[v(P + 0x1000 * (6 + i)) for i in range(4)], None)
    assert st == FB_ERR_HEADDIM
    # with_stats: L misaligned
    ptrs = [v(P + 0x1000 * i) for i in range(10)]
    ptrs[8] = v(P + 0x8002)
    st = lib.bob_attention_with_stats(*ptrs, 0.125, 0, 1, 1, 64, 64, FB_BF16, *[v(P + 0x1000 * (10 + i)) for i in range(6)],
                                      v(P), 1 << 40, None)
    assert st == FB_ERR_ARG


def test_probe_argument_checks(lib):
    """The measurement probe checks its arguments before any launch."""
    dummy = ctypes.c_void_p(16)
    assert lib.fb_probe_gq_atomics(None, 1, 1, 256, 64, 1, None) == FB_ERR_NULL
    assert lib.fb_probe_gq_atomics(dummy, 1, 1, 256, 96, 1, None) == FB_ERR_HEADDIM
    assert lib.fb_probe_gq_atomics(dummy, 1, 0, 256, 64, 1, None) == FB_ERR_SHAPE
    for bad in (0, 65):
        assert lib.fb_probe_gq_atomics(dummy, 1, 1, 256, 64, bad, None) == FB_ERR_ARG


def test_size_overflow_bounds(lib):
    """B*H*N beyond 2^31 - 256 is rejected (row tile counts and launch ids are int);
    sizes just inside the bound give a finite, linear workspace without overflow."""
    INT_MAX = 2147483647
    assert lib.bob_workspace_bytes(1, 1, INT_MAX, 64, FB_BF16) == 0
    assert lib.bob_workspace_bytes(1, 1, INT_MAX - 127, 64, FB_BF16) == 0
    assert lib.bob_workspace_bytes(65535, 1, 32769, 64, FB_BF16) == 0  # B*H*N just above the bound
    n_max = INT_MAX - 255
    w = lib.bob_workspace_bytes(1, 1, n_max, 128, FB_F32)
    assert w > n_max * 128 * 4  # at least the O buffer, no wrap-around
    assert w < n_max * 1024 * 4
    w2 = lib.bob_workspace_bytes(65535, 1, 32767, 64, FB_BF16)
    assert w2 > 65535 * 32767 * 64 * 2
    v = ctypes.c_void_p
    st = lib.attn_fwd(v(P), v(P + 0x1000), v(P + 0x2000), v(0), 0.125, 0, 1, 1, INT_MAX, 64, FB_BF16,
                      v(P + 0x3000), v(P + 0x4000), None, None)
    assert st == FB_ERR_SHAPE and b"exceeds" in lib.fb_last_error()


def test_alloc_limit_refuses_before_any_hip_call(lib):
    """With an allocation cap below the need, the allocating entry points return
    FB_ERR_OOM from the host checks alone (no device here)."""
    v = ctypes.c_void_p
    ptrs = [v(P + 0x1000 * i) for i in range(11)]
    fb.set_alloc_limit(1024)
    try:
        st = lib.bob_attention(*ptrs[:7], 0.125, 0, 1, 1, 4096, 64, FB_BF16, *ptrs[7:], None)
        assert st == FB_ERR_OOM
        assert b"allocation limit" in lib.fb_last_error()
        # attn_bwd without D_out needs scratch for D
        st = lib.attn_bwd(*[v(P + 0x1000 * i) for i in range(6)], 0.125, 0, 1, 1, 4096, 64, FB_BF16,
                          *[v(P + 0x1000 * (6 + i)) for i in range(4)], None)
        assert st == FB_ERR_OOM
        # argument errors still come first
        bad = list(ptrs)
        bad[0] = v(0)
        assert lib.bob_attention(*bad[:7], 0.125, 0, 1, 1, 4096, 64, FB_BF16, *bad[7:], None) == FB_ERR_NULL
    finally:
        fb.set_alloc_limit(0)
