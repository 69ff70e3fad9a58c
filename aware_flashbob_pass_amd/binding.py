"""ctypes binding of libflashbob.so: argument marshalling only.

Every step of the computation runs in the library's HIP kernels; torch is used
here for device memory (output and workspace allocation) and for the current
HIP stream. There is no fallback: if the library is missing or a call fails,
an exception is raised.
"""

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libflashbob.so")

FB_F32, FB_F16, FB_BF16 = 0, 1, 2
_DT = {torch.float32: FB_F32, torch.float16: FB_F16, torch.bfloat16: FB_BF16}

# C-ABI entry points declared in include/flashbob.h, with their ctypes signatures
_P, _I, _F, _S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int), ("total_ms", ctypes.c_double)]


SIGNATURES = {
    "fb_last_error": (ctypes.c_char_p, []),
    "bob_attention": (_I, [_P] * 7 + [_F, _I, _I, _I, _I, _I, _I] + [_P] * 4 + [_P]),
    "bob_workspace_bytes": (_S, [_I, _I, _I, _I, _I]),
    "bob_attention_noalloc": (_I, [_P] * 7 + [_F, _I, _I, _I, _I, _I, _I] + [_P] * 4 + [_P]),
    "bob_attention_ws": (_I, [_P] * 7 + [_F, _I, _I, _I, _I, _I, _I] + [_P] * 4 + [_P, _S, _P]),
    "bob_attention_fourpass_ws": (_I, [_P] * 7 + [_F, _I, _I, _I, _I, _I, _I] + [_P] * 4 + [_P, _S, _P]),
    "bob_attention_with_stats": (_I, [_P] * 10 + [_F, _I, _I, _I, _I, _I, _I] + [_P] * 6 + [_P, _S, _P]),
    "attn_fwd": (_I, [_P] * 4 + [_F, _I, _I, _I, _I, _I, _I] + [_P] * 3 + [_P]),
    "attn_bwd": (_I, [_P] * 6 + [_F, _I, _I, _I, _I, _I, _I] + [_P] * 4 + [_P]),
    "fb_set_tuning": (_I, [_I, _I]),
    "fb_set_alloc_limit": (_I, [_S]),
    "fb_set_reduction": (_I, [_I]),
    "fb_probe_gq_atomics": (_I, [_P, _I, _I, _I, _I, _I, _P]),
    "fb_profile_start": (None, [ctypes.c_char_p]),
    "fb_profile_stop": (_I, [ctypes.POINTER(KernelTime), _I]),
}

_lib = None


class FlashBoBError(RuntimeError):
    pass


def load_library(path=LIB_PATH):
    """Load libflashbob.so (raises if it is missing: there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FlashBoBError(
            f"{path} is missing: build it with `python -m aware_flashbob_pass_amd.build` "
            "(the HIP library is required; there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status):
    if status != 0:
        msg = load_library().fb_last_error().decode(errors="replace")
        raise FlashBoBError(f"flashbob status {status}: {msg}")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _check_inputs(named, dtype=None):
    ref = None
    for name, t in named:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must have shape [B, H, N, d], got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if ref is None:
            ref = t
        elif t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device:
            raise ValueError(f"{name} does not match shape/dtype/device of {named[0][0]}")
    if ref.dtype not in _DT:
        raise ValueError(f"unsupported dtype {ref.dtype}")
    return ref


def _vec_check(name, t, shape, device):
    if t.dtype != torch.float32 or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or t.device != device:
        raise ValueError(f"{name} must be a contiguous float32 tensor of shape {tuple(shape)} on {device}")


def _tau(tau, d):
    return float(1.0 / math.sqrt(d) if tau is None else tau)


def workspace_bytes(B, H, N, d, dtype):
    return int(load_library().bob_workspace_bytes(B, H, N, d, _DT[dtype]))


def set_tuning(pass1_splits=0, pass2_splits=0):
    _check(load_library().fb_set_tuning(int(pass1_splits), int(pass2_splits)))


def set_reduction(mode=0):
    """Pass 2's split reduction: 0 records + merge kernel, 1 float32 atomics, 2 last
    workgroup merges (see fb_set_reduction in flashbob.h)."""
    _check(load_library().fb_set_reduction(int(mode)))


def probe_gq_atomics(gq, B, H, N, d, splits):
    """Measurement probe: the float32 atomic additions of a schedule that forms gQ in
    pass 2 (see fb_probe_gq_atomics in flashbob.h). gq: [B][H][N][d] float32 on the GPU;
    every element grows by ceil(N / 128)."""
    if gq.dtype != torch.float32 or not gq.is_cuda or gq.numel() != B * H * N * d or not gq.is_contiguous():
        raise ValueError("gq must be a contiguous float32 GPU tensor of B*H*N*d elements")
    _check(load_library().fb_probe_gq_atomics(_ptr(gq), B, H, N, d, splits, _stream()))


def set_alloc_limit(nbytes=0):
    """Cap on each device allocation the library makes itself (0: no cap)."""
    _check(load_library().fb_set_alloc_limit(int(nbytes)))


def bob_attention(q, k, v, do, uq, uk, uv, tau=None, causal=False, workspace=None, out=None):
    """Exact BoB through softmax attention: returns (gQ, gK, gV, gdO).

    Inputs are [B, H, N, d] GPU tensors of one dtype (float32, float16 or
    bfloat16). The workspace is a torch-allocated byte tensor (allocated here
    when not given), so torch's memory statistics see all device memory.
    `out` optionally gives the four output tensors (same shape and dtype).
    """
    ref = _check_inputs([("q", q), ("k", k), ("v", v), ("do", do), ("uq", uq), ("uk", uk), ("uv", uv)])
    B, H, N, d = ref.shape
    lib = load_library()
    dt = _DT[ref.dtype]
    need = int(lib.bob_workspace_bytes(B, H, N, d, dt))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=ref.device)
    if out is None:
        outs = [torch.empty_like(ref) for _ in range(4)]
    else:
        outs = list(out)
        _check_inputs([("q", ref)] + [(f"out[{i}]", t) for i, t in enumerate(outs)])
    _check(lib.bob_attention_ws(*[_ptr(t) for t in (q, k, v, do, uq, uk, uv)], _tau(tau, d), int(bool(causal)),
                                B, H, N, d, dt, *[_ptr(t) for t in outs], _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream()))
    return tuple(outs)


def bob_attention_fourpass(q, k, v, do, uq, uk, uv, tau=None, causal=False, workspace=None, out=None):
    """The same BoB result through the four-pass ablation schedule (bf16/fp16)."""
    ref = _check_inputs([("q", q), ("k", k), ("v", v), ("do", do), ("uq", uq), ("uk", uk), ("uv", uv)])
    B, H, N, d = ref.shape
    lib = load_library()
    dt = _DT[ref.dtype]
    if workspace is None:
        workspace = torch.empty(max(int(lib.bob_workspace_bytes(B, H, N, d, dt)), 1), dtype=torch.uint8,
                                device=ref.device)
    outs = [torch.empty_like(ref) for _ in range(4)] if out is None else list(out)
    _check(lib.bob_attention_fourpass_ws(*[_ptr(t) for t in (q, k, v, do, uq, uk, uv)], _tau(tau, d),
                                         int(bool(causal)), B, H, N, d, dt, *[_ptr(t) for t in outs],
                                         _ptr(workspace), workspace.numel() * workspace.element_size(), _stream()))
    return tuple(outs)


def bob_attention_alloc(q, k, v, do, uq, uk, uv, tau=None, causal=False):
    """As bob_attention, through the entry point that allocates its own workspace."""
    ref = _check_inputs([("q", q), ("k", k), ("v", v), ("do", do), ("uq", uq), ("uk", uk), ("uv", uv)])
    B, H, N, d = ref.shape
    outs = [torch.empty_like(ref) for _ in range(4)]
    _check(load_library().bob_attention(*[_ptr(t) for t in (q, k, v, do, uq, uk, uv)], _tau(tau, d),
                                        int(bool(causal)), B, H, N, d, _DT[ref.dtype], *[_ptr(t) for t in outs],
                                        _stream()))
    return tuple(outs)


def bob_attention_noalloc(q, k, v, do, uq, uk, uv, tau=None, causal=False, out=None):
    """As bob_attention, through the entry point that allocates nothing on the device
    (the library's fixed 64 MiB scratch array); only the outputs are allocated here,
    unless `out` gives them."""
    ref = _check_inputs([("q", q), ("k", k), ("v", v), ("do", do), ("uq", uq), ("uk", uk), ("uv", uv)])
    B, H, N, d = ref.shape
    outs = list(out) if out is not None else [torch.empty_like(ref) for _ in range(4)]
    _check(load_library().bob_attention_noalloc(*[_ptr(t) for t in (q, k, v, do, uq, uk, uv)], _tau(tau, d),
                                                int(bool(causal)), B, H, N, d, _DT[ref.dtype],
                                                *[_ptr(t) for t in outs], _stream()))
    return tuple(outs)


def bob_attention_with_stats(q, k, v, do, uq, uk, uv, o, lse, dvec, tau=None, causal=False,
                             return_scalars=False, workspace=None):
    """Pass 1 + pass 2 from saved statistics O, L (row LSE) and D = rowsum(dO * O).
    Returns (gQ, gK, gV, gdO) and, with return_scalars, also (alpha, E)."""
    ref = _check_inputs([("q", q), ("k", k), ("v", v), ("do", do), ("uq", uq), ("uk", uk), ("uv", uv), ("o", o)])
    B, H, N, d = ref.shape
    _vec_check("lse", lse, (B, H, N), ref.device)
    _vec_check("dvec", dvec, (B, H, N), ref.device)
    lib = load_library()
    dt = _DT[ref.dtype]
    need = int(lib.bob_workspace_bytes(B, H, N, d, dt))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=ref.device)
    outs = [torch.empty_like(ref) for _ in range(4)]
    alpha = torch.empty((B, H, N), dtype=torch.float32, device=ref.device) if return_scalars else None
    e_row = torch.empty((B, H, N), dtype=torch.float32, device=ref.device) if return_scalars else None
    _check(lib.bob_attention_with_stats(*[_ptr(t) for t in (q, k, v, do, uq, uk, uv, o, lse, dvec)], _tau(tau, d),
                                        int(bool(causal)), B, H, N, d, dt, *[_ptr(t) for t in outs], _ptr(alpha),
                                        _ptr(e_row), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                        _stream()))
    if return_scalars:
        return tuple(outs), (alpha, e_row)
    return tuple(outs)


def attn_fwd(q, k, v, tau=None, causal=False, do=None):
    """Forward with statistics: returns (O, L) or, when dO is given, (O, L, D)."""
    ref = _check_inputs([("q", q), ("k", k), ("v", v)] + ([("do", do)] if do is not None else []))
    B, H, N, d = ref.shape
    o = torch.empty_like(ref)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=ref.device)
    dvec = torch.empty((B, H, N), dtype=torch.float32, device=ref.device) if do is not None else None
    _check(load_library().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _tau(tau, d), int(bool(causal)), B, H, N, d,
                                   _DT[ref.dtype], _ptr(o), _ptr(lse), _ptr(dvec), _stream()))
    return (o, lse) if do is None else (o, lse, dvec)


def attn_bwd(q, k, v, o, do, lse, tau=None, causal=False):
    """First backward: returns (dQ, dK, dV, D)."""
    ref = _check_inputs([("q", q), ("k", k), ("v", v), ("o", o), ("do", do)])
    B, H, N, d = ref.shape
    _vec_check("lse", lse, (B, H, N), ref.device)
    outs = [torch.empty_like(ref) for _ in range(3)]
    dvec = torch.empty((B, H, N), dtype=torch.float32, device=ref.device)
    _check(load_library().attn_bwd(*[_ptr(t) for t in (q, k, v, o, do, lse)], _tau(tau, d), int(bool(causal)),
                                   B, H, N, d, _DT[ref.dtype], *[_ptr(t) for t in outs], _ptr(dvec), _stream()))
    return (*outs, dvec)


def profile_start(only=None):
    """Record HIP events around every later launch (only those of kernel `only`, if given)."""
    load_library().fb_profile_start(only.encode() if only else None)


def profile_stop(max_kernels=32):
    """Per-kernel launch counts and total milliseconds since profile_start()."""
    buf = (KernelTime * max_kernels)()
    n = load_library().fb_profile_stop(buf, max_kernels)
    if n < 0:
        _check(n)
    return {buf[i].name.decode(): (buf[i].launches, buf[i].total_ms) for i in range(min(n, max_kernels))}
