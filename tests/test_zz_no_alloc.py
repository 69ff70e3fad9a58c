"""bob_attention_noalloc (the entry point that allocates nothing: its workspace is the
library's fixed device array) against bob_attention_ws with a torch-allocated
workspace, through the C ABI: two calls in a row, the second on a smaller input,
then a shape beyond the array's maximum, which must be refused with nothing launched."""

import ctypes

import pytest
import torch

import workload

pytestmark = pytest.mark.gpu

FB_ERR_WORKSPACE = -5


def _case(fb, w, seed):
    cpu = workload.make_inputs(w, seed)
    g = [cpu[n].cuda() for n in workload.INPUT_NAMES]
    ref = fb.bob_attention(*g, tau=w.scale, causal=w.causal)  # bob_attention_ws, torch workspace
    got = fb.bob_attention_noalloc(*g, tau=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    for name, a, b in zip(("gQ", "gK", "gV", "gdO"), got, ref):
        assert torch.isfinite(a).all(), name
        # same kernels, same split choice: the outputs are bitwise equal
        assert torch.equal(a, b), (name, w.describe())


def test_noalloc_matches_ws_twice_second_smaller():
    import aware_flashbob_pass_amd as fb

    fb.load_library()
    big = workload.custom(1, 1, 16384, 64, "bf16", False, name="noalloc_big")
    assert fb.workspace_bytes(1, 1, 16384, 64, torch.bfloat16) <= 64 << 20
    print(f"noalloc: {big.describe()}", flush=True)
    _case(fb, big, 0)
    small = workload.custom(2, 3, 700, 64, "bf16", True, name="noalloc_small")
    print(f"noalloc: {small.describe()}", flush=True)
    _case(fb, small, 1)


def test_noalloc_other_shapes():
    import aware_flashbob_pass_amd as fb

    fb.load_library()
    for w in (workload.custom(1, 2, 900, 128, "fp16", False), workload.custom(1, 1, 300, 64, "fp32", True),
              workload.WORKLOADS["gpt2_hessian"]):
        print(f"noalloc: {w.describe()}", flush=True)
        _case(fb, w, 2)


def test_noalloc_refuses_shape_beyond_scratch():
    import aware_flashbob_pass_amd as fb
    from aware_flashbob_pass_amd.binding import FB_BF16

    lib = fb.load_library()
    B, H, N, d = 1, 2, 1 << 20, 64
    assert lib.bob_workspace_bytes(B, H, N, d, FB_BF16) > 64 << 20
    bufs = [torch.zeros(1024, dtype=torch.bfloat16, device="cuda") for _ in range(11)]
    ptrs = [ctypes.c_void_p(t.data_ptr()) for t in bufs]
    st = lib.bob_attention_noalloc(*ptrs[:7], 0.125, 0, B, H, N, d, FB_BF16, *ptrs[7:],
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == FB_ERR_WORKSPACE
    assert b"maximum" in lib.fb_last_error()
    torch.cuda.synchronize()
    assert not any(t.any() for t in bufs[7:])
