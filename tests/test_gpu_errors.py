"""Error paths of the allocating entry points on a real device.

bob_attention refuses a workspace larger than the device's free memory with
FB_ERR_OOM before it allocates or launches anything, so the input pointers of
the call below (small real buffers standing for a far larger shape) are never
read: the test checks first, on the host, that the workspace the shape needs
exceeds the device's total memory."""

import ctypes

import pytest
import torch

pytestmark = pytest.mark.gpu

FB_ERR_OOM = -6


def test_bob_attention_oom_when_workspace_exceeds_device_memory():
    import aware_flashbob_pass_amd as fb
    from aware_flashbob_pass_amd.binding import FB_BF16

    lib = fb.load_library()
    B, H, N, d = 65535, 1, 32767, 64  # B*H*N just inside the shape bound
    need = int(lib.bob_workspace_bytes(B, H, N, d, FB_BF16))
    free_b, total_b = torch.cuda.mem_get_info()
    print(f"workspace {need} bytes, device total {total_b}, free {free_b}", flush=True)
    assert need > total_b  # the library must refuse it before allocating
    bufs = [torch.zeros(4096, dtype=torch.bfloat16, device="cuda") for _ in range(11)]
    ptrs = [ctypes.c_void_p(t.data_ptr()) for t in bufs]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = lib.bob_attention(*ptrs[:7], 0.125, 0, B, H, N, d, FB_BF16, *ptrs[7:], stream)
    assert st == FB_ERR_OOM
    assert b"free on the device" in lib.fb_last_error()
    torch.cuda.synchronize()
    for t in bufs:
        assert not t.any()  # nothing was written
    # the library still works after the refusal
    import workload
    w = workload.custom(1, 1, 100, 64, "bf16", False)
    cpu = workload.make_inputs(w, 0)
    g = [cpu[n].cuda() for n in workload.INPUT_NAMES]
    out = fb.bob_attention_alloc(*g, tau=w.scale)
    torch.cuda.synchronize()
    assert all(torch.isfinite(o).all() for o in out)
