"""Double backward through the autograd integration (attn_fwd -> attn_bwd ->
bob_attention_with_stats) against the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle
import workload
from workload import to_f64

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-4, "bf16": 2e-2, "fp16": 2e-2}


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / np.linalg.norm(b))


@pytest.mark.parametrize("dtype,d,causal,N", [("fp32", 64, False, 200), ("bf16", 64, True, 300),
                                              ("bf16", 128, False, 160), ("fp16", 64, True, 257)])
def test_double_backward_matches_oracle(dtype, d, causal, N):
    import aware_flashbob_pass_amd as fb

    w = workload.custom(2, 2, N, d, dtype, causal)
    cpu = workload.make_inputs(w, 11)
    g = {k: v.cuda() for k, v in cpu.items()}
    q, k, v, do = (g[n].clone().requires_grad_(True) for n in ("Q", "K", "V", "dO"))
    o = fb.attention(q, k, v, tau=w.scale, causal=causal)
    dq, dk, dv = torch.autograd.grad(o, (q, k, v), grad_outputs=do, create_graph=True)
    s = (dq * g["UQ"]).sum() + (dk * g["UK"]).sum() + (dv * g["UV"]).sum()
    gq, gk, gv, gdo = torch.autograd.grad(s, (q, k, v, do))
    torch.cuda.synchronize()
    arrs = [to_f64(cpu[n]) for n in workload.INPUT_NAMES]
    o_ref, _ = oracle.attention_forward(*arrs[:3], w.scale, causal)
    first = oracle.first_backward(*arrs[:4], w.scale, causal)
    ref = oracle.bob(*arrs, w.scale, causal)
    tol = TOL[dtype]
    assert rel(to_f64(o.detach().cpu()), o_ref) <= tol
    for got, exp in zip((dq, dk, dv), first[:3]):
        assert rel(to_f64(got.detach().cpu()), exp) <= tol
    for got, key in zip((gq, gk, gv, gdo), ("gQ", "gK", "gV", "gdO")):
        assert rel(to_f64(got.cpu()), ref[key]) <= tol, key


def test_hessian_vector_product_is_bob():
    """A Hessian-vector product of a linear readout of attention, the quantity
    Sophia-style Hessian estimation samples, equals BoB with U = the vector."""
    import aware_flashbob_pass_amd as fb

    w = workload.custom(1, 3, 256, 64, "bf16", True)
    cpu = workload.make_inputs(w, 12)
    g = {k: v.cuda() for k, v in cpu.items()}
    q, k, v = (g[n].clone().requires_grad_(True) for n in ("Q", "K", "V"))
    loss = (fb.attention(q, k, v, tau=w.scale, causal=True) * g["dO"]).sum()
    grads = torch.autograd.grad(loss, (q, k, v), create_graph=True)
    hv = torch.autograd.grad(grads, (q, k, v), grad_outputs=(g["UQ"], g["UK"], g["UV"]))
    direct = fb.bob_attention(*[g[n] for n in workload.INPUT_NAMES], tau=w.scale, causal=True)
    torch.cuda.synchronize()
    ref = oracle.bob(*[to_f64(cpu[n]) for n in workload.INPUT_NAMES], w.scale, True)
    # the two paths differ only in D (from the rounded O here, the float32 O in bob_attention)
    for a, b, key in zip(hv, direct[:3], ("gQ", "gK", "gV")):
        assert rel(to_f64(a.cpu()), ref[key]) <= TOL["bf16"]
        assert rel(to_f64(a.cpu()), to_f64(b.cpu())) <= 5e-3


def test_hutchinson_sample_matches_oracle():
    """diag(H) sample u * (H u) with Rademacher u, through the autograd path."""
    import aware_flashbob_pass_amd as fb

    w = workload.custom(2, 2, 200, 64, "bf16", True, sigma={"V": 0.1, "dO": 0.1})
    cpu = workload.make_inputs(w, 13)
    us = [workload.rademacher((2, 2, 200, 64), 50 + i, torch.bfloat16) for i in range(3)]
    g = {k: v.cuda() for k, v in cpu.items()}
    q, k, v = (g[n].clone().requires_grad_(True) for n in ("Q", "K", "V"))
    o = fb.attention(q, k, v, tau=w.scale, causal=True)
    grads = torch.autograd.grad(o, (q, k, v), grad_outputs=g["dO"], create_graph=True)
    hu = torch.autograd.grad(grads, (q, k, v), grad_outputs=tuple(x.cuda() for x in us))
    torch.cuda.synchronize()
    arrs = [to_f64(cpu[n]) for n in ("Q", "K", "V", "dO")] + [to_f64(x) for x in us]
    ref = oracle.bob(*arrs, w.scale, True)
    for got, u, key in zip(hu, us, ("gQ", "gK", "gV")):
        est = to_f64(got.cpu()) * to_f64(u)
        assert rel(est, ref[key] * to_f64(u)) <= TOL["bf16"], key
