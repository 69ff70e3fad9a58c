"""Range of the statistics kernel's 16-bit weight operands (CPU emulation).

The statistics kernel (csrc/attn_fwd.hip) forms each 32-key step's softmax
weights 2^(s - m) against a reference maximum m that it moves only when some
lane's sum of the step's weights reaches a limit (or is not finite); the weights
then become matrix-core operands in the input dtype. For fp16 every weight must
stay below 65504, the largest finite fp16 value, or O, D and every output of the
head turn to inf/NaN.

This test replays that rule on the CPU, wave by wave, with the kernel's lane
layout (lane (n, g) holds query n and keys kappa(r, g) of the step), on inputs
whose row maxima creep up over the keys and then jump (the same recipe as the
GPU test of the statistics kernel). It reads the limits from the kernel source,
checks that the fp16 limit keeps every weight finite in fp16, and checks that
the float32-range limit (the bf16 one) would not, so the emulation can tell the
two apart.
"""

import math
import os
import re

import numpy as np
import pytest
import torch

import workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "aware_flashbob_pass_amd", "csrc", "attn_fwd.hip")
FP16_MAX = 65504.0
LOG2E = 1.4426950408889634


def kernel_limits():
    """(fp16 limit, other limit) as written in lazy_limit<TT>() of the kernel source."""
    text = open(SRC).read()
    m = re.search(r"is_same_v<TT,\s*F16>\s*\?\s*([0-9.eE+]+)f\s*:\s*([0-9.eE+]+)f", text)
    assert m, "lazy_limit<TT>() not found in attn_fwd.hip"
    return float(m.group(1)), float(m.group(2))


def kappa(r, g):
    return ((r >> 2) << 3) + (g << 2) + (r & 3)


def peaked_inputs(d, causal, dtype="fp16", N=1000):
    w = workload.custom(1, 2, N, d, dtype, causal)
    cpu = workload.make_inputs(w, 11)
    k = cpu["K"].float() * torch.linspace(0.5, 3.0, N).view(1, 1, N, 1)
    k[:, :, N - 40:N - 30, :] *= 4.0
    cpu["K"] = k.to(cpu["K"].dtype)
    return w, cpu


def max_weight(q, k, tau, causal, limit, nsplit=1):
    """Largest weight any lane hands to the matrix cores, replaying the kernel's
    lazy rescale rule (scores in float32 from the rounded inputs)."""
    N = q.shape[0]
    cs = np.float32(tau * LOG2E)
    rows_pad = -(-N // 32) * 32
    qp = np.zeros((rows_pad, q.shape[1]), dtype=np.float32)
    qp[:N] = q  # rows past N have zero operands in the kernel: scores 0, never stored
    s_all = (qp @ k.astype(np.float32).T).astype(np.float32)
    keys_of_lane = np.array([[kappa(r, g) for r in range(16)] for g in range(2)])  # [g][r]
    worst = 0.0
    nkt_all = (N + 31) // 32
    for q0 in range(0, N, 32):
        rows = np.arange(q0, q0 + 32)
        nkt = min(nkt_all, (q0 // 128 + 1) * 4) if causal else nkt_all
        for sp in range(nsplit):
            kb, ke = sp * nkt // nsplit, (sp + 1) * nkt // nsplit
            m = np.full(32, -1e30, dtype=np.float32)
            for kt in range(kb, ke):
                k0 = kt * 32
                if causal and k0 > q0 + 31:
                    continue
                sc = np.empty((32, 2, 16), dtype=np.float32)
                for g in range(2):
                    kk = k0 + keys_of_lane[g]
                    ok = np.broadcast_to(kk[None, :] < N, (32, 16))
                    if causal:
                        ok = ok & (kk[None, :] <= rows[:, None])
                    sc[:, g, :] = np.where(ok, s_all[rows][:, np.minimum(kk, N - 1)], -np.inf)

                def weights(mref):
                    with np.errstate(over="ignore", invalid="ignore"):
                        return np.exp2(sc.astype(np.float64) * cs - mref[:, None, None].astype(np.float64))

                p = weights(m)
                lsum = p.sum(axis=2)  # per lane
                if np.any(~(lsum < limit)):
                    mx = np.max(sc, axis=(1, 2)) * cs  # pair maximum: the row's step maximum
                    m = np.maximum(m, mx.astype(np.float32))
                    p = weights(m)
                worst = max(worst, float(np.max(p)))
    return worst


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_fp16_weights_stay_finite(d, causal):
    lim16, lim_other = kernel_limits()
    assert lim16 < FP16_MAX and lim_other >= lim16
    w, cpu = peaked_inputs(d, causal)
    for bh in range(w.B * w.H):
        q = cpu["Q"][0, bh].float().numpy()
        k = cpu["K"][0, bh].float().numpy()
        for nsplit in (1, 8):
            assert max_weight(q, k, w.scale, causal, lim16, nsplit) < FP16_MAX


def test_float32_range_limit_would_overflow_fp16():
    """The rule with the bf16 limit on the same fp16 inputs produces weights that
    fp16 cannot hold: the emulation distinguishes the two limits."""
    _, lim_other = kernel_limits()
    w, cpu = peaked_inputs(64, False)
    worst = max(max_weight(cpu["Q"][0, bh].float().numpy(), cpu["K"][0, bh].float().numpy(), w.scale, False,
                           lim_other) for bh in range(2))
    assert worst > FP16_MAX
    assert math.isfinite(worst)
