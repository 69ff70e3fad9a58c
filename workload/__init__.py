"""Seeded synthetic inputs for exact backward-over-backward attention.

This module only draws random tensors: it holds none of the method's arithmetic
and is shared by the tests, the smoke check and the benchmark. Both the HIP path
and the CPU oracle receive exactly the tensors drawn here (rounded to the
workload's dtype first, then upcast to float64 for the oracle).

Recipe: a CPU torch.Generator seeded with `seed` draws float32 standard normals
of shape (B, H, N, d) for Q, K, V, dO, UQ, UK, UV in that order; each is scaled
by its sigma and rounded to the workload dtype (round-to-nearest-even).
"""

import math
from dataclasses import dataclass, field

import torch

INPUT_NAMES = ("Q", "K", "V", "dO", "UQ", "UK", "UV")

_DTYPES = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str
    causal: bool
    sigma: dict = field(default_factory=dict)  # per-input scale, default 1.0
    tau: float = None  # default 1/sqrt(d)

    @property
    def scale(self):
        return self.tau if self.tau is not None else 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return _DTYPES[self.dtype]

    def describe(self):
        return (f"{self.name}: B={self.B},H={self.H},N={self.N},d={self.d},{self.dtype},"
                f"{'causal' if self.causal else 'non-causal'}")


# The five shapes that the method's evaluation covers: a tiny exactness case, the
# GPT-2-small-shaped Hessian-estimation step (12 heads of width 64, causal), a
# long single head, wide heads at long context, and the 262,144-token endpoint.
_SMALL = {n: 0.1 for n in ("V", "dO", "UQ", "UK", "UV")}
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 1, 256, 64, "fp32", False),
    "gpt2_hessian": Workload("gpt2_hessian", 8, 12, 1024, 64, "bf16", True, _SMALL),
    "long_16k": Workload("long_16k", 1, 1, 16384, 64, "bf16", False),
    "wide_64k": Workload("wide_64k", 1, 4, 65536, 128, "bf16", False),
    "endpoint_256k": Workload("endpoint_256k", 1, 1, 262144, 64, "bf16", False),
}


def make_inputs(w, seed=0):
    """Draw the seven (B, H, N, d) inputs of workload `w` on the CPU, in w's dtype."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(seed))
    out = {}
    for name in INPUT_NAMES:
        x = torch.randn((w.B, w.H, w.N, w.d), generator=gen, dtype=torch.float32)
        sig = w.sigma.get(name, 1.0)
        if sig != 1.0:
            x = x * sig
        out[name] = x.to(w.torch_dtype)
    return out


def rademacher(shape, seed, dtype=torch.float32):
    """Seeded +-1 draws (for Hutchinson probes), exact in every supported dtype."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(seed))
    return (torch.randint(0, 2, shape, generator=gen, dtype=torch.int8) * 2 - 1).to(dtype)


def custom(B, H, N, d, dtype="fp32", causal=False, sigma=None, tau=None, name="custom"):
    """A workload of any shape with the same recipe (used by parity sweeps)."""
    return Workload(name, B, H, N, d, dtype, causal, dict(sigma or {}), tau)


def to_f64(t):
    """Upcast a (rounded) torch tensor to a float64 numpy array for the oracle."""
    return t.detach().to("cpu", torch.float64).numpy()
