"""Seeded synthetic inputs for the attention forward, shared by tests and the benchmark.

This module draws random numbers and casts them; it holds none of the
attention arithmetic. Both the HIP path and the CPU oracle receive the same
host tensors from here (the oracle gets them upcast to float64, which is
exact for float32, bfloat16 and float16).

Recipe (every workload):
  * numpy ``default_rng(seed)`` (PCG64); draws in float32, in the order
    Q, K, V, then the extras below;
  * Q, K, V are iid standard normal, laid out contiguous [B, H, N, D];
  * optional per-row query scale: one factor per (b, h, i) drawn
    uniform in [1, 100), multiplied into the float32 Q row before the cast;
  * optional key padding: kv_len[b] drawn uniform from {0, ..., N}, then one
    batch, drawn uniform from {0, ..., B-1}, is set to kv_len = 0 so that
    every row of it is fully masked;
  * the float32 draws are cast to the working dtype on the CPU with torch
    (round to nearest even);
  * scale = 1/sqrt(D) rounded to float32; the same number goes to both sides.

Output gradients for the backward (``generate_grad_output``): iid standard normal
dO [B, H, N, D] from its own ``default_rng(seed)``, drawn in float32 and cast the
same way.
"""

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    D: int
    dtype: str
    causal: bool
    padding: bool = False
    q_row_scale: bool = False
    seed: int = 0

    def describe(self):
        return {"workload": self.name, "B": self.B, "H": self.H, "N": self.N, "D": self.D,
                "dtype": self.dtype, "causal": self.causal, "padding": self.padding,
                "q_row_scale": self.q_row_scale, "seed": self.seed}


# The five attention-forward workloads, named by what they are.
WORKLOADS = {
    w.name: w for w in [
        Workload("b1h1n256d64-f32-causal", 1, 1, 256, 64, "f32", True, seed=1),
        Workload("b4h16n2048d64-bf16-causal", 4, 16, 2048, 64, "bf16", True, seed=2),
        Workload("b2h32n8192d128-bf16", 2, 32, 8192, 128, "bf16", False, seed=3),
        Workload("b1h16n32768d128-bf16-causal", 1, 16, 32768, 128, "bf16", True, seed=4),
        Workload("b8h8n4096d64-f16-causal-padded", 8, 8, 4096, 64, "f16", True,
                 padding=True, q_row_scale=True, seed=5),
    ]
}

# The workload the headline throughput is quoted on.
HEADLINE = "b2h32n8192d128-bf16"


@dataclass
class Inputs:
    q: torch.Tensor            # [B, H, N, D] CPU tensor in the working dtype
    k: torch.Tensor
    v: torch.Tensor
    kv_len: Optional[np.ndarray]   # int32 [B] or None (every key valid)
    scale: float               # exactly representable in float32
    causal: bool
    meta: dict = field(default_factory=dict)


def softmax_scale(D):
    """1/sqrt(D) rounded to float32, returned as the Python float of that value."""
    return float(np.float32(1.0 / np.sqrt(np.float64(D))))


def generate(B, H, N, D, dtype, *, causal, seed, padding=False, q_row_scale=False):
    """Draw one seeded input set following the module recipe."""
    if dtype not in DTYPES:
        raise ValueError(f"unknown dtype {dtype!r}")
    rng = np.random.default_rng(seed)
    shape = (B, H, N, D)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    meta = {}
    kv_len = None
    if q_row_scale:
        factors = rng.uniform(1.0, 100.0, size=(B, H, N, 1)).astype(np.float32)
        q *= factors
    if padding:
        kv_len = rng.integers(0, N + 1, size=B).astype(np.int32)
        zero_b = int(rng.integers(0, B)) if B > 0 else -1
        if B > 0:
            kv_len[zero_b] = 0
        meta["zero_batch"] = zero_b
    t = DTYPES[dtype]
    return Inputs(q=torch.from_numpy(q).to(t), k=torch.from_numpy(k).to(t), v=torch.from_numpy(v).to(t),
                  kv_len=kv_len, scale=softmax_scale(D), causal=causal, meta=meta)


def generate_workload(w: Workload, *, seed=None):
    return generate(w.B, w.H, w.N, w.D, w.dtype, causal=w.causal, seed=w.seed if seed is None else seed,
                    padding=w.padding, q_row_scale=w.q_row_scale)


def generate_grad_output(B, H, N, D, dtype, *, seed):
    """A seeded output gradient dO [B, H, N, D] in the working dtype (CPU tensor)."""
    if dtype not in DTYPES:
        raise ValueError(f"unknown dtype {dtype!r}")
    rng = np.random.default_rng(seed)
    return torch.from_numpy(rng.standard_normal((B, H, N, D), dtype=np.float32)).to(DTYPES[dtype])


def to_f64(t):
    """Exact upcast of a CPU tensor to a float64 numpy array."""
    return t.to(torch.float64).numpy()
