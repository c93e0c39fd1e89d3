"""Seeded synthetic inputs for exact attention: the workloads and their recipe.

This module holds no attention arithmetic. It draws Q, K, V and dO, shapes them
(scaling, rotary position embedding for the Llama-shaped layer) and rounds them
to the working dtype. Both the fp64 CPU oracle and the GPU library consume the
same rounded tensors, upcast exactly where fp64 is needed.

Recipe (one line per workload):
  * draw Q, K, V, dO in that order, each i.i.d. N(0, 1) in fp32 on the CPU from
    ``torch.Generator().manual_seed(seed)``;
  * multiply by the stated standard deviation;
  * for the Llama-shaped layer, rotate Q and K rows by rotary position
    embedding (base 10000, position = row index, pairs (x_k, x_{k+d/2})),
    evaluated in fp64;
  * round to the dtype with round-to-nearest-even (torch's ``.to``).
Tensors too large to draw on the host (``make_inputs_device``) are drawn the
same way on the GPU from ``torch.Generator(device).manual_seed(seed)``, one
tensor at a time (no rotary embedding, no scaling).

The pages' own test harness (the attention-and-matrix-product essay, section 4)
runs softmax attention on randn(1, 256, 64) with seed 42 and scale 64^-0.5;
the smallest workload below is that shape.
"""
import math
from dataclasses import dataclass, field

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "f32" | "f16" | "bf16"
    causal: bool
    backward: bool
    seed: int
    qkv_std: float = 1.0
    do_std: float = 1.0
    rope: bool = False
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return DTYPES[self.dtype]

    def fwd_flops(self) -> float:
        """4*B*H*N^2*d (two N x N x d contractions); half of it when causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def bwd_flops(self) -> float:
        """10*B*H*N^2*d (five contractions, recompute included); half if causal."""
        f = 10.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f


WORKLOADS = {
    "c1": Workload("c1", 1, 1, 256, 64, "f32", False, False, 43,
                   note="non-causal B1 H1 N256 d64 fp32, forward only"),
    "c2": Workload("c2", 2, 8, 1024, 64, "bf16", False, True, 44,
                   note="non-causal B2 H8 N1024 d64 bf16"),
    "c3": Workload("c3", 4, 32, 2048, 128, "bf16", False, True, 45,
                   note="non-causal B4 H32 N2048 d128 bf16"),
    "c4": Workload("c4", 1, 16, 8192, 64, "f16", True, True, 46, qkv_std=0.5,
                   note="causal B1 H16 N8192 d64 fp16, Q,K,V scaled by 0.5"),
    "c5": Workload("c5", 16, 32, 2048, 128, "bf16", True, True, 47, do_std=0.1,
                   rope=True,
                   note="Llama-2-7B-shaped causal layer B16 H32 N2048 d128 bf16, "
                        "rotary Q/K, dO std 0.1"),
    # Throughput sweep shapes: bf16, d=128, H=16, B*N = 16384 tokens.
    "perf-2k": Workload("perf-2k", 8, 16, 2048, 128, "bf16", False, True, 42),
    "perf-4k": Workload("perf-4k", 4, 16, 4096, 128, "bf16", False, True, 42),
    "perf-8k": Workload("perf-8k", 2, 16, 8192, 128, "bf16", False, True, 42),
    "perf-2k-causal": Workload("perf-2k-causal", 8, 16, 2048, 128, "bf16", True, True, 42),
    "perf-4k-causal": Workload("perf-4k-causal", 4, 16, 4096, 128, "bf16", True, True, 42),
    "perf-8k-causal": Workload("perf-8k-causal", 2, 16, 8192, 128, "bf16", True, True, 42),
}


def custom(name, B, H, N, d, dtype="bf16", causal=False, seed=0, **kw) -> Workload:
    """A workload of any shape (edge-case tests)."""
    return Workload(name, B, H, N, d, dtype, causal, True, seed, **kw)


def _rope_fp64(x: torch.Tensor) -> torch.Tensor:
    """Rotate-half rotary embedding over the last dim, position = row index."""
    *_, N, d = x.shape
    half = d // 2
    x = x.to(torch.float64)
    k = torch.arange(half, dtype=torch.float64)
    theta = torch.pow(torch.tensor(10000.0, dtype=torch.float64), -2.0 * k / d)
    ang = torch.arange(N, dtype=torch.float64)[:, None] * theta[None, :]
    cos, sin = torch.cos(ang), torch.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return torch.cat([a * cos - b * sin, a * sin + b * cos], dim=-1)


def make_inputs(w: Workload, with_do: bool = True) -> dict:
    """Q, K, V (and dO) as CPU tensors in w's dtype, shape [B, H, N, d]."""
    g = torch.Generator().manual_seed(w.seed)
    shape = (w.B, w.H, w.N, w.d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    do = torch.randn(shape, generator=g, dtype=torch.float32) if with_do else None
    if w.qkv_std != 1.0:
        q, k, v = q * w.qkv_std, k * w.qkv_std, v * w.qkv_std
    if do is not None and w.do_std != 1.0:
        do = do * w.do_std
    if w.rope:
        q, k = _rope_fp64(q), _rope_fp64(k)
    dt = w.torch_dtype
    out = {"q": q.to(dt).contiguous(), "k": k.to(dt).contiguous(),
           "v": v.to(dt).contiguous()}
    if do is not None:
        out["do"] = do.to(dt).contiguous()
    return out


def make_inputs_device(w: Workload, device: str = "cuda", with_do: bool = True) -> dict:
    """Q, K, V (and dO) drawn on the device, for shapes too large for the host
    path: each tensor i.i.d. N(0, 1) in fp32 in the order Q, K, V, dO, then
    rounded to w's dtype before the next is drawn."""
    if w.rope or w.qkv_std != 1.0 or w.do_std != 1.0:
        raise ValueError("device-drawn inputs take the plain N(0, 1) recipe only")
    g = torch.Generator(device=device).manual_seed(w.seed)
    shape = (w.B, w.H, w.N, w.d)
    out = {}
    for name in ("q", "k", "v", "do") if with_do else ("q", "k", "v"):
        out[name] = torch.randn(shape, generator=g, dtype=torch.float32,
                                device=device).to(w.torch_dtype)
    return out
