"""Seeded synthetic inputs for the speculative-sampling verify step.

This module draws the inputs only: logit rows, draft tokens and uniforms.  It
holds none of the verify arithmetic (no softmax, no ratio, no inverse CDF), so
both the GPU path and the CPU oracle can consume its output.

Workloads (the pages measure on XSum and HumanEval with Chinchilla 70B and a 4B
draft model; neither models nor datasets are used here - these seeded logit
rows stand in for the two models' outputs):

  tiny      B=1    K=4  V=64     fp32  T=1.0  target 2*z,                     draft target + 0.5*eps
  batch1    B=1    K=4  V=32000  fp32  T=1.0  target 3*z - 1.1*ln(rank),    draft target + 0.7*eps
  small     B=64   K=4  V=32000  bf16  T=1.0  as batch1,                    draft target + 1.0*eps
  headline  B=256  K=8  V=128256 bf16  T=0.8  as batch1,                    draft target + 0.5*eps
  large     B=1024 K=16 V=256000 fp32  T=1.0  as batch1,                    draft target + s_b*eps, s_b~U[0.3,1.5]

z, eps ~ N(0,1) iid per entry; every target and draft row has fresh noise.
rank is one random permutation of 1..V per workload, shared by all rows (a
property of the vocabulary).  Values are rounded once (round-to-nearest-even)
to the storage dtype and both sides read those bytes.

Draft tokens are drawn from softmax(stored_draft / T) with the Gumbel-max
construction in float64: x = argmax_x (z_x / T - log E_x), E_x ~ Exp(1).  That
is an exact sampler for the draft distribution that never forms it.

Uniforms are (r >> 8) * 2**-24 for 32-bit random r: multiples of 2**-24 in
[0, 1), exact in fp32 and fp64.  Slot [b][t] (t < K) drives accept test t,
slot [b][K] the final (residual or bonus) draw.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    K: int
    V: int
    dtype: str            # "f32" or "bf16"
    T: float
    recipe: str           # "gauss" or "zipf"
    scale: float          # gauss: std of target logits
    sigma: float          # draft noise std (fixed)
    sigma_range: Optional[tuple] = None   # per-sequence draft noise std ~ U[lo, hi]

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def elt(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def logit_bytes(self, B: Optional[int] = None) -> int:
        B = self.B if B is None else B
        return B * (2 * self.K + 1) * self.V * self.elt


WORKLOADS = {
    "tiny": Workload("tiny", 1, 4, 64, "f32", 1.0, "gauss", 2.0, 0.5),
    "batch1": Workload("batch1", 1, 4, 32000, "f32", 1.0, "zipf", 0.0, 0.7),
    "small": Workload("small", 64, 4, 32000, "bf16", 1.0, "zipf", 0.0, 1.0),
    "headline": Workload("headline", 256, 8, 128256, "bf16", 0.8, "zipf", 0.0, 0.5),
    "large": Workload("large", 1024, 16, 256000, "f32", 1.0, "zipf", 0.0, 0.0, (0.3, 1.5)),
}


def workload(base: str, **overrides) -> Workload:
    """A named workload with fields overridden (e.g. a smaller B, another V)."""
    return dataclasses.replace(WORKLOADS[base], **overrides)


def _generator(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def uniforms_24bit(shape, g: torch.Generator, device) -> torch.Tensor:
    """(r >> 8) * 2**-24: exact float32 multiples of 2**-24 in [0, 1)."""
    r = torch.randint(0, 1 << 24, shape, generator=g, device=device, dtype=torch.int64)
    return (r.to(torch.float64) * 2.0 ** -24).to(torch.float32)


def gumbel_max_tokens(draft: torch.Tensor, T: float, g: torch.Generator) -> torch.Tensor:
    """Draw one token per row of draft [..., V] from softmax(draft / T) by the
    Gumbel-max construction in float64.  Returns int32 [...]."""
    a = draft.to(torch.float64) / T
    e = torch.empty_like(a).exponential_(generator=g)
    return torch.argmax(a - torch.log(e), dim=-1).to(torch.int32)


def make_inputs(wl: Workload | str, seed: int = 0, device="cpu", B: Optional[int] = None,
                chunk: int = 16) -> dict:
    """Generate one batch of verify inputs on `device`.

    Returns dict(target [B][K+1][V], draft [B][K][V] in the storage dtype,
    tokens [B][K] int32, uniforms [B][K+1] float32, T, workload).
    Generation runs in blocks of `chunk` sequences to bound temporary memory.
    """
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    B = wl.B if B is None else B
    K, V = wl.K, wl.V
    device = torch.device(device)
    g = _generator(device, seed)
    bias = None
    if wl.recipe == "zipf":
        rank = torch.randperm(V, generator=g, device=device).to(torch.float32) + 1.0
        bias = -1.1 * torch.log(rank)
    if wl.sigma_range is not None:
        lo, hi = wl.sigma_range
        sig = lo + (hi - lo) * torch.rand(B, generator=g, device=device, dtype=torch.float64)
        sig = sig.to(torch.float32)
    else:
        sig = torch.full((B,), wl.sigma, device=device, dtype=torch.float32)

    target = torch.empty((B, K + 1, V), dtype=wl.torch_dtype, device=device)
    draft = torch.empty((B, K, V), dtype=wl.torch_dtype, device=device)
    tokens = torch.empty((B, K), dtype=torch.int32, device=device)
    for b0 in range(0, B, chunk):
        b1 = min(B, b0 + chunk)
        n = b1 - b0
        z = torch.randn((n, K + 1, V), generator=g, device=device, dtype=torch.float32)
        if wl.recipe == "gauss":
            t32 = wl.scale * z
        else:
            t32 = 3.0 * z + bias
        del z
        eps = torch.randn((n, K, V), generator=g, device=device, dtype=torch.float32)
        d32 = t32[:, :K, :] + sig[b0:b1, None, None] * eps
        del eps
        target[b0:b1] = t32.to(wl.torch_dtype)
        draft[b0:b1] = d32.to(wl.torch_dtype)
        del t32, d32
        tokens[b0:b1] = gumbel_max_tokens(draft[b0:b1], wl.T, g)
    uniforms = uniforms_24bit((B, K + 1), g, device)
    return dict(target=target, draft=draft, tokens=tokens, uniforms=uniforms, T=wl.T,
                workload=dataclasses.replace(wl, B=B))


def to_host_arrays(inp: dict) -> dict:
    """numpy views for the CPU oracle: float32 logits, or bf16 as raw uint16 bits."""
    def logits(t: torch.Tensor):
        t = t.detach().to("cpu").contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view("uint16")
        return t.numpy()
    return dict(target=logits(inp["target"]), draft=logits(inp["draft"]),
                tokens=inp["tokens"].to("cpu").numpy(), uniforms=inp["uniforms"].to("cpu").numpy(),
                T=inp["T"])
