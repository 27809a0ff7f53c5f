"""Seeded synthetic workloads for PaTH attention (shared by tests, smoke, bench).

This module only draws inputs.  It holds none of the method's arithmetic: no
transition, no score, no softmax.  The distributions follow the workloads the
method is measured on:

* q, k, v ~ N(0, 1) (q, k divided by d**0.25 where stated, which folds the
  usual 1/sqrt(d) into the operands so that the scale argument is 1);
* w_t = normalize(N(0, I_d)): the unit-norm transition direction
  (reading-notes page "PaTH Attention:通过累积 Householder 变换编码位置", s2.1);
* beta_t = 2 * sigmoid(x), x ~ N(0, sigma), optionally clipped below 2
  (s2.1; clipping below 2 for bf16 stability: s5/s6 of the same page), or
  uniform in [lo, hi] for the near-reflection stress case;
* log f_t = logsigmoid(N(3, 1)) for the forget-gate variant (s2.5).

Draws are made in float32 with a seeded torch.Generator and then rounded to
the workload dtype with round-to-nearest-even; beta and log f stay float32.
A (config, tensor, variant) triple fixes the seed, so a CPU draw is
reproducible anywhere; a draw on the GPU is reproducible on one torch build.
"""
from __future__ import annotations

import dataclasses

import torch

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "w": 3, "beta": 4, "logf": 5}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    N: int
    H: int
    L: int
    d: int
    dtype: torch.dtype
    scale: float
    qk_std: float            # std of q and k entries
    beta_sigma: float = 1.0  # beta = 2 sigmoid(N(0, beta_sigma))
    beta_clip: float | None = None
    beta_uniform: tuple[float, float] | None = None
    fox: bool = False
    decode_steps: int = 0

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _cfgs():
    return {
        # tiny single head, fp32; scale 1/sqrt(d)
        "tiny": Workload("tiny", 1, 1, 1, 64, 16, torch.float32, 0.25, 1.0),
        # flip-flop-shaped layer (1 layer, 2 heads, width 64 -> head dim 32)
        "flipflop": Workload("flipflop", 2, 16, 2, 512, 32, torch.bfloat16,
                             32 ** -0.5, 1.0, beta_sigma=1.5, beta_clip=1.98),
        # LM-layer-shaped prefill at the 4096 training context
        "lm": Workload("lm", 3, 4, 24, 4096, 64, torch.bfloat16, 1.0, 64 ** -0.25),
        # PaTH-FoX prefill at the kernel-timing figure's shape (L in 2K..8K)
        "fox": Workload("fox", 4, 32, 32, 2048, 64, torch.bfloat16, 1.0,
                        64 ** -0.25, fox=True),
        # long-context prefill, then decode steps over the rewritten cache
        "long": Workload("long", 5, 1, 32, 32768, 64, torch.bfloat16, 1.0,
                         64 ** -0.25, fox=True, decode_steps=256),
    }


CONFIGS = _cfgs()


def stress(wl: Workload) -> Workload:
    """Near-reflection variant: beta uniform in [1.9, 1.99] for every token."""
    return wl.replace(name=wl.name + "-stress", beta_uniform=(1.9, 1.99))


def _gen(wl: Workload, tensor: str, variant: int, device) -> torch.Generator:
    seed = ((wl.cfg_id * 1000003 + TENSOR_IDS[tensor]) * 7919 + variant) & ((1 << 62) - 1)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def make_inputs(wl: Workload, device="cpu", variant: int = 0, L: int | None = None):
    """Draw q, k, v, w [N,H,L,d] (workload dtype) and beta, logf [N,H,L] (fp32).

    L defaults to wl.L + wl.decode_steps (prompt and decode tokens drawn as one
    sequence).  logf is None unless the workload uses the forget gate.
    """
    L = (wl.L + wl.decode_steps) if L is None else L
    shp = (wl.N, wl.H, L, wl.d)
    f32 = torch.float32

    def normal(name, std=1.0, mean=0.0, shape=shp):
        t = torch.randn(shape, generator=_gen(wl, name, variant, device),
                        dtype=f32, device=device)
        return t.mul_(std).add_(mean) if (std != 1.0 or mean != 0.0) else t

    q = normal("q", wl.qk_std).to(wl.dtype)
    k = normal("k", wl.qk_std).to(wl.dtype)
    v = normal("v").to(wl.dtype)
    w = normal("w")
    w = (w / w.norm(dim=-1, keepdim=True)).to(wl.dtype)
    if wl.beta_uniform is not None:
        lo, hi = wl.beta_uniform
        beta = torch.rand(shp[:3], generator=_gen(wl, "beta", variant, device),
                          dtype=f32, device=device) * (hi - lo) + lo
    else:
        beta = 2.0 * torch.sigmoid(normal("beta", wl.beta_sigma, shape=shp[:3]))
        if wl.beta_clip is not None:
            beta = beta.clamp_max(wl.beta_clip)
    logf = None
    if wl.fox:
        logf = torch.nn.functional.logsigmoid(normal("logf", 1.0, 3.0, shape=shp[:3]))
    return dict(q=q, k=k, v=v, w=w, beta=beta.contiguous(), logf=logf)


def as_slices_f64(t: torch.Tensor, heads=None):
    """[N,H,L,...] tensor -> float64 numpy [S,L,...] for the given flat head ids."""
    t = t.detach()
    flat = t.reshape(t.shape[0] * t.shape[1], *t.shape[2:])
    if heads is not None:
        flat = flat[torch.as_tensor(heads, dtype=torch.long, device=flat.device)]
    return flat.to("cpu", torch.float64).numpy()



def make_frontend_inputs(N, L, Dm, R, H, d, dtype=torch.bfloat16, gate=True, device="cpu",
                         seed=0):
    """Inputs of the parameter front-end: a layer input and the branch weights.

    x ~ N(0, 1) [N, L, Dm]; Wd [R, Dm] and ub, uf [H, Dm] ~ N(0, 1/Dm), so each
    projection of x is ~N(0, 1); Wu [H*d, R] ~ N(0, 1/R); conv taps kc [H*d, 3]
    ~ N(0, 1/3); bb = 0 and bf = 3, so beta = 2 sigma(N(0, 1)) and
    log f = log sigma(N(3, 1)) -- the distributions the attention workloads
    draw beta and log f from directly.  Matrices in `dtype`, kc / bb / bf fp32.
    """
    g = torch.Generator(device=device)
    g.manual_seed((0x5eed * 1000003 + seed) & ((1 << 62) - 1))
    f32 = torch.float32

    def nrm(shape, std):
        return (torch.randn(shape, generator=g, dtype=f32, device=device) * std)

    out = dict(x=nrm((N, L, Dm), 1.0).to(dtype), Wd=nrm((R, Dm), Dm ** -0.5).to(dtype),
               Wu=nrm((H * d, R), R ** -0.5).to(dtype), kc=nrm((H * d, 3), 3 ** -0.5),
               ub=nrm((H, Dm), Dm ** -0.5).to(dtype), bb=torch.zeros(H, dtype=f32, device=device))
    if gate:
        out["uf"] = nrm((H, Dm), Dm ** -0.5).to(dtype)
        out["bf"] = torch.full((H,), 3.0, dtype=f32, device=device)
    return out
