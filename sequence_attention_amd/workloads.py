"""Seeded synthetic inputs shaped like the DiT shard workloads.

This module only draws and shapes random tensors; it holds none of the
method's arithmetic, and both the HIP path and the fp64 oracle are fed from
it.  All draws use one CPU ``torch.Generator`` and float32 ``randn`` (then
round-to-nearest-even to bf16 where the workload is bf16), drawn in the
order Q, K, V, then any further tensors.

The shapes stand in for the pages' model workloads (FLUX.1 at 1024x1024,
Qwen-Image at 1328x1328, Wan 2.1 14B at 720p, a ring shard); no trained
weights, prompts or benchmark items are involved.  Non-causal dense
attention without RoPE makes the internal structure of a joint sequence
irrelevant, so only the lengths matter.
"""

from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    """One DiT shard workload as one rank sees it.

    Attention share: Q [B, Sq, H, D], K/V [B, Skv, H, D], the keys taken in
    ``R`` equal sequential chunks (ring hops; R = 1: one call).
    Ulysses share: sequence S over U ranks with H_total heads before the
    split (U = 1: no permutes).
    """
    name: str
    B: int
    Sq: int
    Skv: int
    H: int           # attention heads of this rank (pad heads included)
    D: int
    R: int           # K/V chunks merged in sequence (ring degree)
    S: int           # sequence covered by the Ulysses group
    H_total: int     # heads before the Ulysses split
    U: int           # Ulysses degree
    rms_qk: bool = False
    note: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def attn_flop(self) -> int:
        """Algorithmic attention FLOP of the rank's share: 4*B*H*Sq*Skv*D."""
        return 4 * self.B * self.H * self.Sq * self.Skv * self.D


WORKLOADS = {
    "tiny": Workload("tiny", B=1, Sq=256, Skv=256, H=4, D=64, R=2, S=256, H_total=4, U=2,
                     note="attention [1,256,4,64]; 2 K/V chunks of 128 merged; U=2 permutes; "
                          "CFG [2,256,256] fp32 g=4"),
    "flux": Workload("flux", B=1, Sq=4608, Skv=4608, H=12, D=128, R=1, S=4608, H_total=24, U=2,
                     rms_qk=True,
                     note="FLUX.1-like 1024x1024: 4096 image + 512 text tokens; U=2 share of 12 heads"),
    "qwen_u4": Workload("qwen_u4", B=2, Sq=7145, Skv=7145, H=6, D=128, R=1, S=7145, H_total=24, U=4,
                        note="Qwen-Image-like 1328x1328: 6889 image + 256 text, CFG pair batched; "
                             "U=4 share of 6 heads, S padded 7145 -> 7148"),
    "qwen_u5": Workload("qwen_u5", B=2, Sq=7145, Skv=7145, H=5, D=128, R=1, S=7145, H_total=24, U=5,
                        note="Qwen-Image-like, 24 heads over U=5: the last rank's 5th head is a zero pad head"),
    "ring": Workload("ring", B=1, Sq=4096, Skv=16384, H=24, D=128, R=4, S=16384, H_total=24, U=1,
                     note="ring shard of S=16384, R=4: 4096 query rows, K/V as 4 chunks of 4096"),
    "wan": Workload("wan", B=1, Sq=75600, Skv=75600, H=5, D=128, R=1, S=75600, H_total=40, U=8,
                    note="Wan-2.1-14B-like 720p: 21x45x80 latent patches; U=8 share of 5 heads; "
                         "permutes of [1,9450,40,128]"),
}


def generator(seed: int = 0) -> torch.Generator:
    return torch.Generator(device="cpu").manual_seed(seed)


def randn(shape, gen: torch.Generator, dtype=torch.bfloat16, mean: float = 0.0,
          std: float = 1.0) -> torch.Tensor:
    """float32 N(mean, std^2) on the CPU, then rounded to ``dtype``."""
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    if mean != 0.0:
        x = x + mean
    return x.to(dtype)


def rms_normalise_heads(x: torch.Tensor, eps: float = 1e-6) -> torch.Tensor:
    """Input recipe for FLUX-like Q/K (per token and head, weight 1), applied
    in float32 before the bf16 cast: x * (mean_d x^2 + eps)^(-1/2)."""
    x = x.float()
    return x * torch.rsqrt(x.pow(2).mean(dim=-1, keepdim=True) + eps)


def attention_inputs(w: Workload, seed: int = 0, dtype=torch.bfloat16, stress: str | None = None,
                     Sq: int | None = None, Skv: int | None = None, H: int | None = None):
    """Q [B,Sq,H,D], K/V [B,Skv,H,D] CPU tensors of the rank's attention share.

    stress (structured variants on the same shapes):
      "sharp"  Q scaled by 8: scores with std ~8, softmax near one-hot;
      "vmean1" V ~ N(1, 1): |O| ~ 1, so an absolute bound bites;
      "huge"   Q and K scaled by 5: scores with std ~25, reaching about +-100
               (exp without a max shift overflows float32);
      "qzero"  Q = 0: O is the mean of V and LSE = ln Skv.
    """
    Sq = w.Sq if Sq is None else Sq
    Skv = w.Skv if Skv is None else Skv
    H = w.H if H is None else H
    g = generator(seed)
    q = torch.randn(w.B, Sq, H, w.D, generator=g, dtype=torch.float32)
    k = torch.randn(w.B, Skv, H, w.D, generator=g, dtype=torch.float32)
    v = torch.randn(w.B, Skv, H, w.D, generator=g, dtype=torch.float32)
    if w.rms_qk:
        q = rms_normalise_heads(q)
        k = rms_normalise_heads(k)
    if stress == "sharp":
        q = q * 8.0
    elif stress == "vmean1":
        v = v + 1.0
    elif stress == "huge":
        q = q * 5.0
        k = k * 5.0
    elif stress == "qzero":
        q = torch.zeros_like(q)
    elif stress is not None:
        raise ValueError(f"unknown stress variant {stress!r}")
    return q.to(dtype), k.to(dtype), v.to(dtype)


def seq_sharded_planes(w: Workload, n_planes: int, S_loc: int, seed: int = 0,
                       dtype=torch.bfloat16):
    """n_planes sequence-sharded tensors [B, S_loc, H_total, D] (one rank's
    Q, K, V or O before the sequence-to-head exchange)."""
    g = generator(seed)
    return [randn((w.B, S_loc, w.H_total, w.D), g, dtype) for _ in range(n_planes)]


def cfg_inputs(shape=(2, 256, 256), seed: int = 0, dtype=torch.float32):
    """Stacked [uncond; cond] predictions for the CFG combine."""
    g = generator(seed)
    return randn(shape, g, dtype)


def rope_tables(S: int, D: int, base: float = 10000.0):
    """cos / sin tables [S, D/2] float32 of the one-axis rotary schedule
    angle(t, i) = t * base^(-2i/D), computed in float64 and rounded once.
    (Image and video tokens use per-axis schedules; those are different
    table contents for the same kernel.)"""
    t = torch.arange(S, dtype=torch.float64)[:, None]
    i = torch.arange(D // 2, dtype=torch.float64)[None, :]
    ang = t * torch.pow(torch.tensor(base, dtype=torch.float64), -2.0 * i / D)
    return torch.cos(ang).to(torch.float32), torch.sin(ang).to(torch.float32)
