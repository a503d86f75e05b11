"""Seeded synthetic workloads for the latent-attention forward path.

This module is shared by the CPU oracle and by the GPU path's tests and
benchmark. It holds shapes, rotary settings given as plain data, and a seeded
random generator. It holds none of the method's arithmetic: no normalisation,
no projection, no rotary frequencies, no attention and no softmax scale.

Shapes and distributions follow the five workloads the project measures:
a tiny prefill, a Kimi-K2-shape prefill at 1k and at 8k tokens, a GLM-5-style
prefill, and a Kimi-K2-shape decode step against an expanded cache. The
tensor roles follow the pages: the query split into a non-rotary and a rotary
part (Kimi-K2 "Query content heads", section "Split content heads"), the
compressed latent and the single rotary key shared by all heads (first page,
"Original context"; GLM-5 "Normalized key-value latent", section "Key-value
compression"), the latent RMSNorm gain and the kv_b_proj weight stored as an
nn.Linear weight of shape [H*(Dn+Dv), R].

Two block workloads start one step earlier, at the hidden states of the
attention block: the query comes from the low-rank query projections with
their RMSNorm, the latent and the shared rotary key from the joint
key-value down-projection, and an output projection follows (Kimi-K2
"Query content heads", the MLA constructor). The hidden size and query rank
are not on the pages; the Kimi-K2 one uses Kimi-K2's published 7168 and
1536, the tiny one 128 and 64; no projection has a bias.

Two further decode workloads (a tiny one and a Kimi-K2-shape one) keep a
compressed-latent cache instead of the expanded one: per token the
normalised latent followed by the rotated shared rotary key (GLM-5
"Normalized key-value latent", section "KV cache"), stored as float16, the
type the latent RMSNorm writes.

Distribution notation N(mu, s2) is read as mean and variance. The RMSNorm
gain 1 + N(0, 0.1) is given for the tiny workload only and is reused for the
others. Draw order per workload: q, latent, k_pe, gain, W, then (decode) the K
cache and the V cache, or the latent cache. Every draw is a float32 standard
normal from a CPU torch.Generator seeded with the workload's seed, scaled,
then rounded to bfloat16 (round to nearest even); the latent cache's draws
are rounded to float16 instead.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class RopeSpec:
    """Rotary settings as plain data (the `rope_scaling` dictionary and base of
    the Kimi-K2 "RoPE coefficients" page, section "Generate RoPE coefficients")."""

    kind: str  # "default" or "yarn"
    base: float
    factor: float = 1.0
    original_max_pos: int = 4096
    beta_fast: float = 32.0
    beta_slow: float = 1.0
    mscale: float = 1.0
    mscale_all_dim: float = 0.0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int  # query tokens per sequence (1 for decode)
    H: int
    R: int  # kv_lora_rank
    Dn: int  # qk_nope_head_dim
    Dr: int  # qk_rope_head_dim
    Dv: int  # v_head_dim
    rope: RopeSpec
    pairing: str  # "half" or "interleaved"
    seed: int
    eps: float = 1e-6
    decode: bool = False
    cache_len: int = 0  # decode: number of cached rows including the new one
    q_pos: int = 0  # decode: position of the new token
    latent_cache: bool = False  # decode: the cache holds latents, not expanded keys/values
    hidden: int = 0  # whole MLA block: hidden size (0: the inputs start at q / latent / k_pe)
    q_lora: int = 0  # whole MLA block: rank of the query down-projection

    @property
    def Dqk(self) -> int:
        return self.Dn + self.Dr

    @property
    def table_len(self) -> int:
        """Rows of the cos/sin table the workload needs (positions 0..max)."""
        return self.cache_len if self.decode else self.T


YARN_KIMI = RopeSpec(kind="yarn", base=50000.0, factor=32.0, original_max_pos=4096,
                     beta_fast=32.0, beta_slow=1.0, mscale=1.0, mscale_all_dim=1.0)

WORKLOADS = {
    "tiny": Workload("tiny", B=1, T=32, H=4, R=64, Dn=32, Dr=16, Dv=32,
                     rope=RopeSpec(kind="default", base=10000.0), pairing="half", seed=0),
    "kimi_k2_1k": Workload("kimi_k2_1k", B=1, T=1024, H=64, R=512, Dn=128, Dr=64, Dv=128,
                           rope=YARN_KIMI, pairing="half", seed=1),
    "kimi_k2_8k": Workload("kimi_k2_8k", B=2, T=8192, H=64, R=512, Dn=128, Dr=64, Dv=128,
                           rope=YARN_KIMI, pairing="half", seed=2),
    "glm5_4k": Workload("glm5_4k", B=1, T=4096, H=64, R=512, Dn=192, Dr=64, Dv=256,
                        rope=RopeSpec(kind="default", base=10000.0), pairing="interleaved", seed=3),
    "kimi_k2_decode": Workload("kimi_k2_decode", B=32, T=1, H=64, R=512, Dn=128, Dr=64, Dv=128,
                               rope=YARN_KIMI, pairing="half", seed=4, decode=True,
                               cache_len=1001, q_pos=1000),
    "tiny_decode_latent": Workload("tiny_decode_latent", B=3, T=1, H=4, R=64, Dn=32, Dr=16, Dv=32,
                                   rope=RopeSpec(kind="default", base=10000.0), pairing="half", seed=6,
                                   decode=True, cache_len=37, q_pos=36, latent_cache=True),
    "kimi_k2_decode_latent": Workload("kimi_k2_decode_latent", B=32, T=1, H=64, R=512, Dn=128, Dr=64, Dv=128,
                                      rope=YARN_KIMI, pairing="half", seed=5, decode=True,
                                      cache_len=1001, q_pos=1000, latent_cache=True),
    "tiny_block": Workload("tiny_block", B=2, T=40, H=4, R=64, Dn=32, Dr=16, Dv=32,
                           rope=RopeSpec(kind="default", base=10000.0), pairing="half", seed=8, hidden=128, q_lora=64),
    "kimi_k2_block_1k": Workload("kimi_k2_block_1k", B=1, T=1024, H=64, R=512, Dn=128, Dr=64, Dv=128,
                                 rope=YARN_KIMI, pairing="half", seed=9, hidden=7168, q_lora=1536),
}

ORDER = ["tiny", "kimi_k2_1k", "kimi_k2_8k", "glm5_4k", "kimi_k2_decode"]


def custom(name: str = "custom", **kw) -> Workload:
    """A workload with arbitrary sizes (tests use it for ragged shapes)."""
    base = dict(B=1, T=8, H=2, R=32, Dn=16, Dr=8, Dv=16,
                rope=RopeSpec(kind="default", base=10000.0), pairing="half", seed=0)
    base.update(kw)
    return Workload(name, **base)


def _normal(gen: torch.Generator, shape, std: float = 1.0, mean: float = 0.0) -> torch.Tensor:
    x = torch.randn(*shape, generator=gen, dtype=torch.float32, device=gen.device)
    if std != 1.0:
        x = x * std
    if mean != 0.0:
        x = x + mean
    return x.to(torch.bfloat16)


def make_inputs(w: Workload, with_cache: bool = True, device: str = "cpu") -> dict:
    """Draw the workload's bf16 inputs on `device` (default the CPU).

    The recipe is the same on every device; a GPU generator gives a different
    (equally seeded) random stream from the CPU one, so tests that compare
    with the oracle draw on the CPU, while benchmarks may draw on the GPU.

    Returns a dict of bf16 tensors on `device`:
      q      [B, H, T, Dn+Dr]   query, rotary part not yet rotated
      latent [B, T, R]          compressed key-value latent (before RMSNorm)
      k_pe   [B, T, Dr]         shared rotary key, not yet rotated
      gain   [R]                latent RMSNorm weight
      W      [H*(Dn+Dv), R]     kv_b_proj weight (nn.Linear layout)
    and for a decode workload, also
      k_cache [B, H, L, Dn+Dr]  expanded key cache, rotary part already rotated
      v_cache [B, H, L, Dv]     expanded value cache
    or, for a latent-cache decode workload,
      latent_cache [B, L, R+Dr] float16: normalised latent, then the rotated
                                shared rotary key
    where the new token's row (slot q_pos) of the cache(s) is the one the
    decode step overwrites.
    """
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)
    if w.hidden:
        # block workload: hidden states and the five projection weights
        # (nn.Linear layout, std 1/sqrt(fan_in)) with the two RMSNorm gains
        return {
            "hidden": _normal(gen, (w.B, w.T, w.hidden)),
            "W_qa": _normal(gen, (w.q_lora, w.hidden), std=1.0 / math.sqrt(w.hidden)),
            "gain_q": _normal(gen, (w.q_lora,), std=math.sqrt(0.1), mean=1.0),
            "W_qb": _normal(gen, (w.H * w.Dqk, w.q_lora), std=1.0 / math.sqrt(w.q_lora)),
            "W_kva": _normal(gen, (w.R + w.Dr, w.hidden), std=1.0 / math.sqrt(w.hidden)),
            "gain": _normal(gen, (w.R,), std=math.sqrt(0.1), mean=1.0),
            "W": _normal(gen, (w.H * (w.Dn + w.Dv), w.R), std=1.0 / math.sqrt(w.R)),
            "W_o": _normal(gen, (w.hidden, w.H * w.Dv), std=1.0 / math.sqrt(w.H * w.Dv)),
        }
    out = {
        "q": _normal(gen, (w.B, w.H, w.T, w.Dqk)),
        "latent": _normal(gen, (w.B, w.T, w.R)),
        "k_pe": _normal(gen, (w.B, w.T, w.Dr)),
        "gain": _normal(gen, (w.R,), std=math.sqrt(0.1), mean=1.0),
        "W": _normal(gen, (w.H * (w.Dn + w.Dv), w.R), std=1.0 / math.sqrt(w.R)),
    }
    if w.decode and with_cache and w.latent_cache:
        x = torch.randn(w.B, w.cache_len, w.R + w.Dr, generator=gen, dtype=torch.float32, device=gen.device)
        out["latent_cache"] = x.to(torch.float16)
    elif w.decode and with_cache:
        out["k_cache"] = _normal(gen, (w.B, w.H, w.cache_len, w.Dqk))
        out["v_cache"] = _normal(gen, (w.B, w.H, w.cache_len, w.Dv))
    return out


def positions(w: Workload, device: Optional[str] = None) -> torch.Tensor:
    """Token positions [B, T] int32: 0..T-1 for prefill, q_pos for decode."""
    if w.decode:
        p = torch.full((w.B, 1), w.q_pos, dtype=torch.int32)
    else:
        p = torch.arange(w.T, dtype=torch.int32).unsqueeze(0).expand(w.B, w.T).contiguous()
    return p if device is None else p.to(device)
