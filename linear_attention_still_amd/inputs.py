"""Seeded synthetic inputs and the workload registry.

This module is shared by the HIP path's tests/bench and by the oracle's
tests. It holds no arithmetic of the method itself: it only draws random
tensors and names the workloads.

Workloads stand in for the activations of one attention layer of a
Llama-3-8B-class model (32 query heads, 8 key/value heads, head dim 128),
the backbone named in the STILL articles' experiment sections. No weights
or datasets are used: every tensor is drawn from a seeded generator.

Value recipe (one reading of "N(0,1) scaled by per-token norms"):
  x = r * z,  z ~ N(0, I_d),  r ~ LogNormal(0, sigma)
drawn independently per (batch, head, position) for each of q, k, v.
A fraction of positions per batch row are outliers: r is multiplied by 8
for q, k and v of every head at those positions.
The feature-map weights are F ~ N(0, 1/d), one d x d matrix per kv head.
The gate is one scalar per query head, g ~ U(0, 1).
The draws are made in float32 and then rounded (round-to-nearest-even) to
the workload's dtype; both implementations consume the rounded tensors.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "bf16"
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    seq_len: int          # prefill length (for decode: the prefilled context)
    window: int           # W
    chunk: int            # C
    budget: int           # m
    t_max: int            # T_max (chunks the budget is spread over)
    sigma: float = 0.5    # LogNormal sigma of the per-token norms
    outlier_frac: float = 0.0
    outlier_scale: float = 8.0
    seed: int = 0
    decode_steps: int = 0  # > 0: decode workload, steps after the prefill

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _tmax(seq_len: int, chunk: int) -> int:
    return -(-seq_len // chunk)


# The five workloads. T_max = L/C (the small workload's lambda = floor(48/8)
# = 6 fixes that reading); the decode workload's window is taken equal to
# the 16K prefill's.
WORKLOADS: Dict[str, Workload] = {
    "small_f32_L256": Workload(
        "small_f32_L256", "f32", 1, 1, 1, 64, 256, 16, 32, 64, _tmax(256, 32),
        sigma=0.5, outlier_frac=0.0, seed=0),
    "gqa_bf16_L4K": Workload(
        "gqa_bf16_L4K", "bf16", 2, 32, 8, 64, 4096, 64, 64, 256, _tmax(4096, 64),
        sigma=0.5, outlier_frac=0.01, seed=1),
    "llama8b_bf16_L16K": Workload(
        "llama8b_bf16_L16K", "bf16", 1, 32, 8, 128, 16384, 64, 64, 512,
        _tmax(16384, 64), sigma=0.5, outlier_frac=0.01, seed=2),
    "decode_bf16_B64_ctx16K": Workload(
        "decode_bf16_B64_ctx16K", "bf16", 64, 32, 8, 128, 16384, 64, 64, 512,
        _tmax(16384, 64), sigma=0.5, outlier_frac=0.01, seed=3, decode_steps=64),
    "llama8b_bf16_L64K": Workload(
        "llama8b_bf16_L64K", "bf16", 1, 32, 8, 128, 65536, 128, 128, 1024,
        _tmax(65536, 128), sigma=0.75, outlier_frac=0.005, seed=4),
}


def _tokens(gen: torch.Generator, shape, sigma: float, outlier_pos,
            outlier_scale: float, device) -> torch.Tensor:
    """r * z with per-(batch, head, position) LogNormal norms r."""
    B, H, L, d = shape
    z = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    r = torch.exp(sigma * torch.randn((B, H, L, 1), generator=gen, device=device,
                                      dtype=torch.float32))
    if outlier_pos is not None:
        scale = torch.ones((B, 1, L, 1), device=device, dtype=torch.float32)
        for b in range(B):
            scale[b, 0, outlier_pos[b], 0] = outlier_scale
        r = r * scale
    return z * r


def make_inputs(wl: Workload, device="cpu", seq_len: Optional[int] = None,
                seed: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Draw q, k, v [B,H,L,d], fmap_w [Hkv,d,d] and gate [Hq] for a workload.

    The draw order is fixed (q, k, v, outlier positions per batch row, then
    fmap_w, then gate) so a (workload, seed, seq_len) triple always gives
    the same tensors on a given device type.
    """
    L = wl.seq_len if seq_len is None else seq_len
    seed = wl.seed if seed is None else seed
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    B, Hq, Hkv, d = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    n_out = int(math.ceil(wl.outlier_frac * L)) if wl.outlier_frac > 0 else 0
    out_pos = None
    if n_out > 0:
        out_pos = [torch.randperm(L, generator=gen, device=device)[:n_out]
                   for _ in range(B)]
    dt = wl.torch_dtype
    q = _tokens(gen, (B, Hq, L, d), wl.sigma, out_pos, wl.outlier_scale, device).to(dt)
    k = _tokens(gen, (B, Hkv, L, d), wl.sigma, out_pos, wl.outlier_scale, device).to(dt)
    v = _tokens(gen, (B, Hkv, L, d), wl.sigma, out_pos, wl.outlier_scale, device).to(dt)
    fmap_w = (torch.randn((Hkv, d, d), generator=gen, device=device,
                          dtype=torch.float32) / math.sqrt(d)).to(dt)
    gate = torch.rand((Hq,), generator=gen, device=device, dtype=torch.float32)
    return {"q": q.contiguous(), "k": k.contiguous(), "v": v.contiguous(),
            "fmap_w": fmap_w.contiguous(), "gate": gate.contiguous()}


def chunk_sweep(base: str = "llama8b_bf16_L16K", chunks=(16, 32, 64, 128)) -> Dict[int, Workload]:
    """The base workload at other chunk sizes C, everything else (window,
    budget, T_max, inputs) unchanged: the chunk-size ablation's axis."""
    wl = WORKLOADS[base]
    return {C: dataclasses.replace(wl, name="%s_C%d" % (base, C), chunk=C) for C in chunks}


def make_grad_output(wl: Workload, device="cpu", seq_len: Optional[int] = None,
                     seed: Optional[int] = None) -> torch.Tensor:
    """An upstream gradient dy [B,Hq,L,d] float32, N(0, 1)."""
    L = wl.seq_len if seq_len is None else seq_len
    gen = torch.Generator(device=device)
    gen.manual_seed((wl.seed if seed is None else seed) + 104729)
    return torch.randn((wl.batch, wl.n_q_heads, L, wl.head_dim), generator=gen, device=device,
                       dtype=torch.float32)


def make_route_scores(wl: Workload, device="cpu", seq_len: Optional[int] = None,
                      seed: Optional[int] = None) -> torch.Tensor:
    """Per-token routing scores [B,Hkv,L] float32, U(0, 1): the draws of
    random routing, handed to the layer as caller-supplied scores."""
    L = wl.seq_len if seq_len is None else seq_len
    gen = torch.Generator(device=device)
    gen.manual_seed((wl.seed if seed is None else seed) + 7919)
    return torch.rand((wl.batch, wl.n_kv_heads, L), generator=gen, device=device,
                      dtype=torch.float32)


def make_out_gate(wl: Workload, shape, device="cpu", seed: Optional[int] = None) -> torch.Tensor:
    """Channel-wise output gates before the sigmoid, of the given shape
    ([B,Hq,L,d] for a prefill, [B,Hq,d] or [n,B,Hq,d] for decode steps), in the
    workload's dtype: N(0, 2^2), so that the sigmoid takes values across its
    range, with one entry in 64 at +-40 (saturated open or shut)."""
    gen = torch.Generator(device=device)
    gen.manual_seed((wl.seed if seed is None else seed) + 15485863)
    g = 2.0 * torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    sat = torch.rand(shape, generator=gen, device=device) < 1.0 / 64
    sign = torch.where(torch.rand(shape, generator=gen, device=device) < 0.5, -1.0, 1.0)
    g = torch.where(sat, 40.0 * sign, g)
    return g.to(torch.bfloat16 if wl.dtype == "bf16" else torch.float32)


def make_decay(wl: Workload, device="cpu", seed: Optional[int] = None, lo: float = 0.9) -> torch.Tensor:
    """Forget factors of the linear state, one per kv head, float32,
    U(lo, 1): from a memory of ~10 tokens (0.9) to none at all (1)."""
    gen = torch.Generator(device=device)
    gen.manual_seed((wl.seed if seed is None else seed) + 32452843)
    return lo + (1.0 - lo) * torch.rand((wl.n_kv_heads,), generator=gen, device=device, dtype=torch.float32)


def make_decode_tokens(wl: Workload, n_steps: int, device="cpu",
                       seed: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """New tokens for n_steps decode steps: q [S,B,Hq,d], k/v [S,B,Hkv,d].

    Same value distribution as the prefill (no outliers), separate stream.
    """
    seed = (wl.seed if seed is None else seed) + 7919
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    B, Hq, Hkv, d = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    dt = wl.torch_dtype
    q = _tokens(gen, (n_steps * B, Hq, 1, d), wl.sigma, None, 1.0,
                device).reshape(n_steps, B, Hq, d).to(dt)
    k = _tokens(gen, (n_steps * B, Hkv, 1, d), wl.sigma, None, 1.0,
                device).reshape(n_steps, B, Hkv, d).to(dt)
    v = _tokens(gen, (n_steps * B, Hkv, 1, d), wl.sigma, None, 1.0,
                device).reshape(n_steps, B, Hkv, d).to(dt)
    return {"q": q.contiguous(), "k": k.contiguous(), "v": v.contiguous()}
