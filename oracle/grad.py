"""Oracle, gradients: the backward of one STILL layer with the routing held
fixed, in float64 on the CPU.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module;
only tests/, the smoke check and the bench's CPU-baseline leg may use it.
It shares no code with the HIP path.

Pages cited (short tag -> page title):
  [P3] "STILL: Content-Aware Intra-Layer Hybrid Attention for Efficient LLM
       Linearization", sections "Delayed Chunk-Level Selection for Unified
       Training-Inference Parallelism", "Content-Aware Routing with Fixed
       Budget", "NP-Map: Norm-Preserving Feature Map"

The pages use one chunk-parallel form for training and inference [P3
"Delayed Chunk-Level Selection ..."]. Training differentiates the layer's
output y with the routing held as a constant (reading: which tokens are kept
is a discrete decision and carries no gradient; the scores that made it are
not differentiated). With the selection fixed, every query's softmax set
A(t) and linear set B(t) are fixed masks and y is an explicit function of
q, k, v, the NP-Map weights F and the gates:

    y_t = (sum_{A(t)} e^{s_tj} v_j + g sum_{B(t)} w_tj v_j)
          / (sum_{A(t)} e^{s_tj} + g sum_{B(t)} w_tj),
    s_tj = scale q_t . k_j,  w_tj = phi(q_t) . phi(k_j),

written out here with torch tensors and differentiated by torch's autograd
(a library routine). The selection comes from the brute-force oracle.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np
import torch

from oracle import bf


def np_map_t(x: torch.Tensor, F: torch.Tensor) -> torch.Tensor:
    """NP-Map of the rows of x [.., d] ([P3 "NP-Map"], the reading of the
    brute-force oracle): ||x|| * softmax(x F) / ||softmax(x F)||."""
    u = torch.softmax(x @ F, dim=-1)
    return x.norm(dim=-1, keepdim=True) * u / u.norm(dim=-1, keepdim=True)


def forward_masked(q, k, v, F, gate, A, Bm, scale):
    """y of one (batch row, kv head) unit: q [G,L,d], k, v [L,d], F [d,d],
    gate [G], A / Bm boolean [L,L] key-set masks (row = query)."""
    s = scale * (q @ k.T)                                   # [G,L,L]
    w = np_map_t(q, F) @ np_map_t(k, F).T                   # [G,L,L]
    m = s.masked_fill(~A, -math.inf).amax(-1, keepdim=True).detach()  # cancels in y
    ea = torch.exp(s - m) * A
    lw = gate[:, None, None] * w * torch.exp(-m) * Bm
    return ((ea + lw) @ v) / (ea.sum(-1, keepdim=True) + lw.sum(-1, keepdim=True))


def gradients(q, k, v, fmap_w, gate, dy, *, window: int, chunk: int, budget: int, t_max: int,
              eps: float = 1e-6, sm_scale: Optional[float] = None,
              sel: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Gradients of sum(y * dy) with respect to q [B,Hq,L,d], k, v
    [B,Hkv,L,d], fmap_w [Hkv,d,d] and gate [Hq], the selection held fixed.

    sel [B,Hkv,n_dec,lam]: the kept positions (default: the brute-force
    oracle's selection on these inputs). Returns dq, dk, dv, dfmap, dgate,
    the output y and sel.
    """
    f64 = lambda a: torch.tensor(np.asarray(a, dtype=np.float64))
    qt, kt, vt, Ft, gt = (f64(a).requires_grad_(True) for a in (q, k, v, fmap_w, gate))
    dyt = f64(dy)
    B, Hq, L, d = qt.shape
    Hkv = kt.shape[1]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d) if sm_scale is None else sm_scale
    if sel is None:
        sel = bf.prefill(q, k, v, fmap_w, gate, window=window, chunk=chunk, budget=budget,
                         t_max=t_max, eps=eps, sm_scale=sm_scale)["sel"]
    ys = []
    for b in range(B):
        rows = []
        for kv in range(Hkv):
            A, Bm = bf.key_sets(L, window, chunk, sel[b, kv].tolist())
            rows.append(forward_masked(qt[b, kv * G:(kv + 1) * G], kt[b, kv], vt[b, kv], Ft[kv],
                                       gt[kv * G:(kv + 1) * G], torch.tensor(A), torch.tensor(Bm),
                                       scale))
        ys.append(torch.cat(rows))
    y = torch.stack(ys)
    (y * dyt).sum().backward()
    g = lambda t: t.grad.detach().numpy().copy()
    return {"dq": g(qt), "dk": g(kt), "dv": g(vt), "dfmap": g(Ft), "dgate": g(gt),
            "y": y.detach().numpy(), "sel": np.asarray(sel)}
