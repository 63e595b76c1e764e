"""Helpers of the GPU parity tests: run the HIP path through the C ABI and the
oracle on the same seeded inputs, and compare them to the stated bars.

Bars: selected indices bit-exact; float32 workloads within 1e-4 max-abs
(outputs and state); bfloat16 workloads within 2e-2 max-abs on the float32
output of the same kernels, and on the bfloat16 output within 2e-2 plus half
a bfloat16 ulp of the reference, with relative L2 <= 1e-2; the state (float32
in both cases) within the dtype's max-abs bar; float32 scores within 1e-5
relative to max(1, |score|).
"""
from __future__ import annotations

import math
import os
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

from linear_attention_still_amd import still
from linear_attention_still_amd.inputs import Workload
from oracle import rec


def n_threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def gpu_prefill(wl: Workload, x: Dict[str, torch.Tensor], fp32_out: bool = False,
                keep_device: bool = False, flags: int = 0, partials: bool = False,
                ext_score: Optional[torch.Tensor] = None,
                out_gate: Optional[torch.Tensor] = None,
                decay: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """still_prefill (or still_prefill_partials, or still_prefill_gated) on
    the GPU; flags are the variant flags; ext_score: the caller's routing
    scores (external route), passed in the score buffer; out_gate: the
    output gate before the sigmoid, [B, Hq, L, d]; decay: the linear
    state's forget factors [Hkv] (still_prefill_decay)."""
    p = still.params_for(wl, fp32_out=fp32_out, flags=flags)
    xd = {k: v.cuda() for k, v in x.items()}
    L = xd["q"].shape[2]
    print("  gpu prefill %s L=%d fp32_out=%s flags=%d partials=%s gated=%s decay=%s"
          % (wl.name, L, fp32_out, flags, partials, out_gate is not None, decay is not None),
          flush=True)
    bufs = still.PrefillBuffers(p, L)
    if ext_score is not None:
        bufs.score.copy_(ext_score)
    out = {}
    if partials:
        B, Hq, d = wl.batch, wl.n_q_heads, wl.head_dim
        out["y_sa"] = torch.full((B, Hq, L, d), float("nan"), device="cuda")
        out["y_la"] = torch.full((B, Hq, L, d), float("nan"), device="cuda")
        out["lse_sa"] = torch.full((B, Hq, L), float("nan"), device="cuda")
        out["lse_la"] = torch.full((B, Hq, L), float("nan"), device="cuda")
        still.still_prefill_partials(p, L, xd["q"], xd["k"], xd["v"], xd["fmap_w"], xd["gate"],
                                     bufs.out, bufs.sel if bufs.sel.numel() else None,
                                     bufs.score, bufs.state, bufs.workspace, out["y_sa"],
                                     out["lse_sa"], out["y_la"], out["lse_la"])
    elif decay is not None:
        still.still_prefill_decay(p, L, xd["q"], xd["k"], xd["v"], xd["fmap_w"], xd["gate"],
                                  decay.cuda(), bufs.out, bufs.sel if bufs.sel.numel() else None,
                                  bufs.score, bufs.state, bufs.workspace)
    elif out_gate is not None:
        still.still_prefill_gated(p, L, xd["q"], xd["k"], xd["v"], xd["fmap_w"], xd["gate"],
                                  out_gate.cuda(), bufs.out, bufs.sel if bufs.sel.numel() else None,
                                  bufs.score, bufs.state, bufs.workspace)
    else:
        still.run_prefill(p, xd, bufs)
    torch.cuda.synchronize()
    out.update({"y": bufs.out, "sel": bufs.sel, "score": bufs.score})
    out.update(still.state_views(p, bufs.state))
    if keep_device:
        out["_state"] = bufs.state
        out["_params"] = p
        return out
    return {k: v.cpu() for k, v in out.items()}


def oracle(wl: Workload, x: Dict[str, torch.Tensor], units=None, merge: str = "one",
           partials: bool = False, route: str = "saliency",
           ext_score=None, decay=None) -> Dict[str, np.ndarray]:
    print("  oracle %s units=%s threads=%d merge=%s route=%s" % (
        wl.name, "all" if units is None else len(units), n_threads(), merge, route), flush=True)
    return rec.prefill(x["q"], x["k"], x["v"], x["fmap_w"], x["gate"], window=wl.window,
                       chunk=wl.chunk, budget=wl.budget, t_max=wl.t_max, units=units,
                       n_threads=n_threads(), merge=merge, partials=partials, route=route,
                       ext_score=ext_score, decay=decay)


def bf16_half_ulp(ref: np.ndarray) -> np.ndarray:
    a = np.abs(ref)
    e = np.floor(np.log2(np.maximum(a, 1e-30)))
    return np.where(a > 0, 2.0 ** (e - 8), 0.0)


def check_outputs(y_gpu: np.ndarray, y_ref: np.ndarray, dtype: str, out_fp32: bool, what=""):
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    worst = float(err.max()) if err.size else 0.0
    rel = float(np.linalg.norm(y_gpu - y_ref) / max(np.linalg.norm(y_ref), 1e-30))
    print("    %s max_abs=%.3e rel_l2=%.3e" % (what, worst, rel), flush=True)
    if dtype == "f32":
        assert worst <= 1e-4, (what, worst)
    elif out_fp32:
        assert worst <= 2e-2, (what, worst)
    else:
        bound = 2e-2 + bf16_half_ulp(y_ref)
        assert np.all(err <= bound), (what, worst)
        assert rel <= 1e-2, (what, rel)


def check_state(got: np.ndarray, ref: np.ndarray, dtype: str, what=""):
    """State (float32 in both dtypes) against the float64 oracle: the
    max-abs bar of the dtype (1e-4 float32, 2e-2 bfloat16) and its relative
    L2 bar (1e-6 float32, 1e-2 bfloat16)."""
    atol = 1e-4 if dtype == "f32" else 2e-2
    err = float(np.abs(got.astype(np.float64) - ref).max()) if ref.size else 0.0
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)) if ref.size else 0.0
    print("    %s max_abs=%.3e (|ref| max %.3g) rel_l2=%.2e"
          % (what, err, float(np.abs(ref).max()) if ref.size else 0, rel), flush=True)
    assert err <= atol, (what, err)
    assert rel <= (1e-6 if dtype == "f32" else 1e-2), (what, rel)


SCORE_RTOL = 1e-5  # float32 score vs the float64 oracle, relative to max(1, |score|)


def check_scores(got: np.ndarray, ref: np.ndarray, what="score"):
    serr = np.abs(got.astype(np.float64) - ref) / np.maximum(1.0, np.abs(ref))
    worst = float(serr.max()) if serr.size else 0.0
    print("    %s max rel err %.3e" % (what, worst), flush=True)
    assert worst <= SCORE_RTOL, (what, worst)


def unit_rows(wl: Workload, units: Sequence[Tuple[int, int]]):
    G = wl.group
    return [(b, kv * G, kv * G + G) for b, kv in units]


def compare_prefill(wl: Workload, g: Dict[str, torch.Tensor], o: Dict[str, np.ndarray],
                    units: Optional[List[Tuple[int, int]]] = None, out_fp32: bool = False,
                    check_state_too: bool = True):
    B, Hkv = wl.batch, wl.n_kv_heads
    units = [(b, kv) for b in range(B) for kv in range(Hkv)] if units is None else units
    U = len(units)
    yg = np.stack([g["y"][b, h0:h1].float().numpy() for b, h0, h1 in unit_rows(wl, units)])
    check_outputs(yg, o["y"], wl.dtype, out_fp32, "y")
    idx = [b * Hkv + kv for b, kv in units]
    # selections: bit-exact
    if o["sel"].size:
        sg = np.stack([g["sel"][b, kv].numpy() for b, kv in units])
        mism = np.argwhere(sg != o["sel"])
        assert mism.size == 0, "selection mismatch at %s" % (mism[:5].tolist(),)
    # scores: float32 evaluation vs float64
    check_scores(np.stack([g["score"][b, kv].numpy() for b, kv in units]), o["score"])
    if not check_state_too:
        return
    check_state(g["S"][idx].numpy(), o["S"], wl.dtype, "S")
    check_state(g["z"][idx].numpy(), o["z"], wl.dtype, "z")
    pend_g = g["pending"][idx].numpy()
    both_nan = np.isnan(pend_g) & np.isnan(o["pending"])
    assert np.array_equal(np.isnan(pend_g), np.isnan(o["pending"]))
    perr = np.where(both_nan, 0.0, np.abs(pend_g - o["pending"]) / np.maximum(1, np.abs(o["pending"])))
    assert float(np.nanmax(perr)) <= 1e-12, float(np.nanmax(perr))
    meta = g["meta"][idx].numpy()
    L = g["y"].shape[2]
    assert np.all(meta[:, 0] == L) and np.all(meta[:, 2] == 0)
    assert np.array_equal(meta[:, 1], o["n_pool"])
    for u in range(U):
        npool = int(o["n_pool"][u])
        flat = o["sel"][u].reshape(-1)
        flat = flat[flat >= 0][:npool]
        assert np.array_equal(g["pool_pos"][idx[u], :npool].numpy(), flat)


def run_decode(wl: Workload, state: torch.Tensor, p, x_dev: Dict[str, torch.Tensor],
               toks: Dict[str, torch.Tensor], L0: int, fp32_out: bool = False):
    """Decode len(toks) steps from position L0 on the GPU; returns outputs
    [S, B, Hq, d] and kept positions [S, B, Hkv, lam] (cpu)."""
    n = toks["q"].shape[0]
    lam = still.still_lambda(p)
    outs, sels = [], []
    odt = torch.float32 if (fp32_out or wl.dtype == "f32") else torch.bfloat16
    for s in range(n):
        out = torch.empty((wl.batch, wl.n_q_heads, wl.head_dim), dtype=odt, device="cuda")
        sel = torch.empty((wl.batch, wl.n_kv_heads, max(lam, 1)), dtype=torch.int32,
                          device="cuda")
        still.still_decode_step(p, L0 + s, toks["q"][s], toks["k"][s], toks["v"][s],
                                x_dev["fmap_w"], x_dev["gate"], state, out,
                                sel if lam > 0 else None)
        outs.append(out)
        sels.append(sel[..., :lam])
    torch.cuda.synchronize()
    return torch.stack(outs).float().cpu(), torch.stack(sels).cpu()


def concat_units(x: Dict[str, torch.Tensor], toks: Dict[str, torch.Tensor], wl: Workload,
                 units: Sequence[Tuple[int, int]]):
    """Per-unit float32 arrays of the prefill tokens followed by the decode
    tokens, in the oracle's unit layout."""
    G = wl.group
    qs, ks, vs, Fs, gs = [], [], [], [], []
    for b, kv in units:
        qp = x["q"][b, kv * G:(kv + 1) * G].float().cpu()
        qd = toks["q"][:, b, kv * G:(kv + 1) * G].float().cpu().permute(1, 0, 2)
        qs.append(torch.cat([qp, qd], dim=1).numpy())
        ks.append(torch.cat([x["k"][b, kv].float().cpu(), toks["k"][:, b, kv].float().cpu()]).numpy())
        vs.append(torch.cat([x["v"][b, kv].float().cpu(), toks["v"][:, b, kv].float().cpu()]).numpy())
        Fs.append(x["fmap_w"][kv].float().cpu().numpy())
        gs.append(x["gate"][kv * G:(kv + 1) * G].float().cpu().numpy())
    return [np.stack(a) for a in (qs, ks, vs, Fs, gs)]
