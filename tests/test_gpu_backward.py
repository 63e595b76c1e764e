"""Parity of the backward (through the C ABI) with the gradient oracle, on
the GPU: gradients of sum(y * dy) with respect to q, k, v, the NP-Map
weights and the gates, the routing held fixed (the forward's selection).

Two checks per shape:
  * the backward alone, fed the oracle's float64 output and branch
    log-normalisers (rounded to float32): its own float32 arithmetic, bar
    1e-4 of the largest gradient entry (float32 data) or 2e-3 (bf16 data:
    the features are float32 either way; the bar covers the float32 sums
    over up to L keys of bf16-sized terms), floors of 1 on the scales;
  * forward and backward chained on the GPU (the forward's float32 output,
    partials and selection): bar 1e-3 (float32) / 2e-2 (bf16) of the largest
    entry, relative L2 1e-4 / 1e-2 (the forward's own output error enters
    delta = dy . y).
Inputs: the workload generator's q, k, v, F, gates; dy ~ N(0, 1), seeded.
"""
import numpy as np
import pytest
import torch

from linear_attention_still_amd import still
from linear_attention_still_amd.inputs import Workload, make_grad_output, make_inputs
from oracle import bf, grad

pytestmark = pytest.mark.gpu


def small(name, dtype, B, Hq, Hkv, d, L, W, C, m, t_max, out=0.01, seed=41):
    return Workload(name, dtype, B, Hq, Hkv, d, L, W, C, m, t_max, sigma=0.5,
                    outlier_frac=out, seed=seed)


SHAPES = [
    small("bw_f32_gqa", "f32", 2, 4, 2, 64, 150, 16, 32, 16 + 3 * 4, 4, out=0.0),
    small("bw_bf16_d128", "bf16", 1, 8, 2, 128, 200, 32, 32, 32 + 4 * 6, 6),
    small("bw_bf16_C16_W8", "bf16", 1, 2, 1, 64, 130, 8, 16, 8 + 7 * 2, 7),
    small("bw_bf16_G1_lam0", "bf16", 2, 2, 2, 64, 97, 16, 32, 16, 5),
    small("bw_bf16_one_token", "bf16", 1, 4, 1, 64, 1, 16, 32, 48, 2),
    # many tiles of both kernels and a ragged tail, the 16K workload's head shape
    small("bw_bf16_L777_d128", "bf16", 1, 8, 2, 128, 777, 64, 64, 64 + 16 * 3, 16),
]
NAMES = ["dq", "dk", "dv", "dfmap", "dgate"]


def gpu_backward(wl, x, sel, y, lse_sa, lse_la, dy):
    p = still.params_for(wl, fp32_out=True)
    L = x["q"].shape[2]
    xd = {k: v.cuda() for k, v in x.items()}
    B, Hq, Hkv, d = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    out = {"dq": torch.full((B, Hq, L, d), float("nan"), device="cuda"),
           "dk": torch.full((B, Hkv, L, d), float("nan"), device="cuda"),
           "dv": torch.full((B, Hkv, L, d), float("nan"), device="cuda"),
           "dfmap": torch.full((Hkv, d, d), float("nan"), device="cuda"),
           "dgate": torch.full((Hq,), float("nan"), device="cuda")}
    ws = torch.empty(still.still_backward_workspace_bytes(p, L), dtype=torch.uint8, device="cuda")
    print("  gpu backward %s L=%d" % (wl.name, L), flush=True)
    still.still_backward(p, L, xd["q"], xd["k"], xd["v"], xd["fmap_w"], xd["gate"],
                         sel.cuda() if sel.numel() else None, y.cuda(), lse_sa.cuda(),
                         lse_la.cuda(), dy.cuda(), out["dq"], out["dk"], out["dv"], out["dfmap"],
                         out["dgate"], ws)
    torch.cuda.synchronize()
    return {k: v.cpu().double().numpy() for k, v in out.items()}


def check(got, ref, max_rel, l2_rel, what):
    for n in NAMES:
        err = np.abs(got[n] - ref[n])
        # floors of 1: a gradient that is exactly 0 (e.g. dq of a lone
        # token, whose output does not depend on q) is met to rounding
        scale = max(float(np.abs(ref[n]).max()), 1.0)
        l2 = float(np.linalg.norm(got[n] - ref[n]) / max(np.linalg.norm(ref[n]), 1.0))
        print("    %s %s max_abs=%.3e (|ref| max %.3g) rel_l2=%.2e"
              % (what, n, float(err.max()), scale, l2), flush=True)
        assert np.all(np.isfinite(got[n])), (what, n)
        assert float(err.max()) <= max_rel * scale, (what, n, float(err.max()), scale)
        assert l2 <= l2_rel, (what, n, l2)


@pytest.mark.parametrize("wl", SHAPES, ids=[w.name for w in SHAPES])
def test_backward_alone_on_oracle_activations(wl):
    x = make_inputs(wl)
    dy = make_grad_output(wl)
    kw = dict(window=wl.window, chunk=wl.chunk, budget=wl.budget, t_max=wl.t_max)
    x64 = {k: v.double().numpy() for k, v in x.items()}
    f = bf.prefill(x64["q"], x64["k"], x64["v"], x64["fmap_w"], x64["gate"], partials=True, **kw)
    ref = grad.gradients(x64["q"], x64["k"], x64["v"], x64["fmap_w"], x64["gate"],
                         dy.double().numpy(), sel=f["sel"], **kw)
    sel = torch.tensor(f["sel"], dtype=torch.int32)
    got = gpu_backward(wl, x, sel, torch.tensor(f["y"], dtype=torch.float32),
                       torch.tensor(f["lse_sa"], dtype=torch.float32),
                       torch.tensor(f["lse_la"], dtype=torch.float32), dy)
    bar = 1e-4 if wl.dtype == "f32" else 2e-3
    check(got, ref, bar, bar, "alone")


@pytest.mark.parametrize("wl", SHAPES[:3], ids=[w.name for w in SHAPES[:3]])
def test_forward_then_backward_on_gpu(wl):
    x = make_inputs(wl)
    dy = make_grad_output(wl)
    L = wl.seq_len
    p = still.params_for(wl, fp32_out=True)
    xd = {k: v.cuda() for k, v in x.items()}
    bufs = still.PrefillBuffers(p, L)
    B, Hq = wl.batch, wl.n_q_heads
    part = {"y_sa": torch.empty((B, Hq, L, wl.head_dim), device="cuda"),
            "y_la": torch.empty((B, Hq, L, wl.head_dim), device="cuda"),
            "lse_sa": torch.empty((B, Hq, L), device="cuda"),
            "lse_la": torch.empty((B, Hq, L), device="cuda")}
    still.still_prefill_partials(p, L, xd["q"], xd["k"], xd["v"], xd["fmap_w"], xd["gate"], bufs.out,
                                 bufs.sel if bufs.sel.numel() else None, bufs.score, bufs.state,
                                 bufs.workspace, part["y_sa"], part["lse_sa"], part["y_la"],
                                 part["lse_la"])
    torch.cuda.synchronize()
    got = gpu_backward(wl, x, bufs.sel.cpu(), bufs.out.cpu(), part["lse_sa"].cpu(),
                       part["lse_la"].cpu(), dy)
    ref = grad.gradients(x["q"].double().numpy(), x["k"].double().numpy(), x["v"].double().numpy(),
                         x["fmap_w"].double().numpy(), x["gate"].double().numpy(), dy.double().numpy(),
                         sel=bufs.sel.cpu().numpy(), window=wl.window, chunk=wl.chunk,
                         budget=wl.budget, t_max=wl.t_max)
    if wl.dtype == "f32":
        check(got, ref, 1e-3, 1e-4, "chained")
    else:
        check(got, ref, 2e-2, 1e-2, "chained")
