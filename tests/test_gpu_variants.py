"""Parity of the branch variants, the branch partials and the routing
metrics with the oracle, on the GPU (through the C ABI).

The variants are the ablation axes the pages discuss: the softmax branch
alone (unkept tokens dropped, the sparse-attention-only alternative of the
STILL article, "Problems with Existing Intra-Layer Hybrid Attention"), the
sum of separately normalised branches (the hybrid-architecture survey, §4
on gating) and the default single normaliser. The partials are the two
branches apart: each normalised output and the natural log of its
normaliser, the linear one without the gate.

Bars: those of the default path (tests/_parity.py) for the outputs, the
selections, scores and state; the branch outputs (float32) within the
dtype's float32-output bar; the log-normalisers within the dtype's max-abs
bar (1e-4 float32, 2e-2 bfloat16: a relative bar on the normaliser), with
-inf exactly where the linear key set is empty.

The routing metrics are the alternatives of the STILL article's routing
ablation ("Ablation Studies"): diagonal attention weight, q.k, key norm,
uniform picks, and caller-supplied scores (random routing's draws, seeded
U(0, 1)); selections bit-exact, scores within the score bar.

The output gate is the channel-wise sigmoid gate of the hybrid-architecture
survey (§4, gating): the entries still_prefill_gated and
still_decode_step_gated against the oracle's output times the sigmoid of the
same seeded gates; the bars of the ungated outputs (the sigmoid lies in
[0, 1], so it shrinks the error with the output).

The forget gate of the linear state (the survey's §2 gated linear
attention, write strength 1): still_prefill_decay and
still_decode_step_decay against the oracle with the same float32 factors
per kv head (seeded U(0.9, 1)); the default path's bars for outputs,
selections, scores and state.
"""
import numpy as np
import pytest
import torch

from linear_attention_still_amd import still
from linear_attention_still_amd.inputs import (WORKLOADS, Workload, make_decay, make_decode_tokens,
                                               make_inputs, make_out_gate, make_route_scores)
from oracle import bf, rec
from tests import _parity as P

pytestmark = pytest.mark.gpu


def small(name, dtype, B, Hq, Hkv, d, L, W, C, m, t_max, out=0.01, seed=13):
    return Workload(name, dtype, B, Hq, Hkv, d, L, W, C, m, t_max, sigma=0.5,
                    outlier_frac=out, seed=seed)


SHAPES = [
    small("f32_gqa_ragged", "f32", 2, 4, 2, 64, 333, 40, 64, 40 + 6 * 3, 6, out=0.0),
    small("bf16_d128_gqa", "bf16", 1, 8, 2, 128, 1000, 64, 64, 64 + 16 * 3, 16),
    small("bf16_C16_W8", "bf16", 1, 2, 1, 64, 300, 8, 16, 8 + 19 * 2, 19),
    small("bf16_G8_C32", "bf16", 1, 8, 1, 64, 300, 32, 32, 32 + 10 * 2, 10),
    small("bf16_G1", "bf16", 2, 3, 3, 64, 260, 32, 32, 32 + 9 * 2, 9),
    small("bf16_W256_C128", "bf16", 1, 4, 1, 128, 900, 256, 128, 256 + 8 * 6, 8),
    small("bf16_pool_global_list", "bf16", 1, 4, 1, 64, 2048, 64, 64, 64 + 36 * 32, 32),
    small("bf16_one_chunk", "bf16", 1, 4, 1, 64, 64, 16, 64, 64, 1),
]
IDS = [w.name for w in SHAPES]


def _units_rows(wl, t):
    """[U, G, ...] of a [B, Hq, ...] tensor, in the oracle's unit order."""
    G = wl.group
    a = t.float().cpu().numpy()
    return np.stack([a[b, kv * G:(kv + 1) * G] for b in range(wl.batch)
                     for kv in range(wl.n_kv_heads)])


def check_lse(got, ref, dtype, what):
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), what
    fin = np.isfinite(ref)
    assert np.all(np.isfinite(got[fin])), what
    err = float(np.abs(got[fin] - ref[fin]).max()) if fin.any() else 0.0
    print("    %s max_abs=%.3e" % (what, err), flush=True)
    assert err <= (1e-4 if dtype == "f32" else 2e-2), (what, err)


@pytest.mark.parametrize("wl", SHAPES, ids=IDS)
def test_prefill_partials(wl):
    x = make_inputs(wl)
    o = P.oracle(wl, x, partials=True)
    g = P.gpu_prefill(wl, x, fp32_out=(wl.dtype == "bf16"), partials=True)
    P.compare_prefill(wl, g, o, out_fp32=(wl.dtype == "bf16"))
    for key in ("y_sa", "y_la"):
        P.check_outputs(_units_rows(wl, g[key]), o[key], wl.dtype, True, key)
    la_empty = np.isneginf(o["lse_la"])
    assert np.all(_units_rows(wl, g["y_la"])[la_empty] == 0)
    for key in ("lse_sa", "lse_la"):
        check_lse(_units_rows(wl, g[key]), o[key], wl.dtype, key)
    # the default walk gives the same merged output as the separate one; the
    # selection work is the same, the state scan may group chunks otherwise
    d = P.gpu_prefill(wl, x, fp32_out=(wl.dtype == "bf16"))
    P.check_outputs(d["y"].float().numpy(), g["y"].float().numpy().astype(np.float64), wl.dtype,
                    True, "two walks")
    for k in ("sel", "score", "pool_k"):
        assert torch.equal(d[k], g[k]), k
    assert np.array_equal(d["pending"].numpy(), g["pending"].numpy(), equal_nan=True)
    for k in ("S", "z"):
        diff = (d[k] - g[k]).abs().max().item()
        assert diff <= 1e-5 * max(1.0, d[k].abs().max().item()), (k, diff)


@pytest.mark.parametrize("variant", ["sum", "softmax_only"])
@pytest.mark.parametrize("wl", SHAPES, ids=IDS)
def test_prefill_merge_variants(wl, variant):
    flags = still.STILL_FLAG_MERGE_SUM if variant == "sum" else still.STILL_FLAG_SOFTMAX_ONLY
    x = make_inputs(wl)
    o = P.oracle(wl, x, merge=variant)
    g = P.gpu_prefill(wl, x, fp32_out=(wl.dtype == "bf16"), flags=flags)
    P.compare_prefill(wl, g, o, out_fp32=(wl.dtype == "bf16"))
    if wl.dtype == "bf16":
        g2 = P.gpu_prefill(wl, x, fp32_out=False, flags=flags)
        P.compare_prefill(wl, g2, o, out_fp32=False, check_state_too=False)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("variant", ["partials", "sum", "softmax_only"])
def test_llama8b_L16K_variants_sampled_units(variant):
    """The 16K workload (batch 1, 32 query / 8 kv heads, d = 128) in each
    variant; the oracle checks two kv-head units."""
    wl = WORKLOADS["llama8b_bf16_L16K"]
    x = make_inputs(wl)
    units = [(0, 2), (0, 7)]
    merge = "one" if variant == "partials" else variant
    flags = {"partials": 0, "sum": still.STILL_FLAG_MERGE_SUM,
             "softmax_only": still.STILL_FLAG_SOFTMAX_ONLY}[variant]
    o = P.oracle(wl, x, units=units, merge=merge, partials=variant == "partials")
    g = P.gpu_prefill(wl, x, fp32_out=True, flags=flags, partials=variant == "partials")
    P.compare_prefill(wl, g, o, units=units, out_fp32=True)
    if variant == "partials":
        rows = P.unit_rows(wl, units)
        for key in ("y_sa", "y_la"):
            got = np.stack([g[key][b, h0:h1].numpy() for b, h0, h1 in rows])
            P.check_outputs(got, o[key], "bf16", True, key)
        for key in ("lse_sa", "lse_la"):
            got = np.stack([g[key][b, h0:h1].numpy() for b, h0, h1 in rows])
            check_lse(got, o[key], "bf16", key)


DECODE_SHAPES = [
    (small("dec_f32", "f32", 1, 2, 1, 64, 90, 16, 32, 16 + 4 * 6, 6, out=0.0), 90, 70),
    (small("dec_bf16_d128", "bf16", 2, 8, 2, 128, 256, 64, 64, 64 + 8 * 2, 8), 256, 130),
    (small("dec_bf16_W_gt_C", "bf16", 1, 2, 1, 64, 70, 48, 16, 48 + 2 * 12, 12), 70, 60),
]


@pytest.mark.parametrize("case", DECODE_SHAPES, ids=[c[0].name for c in DECODE_SHAPES])
def test_decode_softmax_only(case):
    """Prefill and decode with the softmax branch alone; the oracle runs the
    same variant over all L0 + n tokens (the state is still maintained)."""
    wl, L0, n = case
    x = make_inputs(wl, seq_len=L0)
    toks = make_decode_tokens(wl, n)
    flags = still.STILL_FLAG_SOFTMAX_ONLY
    g = P.gpu_prefill(wl, x, keep_device=True, flags=flags)
    p = still.params_for(wl, fp32_out=True, flags=flags)
    xd = {k: v.cuda() for k, v in x.items()}
    td = {k: v.cuda() for k, v in toks.items()}
    outs, sels = P.run_decode(wl, g["_state"], p, xd, td, L0, fp32_out=True)
    units = [(b, kv) for b in range(wl.batch) for kv in range(wl.n_kv_heads)]
    qs, ks, vs, Fs, gs = P.concat_units(x, toks, wl, units)
    o = rec.run_units(qs, ks, vs, Fs, gs, window=wl.window, chunk=wl.chunk, budget=wl.budget,
                      t_max=wl.t_max, n_threads=P.n_threads(), merge="softmax_only")
    G = wl.group
    yg = np.stack([outs[:, b, kv * G:(kv + 1) * G].numpy().transpose(1, 0, 2) for b, kv in units])
    P.check_outputs(yg, o["y"][:, :, L0:], wl.dtype, True, "decode y")
    for s in range(n):
        t = L0 + s
        if t % wl.chunk == 0 and o["lam"] > 0:
            got = np.stack([sels[s, b, kv].numpy() for b, kv in units])
            assert np.array_equal(got, o["sel"][:, t // wl.chunk - 1]), s
    sv = still.state_views(p, g["_state"])
    P.check_state(sv["S"].cpu().numpy(), o["S"], wl.dtype, "decode S")
    P.check_state(sv["z"].cpu().numpy(), o["z"], wl.dtype, "decode z")



ROUTES = ["diag", "qk", "keynorm", "uniform", "external"]
ROUTE_SHAPES = [SHAPES[0], SHAPES[1], SHAPES[2], SHAPES[5], SHAPES[6]]


@pytest.mark.parametrize("route", ROUTES)
@pytest.mark.parametrize("wl", ROUTE_SHAPES, ids=[w.name for w in ROUTE_SHAPES])
def test_prefill_routing_metrics(wl, route):
    x = make_inputs(wl)
    ext = make_route_scores(wl) if route == "external" else None
    o = P.oracle(wl, x, route=route, ext_score=ext)
    g = P.gpu_prefill(wl, x, fp32_out=(wl.dtype == "bf16"), flags=still.route_flag(route),
                      ext_score=ext)
    P.compare_prefill(wl, g, o, out_fp32=(wl.dtype == "bf16"))
    if ext is not None:  # an input: not written
        assert torch.equal(g["score"], ext)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("route", ROUTES)
def test_llama8b_L16K_routing_sampled_units(route):
    wl = WORKLOADS["llama8b_bf16_L16K"]
    x = make_inputs(wl)
    ext = make_route_scores(wl) if route == "external" else None
    units = [(0, 1), (0, 6)]
    o = P.oracle(wl, x, units=units, route=route, ext_score=ext)
    g = P.gpu_prefill(wl, x, fp32_out=True, flags=still.route_flag(route), ext_score=ext)
    P.compare_prefill(wl, g, o, units=units, out_fp32=True)


@pytest.mark.parametrize("route", ["diag", "qk", "keynorm", "uniform"])
@pytest.mark.parametrize("case", DECODE_SHAPES[:2], ids=[c[0].name for c in DECODE_SHAPES[:2]])
def test_decode_routing_metrics(case, route):
    """Prefill and decode under an alternative routing metric; the oracle
    runs the same metric over all L0 + n tokens."""
    wl, L0, n = case
    x = make_inputs(wl, seq_len=L0)
    toks = make_decode_tokens(wl, n)
    flags = still.route_flag(route)
    g = P.gpu_prefill(wl, x, keep_device=True, flags=flags)
    p = still.params_for(wl, fp32_out=True, flags=flags)
    xd = {k: v.cuda() for k, v in x.items()}
    td = {k: v.cuda() for k, v in toks.items()}
    outs, sels = P.run_decode(wl, g["_state"], p, xd, td, L0, fp32_out=True)
    units = [(b, kv) for b in range(wl.batch) for kv in range(wl.n_kv_heads)]
    qs, ks, vs, Fs, gs = P.concat_units(x, toks, wl, units)
    o = rec.run_units(qs, ks, vs, Fs, gs, window=wl.window, chunk=wl.chunk, budget=wl.budget,
                      t_max=wl.t_max, n_threads=P.n_threads(), route=route)
    G = wl.group
    yg = np.stack([outs[:, b, kv * G:(kv + 1) * G].numpy().transpose(1, 0, 2) for b, kv in units])
    P.check_outputs(yg, o["y"][:, :, L0:], wl.dtype, True, "decode y")
    for s in range(n):
        t = L0 + s
        if t % wl.chunk == 0 and o["lam"] > 0:
            got = np.stack([sels[s, b, kv].numpy() for b, kv in units])
            assert np.array_equal(got, o["sel"][:, t // wl.chunk - 1]), s
    sv = still.state_views(p, g["_state"])
    P.check_state(sv["S"].cpu().numpy(), o["S"], wl.dtype, "decode S")
    pend = sv["pending"].cpu().numpy()
    assert np.array_equal(np.isnan(pend), np.isnan(o["pending"]))
    ok = ~np.isnan(pend)
    assert np.allclose(pend[ok], o["pending"][ok], rtol=1e-12, atol=1e-12)


GATE_SHAPES = [SHAPES[0], SHAPES[1], SHAPES[3], SHAPES[5], SHAPES[6]]


@pytest.mark.parametrize("merge", ["one", "sum"])
@pytest.mark.parametrize("wl", GATE_SHAPES, ids=[w.name for w in GATE_SHAPES])
def test_prefill_output_gate(wl, merge):
    """still_prefill_gated: out = y * sigmoid(out_gate), in the walk's output
    stage (the single-normaliser walk and the kept-apart branches of the sum
    merge); selections, scores and state as ungated."""
    x = make_inputs(wl)
    L = x["q"].shape[2]
    og = make_out_gate(wl, (wl.batch, wl.n_q_heads, L, wl.head_dim))
    o = dict(P.oracle(wl, x, merge=merge))
    o["y"] = bf.output_gate(o["y"], _units_rows(wl, og))
    flags = still.STILL_FLAG_MERGE_SUM if merge == "sum" else 0
    g = P.gpu_prefill(wl, x, fp32_out=(wl.dtype == "bf16"), flags=flags, out_gate=og)
    P.compare_prefill(wl, g, o, out_fp32=(wl.dtype == "bf16"))
    if wl.dtype == "bf16":
        g2 = P.gpu_prefill(wl, x, fp32_out=False, flags=flags, out_gate=og)
        P.compare_prefill(wl, g2, o, out_fp32=False, check_state_too=False)


@pytest.mark.timeout(900)
def test_llama8b_L16K_output_gate_sampled_unit():
    """The 16K workload (batch 1, 32 query / 8 kv heads, d = 128) gated, bf16
    output as the walk's tiled store writes it; the oracle checks one unit."""
    wl = WORKLOADS["llama8b_bf16_L16K"]
    x = make_inputs(wl)
    og = make_out_gate(wl, (wl.batch, wl.n_q_heads, wl.seq_len, wl.head_dim))
    units = [(0, 5)]
    o = dict(P.oracle(wl, x, units=units))
    G = wl.group
    o["y"] = bf.output_gate(o["y"], og[0, 5 * G:6 * G].float().numpy()[None])
    g = P.gpu_prefill(wl, x, fp32_out=False, out_gate=og)
    P.compare_prefill(wl, g, o, units=units, out_fp32=False)


@pytest.mark.parametrize("case", DECODE_SHAPES, ids=[c[0].name for c in DECODE_SHAPES])
def test_decode_output_gate(case):
    """Ungated prefill, then still_decode_step_gated steps (chunk boundaries
    included); outputs against the oracle's run over all L0 + n tokens, gated."""
    wl, L0, n = case
    x = make_inputs(wl, seq_len=L0)
    toks = make_decode_tokens(wl, n)
    og = make_out_gate(wl, (n, wl.batch, wl.n_q_heads, wl.head_dim), seed=wl.seed + 1)
    g = P.gpu_prefill(wl, x, keep_device=True)
    p = still.params_for(wl, fp32_out=True)
    xd = {k: v.cuda() for k, v in x.items()}
    td = {k: v.cuda() for k, v in toks.items()}
    ogd = og.cuda()
    lam = still.still_lambda(p)
    outs, sels = [], []
    for s in range(n):
        out = torch.empty((wl.batch, wl.n_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
        sel = torch.empty((wl.batch, wl.n_kv_heads, max(lam, 1)), dtype=torch.int32, device="cuda")
        still.still_decode_step_gated(p, L0 + s, td["q"][s], td["k"][s], td["v"][s], xd["fmap_w"],
                                      xd["gate"], ogd[s], g["_state"], out,
                                      sel if lam > 0 else None)
        outs.append(out)
        sels.append(sel[..., :lam])
    torch.cuda.synchronize()
    outs, sels = torch.stack(outs).cpu(), torch.stack(sels).cpu()
    units = [(b, kv) for b in range(wl.batch) for kv in range(wl.n_kv_heads)]
    qs, ks, vs, Fs, gs = P.concat_units(x, toks, wl, units)
    o = rec.run_units(qs, ks, vs, Fs, gs, window=wl.window, chunk=wl.chunk, budget=wl.budget,
                      t_max=wl.t_max, n_threads=P.n_threads())
    G = wl.group
    gate_u = np.stack([og[:, b, kv * G:(kv + 1) * G].float().numpy().transpose(1, 0, 2)
                       for b, kv in units])
    yg = np.stack([outs[:, b, kv * G:(kv + 1) * G].numpy().transpose(1, 0, 2) for b, kv in units])
    P.check_outputs(yg, bf.output_gate(o["y"][:, :, L0:], gate_u), wl.dtype, True, "gated decode y")
    for s in range(n):
        t = L0 + s
        if t % wl.chunk == 0 and o["lam"] > 0:
            got = np.stack([sels[s, b, kv].numpy() for b, kv in units])
            assert np.array_equal(got, o["sel"][:, t // wl.chunk - 1]), s


DECAY_SHAPES = [SHAPES[0], SHAPES[1], SHAPES[2], SHAPES[3], SHAPES[5], SHAPES[6]]


@pytest.mark.parametrize("wl", DECAY_SHAPES, ids=[w.name for w in DECAY_SHAPES])
def test_prefill_decay(wl):
    """still_prefill_decay: the linear keys and the state decay per token;
    outputs, selections, scores and the exported state (held at the first
    position past it) against the oracle."""
    x = make_inputs(wl)
    dec = make_decay(wl)
    o = P.oracle(wl, x, decay=dec.numpy())
    g = P.gpu_prefill(wl, x, fp32_out=(wl.dtype == "bf16"), decay=dec)
    P.compare_prefill(wl, g, o, out_fp32=(wl.dtype == "bf16"))
    if wl.dtype == "bf16":
        g2 = P.gpu_prefill(wl, x, fp32_out=False, decay=dec)
        P.compare_prefill(wl, g2, o, out_fp32=False, check_state_too=False)


@pytest.mark.timeout(900)
def test_llama8b_L16K_decay_sampled_units():
    """The 16K workload with slow forget factors U(0.99, 1) (the state
    spans hundreds of chunks); the oracle checks two kv-head units."""
    wl = WORKLOADS["llama8b_bf16_L16K"]
    x = make_inputs(wl)
    dec = make_decay(wl, lo=0.99)
    units = [(0, 1), (0, 6)]
    o = P.oracle(wl, x, units=units, decay=dec.numpy())
    g = P.gpu_prefill(wl, x, fp32_out=True, decay=dec)
    P.compare_prefill(wl, g, o, units=units, out_fp32=True)


@pytest.mark.parametrize("case", DECODE_SHAPES, ids=[c[0].name for c in DECODE_SHAPES])
def test_decode_decay(case):
    """still_prefill_decay, then still_decode_step_decay steps over chunk
    boundaries (the fold moves the state on by gamma^C); outputs, kept
    positions and the state against the oracle's run over L0 + n tokens."""
    wl, L0, n = case
    x = make_inputs(wl, seq_len=L0)
    toks = make_decode_tokens(wl, n)
    dec = make_decay(wl, seed=wl.seed + 2)
    g = P.gpu_prefill(wl, x, keep_device=True, decay=dec)
    p = still.params_for(wl, fp32_out=True)
    xd = {k: v.cuda() for k, v in x.items()}
    td = {k: v.cuda() for k, v in toks.items()}
    dd = dec.cuda()
    lam = still.still_lambda(p)
    outs, sels = [], []
    for s in range(n):
        out = torch.empty((wl.batch, wl.n_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
        sel = torch.empty((wl.batch, wl.n_kv_heads, max(lam, 1)), dtype=torch.int32, device="cuda")
        still.still_decode_step_decay(p, L0 + s, td["q"][s], td["k"][s], td["v"][s], xd["fmap_w"],
                                      xd["gate"], dd, g["_state"], out, sel if lam > 0 else None)
        outs.append(out)
        sels.append(sel[..., :lam])
    torch.cuda.synchronize()
    outs, sels = torch.stack(outs).cpu(), torch.stack(sels).cpu()
    units = [(b, kv) for b in range(wl.batch) for kv in range(wl.n_kv_heads)]
    qs, ks, vs, Fs, gs = P.concat_units(x, toks, wl, units)
    o = rec.run_units(qs, ks, vs, Fs, gs, window=wl.window, chunk=wl.chunk, budget=wl.budget,
                      t_max=wl.t_max, n_threads=P.n_threads(),
                      decay=np.array([dec[kv].item() for _, kv in units], np.float32))
    G = wl.group
    yg = np.stack([outs[:, b, kv * G:(kv + 1) * G].numpy().transpose(1, 0, 2) for b, kv in units])
    P.check_outputs(yg, o["y"][:, :, L0:], wl.dtype, True, "decay decode y")
    for s in range(n):
        t = L0 + s
        if t % wl.chunk == 0 and o["lam"] > 0:
            got = np.stack([sels[s, b, kv].numpy() for b, kv in units])
            assert np.array_equal(got, o["sel"][:, t // wl.chunk - 1]), s
    sv = still.state_views(p, g["_state"])
    P.check_state(sv["S"].cpu().numpy(), o["S"], wl.dtype, "decay decode S")
    P.check_state(sv["z"].cpu().numpy(), o["z"], wl.dtype, "decay decode z")
