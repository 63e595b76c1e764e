"""Parity of the HIP path (through the C ABI) with the oracle, on the GPU.

Every input is seeded and synthetic (linear_attention_still_amd.inputs).
Small shapes are compared element by element over every unit; the full
workloads are compared over every unit where the oracle finishes in seconds
and over sampled (batch row, kv head) units otherwise, in the launch
configuration the bench uses.
"""
import numpy as np
import pytest
import torch

from linear_attention_still_amd import still
from linear_attention_still_amd.inputs import WORKLOADS, Workload, make_decode_tokens, make_inputs
from oracle import rec
from tests import _parity as P

pytestmark = pytest.mark.gpu


def small(name, dtype, B, Hq, Hkv, d, L, W, C, m, t_max, sigma=0.5, out=0.01, seed=11):
    # float32 shapes carry no 8x outliers, like the float32 workload: logits of
    # ~1e3 between two outliers hold ~1e-4 of float32 rounding on their own
    return Workload(name, dtype, B, Hq, Hkv, d, L, W, C, m, t_max, sigma=sigma,
                    outlier_frac=out, seed=seed)


SHAPES = [
    small("f32_d64_W16_C32", "f32", 1, 2, 1, 64, 200, 16, 32, 64, 7, out=0.0),
    small("f32_gqa_ragged", "f32", 2, 4, 2, 64, 333, 40, 64, 40 + 6 * 3, 6, out=0.0),
    small("bf16_d64_W64_C64", "bf16", 1, 4, 1, 64, 600, 64, 64, 64 + 3 * 10, 10),
    small("bf16_d128_ragged", "bf16", 1, 8, 2, 128, 1000, 64, 64, 64 + 16 * 3, 16),
    small("bf16_W_lt_C", "bf16", 1, 4, 2, 128, 700, 16, 64, 16 + 11 * 2, 11),
    small("bf16_W_gt_C", "bf16", 1, 2, 1, 64, 500, 96, 32, 96 + 16 * 2, 16),
    small("bf16_lambda0", "bf16", 1, 4, 1, 128, 400, 32, 32, 32, 13),
    small("bf16_full_softmax", "bf16", 1, 4, 1, 64, 256, 32, 32, 32 + 8 * 32, 8),
    small("bf16_C128_split_heads", "bf16", 1, 4, 1, 128, 700, 128, 128, 128 + 6 * 4, 6),
    small("bf16_C16_W8", "bf16", 1, 2, 1, 64, 300, 8, 16, 8 + 19 * 2, 19),
    small("bf16_G8", "bf16", 1, 8, 1, 64, 300, 32, 32, 32 + 10 * 2, 10),
    small("bf16_G1", "bf16", 2, 3, 3, 64, 260, 32, 32, 32 + 9 * 2, 9),
    small("bf16_budget_fills", "bf16", 1, 4, 1, 64, 640, 16, 32, 16 + 6 * 2, 3),
    small("bf16_W1_ties", "bf16", 1, 2, 1, 64, 160, 1, 32, 1 + 5 * 4, 5),
    small("bf16_one_token", "bf16", 1, 4, 1, 64, 1, 16, 32, 64, 4),
    small("bf16_one_chunk", "bf16", 1, 4, 1, 64, 64, 16, 64, 64, 1),
    small("bf16_one_decided", "bf16", 1, 4, 1, 64, 65, 16, 64, 80, 1),
    # more than 1024 kept tokens: the walk reads pool positions from the
    # global list instead of LDS (m - W = 36 * 32 = 1152, lambda = 36)
    small("bf16_pool_global_list", "bf16", 1, 4, 1, 64, 2048, 64, 64, 64 + 36 * 32, 32),
    # the widest window (W = 256) with the widest chunk
    small("bf16_W256_C128", "bf16", 1, 4, 1, 128, 900, 256, 128, 256 + 8 * 6, 8),
]


@pytest.mark.parametrize("wl", SHAPES, ids=[w.name for w in SHAPES])
def test_prefill_parity_shapes(wl):
    x = make_inputs(wl)
    o = P.oracle(wl, x)
    g = P.gpu_prefill(wl, x, fp32_out=(wl.dtype == "bf16"))
    P.compare_prefill(wl, g, o, out_fp32=(wl.dtype == "bf16"))
    if wl.dtype == "bf16":
        g2 = P.gpu_prefill(wl, x, fp32_out=False)
        P.compare_prefill(wl, g2, o, out_fp32=False, check_state_too=False)


def test_small_f32_workload():
    wl = WORKLOADS["small_f32_L256"]
    x = make_inputs(wl)
    P.compare_prefill(wl, P.gpu_prefill(wl, x), P.oracle(wl, x))


@pytest.mark.timeout(600)
def test_gqa_L4K_workload():
    wl = WORKLOADS["gqa_bf16_L4K"]
    x = make_inputs(wl)
    o = P.oracle(wl, x)
    P.compare_prefill(wl, P.gpu_prefill(wl, x, fp32_out=True), o, out_fp32=True)
    P.compare_prefill(wl, P.gpu_prefill(wl, x), o, check_state_too=False)


@pytest.mark.timeout(600)
def test_llama8b_L16K_workload():
    wl = WORKLOADS["llama8b_bf16_L16K"]
    x = make_inputs(wl)
    o = P.oracle(wl, x)
    P.compare_prefill(wl, P.gpu_prefill(wl, x, fp32_out=True), o, out_fp32=True)
    P.compare_prefill(wl, P.gpu_prefill(wl, x), o, check_state_too=False)


@pytest.mark.timeout(900)
def test_llama8b_L64K_workload():
    """Every (batch row, kv head) unit of the 64K workload against the oracle."""
    wl = WORKLOADS["llama8b_bf16_L64K"]
    x = make_inputs(wl)
    o = P.oracle(wl, x)
    P.compare_prefill(wl, P.gpu_prefill(wl, x, fp32_out=True), o, out_fp32=True)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["llama8b_bf16_L16K", "llama8b_bf16_L64K"])
def test_softmax_branch_alone_full_size(name):
    """With every gate at 0 the output is the softmax branch alone over the
    window, own-chunk prefix and kept pool (no linear weight enters), so the
    kept-pool gather path is checked at full size without being diluted by
    the linear branch's mass."""
    wl = WORKLOADS[name]
    x = make_inputs(wl)
    x["gate"] = torch.zeros_like(x["gate"])
    o = P.oracle(wl, x)
    P.compare_prefill(wl, P.gpu_prefill(wl, x, fp32_out=True), o, out_fp32=True,
                      check_state_too=False)


def test_prefill_deterministic():
    wl = WORKLOADS["gqa_bf16_L4K"]
    x = make_inputs(wl)
    a = P.gpu_prefill(wl, x)
    b = P.gpu_prefill(wl, x)
    for k in ("y", "sel", "score", "S", "z", "pending", "ring_k", "pool_k"):
        assert torch.equal(a[k], b[k]), k


@pytest.mark.timeout(600)
@pytest.mark.parametrize("env", [("STILL_HEADS_PER_WAVE", "1"), ("STILL_CHUNKS_PER_WG", "1")],
                         ids=["one_head_per_wave", "one_chunk_per_workgroup"])
def test_prefill_launch_variants_agree(env, monkeypatch):
    """The attention walk's launch shape (heads per wave, chunks per
    workgroup) changes only which workgroup computes a row, not the
    arithmetic of a row: outputs, selections and the exported state match
    the default launch exactly (the chunk split changes the state scan's
    grouping, so S and z are compared to float32 rounding there)."""
    wl = WORKLOADS["gqa_bf16_L4K"]
    x = make_inputs(wl)
    a = P.gpu_prefill(wl, x)
    monkeypatch.setenv(*env)
    b = P.gpu_prefill(wl, x)
    for k in ("sel", "score", "pending", "ring_k", "pool_k"):
        assert torch.equal(a[k], b[k]), k
    if env[0] == "STILL_HEADS_PER_WAVE":
        for k in ("y", "S", "z"):
            assert torch.equal(a[k], b[k]), k
    else:
        # float32-level differences in the state can move a bf16 output
        # across a rounding boundary: one bf16 step (at most 2^-7 of the
        # value) per element on top of the float32-level bar
        for k in ("y", "S", "z"):
            af, bf = a[k].float(), b[k].float()
            ref = af.abs().max().item()
            tol = 1e-5 * max(ref, 1.0)
            if k == "y" and a[k].dtype == torch.bfloat16:
                excess = ((af - bf).abs() - 2.0 ** -7 * af.abs()).max().item()
            else:
                excess = (af - bf).abs().max().item()
            assert excess <= tol, (k, excess)


DECODE_SHAPES = [
    # (workload, prefill length, decode steps)
    (small("dec_f32", "f32", 1, 2, 1, 64, 90, 16, 32, 16 + 4 * 6, 6, out=0.0), 90, 70),
    (small("dec_bf16_d128", "bf16", 2, 8, 2, 128, 256, 64, 64, 64 + 8 * 2, 8), 256, 130),
    (small("dec_bf16_W_lt_C", "bf16", 1, 4, 1, 64, 100, 16, 32, 16 + 3 * 10, 10), 100, 75),
    (small("dec_bf16_W_gt_C", "bf16", 1, 2, 1, 64, 70, 48, 16, 48 + 2 * 12, 12), 70, 60),
    (small("dec_bf16_fill", "bf16", 1, 4, 1, 64, 96, 8, 16, 8 + 2 * 4, 4), 96, 80),
    (small("dec_bf16_G1", "bf16", 2, 2, 2, 128, 150, 32, 32, 32 + 7 * 3, 7), 150, 70),
    (small("dec_bf16_G8", "bf16", 1, 8, 1, 128, 200, 64, 64, 64 + 5 * 4, 5), 200, 70),
    (small("dec_bf16_W256_C128", "bf16", 1, 4, 1, 128, 400, 256, 128, 256 + 5 * 8, 5), 400, 140),
]


@pytest.mark.parametrize("case", DECODE_SHAPES, ids=[c[0].name for c in DECODE_SHAPES])
def test_decode_matches_prefill_of_extended_sequence(case):
    """Prefill L0 tokens, decode n more one by one; the oracle runs the layer
    over all L0 + n tokens (prefill and decode share one rule)."""
    wl, L0, n = case
    x = make_inputs(wl, seq_len=L0)
    toks = make_decode_tokens(wl, n)
    g = P.gpu_prefill(wl, x, keep_device=True)
    p = still.params_for(wl, fp32_out=(wl.dtype == "bf16"))
    xd = {k: v.cuda() for k, v in x.items()}
    td = {k: v.cuda() for k, v in toks.items()}
    outs, sels = P.run_decode(wl, g["_state"], p, xd, td, L0, fp32_out=(wl.dtype == "bf16"))
    units = [(b, kv) for b in range(wl.batch) for kv in range(wl.n_kv_heads)]
    qs, ks, vs, Fs, gs = P.concat_units(x, toks, wl, units)
    o = rec.run_units(qs, ks, vs, Fs, gs, window=wl.window, chunk=wl.chunk, budget=wl.budget,
                      t_max=wl.t_max, n_threads=P.n_threads())
    G = wl.group
    yg = np.stack([outs[:, b, kv * G:(kv + 1) * G].numpy().transpose(1, 0, 2) for b, kv in units])
    P.check_outputs(yg, o["y"][:, :, L0:], wl.dtype, True, "decode y")
    lam = o["lam"]
    for s in range(n):
        t = L0 + s
        if t % wl.chunk == 0 and lam > 0:
            want = o["sel"][:, t // wl.chunk - 1]
            got = np.stack([sels[s, b, kv].numpy() for b, kv in units])
            assert np.array_equal(got, want), (s, got, want)
    sv = still.state_views(p, g["_state"])
    P.check_state(sv["S"].cpu().numpy(), o["S"], wl.dtype, "decode S")
    P.check_state(sv["z"].cpu().numpy(), o["z"], wl.dtype, "decode z")
    meta = sv["meta"].cpu().numpy()
    assert np.all(meta[:, 0] == L0 + n) and np.all(meta[:, 2] == 0)
    assert np.array_equal(meta[:, 1], o["n_pool"])
    pend = sv["pending"].cpu().numpy()
    assert np.array_equal(np.isnan(pend), np.isnan(o["pending"]))
    ok = ~np.isnan(pend)
    assert np.allclose(pend[ok], o["pending"][ok], rtol=1e-12, atol=1e-12)


@pytest.mark.timeout(900)
def test_decode_workload_sampled_units():
    """Batch 64 at 16K context: prefill on the GPU, 64 decode steps (one
    chunk-boundary decision); the oracle checks 16 units spread over the
    batch rows and kv heads."""
    wl = WORKLOADS["decode_bf16_B64_ctx16K"]
    L0, n = wl.seq_len, wl.decode_steps
    x = make_inputs(wl, device="cuda")
    toks = make_decode_tokens(wl, n, device="cuda")
    p = still.params_for(wl, fp32_out=True)
    print("  gpu prefill B=64 L=16384", flush=True)
    bufs = still.PrefillBuffers(p, L0)
    still.run_prefill(p, x, bufs)
    outs, sels = P.run_decode(wl, bufs.state, p, x, toks, L0, fp32_out=True)
    units = [(b, (3 * i) % wl.n_kv_heads) for i, b in
             enumerate([0, 4, 9, 13, 17, 21, 26, 30, 33, 37, 42, 46, 50, 55, 59, 63])]
    qs, ks, vs, Fs, gs = P.concat_units(x, toks, wl, units)
    print("  oracle %d units, %d tokens" % (len(units), L0 + n), flush=True)
    o = rec.run_units(qs, ks, vs, Fs, gs, window=wl.window, chunk=wl.chunk, budget=wl.budget,
                      t_max=wl.t_max, n_threads=P.n_threads())
    G = wl.group
    yg = np.stack([outs[:, b, kv * G:(kv + 1) * G].numpy().transpose(1, 0, 2) for b, kv in units])
    P.check_outputs(yg, o["y"][:, :, L0:], "bf16", True, "decode y")
    got = np.stack([sels[0, b, kv].numpy() for b, kv in units])
    assert np.array_equal(got, o["sel"][:, L0 // wl.chunk - 1])
    sv = still.state_views(p, bufs.state)
    idx = [b * wl.n_kv_heads + kv for b, kv in units]
    P.check_state(sv["S"][idx].cpu().numpy(), o["S"], "bf16", "S")
    P.check_state(sv["z"][idx].cpu().numpy(), o["z"], "bf16", "z")


def test_prefill_then_decode_equals_longer_prefill():
    """GPU only: prefill(L1) + decode to L gives the outputs, kept positions
    and state of prefill(L)."""
    wl = small("pd", "bf16", 1, 4, 2, 128, 320, 64, 64, 64 + 5 * 2, 5)
    L1 = 190
    x = make_inputs(wl)
    xs = {k: (v[:, :, :L1].contiguous() if k in ("q", "k", "v") else v) for k, v in x.items()}
    toks = {k: x[k][:, :, L1:].permute(2, 0, 1, 3).contiguous() for k in ("q", "k", "v")}
    full = P.gpu_prefill(wl, x, fp32_out=True)
    g = P.gpu_prefill(wl, xs, keep_device=True)
    p = still.params_for(wl, fp32_out=True)
    xd = {k: v.cuda() for k, v in x.items()}
    td = {k: v.cuda() for k, v in toks.items()}
    outs, sels = P.run_decode(wl, g["_state"], p, xd, td, L1, fp32_out=True)
    err = (outs.permute(1, 2, 0, 3) - full["y"][:, :, L1:]).abs().max().item()
    assert err <= 2e-2, err
    sv = still.state_views(p, g["_state"])
    assert torch.equal(sv["pool_pos"].cpu(), full["pool_pos"])
    assert (sv["S"].cpu() - full["S"]).abs().max().item() <= 2e-2


def test_decode_position_mismatch_sets_error_word():
    """A decode step whose position does not follow the state sets the
    state's error word (meta[2] = STILL_ESTATE), writes nothing else, and
    later steps are skipped until the state is reset."""
    wl = small("dec_err", "bf16", 1, 4, 1, 64, 100, 16, 32, 16 + 3 * 10, 10)
    x = make_inputs(wl)
    toks = make_decode_tokens(wl, 2)
    g = P.gpu_prefill(wl, x, keep_device=True)
    p = g["_params"]
    before = g["_state"].clone()
    xd = {k: v.cuda() for k, v in x.items()}
    out = torch.full((wl.batch, wl.n_q_heads, wl.head_dim), 7.0, dtype=torch.bfloat16, device="cuda")
    still.still_decode_step(p, 101, toks["q"][0].cuda(), toks["k"][0].cuda(), toks["v"][0].cuda(),
                            xd["fmap_w"], xd["gate"], g["_state"], out)  # the state holds 100
    torch.cuda.synchronize()
    sv = still.state_views(p, g["_state"])
    assert int(sv["meta"][0, 2]) == still.STILL_ESTATE
    assert int(sv["meta"][0, 0]) == 100
    lay = still.still_state_layout_get(p)
    changed = (g["_state"].cpu() != before.cpu()).nonzero().flatten().tolist()
    assert all(lay.meta + 16 <= i < lay.meta + 24 for i in changed), changed
    assert torch.all(out.float() == 7.0)
    # a step at the right position is refused too while the error word is set
    still.still_decode_step(p, 100, toks["q"][1].cuda(), toks["k"][1].cuda(), toks["v"][1].cuda(),
                            xd["fmap_w"], xd["gate"], g["_state"], out)
    torch.cuda.synchronize()
    assert int(still.state_views(p, g["_state"])["meta"][0, 0]) == 100


def test_state_save_restore_resumes_exactly():
    """The decode state is plain device memory: copied to the host and back
    into a fresh buffer, decoding resumes exactly as it would have without
    the interruption (same outputs and kept positions, same final state)."""
    wl = small("dec_resume", "bf16", 2, 8, 2, 128, 190, 64, 64, 64 + 5 * 2, 5)
    x = make_inputs(wl)
    toks = make_decode_tokens(wl, 90)
    g = P.gpu_prefill(wl, x, keep_device=True)
    p = still.params_for(wl)
    xd = {k: v.cuda() for k, v in x.items()}
    td = {k: v.cuda() for k, v in toks.items()}
    saved = g["_state"].cpu()  # the checkpoint, in host memory
    outs_a, sels_a = P.run_decode(wl, g["_state"], p, xd, td, 190)
    restored = saved.cuda()
    outs_b, sels_b = P.run_decode(wl, restored, p, xd, td, 190)
    assert torch.equal(outs_a, outs_b)
    assert torch.equal(sels_a, sels_b)
    assert torch.equal(g["_state"].cpu(), restored.cpu())
