"""The kept pool as an 8-bit store (STILL_FLAG_POOL_FP8), on the GPU through
the C ABI, against the oracle.

The pages' precision work names an fp8 pool K/V; the format is a reading:
OCP E4M3 codes of each kept key and value row divided by a power-of-two
scale 2^e (e the smallest integer with the row's largest magnitude at most
448 * 2^e), e kept as one byte per row. The prefill exports the kept rows in
that form; decode boundaries append them in that form; decode steps read
the kept tokens below the window band from it.

Bars: the stored codes and exponents bit-exact against the oracle's
quantiser applied to the kept tokens' input rows (the division by 2^e is
exact, so both sides take the same rounding decisions); the prefill's own
outputs, selections, scores and state bit-identical to the plain layer's
(the store is read by decode steps only); decode outputs against the
oracle whose queries from the prefill length on read the kept pool below
their band quantised (the default path's bars), selections exact.
"""
import numpy as np
import pytest
import torch

from linear_attention_still_amd import still
from linear_attention_still_amd.inputs import Workload, make_decode_tokens, make_inputs
from oracle import rec
from tests import _parity as P

pytestmark = pytest.mark.gpu


def small(name, dtype, B, Hq, Hkv, d, L, W, C, m, t_max, out=0.01, seed=23):
    return Workload(name, dtype, B, Hq, Hkv, d, L, W, C, m, t_max, sigma=0.5,
                    outlier_frac=out, seed=seed)


# (workload, prefill length, decode steps)
POOL8_SHAPES = [
    (small("p8_bf16_d128_G4", "bf16", 2, 8, 2, 128, 256, 64, 64, 64 + 8 * 2, 8), 256, 130),
    (small("p8_bf16_d128_many", "bf16", 2, 8, 2, 128, 600, 64, 32, 64 + 8 * 20, 20), 600, 100),
    (small("p8_bf16_d64_G1_oddP", "bf16", 2, 2, 2, 64, 150, 32, 32, 32 + 7 * 3, 7), 150, 70),
    (small("p8_bf16_d64_G8", "bf16", 1, 8, 1, 64, 200, 64, 64, 64 + 5 * 4, 5), 200, 70),
    (small("p8_bf16_d128_G2_W_gt_C", "bf16", 1, 4, 2, 128, 170, 48, 16, 48 + 2 * 12, 12), 170, 60),
]


def check_store(p, state, k, n_pool_max=None):
    """Codes and exponent bytes of every stored row against the oracle's
    quantiser of the kept tokens' input rows k [U, L, d] (host, float32)."""
    sv = still.state_views(p, state)
    meta = sv["meta"].cpu().numpy()
    pos = sv["pool_pos"].cpu().numpy()
    n_rows = 0
    for u in range(meta.shape[0]):
        n = int(meta[u, 1])
        n_rows += n
        if n == 0:
            continue
        for name, src in (("k", k[0]), ("v", k[1])):
            codes, exps, _ = rec.e4m3_rows(src[u][pos[u, :n]])
            got = sv["pool_%s8" % name][u, :n].cpu().numpy()
            gexp = sv["pool_%s_exp" % name][u, :n].cpu().numpy().astype(np.int64) - 127
            assert np.array_equal(got, codes), (name, u, np.argwhere(got != codes)[:4])
            assert np.array_equal(gexp, exps.astype(np.int64)), (name, u)
    return n_rows


@pytest.mark.parametrize("case", POOL8_SHAPES, ids=[c[0].name for c in POOL8_SHAPES])
def test_pool8_prefill_and_decode(case):
    wl, L0, n = case
    x = make_inputs(wl, seq_len=L0)
    toks = make_decode_tokens(wl, n)
    g0 = P.gpu_prefill(wl, x, fp32_out=True)  # the plain layer
    g = P.gpu_prefill(wl, x, fp32_out=True, keep_device=True, flags=still.STILL_FLAG_POOL_FP8)
    p = g["_params"]
    for key in ("y", "sel", "score", "S", "z", "pool_pos", "ring_k", "ring_v", "ring_phi", "meta"):
        assert torch.equal(g[key].cpu().view(torch.uint8), g0[key].view(torch.uint8)), key
    units = [(b, kv) for b in range(wl.batch) for kv in range(wl.n_kv_heads)]
    kk = np.stack([np.concatenate([x["k"][b, kv].float().numpy(), toks["k"][:, b, kv].float().numpy()])
                   for b, kv in units])
    vv = np.stack([np.concatenate([x["v"][b, kv].float().numpy(), toks["v"][:, b, kv].float().numpy()])
                   for b, kv in units])
    rows0 = check_store(p, g["_state"], (kk, vv))
    print("    prefill: %d stored rows bit-exact" % rows0, flush=True)

    xd = {k_: v_.cuda() for k_, v_ in x.items()}
    td = {k_: v_.cuda() for k_, v_ in toks.items()}
    lam = still.still_lambda(p)
    outs, sels = [], []
    for s in range(n):
        out = torch.empty((wl.batch, wl.n_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
        sel = torch.empty((wl.batch, wl.n_kv_heads, max(lam, 1)), dtype=torch.int32, device="cuda")
        still.still_decode_step(p, L0 + s, td["q"][s], td["k"][s], td["v"][s], xd["fmap_w"],
                                xd["gate"], g["_state"], out, sel if lam > 0 else None)
        outs.append(out)
        sels.append(sel[..., :lam])
    torch.cuda.synchronize()
    outs, sels = torch.stack(outs).cpu(), torch.stack(sels).cpu()
    rows1 = check_store(p, g["_state"], (kk, vv))
    print("    decode: %d stored rows bit-exact" % rows1, flush=True)
    qs, ks, vs, Fs, gs = P.concat_units(x, toks, wl, units)
    o = rec.run_units(qs, ks, vs, Fs, gs, window=wl.window, chunk=wl.chunk, budget=wl.budget,
                      t_max=wl.t_max, n_threads=P.n_threads(), fp8_from=L0)
    G = wl.group
    yg = np.stack([outs[:, b, kv * G:(kv + 1) * G].numpy().transpose(1, 0, 2) for b, kv in units])
    P.check_outputs(yg, o["y"][:, :, L0:], wl.dtype, True, "pool8 decode y")
    plain = rec.run_units(qs, ks, vs, Fs, gs, window=wl.window, chunk=wl.chunk, budget=wl.budget,
                          t_max=wl.t_max, n_threads=P.n_threads())
    gap = np.abs(o["y"][:, :, L0:] - plain["y"][:, :, L0:]).max()
    print("    oracle 8-bit vs full-precision pool: max |dy| = %.3e" % gap, flush=True)
    for s in range(n):
        t = L0 + s
        if t % wl.chunk == 0 and o["lam"] > 0:
            got = np.stack([sels[s, b, kv].numpy() for b, kv in units])
            assert np.array_equal(got, o["sel"][:, t // wl.chunk - 1]), s


def test_pool8_decode_workload_sampled_units():
    """Batch 64 at 16K context (32/8 heads, d = 128, W = C = 64, budget 512)
    with the 8-bit pool, in the bench's launch configuration: prefill, 64
    decode steps (one chunk-boundary decision); the stored codes of 16 units
    bit-exact, their outputs against the oracle that reads the quantised
    pool, the boundary's selections exact."""
    from linear_attention_still_amd.inputs import WORKLOADS
    wl = WORKLOADS["decode_bf16_B64_ctx16K"]
    L0, n = wl.seq_len, wl.decode_steps
    x = make_inputs(wl, device="cuda")
    toks = make_decode_tokens(wl, n, device="cuda")
    p = still.params_for(wl, fp32_out=True, flags=still.STILL_FLAG_POOL_FP8)
    print("  gpu prefill (8-bit pool) B=64 L=16384", flush=True)
    bufs = still.PrefillBuffers(p, L0)
    still.run_prefill(p, x, bufs)
    outs, sels = P.run_decode(wl, bufs.state, p, x, toks, L0, fp32_out=True)
    units = [(b, (5 * i + 1) % wl.n_kv_heads) for i, b in
             enumerate([1, 5, 8, 12, 16, 20, 25, 29, 34, 38, 41, 45, 51, 54, 58, 62])]
    sv = still.state_views(p, bufs.state)
    meta, pos = sv["meta"].cpu().numpy(), sv["pool_pos"].cpu().numpy()
    for b, kv in units:
        u = b * wl.n_kv_heads + kv
        m = int(meta[u, 1])
        for name, src in (("k", x["k"]), ("v", x["v"])):
            rows = torch.cat([src[b, kv], toks[name][:, b, kv]]).float().cpu().numpy()
            codes, exps, _ = rec.e4m3_rows(rows[pos[u, :m]])
            assert np.array_equal(sv["pool_%s8" % name][u, :m].cpu().numpy(), codes), (name, b, kv)
            assert np.array_equal(sv["pool_%s_exp" % name][u, :m].cpu().numpy().astype(np.int64) - 127,
                                  exps.astype(np.int64)), (name, b, kv)
    qs, ks, vs, Fs, gs = P.concat_units(x, toks, wl, units)
    print("  oracle %d units, %d tokens, 8-bit pool from %d" % (len(units), L0 + n, L0), flush=True)
    o = rec.run_units(qs, ks, vs, Fs, gs, window=wl.window, chunk=wl.chunk, budget=wl.budget,
                      t_max=wl.t_max, n_threads=P.n_threads(), fp8_from=L0)
    G = wl.group
    yg = np.stack([outs[:, b, kv * G:(kv + 1) * G].numpy().transpose(1, 0, 2) for b, kv in units])
    P.check_outputs(yg, o["y"][:, :, L0:], "bf16", True, "pool8 decode y (16K)")
    got = np.stack([sels[0, b, kv].numpy() for b, kv in units])
    assert np.array_equal(got, o["sel"][:, L0 // wl.chunk - 1])
