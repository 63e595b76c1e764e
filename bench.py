#!/usr/bin/env python3
"""Throughput of one STILL hybrid-attention layer on one MI355X.

A step is one prefill of the layer (score -> chunk Top-lambda -> window +
kept softmax -> NP-Map linear attention + merge, plus the decode-state
export) over one batch of seeded synthetic inputs shaped like a
Llama-3-8B layer at 16K context (32 query / 8 kv heads, head dim 128,
W = C = 64, budget m = 512). Inputs are resident in HBM before the timed
region. The same JSON line reports the other workloads (the batch-2 4K GQA
prefill, the 64K prefill with its per-token time against the 16K one, and
the latency of the small float32 workload), measured ceilings of the chip
(a device copy and a large bf16 GEMM), a chunk-size sweep of the 16K
workload (C = 16 .. 128, all else unchanged), the backward on the 4K workload, the
decode leg (batch 64 at 16K
context, 64 steps including one chunk-boundary decision) and the float64
oracle's CPU baseline (all usable cores, and one thread).

  python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-decode]
                  [--no-workloads]

One GPU only: --gpus above 1 exits with a message.
"""
import argparse
import json
import math
import os
import sys
import time

METRIC = "hybrid-attn prefill tokens/s/layer at 16K (MFMA %peak); decode tok/s (HBM GB/s)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def algorithmic_work(wl, sel):
    """Algorithmic flops of the layer and of the attention kernel, counted
    from the actual selection (no padding, masked tile halves or
    recomputation): softmax 4d|A(t)| per (head, query); NP-Map 2d^2 per
    query row and per key; linear readout (2d^2 + 2d) per (head, query);
    state update (2d^2 + 2d) per folded token per kv head."""
    import numpy as np
    B, Hkv, G, d = wl.batch, wl.n_kv_heads, wl.group, wl.head_dim
    L, W, C = wl.seq_len, wl.window, wl.chunk
    t = np.arange(L)
    c = t // C
    lo = np.maximum(0, np.minimum(t - W + 1, c * C))
    sum_A = 0
    n_la = 0
    for b in range(B):
        for kv in range(Hkv):
            pool = np.sort(sel[b, kv].reshape(-1))
            pool = pool[pool >= 0]
            a_t = (t - lo + 1) + np.searchsorted(pool, lo)
            sum_A += int(a_t.sum())
            c_last = (L - 1) // C
            last_ok = min(L - 1 - W, c_last * C - 1)
            n_la += max(0, last_ok + 1) - int(np.count_nonzero(pool <= last_ok))
    Hq = B * Hkv * G
    sa = 4 * d * G * sum_A
    phi = 2 * d * d * L * (B * Hkv * G + B * Hkv)
    phi_q = 2 * d * d * L * Hq
    readout = (2 * d * d + 2 * d) * L * Hq
    update = (2 * d * d + 2 * d) * n_la
    total = sa + phi + readout + update
    attend = sa + phi_q + readout
    return {"total": total, "attend": attend, "sa": sa, "phi": phi, "readout": readout,
            "update": update, "sum_A": sum_A}


HERE = os.path.dirname(os.path.abspath(__file__))
COMMON = ("linear_attention_still_amd/csrc/still_common.h", "linear_attention_still_amd/csrc/still_api.hip")
PREFILL_SOURCES = ("linear_attention_still_amd/csrc/still_prefill.hip",) + COMMON
DECODE_SOURCES = ("linear_attention_still_amd/csrc/still_decode.hip",) + COMMON


def measured_traffic(kernel, profile, sources):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary `profiles/<profile>`, or None when the kernel sources changed
    since the counters were taken."""
    import hashlib
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(HERE, f), "rb") as fh:
            h.update(fh.read())
    sha = h.hexdigest()[:16]
    try:
        with open(os.path.join(HERE, "profiles", profile)) as fh:
            for line in fh:
                if line.startswith("traffic %s " % kernel):
                    kv = dict(x.split("=") for x in line.split()[2:])
                    if kv.get("source_sha256") == sha:
                        return int(kv["bytes_per_launch"])
    except OSError:
        pass
    return None


def run_prefill_bench(torch, still, inputs, name, steps, warmup, breakdown=True):
    """Times `steps` prefills of workload `name` (inputs resident in HBM),
    with HIP events around the attention kernel only; then, if breakdown,
    a second set of steps with events around every kernel."""
    wl = inputs.WORKLOADS[name] if isinstance(name, str) else name
    p = still.params_for(wl)
    x = inputs.make_inputs(wl, device="cuda")
    bufs = still.PrefillBuffers(p, wl.seq_len)
    nk = len(still.PREFILL_KERNELS)
    ai = still.PREFILL_KERNELS.index("attend")
    for _ in range(warmup):
        still.run_prefill(p, x, bufs)
    torch.cuda.synchronize()

    def events(n):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n)] for _ in range(steps)]
        for evs in ev:  # create the handles
            for e in evs:
                e.record()
        return ev

    def run(evs):
        still.still_prefill_timed(p, wl.seq_len, x["q"], x["k"], x["v"], x["fmap_w"], x["gate"],
                                  bufs.out, bufs.sel if bufs.sel.numel() else None, bufs.score,
                                  bufs.state, bufs.workspace, evs)

    # timed region: the prefill with HIP events around the attention kernel
    # only (each recorded event drains the stream, so events around every
    # kernel would slow the step they measure)
    ev_a = events(2)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        run([None] * (2 * ai) + ev_a[s])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    attend_ms = sum(e0.elapsed_time(e1) for e0, e1 in ev_a) / steps
    ms = None
    if breakdown:
        # per-kernel breakdown, after the timed region: events around every kernel
        ev = events(2 * nk)
        torch.cuda.synchronize()
        for s in range(steps):
            run(ev[s])
        torch.cuda.synchronize()
        ms = {k: sum(ev[s][2 * i].elapsed_time(ev[s][2 * i + 1]) for s in range(steps)) / steps
              for i, k in enumerate(still.PREFILL_KERNELS)}
        ms["attend"] = attend_ms  # the timed region's own measurement
        # F^T is made by extra workgroups of the score launch: its pair of
        # events is recorded back to back and times nothing
        ms.pop("fmap_transpose", None)
    work = algorithmic_work(wl, bufs.sel.cpu().numpy())
    step_s = elapsed / steps
    att_tf = work["attend"] / (attend_ms * 1e-3) / 1e12
    out = {"workload": wl.name, "batch": wl.batch, "seq_len": wl.seq_len, "steps": steps,
           "ms_per_step": step_s * 1e3, "tokens_per_s": wl.batch * wl.seq_len / step_s,
           "attend_ms": attend_ms, "attend_tflops": att_tf,
           "attend_mfma_frac": att_tf / PEAK_BF16_TFLOPS,
           "layer_tflop": work["total"] / 1e12,
           "layer_mfma_frac": work["total"] / step_s / 1e12 / PEAK_BF16_TFLOPS,
           "hbm_floor_mb": (2 * wl.batch * wl.n_q_heads + 2 * wl.batch * wl.n_kv_heads) *
           wl.seq_len * wl.head_dim * 2 / 1e6}
    if ms is not None:
        out["kernels_ms"] = ms
    return wl, x, bufs, out, work


PEAK_FP32_VECTOR_TFLOPS = 157.3  # MI355X float32 vector


def backward_work(wl, lam, cap_chunks):
    """Algorithmic flops of still_backward's chunked form: every pair it
    visits one by one (band pairs, key in [b_c, t], from both sides: 22 d;
    kept-pool pairs: 10 d from the query side, 8 d from the kept-key pass),
    the chunk state terms (2 d^2 per head and query, 4 d^2 per kv head and
    key), the chunk deltas (2 d^2 per key, 2 d^2 per head and query) and the
    row work (8 d^2 per q or k row: features, their recompute, F dz, x^T dz)."""
    L, C, W, d = wl.seq_len, wl.chunk, wl.window, wl.head_dim
    band = pool = 0
    for c in range((L + C - 1) // C):
        x = c * C - W + 1
        cf = x // C if x >= 0 else 0
        t1 = min(L, c * C + C)
        n = t1 - c * C
        band += sum(t - cf * C + 1 for t in range(c * C, t1))
        pool += n * min(cf, cap_chunks) * lam
    B, Hq, Hkv = wl.batch, wl.n_q_heads, wl.n_kv_heads
    return (B * Hq * (band * 22 * d + pool * 18 * d) + B * Hq * L * 4 * d * d
            + B * Hkv * L * 6 * d * d + B * (Hq + Hkv) * L * 8 * d * d)


def run_backward_bench(torch, still, inputs, name, steps=5):
    """Time of the backward (gradients of q, k, v, F, gates) after a forward
    with partials, against the float32 vector peak (see backward_work)."""
    wl = inputs.WORKLOADS[name]
    p = still.params_for(wl, fp32_out=True)
    L, B, Hq, Hkv, d = wl.seq_len, wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    x = inputs.make_inputs(wl, device="cuda")
    dy = inputs.make_grad_output(wl, device="cuda")
    bufs = still.PrefillBuffers(p, L)
    lse_sa = torch.empty((B, Hq, L), device="cuda")
    lse_la = torch.empty((B, Hq, L), device="cuda")
    y_sa = torch.empty((B, Hq, L, d), device="cuda")
    y_la = torch.empty((B, Hq, L, d), device="cuda")
    still.still_prefill_partials(p, L, x["q"], x["k"], x["v"], x["fmap_w"], x["gate"], bufs.out,
                                 bufs.sel, bufs.score, bufs.state, bufs.workspace, y_sa, lse_sa,
                                 y_la, lse_la)
    del y_sa, y_la
    g = {"dq": torch.empty((B, Hq, L, d), device="cuda"),
         "dk": torch.empty((B, Hkv, L, d), device="cuda"),
         "dv": torch.empty((B, Hkv, L, d), device="cuda"),
         "dfmap": torch.empty((Hkv, d, d), device="cuda"), "dgate": torch.empty((Hq,), device="cuda")}
    ws = torch.empty(still.still_backward_workspace_bytes(p, L), dtype=torch.uint8, device="cuda")

    def run():
        still.still_backward(p, L, x["q"], x["k"], x["v"], x["fmap_w"], x["gate"], bufs.sel,
                             bufs.out, lse_sa, lse_la, dy, g["dq"], g["dk"], g["dv"], g["dfmap"],
                             g["dgate"], ws)
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    lam = still.still_lambda(p)
    cap = (wl.budget - wl.window) // lam if lam > 0 else 0
    flops = backward_work(wl, lam, cap)
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": wl.name, "steps": steps, "ms": ms, "tokens_per_s": B * L / (ms * 1e-3),
            "form": "chunked (prefix / suffix chunk states, band and kept-pool pairs one by one), "
                    "float32 vector ALU",
            "flops_per_launch": flops, "tflops": tf,
            "roofline": {"bound": "alu", "achieved": tf, "peak": PEAK_FP32_VECTOR_TFLOPS,
                         "unit": "TFLOP/s", "frac": tf / PEAK_FP32_VECTOR_TFLOPS}}


def run_latency_bench(torch, still, inputs, name, reps=50):
    """Wall time of one synchronised prefill of a small workload (median)."""
    wl = inputs.WORKLOADS[name]
    p = still.params_for(wl)
    x = inputs.make_inputs(wl, device="cuda")
    bufs = still.PrefillBuffers(p, wl.seq_len)
    for _ in range(5):
        still.run_prefill(p, x, bufs)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        still.run_prefill(p, x, bufs)
        torch.cuda.synchronize()
        ts.append(time.perf_counter() - t0)
    ts.sort()
    return {"workload": wl.name, "reps": reps, "median_ms": ts[len(ts) // 2] * 1e3,
            "min_ms": ts[0] * 1e3}


def measured_ceilings(torch):
    """What the chip reaches on plain work: a device copy (HBM read + write)
    and a large bf16 GEMM (hipBLASLt through torch)."""
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * n * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    m = 8192
    a = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    b = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    for _ in range(3):
        c = a @ b
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    gemm_tf = 2 * m ** 3 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b, c
    torch.cuda.empty_cache()
    return {"copy_gbs": copy_gbs, "copy_frac_of_spec": copy_gbs / PEAK_HBM_GBS,
            "gemm_bf16_tflops": gemm_tf, "gemm_frac_of_spec": gemm_tf / PEAK_BF16_TFLOPS,
            "gemm_shape": [m, m, m]}


def run_decode_bench(torch, still, inputs, n_steps):
    wl = inputs.WORKLOADS["decode_bf16_B64_ctx16K"]
    p = still.params_for(wl)
    x = inputs.make_inputs(wl, device="cuda")
    bufs = still.PrefillBuffers(p, wl.seq_len)
    still.run_prefill(p, x, bufs)
    del bufs.out, bufs.workspace
    toks = inputs.make_decode_tokens(wl, n_steps + 8, device="cuda")
    out = torch.empty((wl.batch, wl.n_q_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    sel = torch.empty((wl.batch, wl.n_kv_heads, still.still_lambda(p)), dtype=torch.int32,
                      device="cuda")
    # warm-up on a copy of the state
    st2 = bufs.state.clone()
    for s in range(8):
        still.still_decode_step(p, wl.seq_len + s, toks["q"][s], toks["k"][s], toks["v"][s],
                                x["fmap_w"], x["gate"], st2, out, sel)
    torch.cuda.synchronize()
    del st2
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for s in range(n_steps):
        still.still_decode_step(p, wl.seq_len + s, toks["q"][8 + s], toks["k"][8 + s],
                                toks["v"][8 + s], x["fmap_w"], x["gate"], bufs.state, out, sel)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = e0.elapsed_time(e1) / n_steps
    paged_ms = run_decode_paged(torch, still, wl, x, toks, n_steps)
    pool8_ms = run_decode_pool8(torch, still, wl, x, toks, n_steps)
    d, units = wl.head_dim, wl.batch * wl.n_kv_heads
    n_pool = 256  # 255 kept after the prefill, +1 at the boundary of step 0
    per_unit = (wl.window + n_pool) * 2 * d * 2 + d * d * 4 + d * 4
    io = (wl.batch * wl.n_q_heads * d * 2) * 2 + wl.batch * wl.n_kv_heads * d * 2 * 2
    step_bytes = units * per_unit + io
    # the 8-bit pool: codes and an exponent byte per kept row, the window band at bf16
    per_unit8 = wl.window * 2 * d * 2 + n_pool * 2 * (d + 1) + d * d * 4 + d * 4
    step_bytes8 = units * per_unit8 + io
    return {"workload": wl.name, "batch": wl.batch, "context": wl.seq_len, "steps": n_steps,
            "ms_per_step": step_ms, "tokens_per_s": wl.batch / (step_ms * 1e-3),
            "wall_s": wall, "algorithmic_bytes_per_step": step_bytes,
            "hbm_gbs": step_bytes / (step_ms * 1e-3) / 1e9,
            "hbm_frac": step_bytes / (step_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "traffic": measured_traffic("decode_kernel", "decode_llama8b_B64_ctx16K.md",
                                        DECODE_SOURCES),
            "pool8": {"ms_per_step": pool8_ms, "vs_full_pool": pool8_ms / step_ms,
                      "algorithmic_bytes_per_step": step_bytes8,
                      "hbm_gbs": step_bytes8 / (pool8_ms * 1e-3) / 1e9,
                      "hbm_frac": step_bytes8 / (pool8_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                      "layout": "kept K/V rows as E4M3 codes, one power-of-two scale byte per row"},
            "paged": {"ms_per_step": paged_ms, "hbm_gbs": step_bytes / (paged_ms * 1e-3) / 1e9,
                      "vs_unpaged": paged_ms / step_ms,
                      "layout": "kept pool in 16-row pages of a shared arena, "
                                "each unit's pages a seeded random permutation"}}


def run_decode_pool8(torch, still, wl, x, toks, n_steps):
    """The same decode steps with the kept pool as an 8-bit store
    (STILL_FLAG_POOL_FP8): a prefill of the same inputs with that flag,
    then the timed steps. Returns ms per step."""
    p = still.params_for(wl, flags=still.STILL_FLAG_POOL_FP8)
    bufs = still.PrefillBuffers(p, wl.seq_len)
    still.run_prefill(p, x, bufs)
    del bufs.out, bufs.workspace
    out = torch.empty((wl.batch, wl.n_q_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    sel = torch.empty((wl.batch, wl.n_kv_heads, still.still_lambda(p)), dtype=torch.int32,
                      device="cuda")
    st2 = bufs.state.clone()
    for s in range(8):
        still.still_decode_step(p, wl.seq_len + s, toks["q"][s], toks["k"][s], toks["v"][s],
                                x["fmap_w"], x["gate"], st2, out, sel)
    torch.cuda.synchronize()
    del st2
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for s in range(n_steps):
        still.still_decode_step(p, wl.seq_len + s, toks["q"][8 + s], toks["k"][8 + s],
                                toks["v"][8 + s], x["fmap_w"], x["gate"], bufs.state, out, sel)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n_steps


def run_decode_paged(torch, still, wl, x, toks, n_steps):
    """The same decode steps with the kept pool in pages
    (STILL_FLAG_PAGED_POOL): a paged prefill of the same inputs, every
    unit's pages mapped to a seeded permutation of the arena's pages, then
    the timed steps through still_decode_step_paged. Returns ms per step."""
    p = still.params_for(wl, flags=still.STILL_FLAG_PAGED_POOL)
    units, width = wl.batch * wl.n_kv_heads, still.pool_table_width(p)
    rows = still.STILL_POOL_PAGE_ROWS
    pages = torch.zeros((units * width, 2, rows, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    gen = torch.Generator().manual_seed(7)
    table = torch.randperm(units * width, generator=gen).to(torch.int32).view(units, width).cuda()
    bufs = still.PrefillBuffers(p, wl.seq_len)
    still.still_prefill_paged(p, wl.seq_len, x["q"], x["k"], x["v"], x["fmap_w"], x["gate"], bufs.out,
                              bufs.sel, bufs.score, bufs.state, pages, table, bufs.workspace)
    del bufs.out, bufs.workspace
    out = torch.empty((wl.batch, wl.n_q_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    sel = torch.empty((wl.batch, wl.n_kv_heads, still.still_lambda(p)), dtype=torch.int32,
                      device="cuda")
    st2 = bufs.state.clone()
    for s in range(8):
        still.still_decode_step_paged(p, wl.seq_len + s, toks["q"][s], toks["k"][s], toks["v"][s],
                                      x["fmap_w"], x["gate"], st2, pages, table, out, sel)
    torch.cuda.synchronize()
    del st2
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for s in range(n_steps):
        still.still_decode_step_paged(p, wl.seq_len + s, toks["q"][8 + s], toks["k"][8 + s],
                                      toks["v"][8 + s], x["fmap_w"], x["gate"], bufs.state, pages,
                                      table, out, sel)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n_steps


def run_cpu_baseline(wl, x):
    """The float64 recurrent oracle on the host cores: the whole 16K layer
    on every usable core (one (batch row, kv head) unit per thread), and two
    units on one thread, scaled to the layer."""
    from oracle import rec
    cores = len(os.sched_getaffinity(0))
    units = [(b, kv) for b in range(wl.batch) for kv in range(wl.n_kv_heads)]
    threads = max(1, min(cores, len(units)))
    xc = {k: v.cpu() for k, v in x.items()}

    def timed(us, n_threads):
        t0 = time.perf_counter()
        rec.prefill(xc["q"], xc["k"], xc["v"], xc["fmap_w"], xc["gate"], window=wl.window,
                    chunk=wl.chunk, budget=wl.budget, t_max=wl.t_max, units=us, n_threads=n_threads)
        return time.perf_counter() - t0

    wall_all = timed(units, threads)
    one = units[:2]
    wall_one = timed(one, 1) * len(units) / len(one)
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    tokens = wl.batch * wl.seq_len
    return {"value": tokens / wall_all, "unit": "tokens/s/layer", "cores": threads,
            "kind": "oracle", "usable_cores": cores, "cpu_model": model or "unknown",
            "wall_s_all_threads": wall_all, "wall_s_one_thread_est": wall_one,
            "one_thread_tokens_per_s": tokens / wall_one,
            "sample": "whole 16K layer (%d kv-head units, %d threads), float64 recurrent oracle "
                      "(%.1f s); one thread: 2 units timed, scaled to %d (%.1f s)"
                      % (len(units), threads, wall_all, len(units), wall_one)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--decode-steps", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the 4K / 64K prefill lines, the small-workload latency and the "
                         "measured ceilings")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes (HBM counter "
                         "calibration for rocprofv3 --pmc)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one MI355X: the layer runs on a single GPU and --gpus %d is "
              "not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_bytes > 0:
        src = torch.ones(args.copy_bytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_bytes, "launches": 3}))
        return
    from linear_attention_still_amd import inputs, still

    wl, x, bufs, c3, work = run_prefill_bench(torch, still, inputs, "llama8b_bf16_L16K",
                                              args.steps, args.warmup)
    tokens = wl.batch * wl.seq_len
    step_s = c3["ms_per_step"] * 1e-3
    achieved = work["attend"] / (c3["attend_ms"] * 1e-3) / 1e12
    res = {
        "metric": METRIC, "value": tokens / step_s, "unit": "tokens/s/layer", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": c3["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "seq_len": wl.seq_len,
                   "q_heads": wl.n_q_heads, "kv_heads": wl.n_kv_heads,
                   "head_dim": wl.head_dim, "window": wl.window, "chunk": wl.chunk,
                   "budget": wl.budget, "t_max": wl.t_max},
        "roofline": {"bound": "mfma", "kernel": "attend", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": measured_traffic("attend_kernel", "prefill_llama8b_L16K.md",
                                                 PREFILL_SOURCES),
                     "flops_per_launch": work["attend"]},
        "layer": {"algorithmic_tflop": work["total"] / 1e12,
                  "tflops": work["total"] / step_s / 1e12,
                  "mfma_frac": work["total"] / step_s / 1e12 / PEAK_BF16_TFLOPS,
                  "hbm_floor_mb": c3["hbm_floor_mb"]},
        "kernels_ms": c3["kernels_ms"],
    }
    del x, bufs
    torch.cuda.empty_cache()
    if not args.no_workloads:
        others = {}
        for name, steps, warmup in (("gqa_bf16_L4K", args.steps, 5),
                                    ("llama8b_bf16_L64K", max(3, args.steps // 4), 3)):
            _, xo, bo, r, _ = run_prefill_bench(torch, still, inputs, name, steps, warmup,
                                                breakdown=(name == "llama8b_bf16_L64K"))
            others[name] = r
            del xo, bo
            torch.cuda.empty_cache()
        c5 = others["llama8b_bf16_L64K"]
        c5["per_token_time_vs_16K"] = (c5["ms_per_step"] / c5["seq_len"]) / (
            c3["ms_per_step"] / c3["seq_len"])
        others["small_f32_L256"] = run_latency_bench(torch, still, inputs, "small_f32_L256")
        res["workloads"] = others
        res["ceilings"] = measured_ceilings(torch)
        # chunk-size sweep of the 16K workload (window, budget, T_max and
        # inputs unchanged; lambda = min(C, (m - W) / T_max))
        sweep = {}
        for C, wc in inputs.chunk_sweep().items():
            _, xs, bs, r, _ = run_prefill_bench(torch, still, inputs, wc, args.steps, 5)
            sweep[str(C)] = {"ms_per_step": r["ms_per_step"], "tokens_per_s": r["tokens_per_s"],
                             "lambda": still.still_lambda(still.params_for(wc)),
                             "attend_mfma_frac": r["attend_mfma_frac"],
                             "kernels_ms": r["kernels_ms"]}
            del xs, bs
            torch.cuda.empty_cache()
        res["chunk_sweep"] = sweep
    if not args.no_decode:
        res["decode"] = run_decode_bench(torch, still, inputs, args.decode_steps)
    if not args.no_workloads:
        res["backward"] = run_backward_bench(torch, still, inputs, "gqa_bf16_L4K")
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        xc = inputs.make_inputs(wl, device="cuda")
        res["cpu_baseline"] = run_cpu_baseline(wl, xc)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
