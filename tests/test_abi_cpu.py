"""C-ABI checks that need no GPU: the library loads, exports every function
the header declares, and validates arguments on the host before any launch.
"""
import ctypes
import os
import re

import pytest

from linear_attention_still_amd import still
from linear_attention_still_amd.inputs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    with open(os.path.join(ROOT, "include", "still.h")) as fh:
        text = fh.read()
    return sorted(set(re.findall(r"^\s*(?:int|int64_t|const char\*)\s+(still_\w+)\s*\(",
                                 text, re.M)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert {"still_prefill", "still_decode_step", "still_lambda", "still_state_bytes",
            "still_workspace_bytes", "still_state_layout_get", "still_status_str"} <= set(names)
    L = still.lib()
    for n in names:
        assert hasattr(L, n), n


def test_struct_sizes_match_header():
    assert ctypes.sizeof(still.still_params) == 13 * 4
    assert ctypes.sizeof(still.still_state_layout) == 12 * 8 + 8


def base_params(**kw):
    wl = WORKLOADS["llama8b_bf16_L16K"]
    p = still.params_for(wl)
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def test_lambda_values():
    assert still.still_lambda(still.params_for(WORKLOADS["small_f32_L256"])) == 6
    assert still.still_lambda(still.params_for(WORKLOADS["gqa_bf16_L4K"])) == 3
    assert still.still_lambda(still.params_for(WORKLOADS["llama8b_bf16_L16K"])) == 1
    assert still.still_lambda(still.params_for(WORKLOADS["llama8b_bf16_L64K"])) == 1
    assert still.still_lambda(base_params(budget=64 + 64 * 1000, t_max=2)) == 64  # capped at C
    assert still.still_lambda(base_params(budget=64)) == 0


@pytest.mark.parametrize("field,value,rc", [
    ("abi_version", 2, still.STILL_EINVAL),
    ("dtype", 7, still.STILL_EINVAL),
    ("batch", 0, still.STILL_EINVAL),
    ("n_q_heads", 30, still.STILL_EINVAL),
    ("window", 0, still.STILL_EINVAL),
    ("budget", 10, still.STILL_EINVAL),
    ("t_max", 0, still.STILL_EINVAL),
    ("head_dim", 96, still.STILL_EUNSUPPORTED),
    ("chunk", 48, still.STILL_EUNSUPPORTED),
    ("window", 300, still.STILL_EUNSUPPORTED),
])
def test_invalid_params_rejected(field, value, rc):
    p = base_params(**{field: value})
    L = still.lib()
    assert L.still_lambda(ctypes.byref(p)) == rc
    assert L.still_state_bytes(ctypes.byref(p)) == rc
    assert L.still_workspace_bytes(ctypes.byref(p), 1024) == rc


def test_f32_head_dim_128_unsupported():
    p = still.make_params(dtype="f32", batch=1, n_q_heads=1, n_kv_heads=1, head_dim=128,
                          window=16, chunk=32, budget=64, t_max=8)
    assert still.lib().still_lambda(ctypes.byref(p)) == still.STILL_EUNSUPPORTED


def test_state_layout_and_sizes():
    p = still.params_for(WORKLOADS["decode_bf16_B64_ctx16K"])
    lay = still.still_state_layout_get(p)
    assert lay.ring_slots == 64 + 2 * 64 and lay.pool_slots == 512 - 64
    offs = [lay.S, lay.z, lay.pool_k, lay.pool_v, lay.pool_pos, lay.ring_k, lay.ring_v,
            lay.ring_phi, lay.ring_flag, lay.pending, lay.meta]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert lay.pool_v - lay.pool_k >= 448 * 128 * 2
    assert lay.unit_bytes >= lay.meta + 32
    assert still.still_state_bytes(p) == lay.unit_bytes * 64 * 8
    assert still.still_workspace_bytes(p, 0) == 0
    assert still.still_workspace_bytes(p, 16384) > 64 * 8 * 16384 * 9


def test_prefill_validates_before_any_launch():
    """Null pointers, bad lengths and a short workspace are rejected on the
    host (these calls make no HIP call, so they work without a GPU)."""
    p = still.params_for(WORKLOADS["small_f32_L256"])
    L = still.lib()
    fake = ctypes.c_void_p(1 << 20)
    args = [fake] * 10
    ws = still.still_workspace_bytes(p, 256)
    rc = L.still_prefill(ctypes.byref(p), 256, *([None] + args[1:]), ws, None)
    assert rc == still.STILL_EINVAL
    rc = L.still_prefill(ctypes.byref(p), 0, *args, ws, None)
    assert rc == still.STILL_EINVAL
    rc = L.still_prefill(ctypes.byref(p), 256, *args, ws - 1, None)
    assert rc == still.STILL_EWORKSPACE
    odd = ctypes.c_void_p((1 << 20) + 4)
    rc = L.still_prefill(ctypes.byref(p), 256, *([odd] + args[1:]), ws, None)
    assert rc == still.STILL_EINVAL


def test_decode_validates_before_any_launch():
    p = still.params_for(WORKLOADS["decode_bf16_B64_ctx16K"])
    L = still.lib()
    fake = ctypes.c_void_p(1 << 20)
    rc = L.still_decode_step(ctypes.byref(p), 0, *([fake] * 9), 0, None)
    assert rc == still.STILL_EINVAL
    rc = L.still_decode_step(ctypes.byref(p), 16384, *([None] + [fake] * 8), 0, None)
    assert rc == still.STILL_EINVAL


def test_status_strings():
    for rc in (0, -1, -2, -3, -4, -5):
        assert still.still_status_str(rc) != "unknown status"
    assert still.still_status_str(42) == "unknown status"


def test_noalloc_rejects_oversize_before_any_hip_call():
    """still_prefill_noalloc refuses a problem whose workspace exceeds its
    static scratch before touching the device (runs without a GPU)."""
    p = still.make_params(dtype="bf16", batch=4, n_q_heads=32, n_kv_heads=8, head_dim=128,
                          window=128, chunk=128, budget=1024, t_max=512)
    assert still.still_workspace_bytes(p, 65536) > still.still_noalloc_scratch_bytes()
    rc = still.lib().still_prefill_noalloc(ctypes.byref(p), 65536, *([ctypes.c_void_p(256)] * 10))
    assert rc == still.STILL_ESCRATCH
    assert "scratch" in still.still_status_str(rc)


def test_branch_flags_validated_before_any_hip_call():
    """Unknown flag bits and the two merges at once are rejected by every
    entry; the separate-branch partials refuse the softmax-only variant; the
    decode step refuses the sum merge (it keeps one normaliser)."""
    L = still.lib()
    fake = ctypes.c_void_p(1 << 20)
    wl = WORKLOADS["small_f32_L256"]
    for bad in (still.STILL_FLAG_SOFTMAX_ONLY | still.STILL_FLAG_MERGE_SUM, 8, 1 << 31):
        p = still.params_for(wl, flags=bad)
        assert L.still_lambda(ctypes.byref(p)) == still.STILL_EINVAL
        assert L.still_workspace_bytes(ctypes.byref(p), 256) == still.STILL_EINVAL
        assert L.still_prefill(ctypes.byref(p), 256, *([fake] * 10), 1 << 30, None) == still.STILL_EINVAL
    p = still.params_for(wl, flags=still.STILL_FLAG_SOFTMAX_ONLY)
    ws = still.still_workspace_bytes(p, 256)
    rc = L.still_prefill_partials(ctypes.byref(p), 256, *([fake] * 10), ws, None, *([fake] * 4))
    assert rc == still.STILL_EINVAL
    p = still.params_for(wl)
    rc = L.still_prefill_partials(ctypes.byref(p), 256, *([fake] * 10), ws, None, fake, None, fake, fake)
    assert rc == still.STILL_EINVAL  # all four partial outputs are required
    p = still.params_for(WORKLOADS["decode_bf16_B64_ctx16K"], flags=still.STILL_FLAG_MERGE_SUM)
    rc = L.still_decode_step(ctypes.byref(p), 16384, *([fake] * 9), 0, None)
    assert rc == still.STILL_EUNSUPPORTED


def test_routing_flags_validated_before_any_hip_call():
    """Routing metrics above the last one are rejected; the caller's scores
    (external routing) are a required prefill input and are refused by the
    decode step."""
    L = still.lib()
    fake = ctypes.c_void_p(1 << 20)
    wl = WORKLOADS["small_f32_L256"]
    for r in range(6):
        p = still.params_for(wl, flags=still.route_flag(list(still.ROUTES)[r]))
        assert L.still_lambda(ctypes.byref(p)) >= 0
    p = still.params_for(wl, flags=6 << 8)
    assert L.still_lambda(ctypes.byref(p)) == still.STILL_EINVAL
    p = still.params_for(wl, flags=still.route_flag("external"))
    ws = still.still_workspace_bytes(p, 256)
    args = [fake] * 10
    args[7] = None  # no score buffer
    assert L.still_prefill(ctypes.byref(p), 256, *args, ws, None) == still.STILL_EINVAL
    p = still.params_for(WORKLOADS["decode_bf16_B64_ctx16K"], flags=still.route_flag("external"))
    rc = L.still_decode_step(ctypes.byref(p), 16384, *([fake] * 9), 0, None)
    assert rc == still.STILL_EUNSUPPORTED


def test_ragged_entries_validate_before_any_hip_call():
    """Varlen prefill checks every row's length (and the kept-index buffer a
    later row would need) before the first row runs; multi-token decode
    checks its token count and host position."""
    L = still.lib()
    fake = ctypes.c_void_p(1 << 20)
    wl = WORKLOADS["small_f32_L256"]
    p = still.make_params(dtype="bf16", batch=3, n_q_heads=8, n_kv_heads=2, head_dim=128,
                          window=64, chunk=64, budget=64 + 48, t_max=16)
    lens = [300, 1, 777]
    ws = still.still_workspace_bytes_varlen(p, lens)
    p1 = still.make_params(dtype="bf16", batch=1, n_q_heads=8, n_kv_heads=2, head_dim=128,
                           window=64, chunk=64, budget=64 + 48, t_max=16)
    assert ws == still.still_workspace_bytes(p1, 777)
    for bad in ([300, 0, 777], [300, -5, 1]):
        assert L.still_workspace_bytes_varlen(ctypes.byref(p), still._lens(bad)) == still.STILL_EINVAL
        assert L.still_prefill_varlen(ctypes.byref(p), still._lens(bad), *([fake] * 10), ws,
                                      None) == still.STILL_EINVAL
    assert L.still_prefill_varlen(ctypes.byref(p), still._lens(lens), *([fake] * 10), ws - 1,
                                  None) == still.STILL_EWORKSPACE
    args = [fake] * 10
    args[6] = None  # no kept-index buffer: row 0 already decides chunks
    assert L.still_prefill_varlen(ctypes.byref(p), still._lens(lens), *args, ws,
                                  None) == still.STILL_EINVAL
    p = still.params_for(WORKLOADS["decode_bf16_B64_ctx16K"])
    f8 = [fake] * 8  # q, k, v, fmap_w, gate, state, out, sel_new (then the stream)
    assert L.still_decode_tokens(ctypes.byref(p), 16384, None, 0, *f8, None) == still.STILL_EINVAL
    assert L.still_decode_tokens(ctypes.byref(p), 0, None, 4, *f8, None) == still.STILL_EINVAL
    odd = ctypes.c_void_p((1 << 20) + 2)
    assert L.still_decode_tokens(ctypes.byref(p), 0, odd, 4, *f8, None) == still.STILL_EINVAL


def test_gated_entries_validate_before_any_hip_call():
    """The output-gated prefill and decode step require their gate and a
    16-byte aligned one; their other checks are those of the plain entries."""
    L = still.lib()
    fake = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 8)
    p = still.params_for(WORKLOADS["small_f32_L256"])
    ws = still.still_workspace_bytes(p, 256)
    args = [fake] * 11  # q, k, v, fmap_w, gate, out_gate, out, sel_idx, score, state, workspace
    for bad in (None, odd):
        args[5] = bad
        assert L.still_prefill_gated(ctypes.byref(p), 256, *args, ws, None) == still.STILL_EINVAL
    args[5] = fake
    assert L.still_prefill_gated(ctypes.byref(p), 256, *args, ws - 1, None) == still.STILL_EWORKSPACE
    p = still.params_for(WORKLOADS["decode_bf16_B64_ctx16K"])
    f9 = [fake] * 9  # q, k, v, fmap_w, gate, out_gate | decay, state, out, sel_new (then the stream)
    for bad in (None, odd):
        f9[5] = bad
        assert L.still_decode_step_gated(ctypes.byref(p), 16384, *f9, None) == still.STILL_EINVAL
    f9[5] = fake
    assert L.still_decode_step_gated(ctypes.byref(p), 0, *f9, None) == still.STILL_EINVAL
    p = still.params_for(WORKLOADS["decode_bf16_B64_ctx16K"], flags=still.STILL_FLAG_MERGE_SUM)
    assert L.still_decode_step_gated(ctypes.byref(p), 16384, *f9, None) == still.STILL_EUNSUPPORTED


def test_decay_entries_validate_before_any_hip_call():
    """The forget-gated prefill and decode step require their factors, 16-byte
    aligned; their other checks are those of the plain entries."""
    L = still.lib()
    fake = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 4)
    p = still.params_for(WORKLOADS["small_f32_L256"])
    ws = still.still_workspace_bytes(p, 256)
    args = [fake] * 11  # q, k, v, fmap_w, gate, decay, out, sel_idx, score, state, workspace
    for bad in (None, odd):
        args[5] = bad
        assert L.still_prefill_decay(ctypes.byref(p), 256, *args, ws, None) == still.STILL_EINVAL
    args[5] = fake
    assert L.still_prefill_decay(ctypes.byref(p), 256, *args, ws - 1, None) == still.STILL_EWORKSPACE
    p = still.params_for(WORKLOADS["decode_bf16_B64_ctx16K"])
    f9 = [fake] * 9
    for bad in (None, odd):
        f9[5] = bad
        assert L.still_decode_step_decay(ctypes.byref(p), 16384, *f9, None) == still.STILL_EINVAL
    f9[5] = fake
    p = still.params_for(WORKLOADS["decode_bf16_B64_ctx16K"], flags=still.STILL_FLAG_MERGE_SUM)
    assert L.still_decode_step_decay(ctypes.byref(p), 16384, *f9, None) == still.STILL_EUNSUPPORTED


def test_decay_refuses_the_sum_merge():
    L = still.lib()
    fake = ctypes.c_void_p(1 << 20)
    p = still.params_for(WORKLOADS["small_f32_L256"], flags=still.STILL_FLAG_MERGE_SUM)
    ws = still.still_workspace_bytes(p, 256)
    assert L.still_prefill_decay(ctypes.byref(p), 256, *([fake] * 11), ws, None) == still.STILL_EUNSUPPORTED


def test_paged_entries_validate_before_any_hip_call():
    """The paged flag and the paged entries go together; the arena is 16-byte
    aligned and its page count fits 31-bit byte offsets; the table is int32
    aligned. The other checks are those of the plain entries."""
    L = still.lib()
    fake = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 8)
    wl = WORKLOADS["small_f32_L256"]
    plain = still.params_for(wl)
    p = still.params_for(wl, flags=still.STILL_FLAG_PAGED_POOL)
    ws = still.still_workspace_bytes(p, 256)
    page_bytes = 2 * still.STILL_POOL_PAGE_ROWS * wl.head_dim * 4

    def pre(pp, arena=fake, table=fake, n_pages=4, wsb=ws):
        # q, k, v, fmap_w, gate, out, sel_idx, score, state, then the pages
        return L.still_prefill_paged(ctypes.byref(pp), 256, *([fake] * 9), arena, table, n_pages,
                                     fake, wsb, None)
    assert pre(plain) == still.STILL_EINVAL  # paged entry, unpaged params
    args = [fake] * 9
    assert L.still_prefill(ctypes.byref(p), 256, *args, fake, ws, None) == still.STILL_EINVAL
    assert pre(p, arena=None) == still.STILL_EINVAL
    assert pre(p, arena=odd) == still.STILL_EINVAL
    assert pre(p, table=None) == still.STILL_EINVAL
    assert pre(p, table=ctypes.c_void_p((1 << 20) + 2)) == still.STILL_EINVAL
    assert pre(p, n_pages=0) == still.STILL_EINVAL
    assert pre(p, n_pages=(1 << 31) // page_bytes) == still.STILL_EINVAL
    assert pre(p, wsb=ws - 1) == still.STILL_EWORKSPACE

    pd = still.params_for(WORKLOADS["decode_bf16_B64_ctx16K"])
    pdp = still.params_for(WORKLOADS["decode_bf16_B64_ctx16K"], flags=still.STILL_FLAG_PAGED_POOL)

    def dec(pp, arena=fake, n_pages=4, pos=16384):
        # q, k, v, fmap_w, gate, state, then the pages, out, sel_new
        return L.still_decode_step_paged(ctypes.byref(pp), pos, *([fake] * 6), arena, fake, n_pages,
                                         fake, fake, None)
    assert dec(pd) == still.STILL_EINVAL
    assert L.still_decode_step(ctypes.byref(pdp), 16384, *([fake] * 9), 1 << 30, None) == still.STILL_EINVAL
    assert dec(pdp, arena=odd) == still.STILL_EINVAL
    assert dec(pdp, n_pages=0) == still.STILL_EINVAL
    assert dec(pdp, pos=0) == still.STILL_EINVAL
    # the ragged and allocation-free entries keep their pool in the state
    assert L.still_prefill_noalloc(ctypes.byref(p), 256, *args, None) == still.STILL_EINVAL


def test_paged_params_state_and_limits():
    """A paged pool leaves its rows out of the state; a table wider than 256
    pages per unit is refused."""
    wl = WORKLOADS["small_f32_L256"]
    plain = still.params_for(wl)
    p = still.params_for(wl, flags=still.STILL_FLAG_PAGED_POOL)
    P = wl.budget - wl.window
    units = wl.batch * wl.n_kv_heads
    assert still.still_state_bytes(plain) - still.still_state_bytes(p) >= 2 * P * wl.head_dim * 4 * units
    lay = still.still_state_layout_get(p)
    assert lay.pool_k == lay.pool_v
    big = still.make_params(dtype="bf16", batch=1, n_q_heads=8, n_kv_heads=1, head_dim=128,
                            window=64, chunk=64, budget=64 + 256 * 16 + 1, t_max=128,
                            flags=still.STILL_FLAG_PAGED_POOL)
    with pytest.raises(still.StillError):
        still.still_state_bytes(big)
    ok = still.make_params(dtype="bf16", batch=1, n_q_heads=8, n_kv_heads=1, head_dim=128,
                           window=64, chunk=64, budget=64 + 256 * 16, t_max=128,
                           flags=still.STILL_FLAG_PAGED_POOL)
    assert still.pool_table_width(ok) == 256
    assert still.still_state_bytes(ok) > 0


def test_pool_rows_counts_lambda_rows_per_decided_chunk():
    """Chunk c is decided once chunk c + 1 has begun: after n tokens,
    (n - 1) // C chunks are decided, each adding lambda rows until the
    budget's chunks are used up."""
    wl = WORKLOADS["small_f32_L256"]
    p = still.params_for(wl)
    lam, C = still.still_lambda(p), wl.chunk
    cap = (wl.budget - wl.window) // lam
    for n in (0, 1, C, C + 1, 2 * C, 2 * C + 1, 5 * C + 3, 10 ** 6):
        n_dec = (n - 1) // C if n > 0 else 0
        assert still.still_pool_rows(p, n) == lam * min(n_dec, cap), n
    with pytest.raises(still.StillError):
        still.still_pool_rows(p, -1)


def test_pool_fp8_params_and_layout():
    """The 8-bit pool takes bf16 data and an unpaged pool; its pool regions
    hold (budget - window) rows of head_dim codes plus one exponent byte
    per row."""
    wl = WORKLOADS["decode_bf16_B64_ctx16K"]
    plain = still.params_for(wl)
    p8 = still.params_for(wl, flags=still.STILL_FLAG_POOL_FP8)
    P, d = wl.budget - wl.window, wl.head_dim
    lay, lay0 = still.still_state_layout_get(p8), still.still_state_layout_get(plain)
    assert lay.pool_v - lay.pool_k >= P * (d + 1) and lay.pool_v - lay.pool_k < P * (d + 1) + 256
    assert lay0.pool_v - lay0.pool_k >= P * d * 2
    assert still.still_state_bytes(p8) < still.still_state_bytes(plain)
    with pytest.raises(still.StillError):
        still.still_state_bytes(still.params_for(WORKLOADS["small_f32_L256"], flags=still.STILL_FLAG_POOL_FP8))
    with pytest.raises(still.StillError):
        still.still_state_bytes(still.params_for(
            wl, flags=still.STILL_FLAG_POOL_FP8 | still.STILL_FLAG_PAGED_POOL))
