"""The kept pool in pages (still_prefill_paged, still_decode_step_paged), on
the GPU through the C ABI.

The kept tokens of the STILL article ("Delayed Chunk-Level Selection", the
budget of kept tokens) live, with STILL_FLAG_PAGED_POOL, in an arena of
16-row pages that the caller owns, reached through a page table per unit.
Paging moves rows, not arithmetic: every output, selection, score, state
word and kept row must equal the unpaged path's bit for bit (the unpaged
path is the one the parity tests hold to the oracle), and the decode
outputs are also checked against the oracle itself, to the default path's
bars.

The tables map the units' pages to a seeded permutation of the arena's pages
(so that a unit's rows are scattered), and the decode run maps them lazily:
only the pages of still_pool_rows(p, pos + 1) rows, before the step at pos.
A needed page left unmapped sets the unit's error word (meta[2] =
STILL_ESTATE) and the step leaves the state as it was.
"""
import numpy as np
import pytest
import torch

from linear_attention_still_amd import still
from linear_attention_still_amd.inputs import WORKLOADS, Workload, make_decode_tokens, make_inputs
from oracle import rec
from tests import _parity as P

pytestmark = pytest.mark.gpu

ROWS = still.STILL_POOL_PAGE_ROWS


def small(name, dtype, B, Hq, Hkv, d, L, W, C, m, t_max, out=0.01, seed=17):
    return Workload(name, dtype, B, Hq, Hkv, d, L, W, C, m, t_max, sigma=0.5,
                    outlier_frac=out, seed=seed)


# (workload, prefill length, decode steps): pools of 2, 1 and 10 pages per
# unit; the last fills its budget during the decode run.
PAGED_SHAPES = [
    (small("pg_f32", "f32", 1, 2, 1, 64, 90, 16, 32, 16 + 4 * 6, 6, out=0.0), 90, 70),
    (small("pg_bf16_d128", "bf16", 2, 8, 2, 128, 256, 64, 64, 64 + 8 * 2, 8), 256, 130),
    (small("pg_bf16_many_pages", "bf16", 2, 8, 2, 128, 600, 64, 32, 64 + 8 * 20, 20), 600, 100),
]


class Arena:
    """n_pages pages [n_pages, 2, ROWS, d] (key rows then value rows) and a
    table [U, width] of int32, -1 where no page is mapped."""

    def __init__(self, p, spare: int = 3, seed: int = 0):
        self.U = p.batch * p.n_kv_heads
        self.width = still.pool_table_width(p)
        self.n_pages = self.U * self.width + spare
        dt = torch.float32 if p.dtype == still.STILL_DTYPE_F32 else torch.bfloat16
        self.pages = torch.zeros((self.n_pages, 2, ROWS, p.head_dim), dtype=dt, device="cuda")
        gen = torch.Generator().manual_seed(seed)
        perm = torch.randperm(self.n_pages, generator=gen)[:self.U * self.width]
        self.assign = perm.view(self.U, self.width).to(torch.int32)
        self.table_host = torch.full((self.U, self.width), -1, dtype=torch.int32)
        self.table = self.table_host.cuda()

    def map_rows(self, n_rows: int):
        """Maps the pages of pool rows [0, n_rows) of every unit."""
        n = -(-n_rows // ROWS)
        self.table_host[:, :n] = self.assign[:, :n]
        self.table.copy_(self.table_host)

    def rows(self, n_rows: int):
        """Pool keys and values [U, n_rows, d] read back through the table."""
        idx = torch.arange(n_rows)
        pg = self.table_host[:, idx // ROWS].long().cuda()
        off = (idx % ROWS).cuda()
        return self.pages[pg, 0, off], self.pages[pg, 1, off]


def paged_params(wl, fp32_out=True):
    return still.params_for(wl, fp32_out=fp32_out, flags=still.STILL_FLAG_PAGED_POOL)


def paged_prefill(wl, xd, arena, fp32_out=True):
    p = paged_params(wl, fp32_out)
    L = xd["q"].shape[2]
    print("  gpu paged prefill %s L=%d pages=%d" % (wl.name, L, arena.n_pages), flush=True)
    bufs = still.PrefillBuffers(p, L)
    still.still_prefill_paged(p, L, xd["q"], xd["k"], xd["v"], xd["fmap_w"], xd["gate"], bufs.out,
                              bufs.sel if bufs.sel.numel() else None, bufs.score, bufs.state,
                              arena.pages, arena.table, bufs.workspace)
    torch.cuda.synchronize()
    return p, bufs


STATE_KEYS = ("S", "z", "pool_pos", "ring_k", "ring_v", "ring_phi", "ring_flag", "pending", "meta")


def assert_same_state(p_paged, st_paged, p_plain, st_plain, arena, n_rows, what):
    a, b = still.state_views(p_paged, st_paged), still.state_views(p_plain, st_plain)
    for key in STATE_KEYS:  # bit patterns (unused pending slots hold NaN)
        assert torch.equal(a[key].view(torch.uint8), b[key].view(torch.uint8)), "%s: %s" % (what, key)
    pk, pv = arena.rows(n_rows)
    assert torch.equal(pk, b["pool_k"][:, :n_rows]), "%s: pool keys" % what
    assert torch.equal(pv, b["pool_v"][:, :n_rows]), "%s: pool values" % what


@pytest.mark.parametrize("case", PAGED_SHAPES, ids=[c[0].name for c in PAGED_SHAPES])
def test_paged_prefill_and_decode_match_unpaged(case):
    """Prefill, then decode steps over chunk boundaries with the pages mapped
    as the pool grows: bitwise equal to the unpaged path at every step, and
    the decode outputs and selections against the oracle."""
    wl, L0, n = case
    x = make_inputs(wl, seq_len=L0)
    toks = make_decode_tokens(wl, n)
    xd = {k: v.cuda() for k, v in x.items()}
    td = {k: v.cuda() for k, v in toks.items()}
    g = P.gpu_prefill(wl, x, fp32_out=True, keep_device=True)
    p0 = g["_params"]
    arena = Arena(p0, seed=wl.seed)
    n_rows = still.still_pool_rows(p0, L0)
    arena.map_rows(n_rows)
    p, bufs = paged_prefill(wl, xd, arena)
    assert torch.equal(bufs.out, g["y"])
    assert torch.equal(bufs.sel, g["sel"])
    assert torch.equal(bufs.score, g["score"])
    assert_same_state(p, bufs.state, p0, g["_state"], arena, n_rows, "prefill")
    assert int(still.state_views(p, bufs.state)["meta"][:, 2].abs().max()) == 0

    lam = still.still_lambda(p)
    B, Hq, Hkv, d = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    outs, sels = [], []
    for s in range(n):
        pos = L0 + s
        arena.map_rows(still.still_pool_rows(p, pos + 1))
        out_a = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
        out_b = torch.empty_like(out_a)
        sel_a = torch.empty((B, Hkv, max(lam, 1)), dtype=torch.int32, device="cuda")
        sel_b = torch.empty_like(sel_a)
        still.still_decode_step_paged(p, pos, td["q"][s], td["k"][s], td["v"][s], xd["fmap_w"],
                                      xd["gate"], bufs.state, arena.pages, arena.table, out_a,
                                      sel_a if lam > 0 else None)
        still.still_decode_step(p0, pos, td["q"][s], td["k"][s], td["v"][s], xd["fmap_w"],
                                xd["gate"], g["_state"], out_b, sel_b if lam > 0 else None)
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b), "step %d" % s
        if lam > 0 and pos % wl.chunk == 0:
            assert torch.equal(sel_a[..., :lam], sel_b[..., :lam]), "step %d" % s
        outs.append(out_a)
        sels.append(sel_a[..., :lam])
    n_rows = still.still_pool_rows(p, L0 + n)
    assert_same_state(p, bufs.state, p0, g["_state"], arena, n_rows, "decode")
    print("    %d decode steps bitwise equal; %d pool rows in %d pages per unit"
          % (n, n_rows, -(-n_rows // ROWS)), flush=True)

    outs, sels = torch.stack(outs).cpu(), torch.stack(sels).cpu()
    units = [(b, kv) for b in range(B) for kv in range(Hkv)]
    qs, ks, vs, Fs, gs = P.concat_units(x, toks, wl, units)
    o = rec.run_units(qs, ks, vs, Fs, gs, window=wl.window, chunk=wl.chunk, budget=wl.budget,
                      t_max=wl.t_max, n_threads=P.n_threads())
    G = wl.group
    yg = np.stack([outs[:, b, kv * G:(kv + 1) * G].numpy().transpose(1, 0, 2) for b, kv in units])
    P.check_outputs(yg, o["y"][:, :, L0:], wl.dtype, True, "paged decode y")
    for s in range(n):
        t = L0 + s
        if t % wl.chunk == 0 and o["lam"] > 0:
            got = np.stack([sels[s, b, kv].numpy() for b, kv in units])
            assert np.array_equal(got, o["sel"][:, t // wl.chunk - 1]), s


def test_paged_prefill_full_size_matches_unpaged():
    """The 16K-token Llama-8B-shaped prefill (32 query heads, 8 kv heads,
    d = 128, W = C = 64, budget 512) through the paged entry, in the launch
    configuration of the plain one: every output, score, selection, state
    word and kept row equal to the unpaged run's."""
    wl = WORKLOADS["llama8b_bf16_L16K"]
    x = make_inputs(wl, device="cuda")
    g = P.gpu_prefill(wl, x, fp32_out=False, keep_device=True)
    p0 = g["_params"]
    arena = Arena(p0, seed=5)
    n_rows = still.still_pool_rows(p0, wl.seq_len)
    assert n_rows == (wl.seq_len - 1) // wl.chunk  # lambda = 1: one row per decided chunk
    arena.map_rows(n_rows)
    p, bufs = paged_prefill(wl, x, arena, fp32_out=False)
    assert torch.equal(bufs.out, g["y"])
    assert torch.equal(bufs.sel, g["sel"])
    assert torch.equal(bufs.score, g["score"])
    assert_same_state(p, bufs.state, p0, g["_state"], arena, n_rows, "16K prefill")


def test_unmapped_page_sets_the_error_word():
    """A pool row without a page: the prefill marks the unit (meta[2] =
    STILL_ESTATE, other units clean); a decode step whose boundary appends
    into an unmapped page marks the unit and leaves the position where it
    was, and every later step on that state does nothing."""
    wl, L0, _ = PAGED_SHAPES[2]
    x = make_inputs(wl, seq_len=L0)
    xd = {k: v.cuda() for k, v in x.items()}
    p = paged_params(wl)
    n_rows = still.still_pool_rows(p, L0)
    assert n_rows % ROWS == 0  # the next boundary opens a new page

    arena = Arena(p, seed=1)
    arena.map_rows(n_rows)
    arena.table_host[1, (n_rows - 1) // ROWS] = -1  # unit 1 misses its last needed page
    arena.table.copy_(arena.table_host)
    _, bufs = paged_prefill(wl, xd, arena)
    meta = still.state_views(p, bufs.state)["meta"].cpu()
    assert int(meta[1, 2]) == still.STILL_ESTATE
    assert all(int(meta[u, 2]) == 0 for u in range(arena.U) if u != 1)

    arena = Arena(p, seed=2)
    arena.map_rows(n_rows)  # but not the page the next boundary needs
    _, bufs = paged_prefill(wl, xd, arena)
    toks = make_decode_tokens(wl, wl.chunk + 2)
    td = {k: v.cuda() for k, v in toks.items()}
    B, Hq, d = wl.batch, wl.n_q_heads, wl.head_dim
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    lam = still.still_lambda(p)
    sel = torch.empty((B, wl.n_kv_heads, lam), dtype=torch.int32, device="cuda")
    t_b = -(-L0 // wl.chunk) * wl.chunk  # first chunk boundary at or after L0
    for s in range(t_b - L0 + 2):
        still.still_decode_step_paged(p, L0 + s, td["q"][s], td["k"][s], td["v"][s], xd["fmap_w"],
                                      xd["gate"], bufs.state, arena.pages, arena.table, out, sel)
    torch.cuda.synchronize()
    meta = still.state_views(p, bufs.state)["meta"].cpu()
    for u in range(arena.U):
        assert int(meta[u, 2]) == still.STILL_ESTATE, u
        assert int(meta[u, 0]) == t_b, u  # the boundary step and those after it were skipped
        assert int(meta[u, 1]) == n_rows, u
