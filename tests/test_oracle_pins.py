"""Pins of the oracle against facts fixed outside it (CPU only).

Each test checks the oracle against something other than itself: a
hand-worked example, a closed form, a library routine a special case reduces
to (scipy's relative entropy, torch's scaled-dot-product attention and
softmax), invariants the pages state, or the other oracle form on random
tiny shapes. Citations name the article "STILL: Content-Aware Intra-Layer
Hybrid Attention for Efficient LLM Linearization" by section.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import rel_entr, softmax as sp_softmax

from oracle import bf, rec

HERE = os.path.dirname(os.path.abspath(__file__))
EPS = 1e-6


def rand_inputs(rng, B, Hq, Hkv, L, d, sigma=0.5, outliers=0):
    def tok(H):
        z = rng.standard_normal((B, H, L, d))
        r = np.exp(sigma * rng.standard_normal((B, H, L, 1)))
        if outliers:
            for b in range(B):
                r[b, :, rng.choice(L, outliers, replace=False)] *= 8.0
        return (z * r).astype(np.float32).astype(np.float64)
    q, k, v = tok(Hq), tok(Hkv), tok(Hkv)
    F = (rng.standard_normal((Hkv, d, d)) / math.sqrt(d)).astype(np.float32).astype(np.float64)
    g = rng.uniform(0, 1, Hq).astype(np.float32).astype(np.float64)
    return q, k, v, F, g


def phi_torch(x, F):
    """NP-Map via torch's softmax: ||x|| * softmax(xF) / ||softmax(xF)||."""
    x = torch.as_tensor(x, dtype=torch.float64)
    u = torch.softmax(x @ torch.as_tensor(F, dtype=torch.float64), dim=-1)
    return (x.norm(dim=-1, keepdim=True) * u / u.norm(dim=-1, keepdim=True)).numpy()


def sdpa(q, k, v, mask, scale):
    """torch's scaled-dot-product attention in fp64 on the CPU."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.as_tensor(q), torch.as_tensor(k), torch.as_tensor(v),
        attn_mask=torch.as_tensor(mask), scale=scale).numpy()


# ---------------------------------------------------------------- score ----

def test_score_hand_example():
    """W = 2, logits (0, ln 3) with the token last: p = 3/4, so the score is
    the two-point KL 3/4 ln(3/4 / eps) + 1/4 ln(1/4 / (1 - eps))."""
    s = np.array([0.0, math.log(3.0)])
    want = 0.75 * math.log(0.75 / EPS) + 0.25 * math.log(0.25 / (1 - EPS))
    assert bf.saliency_kl(s, 1, EPS) == pytest.approx(want, rel=1e-14)


@pytest.mark.parametrize("n", [2, 3, 16, 64])
def test_score_is_bernoulli_relative_entropy(n):
    """The literal KL over the window equals KL(Bern(p) || Bern(eps)) with
    p the self entry of the window softmax (scipy's rel_entr)."""
    rng = np.random.default_rng(n)
    for _ in range(20):
        s = rng.standard_normal(n) * rng.uniform(0.1, 10)
        idx = int(rng.integers(n))
        p = sp_softmax(s)[idx]
        want = rel_entr(p, EPS) + rel_entr(1 - p, 1 - EPS)
        assert bf.saliency_kl(s, idx, EPS) == pytest.approx(want, rel=1e-10, abs=1e-12)


def test_score_single_key_window():
    assert bf.saliency_kl(np.array([3.7]), 0, EPS) == pytest.approx(math.log(1 / EPS), rel=1e-15)


def test_score_monotone_in_self_probability():
    """Proposition 1 (section "Theoretical Guarantee"): the score increases
    with the local self-attention probability p for p > eps."""
    p_vals = np.linspace(2 * EPS, 1.0, 400)
    scores = []
    for p in p_vals:
        # window of 4: self logit chosen so the self probability is p
        others = np.zeros(3)
        s_self = math.log(p / (1 - p) * 3.0) if p < 1 else 50.0
        scores.append(bf.saliency_kl(np.concatenate([others, [s_self]]), 3, EPS))
    assert np.all(np.diff(scores) > 0)


# --------------------------------------------------------------- NP-Map ----

def test_np_map_properties():
    """Section "NP-Map": direction from the learned map, norm re-injected,
    non-negative features."""
    rng = np.random.default_rng(1)
    d = 32
    F = rng.standard_normal((d, d)) / math.sqrt(d)
    for scale in [1e-3, 1.0, 30.0]:
        x = rng.standard_normal(d) * scale
        f = bf.np_map(x, F)
        assert np.linalg.norm(f) == pytest.approx(np.linalg.norm(x), rel=1e-12)
        assert np.all(f > 0)
        np.testing.assert_allclose(f, phi_torch(x, F), rtol=1e-12)
    assert np.all(bf.np_map(np.zeros(d), F) == 0)


# --------------------------------------------------- hand-worked example ----

def _hand():
    with open(os.path.join(HERE, "golden", "hand_example.json")) as fh:
        fx = json.load(fh)
    env = {"sqrt2*ln2": math.sqrt(2) * math.log(2), "sqrt2*ln3": math.sqrt(2) * math.log(3)}
    conv = lambda a: np.array(json.loads(json.dumps(a)), dtype=object)

    def num(a):
        return np.vectorize(lambda e: env[e] if isinstance(e, str) else float(e))(conv(a)).astype(np.float64)
    ins = {k: num(v) for k, v in fx["inputs"].items()}
    return fx, ins


def _hand_expected():
    r2, l3 = math.sqrt(2), math.log(3)
    v = np.array([[1, 0], [0, 1], [2, 2], [-1, 3]], dtype=np.float64)
    y = np.zeros((4, 2))
    y[0] = v[0]
    y[1] = (v[0] + 4 * v[1]) / 5
    y[2] = (v[2] + (r2 / 2) * v[0] + r2 * v[1]) / (1 + 3 * r2 / 2)
    y[3] = (3 * v[2] + v[3] / 3 + (r2 / 2) * l3 * v[0] + r2 * l3 * v[1]) / (3 + 1 / 3 + 1.5 * r2 * l3)
    S = np.array([[1 / r2, r2], [1 / r2, r2]])
    z = np.array([3 / r2, 3 / r2])
    return y, S, z


@pytest.mark.parametrize("form", ["bf", "rec"])
def test_hand_worked_example(form):
    fx, ins = _hand()
    p = fx["params"]
    kw = dict(window=p["window"], chunk=p["chunk"], budget=p["budget"], t_max=p["t_max"], eps=p["eps"])
    run = bf.prefill if form == "bf" else rec.prefill
    o = run(ins["q"], ins["k"], ins["v"], ins["fmap_w"], ins["gate"], **kw)
    y, S, z = _hand_expected()
    # rec's inputs pass through float32: sqrt2*ln2 etc. are rounded there
    tol = 1e-12 if form == "bf" else 1e-6
    np.testing.assert_allclose(o["y"].reshape(4, 2), y, atol=tol)
    np.testing.assert_allclose(o["S"].reshape(2, 2), S, atol=tol)
    np.testing.assert_allclose(o["z"].reshape(2), z, atol=tol)
    np.testing.assert_allclose(o["score"].reshape(4), math.log(1 / EPS), rtol=1e-14)
    np.testing.assert_allclose(o["pending"].reshape(2), math.log(1 / EPS), rtol=1e-14)
    assert o["lam"] == 0


# ---------------------------------------------- textbook reductions --------

@pytest.mark.parametrize("form", ["bf", "rec"])
@pytest.mark.parametrize("W,C,L", [(4, 8, 40), (8, 8, 33), (12, 4, 29)])
def test_everything_kept_is_causal_softmax(form, W, C, L):
    """lambda = C (m - W >= T_max C): every decided chunk is kept whole, the
    linear branch is empty and the layer is causal softmax attention."""
    rng = np.random.default_rng(W * 100 + C)
    q, k, v, F, g = rand_inputs(rng, 1, 2, 1, L, 16)
    t_max = -(-L // C)
    run = bf.prefill if form == "bf" else rec.prefill
    o = run(q, k, v, F, g, window=W, chunk=C, budget=W + t_max * C, t_max=t_max)
    assert o["lam"] == C
    y = o["y"] if form == "bf" else o["y"][None, :, :, :].reshape(1, 2, L, 16)
    causal = np.tril(np.ones((L, L), dtype=bool))
    want = sdpa(q, np.repeat(k, 2, 1), np.repeat(v, 2, 1), causal, 1 / 4.0)
    np.testing.assert_allclose(y, want, atol=1e-12)


def test_gate_zero_is_softmax_over_kept_and_window():
    """g = 0: the output is softmax attention restricted to A(t) (window,
    own chunk, kept tokens); checked with torch's masked SDPA."""
    rng = np.random.default_rng(5)
    L, C, W = 48, 8, 5
    q, k, v, F, g = rand_inputs(rng, 1, 1, 1, L, 16)
    o = bf.prefill(q, k, v, F, np.zeros(1), window=W, chunk=C, budget=W + 12, t_max=6)
    A, _ = bf.key_sets(L, W, C, o["sel"][0, 0].tolist())
    want = sdpa(q, k, v, A, 1 / 4.0)
    np.testing.assert_allclose(o["y"], want, atol=1e-12)


@pytest.mark.parametrize("W,C", [(3, 8), (8, 8), (10, 4)])
def test_nothing_kept_gate_zero_is_sliding_window(W, C):
    """lambda = 0 and g = 0 reduce to sliding-window (plus own chunk)
    softmax attention, the positional routing the pages contrast with."""
    rng = np.random.default_rng(W + C)
    L = 37
    q, k, v, F, _ = rand_inputs(rng, 1, 1, 1, L, 8)
    o = bf.prefill(q, k, v, F, np.zeros(1), window=W, chunk=C, budget=W, t_max=5)
    i, j = np.indices((L, L))
    mask = (j <= i) & ((j >= i - W + 1) | (j // C == i // C))
    np.testing.assert_allclose(o["y"], sdpa(q, k, v, mask, 1 / math.sqrt(8)), atol=1e-12)


def test_linear_branch_is_masked_linear_attention():
    """With nothing kept, the linear branch is the textbook quadratic form
    of (NP-Map) linear attention over keys outside the window and chunk:
    (M * phi(Q) phi(K)^T) V / row sums, taken without the gate; the default
    output merges it with the softmax branch under one normaliser and the
    sum merge [P4 §4] adds it scaled by the gate."""
    rng = np.random.default_rng(7)
    L, C, W, d = 40, 8, 6, 16
    q, k, v, F, g = rand_inputs(rng, 1, 1, 1, L, d)
    kw = dict(window=W, chunk=C, budget=W, t_max=5, partials=True)
    o = bf.prefill(q, k, v, F, g, **kw)
    pq, pk = phi_torch(q[0, 0], F[0]), phi_torch(k[0, 0], F[0])
    i, j = np.indices((L, L))
    M = (j <= i - W) & (j // C < i // C)
    Wm = M * (pq @ pk.T)
    rows = M.any(1)
    want = (Wm @ v[0, 0])[rows] / Wm.sum(1, keepdims=True)[rows]
    np.testing.assert_allclose(o["y_la"][0, 0][rows], want, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(o["lse_la"][0, 0][rows], np.log(Wm.sum(1)[rows]), rtol=1e-13)
    assert np.all(o["y_la"][0, 0][~rows] == 0) and np.all(o["lse_la"][0, 0][~rows] == -np.inf)
    # the merge: one normaliser over exp(logits) and g * <phi, phi>
    za, zl = np.exp(o["lse_sa"][0, 0][rows]), g[0] * Wm.sum(1)[rows]
    mix = (za[:, None] * o["y_sa"][0, 0][rows] + zl[:, None] * want) / (za + zl)[:, None]
    np.testing.assert_allclose(o["y"][0, 0][rows], mix, rtol=1e-10, atol=1e-12)
    # the sum merge: y_SA + g y_LA, y_SA alone where the linear set is empty
    for run in (bf.prefill, rec.prefill):
        s_ = run(q, k, v, F, g, merge="sum", **kw)
        y_s = s_["y"].reshape(L, d)
        np.testing.assert_allclose(y_s[rows], o["y_sa"][0, 0][rows] + g[0] * want,
                                   rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(y_s[~rows], o["y_sa"][0, 0][~rows], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("form", ["bf", "rec"])
def test_softmax_only_is_masked_softmax(form):
    """The sparse-attention-only variant ([P3 "Problems with Existing
    Intra-Layer Hybrid Attention"]) with a non-zero gate: torch's masked SDPA
    over A(t) (window, own chunk, kept tokens), and the softmax partial's
    log-normaliser is torch's logsumexp of the masked logits; the exported
    state is the same as the default merge's."""
    rng = np.random.default_rng(17)
    L, C, W, d = 56, 8, 5, 16
    q, k, v, F, g = rand_inputs(rng, 1, 2, 1, L, d)
    kw = dict(window=W, chunk=C, budget=W + 12, t_max=6, partials=True)
    run = bf.prefill if form == "bf" else rec.prefill
    o = run(q, k, v, F, g, merge="softmax_only", **kw)
    d1 = run(q, k, v, F, g, **kw)
    sel = o["sel"][0, 0] if form == "bf" else o["sel"][0]
    A, _ = bf.key_sets(L, W, C, sel.tolist())
    want = sdpa(q, np.repeat(k, 2, 1), np.repeat(v, 2, 1), A, 1 / 4.0)
    np.testing.assert_allclose(o["y"].reshape(want.shape), want, atol=1e-12)
    np.testing.assert_allclose(o["y_sa"].reshape(want.shape), want, atol=1e-12)
    logits = torch.as_tensor(q[0]) @ torch.as_tensor(k[0, 0]).T / 4.0
    lse = torch.logsumexp(logits.masked_fill(~torch.as_tensor(A), -math.inf), -1).numpy()
    np.testing.assert_allclose(o["lse_sa"].reshape(lse.shape), lse, rtol=1e-13, atol=1e-13)
    for key in ("S", "z", "score", "sel", "y_la", "lse_la"):
        np.testing.assert_array_equal(o[key], d1[key])
    assert not np.allclose(o["y"], d1["y"])  # the gate is not 0: the variants differ


def test_gate_zero_merges_coincide():
    """g = 0 turns the linear branch off in every merge: the default, the
    sum and the softmax-only outputs are equal."""
    rng = np.random.default_rng(23)
    q, k, v, F, _ = rand_inputs(rng, 1, 2, 1, 45, 8, outliers=2)
    kw = dict(window=6, chunk=8, budget=6 + 8, t_max=4)
    ys = [rec.prefill(q, k, v, F, np.zeros(2), merge=mg, **kw)["y"]
          for mg in ("one", "sum", "softmax_only")]
    np.testing.assert_array_equal(ys[0], ys[1])
    np.testing.assert_array_equal(ys[0], ys[2])


# ------------------------------------------------------------ invariants ----

def _check_selection(o, L, W, C, m):
    lam, n_dec = o["lam"], o["n_dec"]
    for b in range(o["sel"].shape[0]):
        for kv in range(o["sel"].shape[1]):
            pool = 0
            sc = o["score"][b, kv]
            for c in range(n_dec):
                row = [int(j) for j in o["sel"][b, kv, c] if j >= 0]
                lam_c = lam if pool + lam <= m - W else 0
                assert len(row) == lam_c
                assert row == sorted(row) and len(set(row)) == len(row)
                assert all(c * C <= j < (c + 1) * C for j in row)
                rest = [j for j in range(c * C, (c + 1) * C) if j not in row]
                if row and rest:
                    worst_kept = min(row, key=lambda j: (sc[j], -j))
                    best_left = max(rest, key=lambda j: (sc[j], -j))
                    assert (sc[worst_kept], -worst_kept) > (sc[best_left], -best_left)
                pool += lam_c
            assert pool == o["n_pool"][b, kv] <= m - W


def test_selection_invariants_and_state_excludes_kept():
    """Exactly lambda kept per decided chunk while the budget lasts, the
    kept ones outrank the rest, none enters the linear state."""
    rng = np.random.default_rng(11)
    L, C, W, m, tm, d = 70, 8, 5, 5 + 12, 4, 8   # lam = 3; pool fills at 4 chunks
    q, k, v, F, g = rand_inputs(rng, 2, 4, 2, L, d)
    o = bf.prefill(q, k, v, F, g, window=W, chunk=C, budget=m, t_max=tm)
    assert o["lam"] == 3 and o["n_dec"] == 8
    _check_selection(o, L, W, C, m)
    for b in range(2):
        for kv in range(2):
            kept = {int(j) for j in o["sel"][b, kv].ravel() if j >= 0}
            c_last = (L - 1) // C
            cf = bf.full_chunks_out_of_window(c_last, W, C)
            folded = [j for j in range(cf * C) if j not in kept]
            pk = phi_torch(k[b, kv], F[kv])
            want_S = pk[folded].T @ v[b, kv][folded]
            np.testing.assert_allclose(o["S"][b, kv], want_S, rtol=1e-11, atol=1e-11)
            np.testing.assert_allclose(o["z"][b, kv], pk[folded].sum(0), rtol=1e-12)
            with_kept = pk[:cf * C].T @ v[b, kv][:cf * C]
            assert np.abs(with_kept - o["S"][b, kv]).max() > 1e-3


def test_tie_rule_lower_index_first():
    """W = 1: every window holds only the token, p = 1 and all scores tie;
    ties go to the lower position, so each chunk keeps its first lambda."""
    rng = np.random.default_rng(3)
    L, C = 40, 8
    q, k, v, F, g = rand_inputs(rng, 1, 2, 1, L, 8)
    for run in (bf.prefill, rec.prefill):
        o = run(q, k, v, F, g, window=1, chunk=C, budget=1 + 2 * 5, t_max=5)
        sel = np.asarray(o["sel"]).reshape(-1, 2)
        want = np.array([[c * C, c * C + 1] for c in range(4)])
        np.testing.assert_array_equal(sel, want)
        np.testing.assert_allclose(np.asarray(o["score"]).ravel(), 2 * math.log(1 / EPS), rtol=1e-14)


def test_output_is_convex_combination():
    rng = np.random.default_rng(13)
    L = 50
    q, k, v, F, g = rand_inputs(rng, 1, 2, 1, L, 8, outliers=3)
    o = bf.prefill(q, k, v, F, g, window=4, chunk=8, budget=4 + 6, t_max=6)
    vv = v[0, 0]
    for t in range(L):
        lo, hi = vv[:t + 1].min(0), vv[:t + 1].max(0)
        for h in range(2):
            assert np.all(o["y"][0, h, t] >= lo - 1e-12) and np.all(o["y"][0, h, t] <= hi + 1e-12)


def test_causality_and_prefix_consistency():
    """Changing tokens after position t0 changes no output, score or
    decision made by t0 (decode of later tokens continues the prefill)."""
    rng = np.random.default_rng(17)
    L, t0, C, W = 56, 30, 8, 6
    q, k, v, F, g = rand_inputs(rng, 1, 2, 1, L, 8)
    kw = dict(window=W, chunk=C, budget=W + 9, t_max=3)
    a = rec.prefill(q, k, v, F, g, **kw)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for x in (q2, k2, v2):
        x[:, :, t0 + 1:] = rng.standard_normal(x[:, :, t0 + 1:].shape)
    b = rec.prefill(q2, k2, v2, F, g, **kw)
    np.testing.assert_array_equal(a["y"][..., :t0 + 1, :], b["y"][..., :t0 + 1, :])
    np.testing.assert_array_equal(a["score"][..., :t0 + 1], b["score"][..., :t0 + 1])
    n_decided = t0 // C
    np.testing.assert_array_equal(a["sel"][:, :n_decided], b["sel"][:, :n_decided])
    c = rec.prefill(q[:, :, :t0 + 1], k[:, :, :t0 + 1], v[:, :, :t0 + 1], F, g, **kw)
    np.testing.assert_array_equal(c["y"], a["y"][..., :t0 + 1, :])


def test_gqa_group_and_permutations():
    """G = 1 is multi-head attention; permuting batch rows or kv groups
    (with their heads, map weights and gates) permutes the outputs."""
    rng = np.random.default_rng(19)
    L = 24
    q, k, v, F, g = rand_inputs(rng, 2, 4, 2, L, 8)
    kw = dict(window=3, chunk=4, budget=3 + 6, t_max=6)
    o = bf.prefill(q, k, v, F, g, **kw)
    # each kv group alone, as G = 2 MHA-like runs
    for kv in range(2):
        oo = bf.prefill(q[:, 2 * kv:2 * kv + 2], k[:, kv:kv + 1], v[:, kv:kv + 1], F[kv:kv + 1],
                        g[2 * kv:2 * kv + 2], **kw)
        np.testing.assert_allclose(oo["y"], o["y"][:, 2 * kv:2 * kv + 2], atol=1e-14)
    perm_q = [2, 3, 0, 1]
    op = bf.prefill(q[::-1][:, perm_q], k[::-1][:, ::-1], v[::-1][:, ::-1], F[::-1], g[perm_q], **kw)
    np.testing.assert_allclose(op["y"], o["y"][::-1][:, perm_q], atol=1e-14)
    np.testing.assert_array_equal(op["sel"], o["sel"][::-1][:, ::-1])
    # G = 1: one query head per kv head
    o1 = bf.prefill(q[:, :1], k[:, :1], v[:, :1], F[:1], g[:1], **kw)
    o1b = bf.prefill(q[:, :1], k[:, :1], v[:, :1], F[:1], g[:1], **kw)
    np.testing.assert_array_equal(o1["y"], o1b["y"])


CASES = [
    # (B, Hq, Hkv, L, d, W, C, m, t_max, outliers)
    (1, 1, 1, 64, 8, 4, 8, 4 + 8, 8, 0),          # W < C, lam = 1
    (1, 2, 1, 61, 8, 8, 8, 8 + 14, 7, 2),         # W = C, ragged L
    (2, 4, 2, 45, 8, 11, 4, 11 + 24, 6, 1),       # W > C, lam = 4 = C
    (1, 2, 2, 50, 16, 5, 8, 5 + 3, 7, 0),         # lam = 0
    (1, 3, 1, 77, 8, 6, 8, 6 + 8, 2, 2),          # lam = 4, budget fills
    (1, 2, 1, 1, 8, 4, 8, 12, 1, 0),              # one token
    (1, 2, 1, 8, 8, 4, 8, 12, 1, 0),              # one chunk, nothing decided
    (1, 2, 1, 9, 8, 2, 8, 12, 1, 0),              # one decided chunk
]


@pytest.mark.parametrize("case", CASES)
def test_recurrent_matches_brute_force(case):
    """The two oracle forms (explicit sets vs. token-by-token recurrence)
    agree to fp64 rounding on tiny shapes covering the edge cases."""
    B, Hq, Hkv, L, d, W, C, m, tm, nout = case
    rng = np.random.default_rng(sum(case))
    q, k, v, F, g = rand_inputs(rng, B, Hq, Hkv, L, d, outliers=nout)
    kw = dict(window=W, chunk=C, budget=m, t_max=tm)
    a = bf.prefill(q, k, v, F, g, **kw)
    r = rec.prefill(q, k, v, F, g, **kw)
    G = Hq // Hkv
    U = B * Hkv
    np.testing.assert_allclose(r["y"], a["y"].reshape(B, Hkv, G, L, d).reshape(U, G, L, d),
                               rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(r["score"], a["score"].reshape(U, L), rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(r["sel"], a["sel"].reshape(U, a["n_dec"], a["lam"]))
    np.testing.assert_allclose(r["S"], a["S"].reshape(U, d, d), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(r["z"], a["z"].reshape(U, d), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["pending"], a["pending"].reshape(U, C), rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(r["n_pool"], a["n_pool"].reshape(U))
    _check_selection(a, L, W, C, m)


@pytest.mark.parametrize("merge", ["one", "sum", "softmax_only"])
@pytest.mark.parametrize("case", CASES[:5] + CASES[7:])
def test_variants_recurrent_matches_brute_force(case, merge):
    """Both oracle forms agree on the three merges and on the branch
    partials (recurrence over the state vs. explicit sets)."""
    B, Hq, Hkv, L, d, W, C, m, tm, nout = case
    rng = np.random.default_rng(sum(case) + 1)
    q, k, v, F, g = rand_inputs(rng, B, Hq, Hkv, L, d, outliers=nout)
    kw = dict(window=W, chunk=C, budget=m, t_max=tm, merge=merge, partials=True)
    a = bf.prefill(q, k, v, F, g, **kw)
    r = rec.prefill(q, k, v, F, g, **kw)
    G = Hq // Hkv
    U = B * Hkv
    for key in ("y", "y_sa", "y_la"):
        np.testing.assert_allclose(r[key], a[key].reshape(B, Hkv, G, L, d).reshape(U, G, L, d),
                                   rtol=1e-11, atol=1e-12, err_msg=key)
    for key in ("lse_sa", "lse_la"):
        np.testing.assert_allclose(r[key], a[key].reshape(U, G, L), rtol=1e-12, atol=1e-12,
                                   err_msg=key)


# ------------------------------------------------------ routing metrics ----

def _topk_selection(score_t, L, C, lam):
    """Per decided chunk, the lam positions with the largest scores by
    torch.topk (distinct scores), ascending."""
    n_dec = (L - 1) // C
    out = []
    for c in range(n_dec):
        _, idx = torch.topk(score_t[c * C:(c + 1) * C], lam)
        out.append(sorted((idx + c * C).tolist()))
    return np.array(out).reshape(n_dec, lam)


@pytest.mark.parametrize("route", ["diag", "qk", "keynorm", "external"])
@pytest.mark.parametrize("form", ["bf", "rec"])
def test_routing_metric_scores_and_selection(route, form):
    """The routing-metric alternatives [P3 "Ablation Studies"]: the scores
    are torch's window softmax weight on the token itself (diag), torch's
    scaled self dot product (qk), torch's vector norm (keynorm) or the given
    draws (external), summed over the group's heads where per query head;
    each decided chunk keeps torch.topk of them (the budget never fills)."""
    rng = np.random.default_rng(31)
    B, Hq, Hkv, L, d, W, C = 1, 2, 1, 50, 8, 6, 8
    q, k, v, F, g = rand_inputs(rng, B, Hq, Hkv, L, d)
    m = W + 6 * 3  # lambda = 18 / 6 = 3 for each of the six decided chunks
    ext = rng.uniform(0, 1, (B, Hkv, L)).astype(np.float32)
    kw = dict(window=W, chunk=C, budget=m, t_max=6, route=route, ext_score=ext)
    o = (bf.prefill if form == "bf" else rec.prefill)(q, k, v, F, g, **kw)
    lam = o["lam"]
    assert lam == 3
    qt, kt = torch.as_tensor(q[0]), torch.as_tensor(k[0, 0])
    scale = 1 / math.sqrt(d)
    if route == "diag":
        i, j = np.indices((L, L))
        band = torch.as_tensor((j <= i) & (j >= i - W + 1))
        p = torch.softmax((qt @ kt.T * scale).masked_fill(~band, -math.inf), -1)
        want = torch.diagonal(p, dim1=-2, dim2=-1).sum(0)
    elif route == "qk":
        want = (qt * kt).sum(-1).sum(0) * scale
    elif route == "keynorm":
        want = torch.linalg.vector_norm(kt, dim=-1)
    else:
        want = torch.as_tensor(ext[0, 0], dtype=torch.float64)
    np.testing.assert_allclose(o["score"].reshape(L), want.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(o["sel"].reshape(-1, lam), _topk_selection(want, L, C, lam))
    # the state holds the unselected tokens whatever ranked them
    _check_selection(o if form == "bf" else bf.prefill(q, k, v, F, g, **kw), L, W, C, m)


def test_uniform_routing_hand_example():
    """Uniform routing, C = 16, lambda = 6: every decided chunk keeps the
    offsets floor(16 i / 6) = 0, 2, 5, 8, 10, 13; the last chunk's scores are
    1 at those offsets and 0 elsewhere."""
    rng = np.random.default_rng(3)
    L, C, W = 60, 16, 4
    q, k, v, F, g = rand_inputs(rng, 1, 1, 1, L, 8)
    offs = [0, 2, 5, 8, 10, 13]
    for run in (bf.prefill, rec.prefill):
        o = run(q, k, v, F, g, window=W, chunk=C, budget=W + 6 * 3, t_max=3, route="uniform")
        assert o["lam"] == 6
        sel = o["sel"].reshape(3, 6)
        for c in range(3):
            assert sel[c].tolist() == [c * C + x for x in offs]
        pend = o["pending"].reshape(-1)[:L - 3 * C]
        assert pend.tolist() == [1.0 if x in offs else 0.0 for x in range(L - 3 * C)]


@pytest.mark.parametrize("route", ["diag", "qk", "keynorm", "uniform", "external"])
@pytest.mark.parametrize("case", CASES[:5] + CASES[7:])
def test_routes_recurrent_matches_brute_force(case, route):
    B, Hq, Hkv, L, d, W, C, m, tm, nout = case
    rng = np.random.default_rng(sum(case) + 2)
    q, k, v, F, g = rand_inputs(rng, B, Hq, Hkv, L, d, outliers=nout)
    ext = rng.uniform(0, 1, (B, Hkv, L)).astype(np.float32)
    kw = dict(window=W, chunk=C, budget=m, t_max=tm, route=route, ext_score=ext)
    a = bf.prefill(q, k, v, F, g, **kw)
    r = rec.prefill(q, k, v, F, g, **kw)
    G, U = Hq // Hkv, B * Hkv
    np.testing.assert_allclose(r["score"], a["score"].reshape(U, L), rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(r["sel"], a["sel"].reshape(U, a["n_dec"], a["lam"]))
    np.testing.assert_allclose(r["y"], a["y"].reshape(U, G, L, d), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(r["S"], a["S"].reshape(U, d, d), rtol=1e-11, atol=1e-11)
    _check_selection(a, L, W, C, m)


@pytest.mark.parametrize("W,C,L", [(5, 8, 70), (8, 8, 61), (20, 4, 45), (1, 16, 50)])
def test_exported_state_plus_ring_is_last_query_linear_set(W, C, L):
    """The exported state S, z (the unkept tokens of the chunks wholly before
    every window of the last chunk) plus the decided, unkept, out-of-window
    tokens after that boundary (kept explicitly in the recent-token ring) sum
    to phi(k) v^T over B(L-1), the last query's linear set built by
    key_sets; the boundary lies on a chunk start at or before the last
    query's window, i.e. cf C <= L - W (for L > W) and cf C <= (c_last - 1) C."""
    rng = np.random.default_rng(W * 100 + C + L)
    q, k, v, F, g = rand_inputs(rng, 1, 2, 1, L, 8)
    o = bf.prefill(q, k, v, F, g, window=W, chunk=C, budget=W + 3 * 4, t_max=4)
    c_last = (L - 1) // C
    cf = bf.full_chunks_out_of_window(c_last, W, C)
    assert cf * C <= max(0, c_last * C - W + 1) and cf * C % C == 0
    assert (cf + 1) * C > c_last * C - W + 1  # the largest such chunk boundary
    _, Bm = bf.key_sets(L, W, C, o["sel"][0, 0].tolist())
    lin = np.nonzero(Bm[L - 1])[0]
    pk = phi_torch(k[0, 0], F[0])
    ring = [j for j in lin if j >= cf * C]
    want_S = pk[lin].T @ v[0, 0][lin]
    got_S = o["S"][0, 0] + (pk[ring].T @ v[0, 0][ring] if ring else 0.0)
    np.testing.assert_allclose(got_S, want_S, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(o["z"][0, 0] + pk[ring].sum(0), pk[lin].sum(0), rtol=1e-12, atol=1e-12)
    assert all(j < cf * C for j in lin if j not in ring)


# ---- channel-wise sigmoid output gate [P4 §4 Gating Mechanism] -------------
def test_output_gate_pins():
    """Pins of the gated output against what the sigmoid fixes, not its
    formula: a zero gate halves the output exactly; gates g and -g split the
    output into two parts that add up to it (sigmoid(g) + sigmoid(-g) = 1);
    a large positive gate leaves it unchanged and a large negative one
    closes it; one value worked by hand: sigmoid(ln 3) = 3/4."""
    rng = np.random.default_rng(7)
    y = rng.standard_normal((2, 3, 5, 8))
    g = rng.standard_normal(y.shape) * 3.0
    assert np.array_equal(bf.output_gate(y, np.zeros_like(y)), y / 2)
    np.testing.assert_allclose(bf.output_gate(y, g) + bf.output_gate(y, -g), y, rtol=0, atol=1e-15)
    np.testing.assert_allclose(bf.output_gate(y, np.full_like(y, 50.0)), y, rtol=1e-15, atol=0)
    assert np.abs(bf.output_gate(y, np.full_like(y, -800.0))).max() == 0.0
    np.testing.assert_allclose(bf.output_gate(np.array([4.0]), np.array([math.log(3.0)])), [3.0], rtol=1e-15)
    # element by element: each output entry depends on its own gate entry only
    g2 = g.copy()
    g2[1, 2, 3, 4] += 1.0
    d = bf.output_gate(y, g2) - bf.output_gate(y, g)
    d[1, 2, 3, 4] = 0.0
    assert np.abs(d).max() == 0.0


# ---------------------------------------------------------- decay gate ----
# Reading of the forget gate of gated linear attention (the hybrid-
# architecture survey, §2: the state decays by gamma every token, write
# strength 1), applied to STILL's linear state: the linear key j of query t
# is weighted gamma^(t - j); the exported state holds gamma^(R - j), R the
# first position past it.


@pytest.mark.parametrize("form", ["bf", "rec"])
def test_decay_one_is_the_plain_layer(form):
    """gamma = 1 gives the plain layer exactly (outputs and exported state)."""
    rng = np.random.default_rng(41)
    q, k, v, F, g = rand_inputs(rng, 1, 4, 2, 70, 8, outliers=1)
    kw = dict(window=6, chunk=8, budget=6 + 4 * 8, t_max=8)
    run = bf.prefill if form == "bf" else rec.prefill
    a = run(q, k, v, F, g, **kw)
    b = run(q, k, v, F, g, decay=np.ones(2, np.float32), **kw)
    for key in ("y", "S", "z"):
        np.testing.assert_array_equal(a[key], b[key])


@pytest.mark.parametrize("form", ["bf", "rec"])
def test_decay_vanishing_is_softmax_only(form):
    """gamma -> 0: every linear key lies at least W tokens back, so its weight
    falls below gamma^W and the output is the softmax branch alone."""
    rng = np.random.default_rng(43)
    q, k, v, F, g = rand_inputs(rng, 1, 4, 2, 70, 8, outliers=1)
    kw = dict(window=6, chunk=8, budget=6 + 4 * 8, t_max=8)
    run = bf.prefill if form == "bf" else rec.prefill
    a = run(q, k, v, F, g, merge="softmax_only", **kw)
    b = run(q, k, v, F, g, decay=np.full(2, 1e-6, np.float32), **kw)
    np.testing.assert_allclose(b["y"], a["y"], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("case", CASES[:5] + CASES[7:])
def test_decay_recurrent_matches_brute_force(case):
    """Both forms agree with a decaying state (the recurrence multiplies its
    state by gamma every token; the explicit form weights gamma^(t - j))."""
    B, Hq, Hkv, L, d, W, C, m, tm, nout = case
    rng = np.random.default_rng(sum(case) + 5)
    q, k, v, F, g = rand_inputs(rng, B, Hq, Hkv, L, d, outliers=nout)
    dec = rng.uniform(0.8, 1.0, Hkv).astype(np.float32)
    kw = dict(window=W, chunk=C, budget=m, t_max=tm, decay=dec)
    a = bf.prefill(q, k, v, F, g, partials=True, **kw)
    r = rec.prefill(q, k, v, F, g, partials=True, **kw)
    G = Hq // Hkv
    U = B * Hkv
    np.testing.assert_allclose(r["y"], a["y"].reshape(U, G, L, d), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(r["y_la"], a["y_la"].reshape(U, G, L, d), rtol=1e-10, atol=1e-11)
    fin = np.isfinite(a["lse_la"].reshape(U, G, L))
    np.testing.assert_array_equal(np.isfinite(r["lse_la"]), fin)
    np.testing.assert_allclose(r["lse_la"][fin], a["lse_la"].reshape(U, G, L)[fin], rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(r["S"], a["S"].reshape(U, d, d), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(r["z"], a["z"].reshape(U, d), rtol=1e-12, atol=1e-12)


def test_decay_geometric_closed_form():
    """Identical keys (one feature vector, tied scores: the lower index is
    kept) and distinct values: the linear branch at query t is the average
    of its values with weights gamma^(t - j) over B(t) = the unkept tokens
    below min(t - W + 1, cC), and the exported z is phi(k) times the sum of
    gamma^(R - j) over the unkept tokens below R = cf C."""
    rng = np.random.default_rng(47)
    L, d, W, C, m, tm, gam = 40, 4, 4, 8, 4 + 2 * 8, 8, np.float32(0.75)
    q, k, v, F, g = rand_inputs(rng, 1, 1, 1, L, d)
    k[:] = k[0, 0, 0]
    r = rec.prefill(q, k, v, F, g, window=W, chunk=C, budget=m, t_max=tm,
                    decay=np.array([gam]), partials=True)
    lam = bf.budget_lambda(W, C, m, tm)
    assert lam == 2
    kept = set()
    for c in range((L - 1) // C):  # ties: the two lowest positions of each chunk
        if len(kept) + lam <= m - W:
            kept.update((c * C, c * C + 1))
    np.testing.assert_array_equal(np.sort(r["sel"].reshape(-1)[r["sel"].reshape(-1) >= 0]), sorted(kept))
    G64 = float(gam)
    for t in range(L):
        c = t // C
        B_t = [j for j in range(min(t - W + 1, c * C)) if j not in kept]
        if not B_t:
            assert r["lse_la"][0, 0, t] == -np.inf
            continue
        w = np.array([G64 ** (t - j) for j in B_t])
        want = (w[:, None] * v[0, 0, B_t]).sum(0) / w.sum()
        np.testing.assert_allclose(r["y_la"][0, 0, t], want, rtol=1e-12, atol=1e-13)
    c_last = (L - 1) // C
    R = bf.full_chunks_out_of_window(c_last, W, C) * C
    geo = sum(G64 ** (R - j) for j in range(R) if j not in kept)
    np.testing.assert_allclose(r["z"][0], geo * bf.np_map(k[0, 0, 0], F[0]), rtol=1e-12)


# ---- the kept pool as an 8-bit store (OCP E4M3 codes, a float32 scale per row)

def test_e4m3_code_points_of_the_format():
    """Fixed points of the OCP E4M3 definition: the largest finite value 448
    is code 0x7E, 1 is 0x38, the smallest normal 2^-6 is 0x08, the smallest
    subnormal 2^-9 is 0x01; with a row maximum of 448 the scale is 2^0, with
    449 it is 2^1 (the smallest power of two that brings the row within 448)."""
    row = np.array([448, 1, 2.0 ** -6, 2.0 ** -9, -448, -1, 0, 0.5], np.float32)
    for codes, e in (rec.e4m3_rows(row[None])[:2], bf.e4m3_row(row)[:2]):
        assert int(np.asarray(e).reshape(-1)[0]) == 0
        assert list(np.asarray(codes).reshape(-1)) == [0x7E, 0x38, 0x08, 0x01, 0xFE, 0xB8, 0x00, 0x30]
    for amax, e in ((449.0, 1), (896.0, 1), (897.0, 2), (224.0, -1), (225.0, 0), (1e-40, -126)):
        assert rec.e4m3_rows(np.array([[amax, 0]], np.float32))[1][0] == e, amax
        assert bf.e4m3_row(np.array([amax, 0], np.float32))[1] == e, amax


def test_e4m3_every_finite_value_round_trips():
    """Every finite E4M3 magnitude (and its negative), in a row whose maximum
    is 448 (scale 1), is stored exactly as its own code."""
    table = bf.e4m3_values()
    assert table[0] == 0 and table[-1] == 448 and np.all(np.diff(table) > 0)
    row = np.concatenate([table, -table[1:]]).astype(np.float32)
    codes, e, vals = rec.e4m3_rows(row[None])
    assert e[0] == 0
    np.testing.assert_array_equal(vals[0], row.astype(np.float64))
    np.testing.assert_array_equal(codes[0][:127], np.arange(127))
    np.testing.assert_array_equal(codes[0][127:], np.arange(1, 127) | 0x80)


def test_e4m3_ties_go_to_the_even_code():
    """Midpoints between neighbouring codes (scale 1) round to the even
    code; just above a midpoint rounds up."""
    table = bf.e4m3_values()
    mids = (table[:-1] + table[1:]) / 2
    row = np.concatenate([[448.0], mids]).astype(np.float32)
    assert np.array_equal(row[1:].astype(np.float64), mids)  # midpoints are exact in float32
    codes = rec.e4m3_rows(row[None])[0][0][1:]
    want = np.where(np.arange(126) % 2 == 0, np.arange(126), np.arange(1, 127))
    np.testing.assert_array_equal(codes, want)
    up = np.nextafter(mids.astype(np.float32), np.float32(np.inf))
    codes = rec.e4m3_rows(np.concatenate([[448.0], up]).astype(np.float32)[None])[0][0][1:]
    np.testing.assert_array_equal(codes, np.arange(1, 127))


def test_e4m3_rows_two_implementations_agree():
    """The recurrent oracle's quantiser (arithmetic on the binade) and the
    brute-force one (nearest entry of the code table) give the same codes,
    scale exponents and values on rows of every magnitude, zero rows
    included; a value is off by at most half a step of the top binade,
    16 times the scale."""
    rng = np.random.default_rng(11)
    X = (rng.standard_normal((300, 64)) * np.exp(rng.uniform(-20, 12, (300, 1)))).astype(np.float32)
    X[5] = 0
    X[6, ::3] = 0
    c, s, v = rec.e4m3_rows(X)
    for i in range(len(X)):
        cb, sb, vb = bf.e4m3_row(X[i])
        assert np.array_equal(cb, c[i]) and sb == s[i] and np.array_equal(vb, v[i]), i
    assert np.all(np.abs(v - X) <= 16.0 * np.exp2(s.astype(np.float64))[:, None])
    amax = np.abs(X).max(axis=1)
    nz = amax > 0
    assert np.all(amax[nz] <= 448 * np.exp2(s[nz].astype(np.float64)))
    assert np.all(amax[nz] > 224 * np.exp2(s[nz].astype(np.float64)))
    assert s[5] == 0 and not c[5].any()


FP8_CASES = [
    # (B, Hq, Hkv, L, d, W, C, m, t_max, fp8_from)
    (1, 2, 1, 60, 8, 4, 8, 4 + 2 * 7, 7, 30),
    (2, 4, 2, 75, 16, 8, 8, 8 + 3 * 9, 9, 40),
    (1, 1, 1, 50, 8, 12, 4, 12 + 1 * 12, 12, 20),
]


@pytest.mark.parametrize("case", FP8_CASES)
def test_fp8_pool_recurrent_matches_brute_force(case):
    """Both forms read the kept pool below the window band in E4M3 from
    fp8_from on: they agree, the queries before fp8_from equal the plain
    layer's exactly, the later ones differ from it (the 8-bit store is
    read), and fp8_from past the end is the plain layer."""
    B, Hq, Hkv, L, d, W, C, m, tm, f = case
    rng = np.random.default_rng(sum(case) + 9)
    q, k, v, F, g = rand_inputs(rng, B, Hq, Hkv, L, d, outliers=1)
    kw = dict(window=W, chunk=C, budget=m, t_max=tm)
    a = bf.prefill(q, k, v, F, g, fp8_from=f, **kw)
    r = rec.prefill(q, k, v, F, g, fp8_from=f, **kw)
    plain = rec.prefill(q, k, v, F, g, **kw)
    G, U = Hq // Hkv, B * Hkv
    np.testing.assert_allclose(r["y"], a["y"].reshape(U, G, L, d), rtol=1e-11, atol=1e-12)
    np.testing.assert_array_equal(r["y"][:, :, :f], plain["y"][:, :, :f])
    assert np.abs(r["y"][:, :, f:] - plain["y"][:, :, f:]).max() > 1e-4
    for key in ("sel", "score", "S", "z"):
        np.testing.assert_array_equal(r[key], plain[key])
    late = rec.prefill(q, k, v, F, g, fp8_from=L, **kw)
    np.testing.assert_array_equal(late["y"], plain["y"])


def test_fp8_pool_leaves_the_band_exact():
    """A kept token still inside a query's window band is read at full
    precision: with the window covering the whole sequence (no kept token
    ever lies below the band) the 8-bit store changes nothing."""
    rng = np.random.default_rng(3)
    L, d = 40, 8
    q, k, v, F, g = rand_inputs(rng, 1, 2, 1, L, d)
    kw = dict(window=L, chunk=8, budget=L + 10, t_max=5)
    np.testing.assert_array_equal(rec.prefill(q, k, v, F, g, fp8_from=0, **kw)["y"],
                                  rec.prefill(q, k, v, F, g, **kw)["y"])
