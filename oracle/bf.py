"""Oracle, brute-force form: the STILL layer's definitions written out in fp64.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module;
only tests/, the smoke check and the bench's CPU-baseline leg may use it.
It shares no code with the HIP path.

Pages cited (short tag -> page title):
  [P2] "NeurIPS 2026|层内混合注意力：告别位置「伪混合」，STILL首个内容感知的层内混合注意力架构"
       (Chinese press article), sections 亮点一 (固定预算路由, 延迟选择与分块并行) and 亮点二
  [P3] "STILL: Content-Aware Intra-Layer Hybrid Attention for Efficient LLM
       Linearization", sections "Content-Aware Routing with Fixed Budget",
       "Delayed Chunk-Level Selection for Unified Training-Inference
       Parallelism", "Self-Saliency Score", "Theoretical Guarantee:
       Local-Global Consistency", "NP-Map: Norm-Preserving Feature Map"

Every query is handled on its own: the key set of each branch is built as an
explicit index set and summed over directly (O(L^2 d) per unit). The state
is summed over its explicit token set. Readings where the pages are silent
(score form, merge rule, NP-Map form, GQA grouping, T_max) are the ones
listed under "Readings" in the design notes; each function names its own.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Tuple

import numpy as np


def budget_lambda(window: int, chunk: int, budget: int, t_max: int) -> int:
    """Tokens kept per completed chunk.

    [P2 固定预算路由], [P3 "Content-Aware Routing with Fixed Budget"]: of the
    per-head budget m, W slots hold the recent window and the other m - W
    are spread over completed chunks, floor((m - W) / T_max) per chunk.
    Reading: the count is capped at C (a chunk has only C tokens).
    """
    if budget < window or t_max < 1 or chunk < 1 or window < 1:
        raise ValueError("need budget >= window >= 1, chunk >= 1, t_max >= 1")
    return min(chunk, (budget - window) // t_max)


def full_chunks_out_of_window(c: int, window: int, chunk: int) -> int:
    """Number of leading chunks lying wholly before the window of every
    query of chunk c: chunk c' qualifies iff its last position
    (c'+1)C - 1 <= cC - W. These are the chunks folded into the exported
    linear-attention state (reading: the state absorbs whole chunks)."""
    x = c * chunk - window + 1
    return max(0, x // chunk) if x >= 0 else 0


def saliency_kl(logits: np.ndarray, self_idx: int, eps: float) -> float:
    """Self-Saliency Score of one token for one head.

    [P3 "Self-Saliency Score"], [P2 亮点二]: two window attention
    distributions are formed, a_diag with the token's own (diagonal) term
    and a_nodiag without it, and the score is a KL-type sensitivity between
    them. Reading (the formula is not printed): KL(a_diag || (1-eps) a_nodiag
    + eps delta_self), eps > 0 small, so that the self entry has mass.
    Computed here literally, entry by entry, from the two softmaxes.
    """
    s = np.asarray(logits, dtype=np.float64)
    n = s.shape[0]
    a_diag = np.exp(s - s.max())
    a_diag /= a_diag.sum()
    a_nodiag = np.zeros(n)
    if n > 1:
        others = np.delete(np.arange(n), self_idx)
        e = np.exp(s[others] - s[others].max())
        a_nodiag[others] = e / e.sum()
    mix = (1.0 - eps) * a_nodiag
    mix[self_idx] += eps
    kl = 0.0
    for j in range(n):
        if a_diag[j] > 0.0:
            kl += a_diag[j] * math.log(a_diag[j] / mix[j])
    return kl


def np_map(x: np.ndarray, F: np.ndarray) -> np.ndarray:
    """NP-Map feature of a row vector x with map weights F [d, d].

    [P3 "NP-Map: Norm-Preserving Feature Map"]: a learned map sets only the
    direction of the feature, the input's own norm ||x|| is put back, and
    the feature is non-negative. Reading: direction = softmax(x F) (a
    Hedgehog-style softmax feature) normalised to unit L2 norm, then scaled
    by ||x||_2. phi(0) = 0.
    """
    x = np.asarray(x, dtype=np.float64)
    a = x @ F
    u = np.exp(a - a.max())
    return np.linalg.norm(x) * u / np.linalg.norm(u)


def prefill(q, k, v, fmap_w, gate, *, window: int, chunk: int, budget: int,
            t_max: int, eps: float = 1e-6, sm_scale: Optional[float] = None,
            partials: bool = False, merge: str = "one", route: str = "saliency",
            ext_score=None, decay=None, fp8_from: int = -1) -> Dict[str, np.ndarray]:
    """One STILL layer over a whole sequence, every query by brute force.

    q [B,Hq,L,d], k/v [B,Hkv,L,d], fmap_w [Hkv,d,d], gate [Hq] (any array
    type convertible to float64). Query head h belongs to kv group h // G.

    Returns y [B,Hq,L,d], score [B,Hkv,L], sel [B,Hkv,n_dec,lam] (ascending
    positions, -1 where a chunk kept fewer), n_pool [B,Hkv], the exported
    state S [B,Hkv,d,d], z [B,Hkv,d], and pending [B,Hkv,C] (scores of the
    undecided chunk's tokens, NaN beyond the sequence end). With
    partials=True also y_sa, lse_sa, y_la, lse_la: each branch normalised
    on its own, lse the natural log of its weight sum, the linear branch
    without the gate (y_la = 0 and lse_la = -inf where B(t) is empty).

    merge (reading where the pages leave it open): "one" = one normaliser
    over exp(logit) and gate * <phi(q), phi(k)>; "sum" = y_SA + gate * y_LA,
    each normalised on its own [P4 §4]; "softmax_only" = y_SA, the linear
    branch dropped and unkept tokens discarded ([P3 "Problems with Existing
    Intra-Layer Hybrid Attention"]: the sparse-attention-only alternative).

    route: the score that ranks a chunk's tokens, the Self-Saliency Score
    ("saliency") or an alternative of the pages' routing-metric ablation
    [P3 "Ablation Studies"]: "diag" (the window softmax's weight on the
    token itself, summed over the group's heads), "qk" (the scaled self
    logit, summed over the heads), "keynorm" (||k_t||), "uniform" (reading:
    evenly spaced offsets floor(i C / lambda) of each chunk score 1, the rest
    0) or "external" (ext_score [B,Hkv,L], e.g. random routing's draws).

    decay [Hkv] (reading of the forget gate of gated linear attention
    [P4 §2], write strength 1, applied to the linear state): the linear key j
    of query t is weighted decay^(t - j); the exported state holds
    decay^(R - j) with R = cf C, the first position past it. None = 1.

    fp8_from: queries t >= fp8_from read the kept tokens that lie below
    their window band (before both the window and the own chunk) from an
    8-bit store, the values of e4m3_row (reading of the pages' fp8 pool);
    -1: never.
    """
    if merge not in ("one", "sum", "softmax_only"):
        raise ValueError("merge must be one, sum or softmax_only")
    if route not in ("saliency", "diag", "qk", "keynorm", "uniform", "external"):
        raise ValueError("unknown route")
    if route == "external" and ext_score is None:
        raise ValueError("route external needs ext_score")
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Fw = np.asarray(fmap_w, dtype=np.float64)
    g_all = np.asarray(gate, dtype=np.float64)
    dec = None if decay is None else np.asarray(np.asarray(decay, dtype=np.float32), dtype=np.float64)
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    W, C, m = window, chunk, budget
    scale = 1.0 / math.sqrt(d) if sm_scale is None else sm_scale
    lam = budget_lambda(W, C, m, t_max)
    n_dec = (L - 1) // C if L > 0 else 0

    y = np.zeros((B, Hq, L, d))
    score = np.zeros((B, Hkv, L))
    sel = -np.ones((B, Hkv, n_dec, lam), dtype=np.int64)
    n_pool = np.zeros((B, Hkv), dtype=np.int64)
    S = np.zeros((B, Hkv, d, d))
    z = np.zeros((B, Hkv, d))
    pending = np.full((B, Hkv, C), np.nan)
    if partials:
        y_sa = np.full((B, Hq, L, d), np.nan)
        lse_sa = np.full((B, Hq, L), np.nan)
        y_la = np.zeros((B, Hq, L, d))
        lse_la = np.full((B, Hq, L), -np.inf)

    pos = np.arange(L)
    chunk_of = pos // C
    for b in range(B):
        for kv in range(Hkv):
            K, V, F = k[b, kv], v[b, kv], Fw[kv]
            if fp8_from >= 0:
                K8 = np.stack([e4m3_row(K[j])[2] for j in range(L)]) if L else K
                V8 = np.stack([e4m3_row(V[j])[2] for j in range(L)]) if L else V
            gam = 1.0 if dec is None else float(dec[kv])
            heads = range(kv * G, kv * G + G)
            # Score of every token, summed over the query heads of the group
            # (reading: routing is per kv head).
            sc = np.zeros(L)
            marks = {(i * C) // lam for i in range(lam)} if lam > 0 else set()
            for t in range(L):
                lo = max(0, t - W + 1)
                if route == "keynorm":
                    sc[t] = math.sqrt(float(K[t] @ K[t]))
                elif route == "uniform":
                    sc[t] = 1.0 if t % C in marks else 0.0
                elif route == "external":
                    sc[t] = float(np.float32(ext_score[b, kv, t]))
                for h in heads if route in ("saliency", "diag", "qk") else ():
                    logits = scale * (K[lo:t + 1] @ q[b, h, t])
                    if route == "saliency":
                        sc[t] += saliency_kl(logits, t - lo, eps)
                    elif route == "diag":
                        e = np.exp(logits - logits.max())
                        sc[t] += e[-1] / e.sum()
                    else:
                        sc[t] += logits[-1]
            score[b, kv] = sc

            # Delayed chunk-level Top-lambda: chunk c is decided when chunk
            # c+1 begins [P3 "Delayed Chunk-Level Selection"], keeping the
            # lambda best by (score desc, position asc); selections are
            # permanent and the pool never exceeds m - W [P2 固定预算路由].
            selected = np.zeros(L, dtype=bool)
            pool = 0
            for c in range(n_dec):
                lam_c = lam if pool + lam <= m - W else 0
                cand = sorted(range(c * C, (c + 1) * C), key=lambda j: (-sc[j], j))
                chosen = sorted(cand[:lam_c])
                selected[chosen] = True
                sel[b, kv, c, :len(chosen)] = chosen
                pool += lam_c
            n_pool[b, kv] = pool

            phik = np.stack([np_map(K[j], F) for j in range(L)]) if L else np.zeros((0, d))
            for t in range(L):
                c = t // C
                in_pool = selected & (chunk_of < c)
                in_a = (pos <= t) & ((pos >= t - W + 1) | (chunk_of == c) | in_pool)
                in_b = (pos <= t) & ~in_a
                ia, ib = np.nonzero(in_a)[0], np.nonzero(in_b)[0]
                Ka, Va = K[ia], V[ia]
                if 0 <= fp8_from <= t:  # the pool below the band, as stored
                    low = in_pool[ia] & (ia < t - W + 1)
                    Ka, Va = np.where(low[:, None], K8[ia], Ka), np.where(low[:, None], V8[ia], Va)
                for h in heads:
                    s = scale * (Ka @ q[b, h, t])
                    w0 = phik[ib] @ np_map(q[b, h, t], F)  # linear weights, no gate
                    if gam != 1.0:
                        w0 = w0 * gam ** (t - ib).astype(np.float64)
                    ea = np.exp(s - s.max())
                    ysa = (ea @ Va) / ea.sum()
                    yla = (w0 @ V[ib]) / w0.sum() if len(ib) and w0.sum() > 0 else np.zeros(d)
                    if merge == "one":
                        w = g_all[h] * w0
                        with np.errstate(divide="ignore"):
                            logw = np.concatenate([s, np.log(w)])
                        mx = logw.max()
                        e = np.exp(logw - mx)
                        vals = np.concatenate([Va, V[ib]])
                        y[b, h, t] = (e @ vals) / e.sum()
                    elif merge == "sum":
                        y[b, h, t] = ysa + g_all[h] * yla
                    else:
                        y[b, h, t] = ysa
                    if partials:
                        y_sa[b, h, t] = ysa
                        lse_sa[b, h, t] = s.max() + math.log(ea.sum())
                        y_la[b, h, t] = yla
                        if len(ib) and w0.sum() > 0:
                            lse_la[b, h, t] = math.log(w0.sum())

            if L:
                c_last = (L - 1) // C
                cf = full_chunks_out_of_window(c_last, W, C)
                folded = (~selected) & (chunk_of < cf)
                wf = gam ** (cf * C - pos[folded]).astype(np.float64) if gam != 1.0 else \
                    np.ones(int(folded.sum()))
                S[b, kv] = (phik[folded] * wf[:, None]).T @ V[folded]
                z[b, kv] = (phik[folded] * wf[:, None]).sum(axis=0)
                pend = pos[chunk_of == c_last]
                pending[b, kv, :len(pend)] = sc[pend]

    out = {"y": y, "score": score, "sel": sel, "n_pool": n_pool, "S": S, "z": z,
           "pending": pending, "lam": lam, "n_dec": n_dec}
    if partials:
        out.update(y_sa=y_sa, lse_sa=lse_sa, y_la=y_la, lse_la=lse_la)
    return out


def e4m3_values() -> np.ndarray:
    """The 127 non-negative finite values of OCP E4M3 by code 0..126 (sign
    bit clear): 4 exponent bits (bias 7), 3 mantissa bits, exponent field 0
    subnormal (m/8 2^-6), code 127 NaN."""
    out = []
    for c in range(127):
        e, m = c >> 3, c & 7
        out.append(m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(out)


def e4m3_row(x) -> Tuple[np.ndarray, int, np.ndarray]:
    """One row as the kept pool's 8-bit store (reading: the pages name an
    fp8 pool, not its format): a power-of-two scale 2^e (an E8M0 exponent as
    in the OCP microscaling formats), e the smallest integer with
    max |x_i| <= 448 2^e (0 for a zero row), at least -126; each x_i / 2^e to
    the nearest E4M3 value, ties to the even code, beyond 448 to 448.
    Returns codes (uint8), e, and the values code 2^e (float64). The
    exponent by search, the code by the nearest entry of the code table."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    e = 0
    if amax > 0:
        e = math.floor(math.log2(amax)) - 9
        while amax > 448 * 2.0 ** e:
            e += 1
        while e > -126 and amax <= 448 * 2.0 ** (e - 1):
            e -= 1
        e = max(e, -126)
    y = x / 2.0 ** e
    table = e4m3_values()
    a = np.abs(y)
    hi = np.clip(np.searchsorted(table, a), 1, 126)  # table[hi - 1] <= a <= table[hi] inside
    lo = hi - 1
    dlo, dhi = a - table[lo], table[hi] - a
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(a >= 448, 126, pick)
    codes = (pick | np.where(y < 0, 0x80, 0)).astype(np.uint8)
    vals = table[pick] * np.where(y < 0, -1.0, 1.0) * 2.0 ** e
    return codes, e, vals


def output_gate(y, gate_out) -> np.ndarray:
    """Channel-wise sigmoid output gate on the attention output.

    [P4 "Synergizing Linear and Sparse Attention: A Deep Dive into Hybrid LLM
    Architectures", §4 Gating Mechanism]: the attention output, on its way
    back to the residual stream, is multiplied element by element by the
    logistic sigmoid of a gate vector of the same shape. Reading: the gate is
    a caller-supplied tensor shaped like the output (one value per token and
    channel, before the sigmoid); the layer's merged output y is gated,
    float64: y * 1 / (1 + exp(-g)).
    """
    g = np.asarray(gate_out, np.float64)
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
    return np.asarray(y, np.float64) * sig


def key_sets(L: int, window: int, chunk: int, sel_rows: List[List[int]]):
    """The softmax (A) and linear (B) key sets of every query, for tests.

    sel_rows[c] lists the positions kept from chunk c. Returns boolean
    matrices A, B of shape [L, L] (row = query, column = key).
    """
    pos = np.arange(L)
    chunk_of = pos // chunk
    selected_chunk = np.full(L, -1)
    for c, row in enumerate(sel_rows):
        for j in row:
            if j >= 0:
                selected_chunk[j] = c
    A = np.zeros((L, L), dtype=bool)
    Bm = np.zeros((L, L), dtype=bool)
    for t in range(L):
        c = t // chunk
        in_pool = (selected_chunk >= 0) & (chunk_of < c)
        A[t] = (pos <= t) & ((pos >= t - window + 1) | (chunk_of == c) | in_pool)
        Bm[t] = (pos <= t) & ~A[t]
    return A, Bm
