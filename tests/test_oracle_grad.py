"""Pins of the gradient oracle (CPU only): central finite differences of
the layer's output (every input element of a tiny case), torch's
scaled-dot-product attention gradients where the gate is 0 (the layer is
then masked softmax attention), and the forward it differentiates equal to
the brute-force oracle's output."""
import math

import numpy as np
import pytest
import torch

from oracle import bf, grad


def inputs(rng, B, Hq, Hkv, L, d):
    q = rng.standard_normal((B, Hq, L, d))
    k = rng.standard_normal((B, Hkv, L, d))
    v = rng.standard_normal((B, Hkv, L, d))
    F = rng.standard_normal((Hkv, d, d)) / math.sqrt(d)
    g = rng.uniform(0.2, 1.0, Hq)
    return q, k, v, F, g


KW = dict(window=3, chunk=4, budget=3 + 6, t_max=3)  # lambda = 2


def loss_of(q, k, v, F, g, dy, sel):
    o = grad.gradients(q, k, v, F, g, dy, sel=sel, **KW)
    return float((o["y"] * dy).sum())


def test_forward_is_the_brute_force_layer():
    rng = np.random.default_rng(1)
    q, k, v, F, g = inputs(rng, 2, 4, 2, 23, 8)
    o = grad.gradients(q, k, v, F, g, np.zeros_like(q), **KW)
    want = bf.prefill(q, k, v, F, g, **KW)["y"]
    np.testing.assert_allclose(o["y"], want, rtol=1e-12, atol=1e-13)


def test_gradients_match_central_differences():
    """Every element of q, k, v, F and the gates: (f(x+h) - f(x-h)) / 2h,
    f = sum(y * dy), with the selection of the unperturbed inputs."""
    rng = np.random.default_rng(2)
    q, k, v, F, g = inputs(rng, 1, 2, 1, 14, 4)
    dy = rng.standard_normal(q.shape)
    o = grad.gradients(q, k, v, F, g, dy, **KW)
    sel = o["sel"]
    assert (sel >= 0).sum() >= 4  # tokens are kept: both branches are live
    h = 1e-6
    args = [q, k, v, F, g]
    names = ["dq", "dk", "dv", "dfmap", "dgate"]
    for ai, name in enumerate(names):
        a = args[ai]
        fd = np.zeros_like(a)
        for idx in np.ndindex(a.shape):
            ap, am = a.copy(), a.copy()
            ap[idx] += h
            am[idx] -= h
            fp = loss_of(*[ap if i == ai else args[i] for i in range(5)], dy, sel)
            fm = loss_of(*[am if i == ai else args[i] for i in range(5)], dy, sel)
            fd[idx] = (fp - fm) / (2 * h)
        scale = max(1.0, float(np.abs(o[name]).max()))
        np.testing.assert_allclose(o[name], fd, rtol=0, atol=2e-7 * scale, err_msg=name)


def test_gate_zero_gradients_are_masked_sdpa_gradients():
    rng = np.random.default_rng(3)
    q, k, v, F, _ = inputs(rng, 1, 2, 1, 30, 8)
    g = np.zeros(2)
    dy = rng.standard_normal(q.shape)
    o = grad.gradients(q, k, v, F, g, dy, **KW)
    A, _ = bf.key_sets(30, KW["window"], KW["chunk"], o["sel"][0, 0].tolist())
    qt, kt, vt = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    y = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.expand(1, 2, 30, 8), vt.expand(1, 2, 30, 8), attn_mask=torch.tensor(A),
        scale=1 / math.sqrt(8))
    (y * torch.tensor(dy)).sum().backward()
    np.testing.assert_allclose(o["dq"], qt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(o["dk"], kt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(o["dv"], vt.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.all(o["dfmap"] == 0)
