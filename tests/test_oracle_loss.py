"""Pins of the oracle's language-model-head cross-entropy (the loss that segment-based peak
cutting splits, [summary] 4.4.2 / [notes] 4.4).

* zero weight: uniform softmax, so the loss is exactly log V and the gradient is zero;
* torch's cross_entropy and autograd (float64, CPU) as an independent implementation;
* pure-Python loops on a tiny case; central finite differences of the loss in h;
* the mean over rows equals the mean of any split into segments (the quantity is additive).
"""
import math

import numpy as np
import torch

import oracle


def test_zero_weight_closed_form():
    rng = np.random.default_rng(1)
    h = rng.standard_normal((7, 5))
    loss, rows, dh = oracle.lm_head_ce(h, np.zeros((11, 5)), rng.integers(0, 11, 7))
    assert abs(loss - math.log(11)) < 1e-15
    np.testing.assert_allclose(rows, math.log(11), rtol=1e-15)
    assert np.all(dh == 0.0)


def test_matches_torch_cross_entropy_and_autograd():
    rng = np.random.default_rng(2)
    T, d, V = 9, 6, 13
    h = rng.standard_normal((T, d))
    w = rng.standard_normal((V, d))
    t = rng.integers(0, V, T)
    loss, rows, dh = oracle.lm_head_ce(h, w, t)
    ht = torch.from_numpy(h).requires_grad_(True)
    lt = torch.nn.functional.cross_entropy(ht @ torch.from_numpy(w).T, torch.from_numpy(t))
    lt.backward()
    assert abs(loss - lt.item()) < 1e-12
    np.testing.assert_allclose(dh, ht.grad.numpy(), rtol=1e-10, atol=1e-13)


def test_brute_force_loops():
    rng = np.random.default_rng(3)
    T, d, V = 3, 2, 4
    h = rng.standard_normal((T, d))
    w = rng.standard_normal((V, d))
    t = [2, 0, 3]
    total = 0.0
    for i in range(T):
        z = [sum(h[i, k] * w[v, k] for k in range(d)) for v in range(V)]
        total += math.log(sum(math.exp(x) for x in z)) - z[t[i]]
    assert abs(oracle.lm_head_ce(h, w, t)[0] - total / T) < 1e-13


def test_finite_differences_and_segment_additivity():
    rng = np.random.default_rng(4)
    T, d, V = 8, 4, 10
    h = rng.standard_normal((T, d))
    w = rng.standard_normal((V, d))
    t = rng.integers(0, V, T)
    loss, rows, dh = oracle.lm_head_ce(h, w, t)
    eps = 1e-6
    for (i, k) in [(0, 0), (3, 2), (7, 3)]:
        hp, hm = h.copy(), h.copy()
        hp[i, k] += eps
        hm[i, k] -= eps
        fd = (oracle.lm_head_ce(hp, w, t)[0] - oracle.lm_head_ce(hm, w, t)[0]) / (2 * eps)
        assert abs(fd - dh[i, k]) < 1e-8
    parts = [oracle.lm_head_ce(h[a:a + 3], w, t[a:a + 3])[1] for a in range(0, T, 3)]
    np.testing.assert_allclose(np.concatenate(parts), rows, rtol=1e-14)


def test_logit_gradient_against_torch_autograd():
    # the logit gradient the oracle returns on request is the gradient of the mean loss with
    # respect to the logits (torch autograd through cross_entropy), each row sums to zero, and
    # dh is that gradient times w
    rng = np.random.default_rng(5)
    T, d, V = 6, 5, 9
    h = rng.standard_normal((T, d))
    w = rng.standard_normal((V, d))
    t = rng.integers(0, V, T)
    loss, rows, dh, g = oracle.lm_head_ce(h, w, t, with_logit_grad=True)
    z = torch.from_numpy(h @ w.T).requires_grad_(True)
    torch.nn.functional.cross_entropy(z, torch.from_numpy(t)).backward()
    np.testing.assert_allclose(g, z.grad.numpy(), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(g.sum(axis=1), 0.0, atol=1e-15)
    np.testing.assert_allclose(dh, g @ w, rtol=1e-13)
    assert (loss, list(rows)) == (oracle.lm_head_ce(h, w, t)[0], list(oracle.lm_head_ce(h, w, t)[1]))
