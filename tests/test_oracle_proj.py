"""Pins of the oracle's permutation-free projections ([notes] 4.4; [summary] 4.4.1).

* pure-Python loop brute force (no matrix products) on tiny cases;
* identity weight: the gathered projection returns exactly the kept rows, in kept order;
* a one-hot weight picks one input column;
* scatter-add leaves every eliminated row bitwise unchanged and equals gather -> dense
  product -> scatter for the kept rows; linearity in the weight.
"""
import numpy as np

import oracle


def _brute_gather(x, w, kept, block):
    B, S, K = x.shape
    N = w.shape[0]
    out = []
    for b in range(B):
        rows = [blk * block + t for blk in kept[b] for t in range(block)]
        yb = [[sum(float(x[b, i, kk]) * float(w[n, kk]) for kk in range(K)) for n in range(N)]
              for i in rows]
        out.append(yb)
    return out


def test_proj_gather_brute_force():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 12, 5))
    w = rng.standard_normal((3, 5))
    kept = [[0, 2], [1, 2]]
    got = oracle.proj_gather(x, w, kept, 4)
    ref = _brute_gather(x, w, kept, 4)
    for b in range(2):
        np.testing.assert_allclose(got[b], np.array(ref[b]), rtol=1e-13)


def test_proj_gather_identity_and_one_hot():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((1, 32, 8))
    kept = [[1, 3]]
    y = oracle.proj_gather(x, np.eye(8), kept, 8)
    np.testing.assert_array_equal(y[0], np.concatenate([x[0, 8:16], x[0, 24:32]]))
    w = np.zeros((1, 8))
    w[0, 5] = 1.0
    y = oracle.proj_gather(x, w, kept, 8)
    np.testing.assert_array_equal(y[0, :, 0], np.concatenate([x[0, 8:16, 5], x[0, 24:32, 5]]))


def test_proj_scatter_add_semantics():
    rng = np.random.default_rng(3)
    B, S, K, N, block = 2, 24, 6, 4, 4
    resid = rng.standard_normal((B, S, N))
    y = rng.standard_normal((B, 12, K))
    w = rng.standard_normal((N, K))
    kept = [[0, 3, 5], [2]]
    out = oracle.proj_scatter_add(resid, y, w, kept, block)
    for b in range(B):
        pos = oracle.token_positions(kept[b], block)
        elim = np.setdiff1d(np.arange(S), pos)
        assert np.array_equal(out[b, elim], resid[b, elim])
        np.testing.assert_allclose(out[b, pos] - resid[b, pos], y[b, :len(pos)] @ w.T, rtol=1e-12)
    # linear in the weight
    w2 = rng.standard_normal((N, K))
    a = oracle.proj_scatter_add(resid, y, w + w2, kept, block) - resid
    c = (oracle.proj_scatter_add(resid, y, w, kept, block) - resid) + \
        (oracle.proj_scatter_add(resid, y, w2, kept, block) - resid)
    np.testing.assert_allclose(a, c, rtol=1e-12, atol=1e-12)
