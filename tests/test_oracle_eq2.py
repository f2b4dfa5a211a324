"""Pins of the oracle's Eq. 2 literal block scores ([summary] 4.2.2 Eq. 2 and 4.2.3).

* a pure-Python loop brute force on tiny cases (no NumPy matrix products);
* closed forms: constant query / key vectors give one value e for every causal element, so
  every score block is e and s_n = (nKB - n) e; all-negative scores give s = 0;
* the maximum (not the sum) over a score block: a single positive query row leaves exactly
  the blocks it touches at its value;
* the causal mask on diagonal blocks: a positive score that only occurs above the diagonal
  does not count;
* positive homogeneity in Q, head-permutation invariance, GQA equals MHA with repeated K.
"""
import math

import numpy as np
import pytest

import oracle


def _brute(q, k, block, scale):
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    nkb = S // block
    out = [[0.0] * nkb for _ in range(B)]
    for b in range(B):
        for n in range(nkb):
            total = 0.0
            for m in range(n, nkb):
                best = None
                for i in range(m * block, (m + 1) * block):
                    for j in range(n * block, (n + 1) * block):
                        if j > i:
                            continue
                        e = 0.0
                        for h in range(Hq):
                            dot = 0.0
                            for d in range(D):
                                dot += float(q[b, i, h, d]) * float(k[b, j, h // G, d])
                            e += max(scale * dot, 0.0)
                        e /= Hq
                        best = e if best is None or e > best else best
                total += best
            out[b][n] = total
    return np.array(out)


@pytest.mark.parametrize("B,S,Hq,Hkv,D,block", [(1, 16, 2, 1, 3, 4), (2, 12, 2, 2, 2, 3),
                                                (1, 16, 4, 2, 4, 8)])
def test_eq2_brute_force_loops(B, S, Hq, Hkv, D, block):
    rng = np.random.default_rng(5)
    q = rng.standard_normal((B, S, Hq, D))
    k = rng.standard_normal((B, S, Hkv, D))
    scale = 1.0 / math.sqrt(D)
    np.testing.assert_allclose(oracle.block_scores_eq2(q, k, block), _brute(q, k, block, scale),
                               rtol=1e-12, atol=1e-14)


def test_eq2_constant_vectors_closed_form():
    S, block, Hq, Hkv, D = 32, 8, 4, 2, 5
    rng = np.random.default_rng(9)
    a = rng.standard_normal((Hq, D))
    c = rng.standard_normal((Hkv, D))
    q = np.broadcast_to(a, (1, S, Hq, D)).copy()
    k = np.broadcast_to(c, (1, S, Hkv, D)).copy()
    scale = 1.0 / math.sqrt(D)
    e = sum(max(scale * float(a[h] @ c[h // 2]), 0.0) for h in range(Hq)) / Hq
    nkb = S // block
    want = np.array([(nkb - n) * e for n in range(nkb)])
    np.testing.assert_allclose(oracle.block_scores_eq2(q, k, block)[0], want, rtol=1e-13)


def test_eq2_all_negative_scores_give_zero():
    S, block, H, D = 24, 6, 3, 4
    v = np.random.default_rng(2).standard_normal((H, D))
    q = np.broadcast_to(-v, (1, S, H, D)).copy()
    k = np.broadcast_to(v, (1, S, H, D)).copy()
    assert np.all(oracle.block_scores_eq2(q, k, block) == 0.0)


def test_eq2_is_a_block_maximum_not_a_sum():
    # every score is -|v|^2 scale except the row of query i_star, whose scores are +|v|^2 scale
    S, block, D = 32, 8, 4
    v = np.array([1.0, -2.0, 0.5, 1.5])
    q = np.broadcast_to(-v, (1, S, 1, D)).copy()
    k = np.broadcast_to(v, (1, S, 1, D)).copy()
    i_star = 19                                          # query block 2
    q[0, i_star, 0] = v
    val = float(v @ v) / math.sqrt(D)
    got = oracle.block_scores_eq2(q, k, block)[0]
    np.testing.assert_allclose(got, [val, val, val, 0.0], rtol=1e-14)


def test_eq2_masked_positive_scores_do_not_count():
    # the only positive score sits above the diagonal of score block (0, 0)
    S, block, D = 16, 8, 3
    v = np.array([1.0, 2.0, -1.0])
    q = np.zeros((1, S, 1, D))
    k = np.broadcast_to(-v, (1, S, 1, D)).copy()
    q[0, 0, 0] = v
    k[0, 1, 0] = v                                       # q_0 . k_1 > 0, but 1 > 0 is masked
    assert np.all(oracle.block_scores_eq2(q, k, block) == 0.0)
    k[0, 0, 0] = v                                       # now an allowed positive element exists
    np.testing.assert_allclose(oracle.block_scores_eq2(q, k, block)[0],
                               [float(v @ v) / math.sqrt(D), 0.0], rtol=1e-14)


def test_eq2_homogeneity_permutation_gqa():
    rng = np.random.default_rng(21)
    B, S, Hq, Hkv, D, block = 1, 32, 4, 2, 6, 8
    q = rng.standard_normal((B, S, Hq, D))
    k = rng.standard_normal((B, S, Hkv, D))
    base = oracle.block_scores_eq2(q, k, block)
    np.testing.assert_allclose(oracle.block_scores_eq2(2.5 * q, k, block), 2.5 * base, rtol=1e-13)
    # swapping the two query heads of one KV group changes nothing
    q2 = q.copy()
    q2[:, :, [0, 1]] = q[:, :, [1, 0]]
    np.testing.assert_allclose(oracle.block_scores_eq2(q2, k, block), base, rtol=1e-13)
    k_rep = np.repeat(k, Hq // Hkv, axis=2)
    np.testing.assert_allclose(oracle.block_scores_eq2(q, k_rep, block), base, rtol=1e-13)


def test_eq2_key_block_subset_matches_full():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 40, 2, 4))
    k = rng.standard_normal((1, 40, 2, 4))
    full = oracle.block_scores_eq2(q, k, 8)
    part = oracle.block_scores_eq2(q, k, 8, key_blocks=[1, 4])
    np.testing.assert_array_equal(part[0, [1, 4]], full[0, [1, 4]])
    assert np.isnan(part[0, [0, 2, 3]]).all()
