"""Pins of the oracle's block scores against things other than itself.

* torch's scaled-dot-product attention (fp64, causal) with V = identity returns the
  causal softmax matrix P itself; its column sums minus the diagonal are the received
  masses of Eq. 1 (self term excluded), so block scores follow from a library routine;
* the closed form at Q = 0: P_ij = 1/(i+1), so M(j) = H_S - H_{j+1} (harmonic numbers,
  computed with exact fractions);
* the checksum sum_j M(j) = S - sum_i P_ii;
* a pure-Python loop brute force on a tiny case; head-permutation invariance; GQA equals
  MHA with repeated K.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def _sdpa_probs(qh, kh):
    """Causal softmax matrix from torch SDPA with V = identity (fp64, CPU)."""
    S, D = qh.shape
    q = torch.from_numpy(qh)[None, None]
    k = torch.from_numpy(kh)[None, None]
    eye = torch.eye(S, dtype=torch.float64)[None, None]
    P = torch.nn.functional.scaled_dot_product_attention(q, k, eye, is_causal=True,
                                                         scale=1.0 / math.sqrt(D))
    return P[0, 0].numpy()


def _scores_via_sdpa(q, k, block):
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    out = np.zeros((B, S // block))
    for b in range(B):
        for h in range(Hq):
            P = _sdpa_probs(q[b, :, h], k[b, :, h // (Hq // Hkv)])
            M = P.sum(axis=0) - np.diag(P)
            out[b] += M.reshape(-1, block).sum(axis=1)
    return out / Hq


@pytest.mark.parametrize("B,S,Hq,Hkv,D,block", [(1, 64, 2, 2, 8, 8), (2, 96, 4, 2, 16, 16),
                                                (1, 128, 3, 1, 8, 32)])
def test_scores_match_library_softmax(B, S, Hq, Hkv, D, block):
    rng = np.random.default_rng(11)
    q = rng.standard_normal((B, S, Hq, D))
    k = rng.standard_normal((B, S, Hkv, D))
    got = oracle.block_scores(q, k, block)
    ref = _scores_via_sdpa(q, k, block)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_scores_closed_form_q_zero():
    S, block, Hq, D = 48, 8, 3, 4
    q = np.zeros((1, S, Hq, D))
    k = np.random.default_rng(3).standard_normal((1, S, Hq, D))
    got = oracle.block_scores(q, k, block)[0]
    H = [Fraction(0)]
    for n in range(1, S + 1):
        H.append(H[-1] + Fraction(1, n))
    M = [H[S] - H[j + 1] for j in range(S)]          # sum_{i=j+1}^{S-1} 1/(i+1)
    ref = [float(sum(M[n * block:(n + 1) * block], Fraction(0))) for n in range(S // block)]
    np.testing.assert_allclose(got, ref, rtol=1e-13)
    # total received mass at Q = 0 is S - H_S
    assert abs(got.sum() - float(S - H[S])) < 1e-11


def test_scores_checksum_and_positivity():
    rng = np.random.default_rng(5)
    S, Hq, D, block = 80, 2, 8, 8
    q = rng.standard_normal((1, S, Hq, D)) * 2
    k = rng.standard_normal((1, S, Hq, D)) * 2
    s = oracle.block_scores(q, k, block)[0]
    diag = sum(np.diag(_sdpa_probs(q[0, :, h], k[0, :, h])).sum() for h in range(Hq)) / Hq
    assert abs(s.sum() - (S - diag)) < 1e-10
    assert np.all(s > 0)


def test_scores_brute_force_loops():
    rng = np.random.default_rng(9)
    S, Hq, D, block = 12, 2, 3, 4
    q = rng.standard_normal((1, S, Hq, D))
    k = rng.standard_normal((1, S, Hq, D))
    sc = 1 / math.sqrt(D)
    ref = [0.0] * (S // block)
    for h in range(Hq):
        for i in range(S):
            logits = [sc * sum(q[0, i, h, d] * k[0, j, h, d] for d in range(D)) for j in range(i + 1)]
            mx = max(logits)
            den = sum(math.exp(x - mx) for x in logits)
            for j in range(i):                        # j != i, j <= i
                ref[j // block] += math.exp(logits[j] - mx) / den / Hq
    np.testing.assert_allclose(oracle.block_scores(q, k, block)[0], ref, rtol=1e-12)


def test_scores_head_permutation_and_gqa():
    rng = np.random.default_rng(21)
    S, Hq, Hkv, D, block = 64, 4, 2, 8, 16
    q = rng.standard_normal((1, S, Hq, D))
    k = rng.standard_normal((1, S, Hkv, D))
    base = oracle.block_scores(q, k, block)
    krep = np.repeat(k, Hq // Hkv, axis=2)
    np.testing.assert_allclose(oracle.block_scores(q, krep, block), base, rtol=1e-13)
    perm = [2, 0, 3, 1]
    np.testing.assert_allclose(oracle.block_scores(q[:, :, perm], krep[:, :, perm], block), base,
                               rtol=1e-13)


def test_received_mass_uniform_sanity():
    # Every query row of a causal softmax sums to 1: total mass received by tokens
    # other than the query itself is S - sum_i P_ii, and P_00 = 1.
    rng = np.random.default_rng(2)
    S, D = 40, 4
    qh = rng.standard_normal((S, D))
    kh = rng.standard_normal((S, D))
    M = oracle.received_mass(qh, kh, 0.5)
    assert M[-1] == 0.0                                # nothing after the last token
    assert M.sum() <= S - 1 + 1e-12
