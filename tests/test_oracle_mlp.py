"""Pins of the oracle's MLP-block token elimination ([summary] 4.2.4; [notes] 4.2, extension of
token elimination to the MLP block): the activation, token and block informativeness, the
gathered-row down projection with in-place residual add, and the composed sparse MLP.

* pure-Python loops with math.exp on tiny inputs;
* torch's float64 relu / silu and matmul as an independent implementation;
* closed forms: a zero gate gives zero activation; silu(ln 3) = (3/4) ln 3; an identity
  first layer makes the ReLU activation the positive part of the input;
* invariants: permuting the units, flipping the sign of the up projection, scaling by c > 0,
  permuting tokens inside a block; eliminated residual rows stay bitwise unchanged;
* with every block kept the sparse MLP equals torch's dense MLP.
"""
import math

import numpy as np
import torch

import oracle


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_activation_and_scores_brute_force():
    rng = np.random.default_rng(11)
    S, K, F, blk = 4, 3, 5, 2
    x = _rand(rng, 1, S, K)
    wg, wu = _rand(rng, F, K), _rand(rng, F, K)
    act = oracle.mlp_activation(x, wg, wu, oracle.MLP_SILU_GATED)
    tok, blocks = [], []
    for i in range(S):
        row = []
        for f in range(F):
            z = sum(x[0, i, k] * wg[f, k] for k in range(K))
            u = sum(x[0, i, k] * wu[f, k] for k in range(K))
            row.append(z / (1.0 + math.exp(-z)) * u)
        assert np.allclose(act[0, i], row, rtol=1e-13, atol=1e-15)
        tok.append(sum(abs(v) for v in row) / F)
    for n in range(S // blk):
        blocks.append(max(tok[n * blk:(n + 1) * blk]))
    np.testing.assert_allclose(oracle.mlp_token_scores(act)[0], tok, rtol=1e-13)
    np.testing.assert_allclose(oracle.mlp_block_scores(act, blk)[0], blocks, rtol=1e-13)

    relu = oracle.mlp_activation(x, wg, None, oracle.MLP_RELU)
    for i in range(S):
        for f in range(F):
            z = sum(x[0, i, k] * wg[f, k] for k in range(K))
            assert abs(relu[0, i, f] - (z if z > 0 else 0.0)) < 1e-14


def test_matches_torch_relu_and_silu():
    rng = np.random.default_rng(12)
    x = _rand(rng, 2, 16, 8)
    wg, wu = _rand(rng, 24, 8), _rand(rng, 24, 8)
    xt, gt, ut = (torch.from_numpy(v) for v in (x, wg, wu))
    ref = torch.nn.functional.silu(xt @ gt.T) * (xt @ ut.T)
    np.testing.assert_allclose(oracle.mlp_activation(x, wg, wu), ref.numpy(), rtol=1e-12,
                               atol=1e-14)
    ref = torch.relu(xt @ gt.T)
    np.testing.assert_allclose(oracle.mlp_activation(x, wg, None, oracle.MLP_RELU), ref.numpy(),
                               rtol=1e-12, atol=1e-14)


def test_closed_forms():
    rng = np.random.default_rng(13)
    x = _rand(rng, 1, 8, 6)
    # zero gate: silu(0) = 0 for every unit, whatever the up projection
    act = oracle.mlp_activation(x, np.zeros((10, 6)), _rand(rng, 10, 6))
    assert np.all(act == 0.0)
    assert np.all(oracle.mlp_block_scores(act, 4) == 0.0)
    # sigmoid(ln 3) = 3/4, so silu(ln 3) * (2 ln 3) = 1.5 (ln 3)^2
    a = oracle.mlp_activation(np.array([[[math.log(3.0)]]]), np.array([[1.0]]), np.array([[2.0]]))
    assert abs(a[0, 0, 0] - 1.5 * math.log(3.0) ** 2) < 1e-14
    # identity first layer (F = K): ReLU activation = positive part; score = its mean over F
    relu = oracle.mlp_activation(x, np.eye(6), None, oracle.MLP_RELU)
    assert np.array_equal(relu, np.maximum(x, 0.0))
    np.testing.assert_allclose(oracle.mlp_token_scores(relu), np.maximum(x, 0).mean(axis=2),
                               rtol=1e-15)


def test_invariants():
    rng = np.random.default_rng(14)
    x = _rand(rng, 2, 12, 5)
    wg, wu = _rand(rng, 9, 5), _rand(rng, 9, 5)
    e = oracle.mlp_token_scores(oracle.mlp_activation(x, wg, wu))
    perm = rng.permutation(9)
    np.testing.assert_allclose(oracle.mlp_token_scores(oracle.mlp_activation(x, wg[perm], wu[perm])),
                               e, rtol=1e-13)
    # magnitude, not the positive part: flipping the up projection changes no score
    np.testing.assert_allclose(oracle.mlp_token_scores(oracle.mlp_activation(x, wg, -wu)), e,
                               rtol=1e-13)
    np.testing.assert_allclose(oracle.mlp_token_scores(oracle.mlp_activation(x, wg, 2.5 * wu)),
                               2.5 * e, rtol=1e-13)
    # block maximum: one of the block's own token scores, and order inside a block is irrelevant
    act = oracle.mlp_activation(x, wg, wu)
    bs = oracle.mlp_block_scores(act, 4)
    for b in range(2):
        for n in range(3):
            seg = e[b, 4 * n:4 * n + 4]
            assert bs[b, n] == seg.max() and bs[b, n] in seg
    sh = act.copy()
    sh[:, 4:8] = sh[:, [6, 4, 7, 5]]
    assert np.array_equal(oracle.mlp_block_scores(sh, 4), bs)


def test_gather_scatter_add_brute_force_and_untouched_rows():
    rng = np.random.default_rng(15)
    B, S, K, N, blk = 2, 8, 3, 4, 2
    resid, a, w = _rand(rng, B, S, N), _rand(rng, B, S, K), _rand(rng, N, K)
    kept = [np.array([0, 2]), np.array([3])]
    out = oracle.proj_gather_scatter_add(resid, a, w, kept, blk)
    for b in range(B):
        pos = set(int(p) for kb in kept[b] for p in range(kb * blk, kb * blk + blk))
        for i in range(S):
            for n in range(N):
                want = resid[b, i, n]
                if i in pos:
                    want += sum(a[b, i, k] * w[n, k] for k in range(K))
                    assert abs(out[b, i, n] - want) < 1e-13
                else:
                    assert out[b, i, n] == want


def test_sparse_forward_keep_all_is_dense_mlp_and_topk_set():
    rng = np.random.default_rng(16)
    B, S, K, F, blk = 2, 16, 6, 12, 4
    x, resid = _rand(rng, B, S, K), _rand(rng, B, S, K)
    wg, wu, wd = _rand(rng, F, K), _rand(rng, F, K), _rand(rng, K, F)
    out, sc, kept = oracle.mlp_sparse_forward(x, wg, wu, wd, resid, blk, oracle.SELECT_TOPK, 1.0)
    xt = torch.from_numpy(x)
    dense = torch.from_numpy(resid) + (torch.nn.functional.silu(xt @ torch.from_numpy(wg).T)
                                       * (xt @ torch.from_numpy(wu).T)) @ torch.from_numpy(wd).T
    np.testing.assert_allclose(out, dense.numpy(), rtol=1e-12, atol=1e-12)

    out, sc, kept = oracle.mlp_sparse_forward(x, wg, wu, wd, resid, blk, oracle.SELECT_TOPK, 0.5)
    for b in range(B):
        order = sorted(range(S // blk), key=lambda n: (-np.float32(sc[b, n]), n))
        assert sorted(order[:2]) == list(kept[b])
        for n in range(S // blk):
            rows = slice(n * blk, (n + 1) * blk)
            if n in kept[b]:
                assert not np.array_equal(out[b, rows], resid[b, rows])
            else:
                assert np.array_equal(out[b, rows], resid[b, rows])
