"""Pins of the oracle's token-sparse attention forward and backward.

* keep everything: equals torch's causal scaled-dot-product attention (fp64) and its
  autograd gradients;
* any kept set: equals torch SDPA run on the gathered kept tokens, scattered back, and
  torch autograd of that; the explicit-mask and compact forms agree;
* closed forms: V = const gives O = const; Q = 0 gives the running mean of kept values,
  LSE = ln(#kept keys <= i) and dV_j = sum_{i >= j} dO_i / (rank(i)+1);
* softmax shift invariance: sum_j dK_j = 0 per KV head;
* central finite differences of L = <dOut, O> on a tiny case;
* eliminated rows: zero output, zero gradients, residual bitwise unchanged.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa(q, k, v, scale):
    """torch causal SDPA, fp64, GQA by repeating K/V. q [S,Hq,D] -> O [S,Hq,D]."""
    Hq, Hkv = q.shape[1], k.shape[1]
    qt = q.permute(1, 0, 2)[None]
    kt = k.repeat_interleave(Hq // Hkv, dim=1).permute(1, 0, 2)[None]
    vt = v.repeat_interleave(Hq // Hkv, dim=1).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    return o[0].permute(1, 0, 2)


def _library_sparse(q, k, v, kept, block, dout=None):
    """Gather kept tokens, torch SDPA (causal over kept ranks), scatter; optional grads."""
    B, S, Hq, D = q.shape
    scale = 1.0 / math.sqrt(D)
    pos = oracle.token_positions(kept, block)
    O = np.zeros(q.shape)
    grads = [np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)]
    for b in range(B):
        qt = torch.tensor(q[b, pos], requires_grad=True)
        kt = torch.tensor(k[b, pos], requires_grad=True)
        vt = torch.tensor(v[b, pos], requires_grad=True)
        o = _sdpa(qt, kt, vt, scale)
        O[b, pos] = o.detach().numpy()
        if dout is not None:
            (o * torch.tensor(dout[b, pos])).sum().backward()
            grads[0][b, pos] = qt.grad.numpy()
            grads[1][b, pos] = kt.grad.numpy()
            grads[2][b, pos] = vt.grad.numpy()
    return O, grads


CASES = [
    # B, S, Hq, Hkv, D, block, kept
    (1, 64, 2, 2, 8, 8, [0, 1, 2, 3, 4, 5, 6, 7]),
    (2, 64, 4, 2, 16, 8, [1, 3, 4, 7]),
    (1, 96, 3, 1, 8, 16, [0, 2, 5]),
    (1, 128, 2, 2, 32, 32, [3]),
    (1, 64, 2, 1, 8, 8, [0, 7]),
]


@pytest.mark.parametrize("B,S,Hq,Hkv,D,block,kept", CASES)
def test_fwd_matches_library_sdpa(B, S, Hq, Hkv, D, block, kept):
    q, k, v = _rand((B, S, Hq, D), 1), _rand((B, S, Hkv, D), 2), _rand((B, S, Hkv, D), 3)
    kept = np.array(kept)
    O, LSE = oracle.attn_fwd_masked(q, k, v, kept, block)
    Oref, _ = _library_sparse(q, k, v, kept, block)
    np.testing.assert_allclose(O, Oref, atol=1e-12, rtol=1e-12)
    Oc, LSEc = oracle.attn_fwd_compact(q, k, v, kept, block)
    np.testing.assert_allclose(Oc, O, atol=1e-12, rtol=1e-12)
    np.testing.assert_array_equal(np.isinf(LSE), np.isinf(LSEc))
    fin = np.isfinite(LSE)
    np.testing.assert_allclose(LSEc[fin], LSE[fin], rtol=1e-12)
    # eliminated rows: zero output, -inf LSE
    elim = np.setdiff1d(np.arange(S), oracle.token_positions(kept, block))
    assert np.all(O[:, elim] == 0) and np.all(np.isneginf(LSE[:, :, elim]))


def test_keep_all_equals_dense_causal():
    B, S, Hq, Hkv, D, block = 1, 64, 4, 2, 16, 8
    q, k, v = _rand((B, S, Hq, D), 4), _rand((B, S, Hkv, D), 5), _rand((B, S, Hkv, D), 6)
    O, _ = oracle.attn_fwd(q, k, v, np.arange(S // block), block)
    ref = _sdpa(torch.tensor(q[0]), torch.tensor(k[0]), torch.tensor(v[0]), 1 / math.sqrt(D))
    np.testing.assert_allclose(O[0], ref.numpy(), atol=1e-12)


def test_fwd_closed_forms():
    B, S, Hq, D, block = 1, 64, 2, 8, 8
    kept = np.array([1, 2, 5, 6])
    pos = oracle.token_positions(kept, block)
    k = _rand((B, S, Hq, D), 7)
    # V = const -> O = const at kept rows
    v = np.full((B, S, Hq, D), 0.375)
    O, _ = oracle.attn_fwd(_rand((B, S, Hq, D), 8), k, v, kept, block)
    np.testing.assert_allclose(O[0, pos], 0.375, rtol=1e-14)
    # Q = 0 -> uniform weights over kept keys <= i
    v = _rand((B, S, Hq, D), 9)
    O, LSE = oracle.attn_fwd(np.zeros((B, S, Hq, D)), k, v, kept, block)
    for r, i in enumerate(pos):
        np.testing.assert_allclose(O[0, i], v[0, pos[:r + 1]].mean(axis=0), atol=1e-13)
        np.testing.assert_allclose(LSE[0, :, i], math.log(r + 1), rtol=1e-14)


def test_residual_add_leaves_eliminated_rows_bitwise():
    B, S, Hq, D, block = 1, 64, 2, 8, 8
    kept = np.array([0, 3, 4])
    q, k, v = _rand((B, S, Hq, D), 10), _rand((B, S, Hq, D), 11), _rand((B, S, Hq, D), 12)
    resid = _rand((B, S, Hq, D), 13).astype(np.float32)
    O, _ = oracle.attn_fwd(q, k, v, kept, block)
    out = oracle.residual_add(resid, O, kept, block)
    elim = np.setdiff1d(np.arange(S), oracle.token_positions(kept, block))
    assert np.array_equal(out[:, elim], resid[:, elim].astype(np.float64))
    pos = oracle.token_positions(kept, block)
    np.testing.assert_allclose(out[:, pos] - resid[:, pos], O[:, pos], atol=1e-12)


@pytest.mark.parametrize("B,S,Hq,Hkv,D,block,kept", CASES)
def test_bwd_matches_library_autograd(B, S, Hq, Hkv, D, block, kept):
    q, k, v = _rand((B, S, Hq, D), 21), _rand((B, S, Hkv, D), 22), _rand((B, S, Hkv, D), 23)
    dout = _rand((B, S, Hq, D), 24)
    kept = np.array(kept)
    dq, dk, dv = oracle.attn_bwd_masked(q, k, v, kept, block, dout)
    _, (rq, rk, rv) = _library_sparse(q, k, v, kept, block, dout)
    np.testing.assert_allclose(dq, rq, atol=1e-11)
    np.testing.assert_allclose(dk, rk, atol=1e-11)
    np.testing.assert_allclose(dv, rv, atol=1e-11)
    cq, ck, cv = oracle.attn_bwd_compact(q, k, v, kept, block, dout)
    np.testing.assert_allclose(cq, dq, atol=1e-12)
    np.testing.assert_allclose(ck, dk, atol=1e-12)
    np.testing.assert_allclose(cv, dv, atol=1e-12)
    elim = np.setdiff1d(np.arange(S), oracle.token_positions(kept, block))
    assert np.all(dq[:, elim] == 0) and np.all(dk[:, elim] == 0) and np.all(dv[:, elim] == 0)
    # softmax shift invariance: sum over keys of dK is zero per KV head
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-11)


def test_bwd_finite_differences():
    B, S, Hq, Hkv, D, block = 1, 32, 2, 1, 8, 8
    kept = np.array([0, 2, 3])
    q, k, v = _rand((B, S, Hq, D), 31), _rand((B, S, Hkv, D), 32), _rand((B, S, Hkv, D), 33)
    dout = _rand((B, S, Hq, D), 34)
    dq, dk, dv = oracle.attn_bwd(q, k, v, kept, block, dout)
    pos = oracle.token_positions(kept, block)

    def loss(qq, kk, vv):
        O, _ = oracle.attn_fwd(qq, kk, vv, kept, block)
        return float((O * dout).sum())

    h = 1e-6
    rng = np.random.default_rng(0)
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        idxs = [tuple(int(rng.integers(0, n)) for n in arr.shape) for _ in range(40)]
        idxs += [(0, int(p), 0, 1) for p in pos[::5]]
        for idx in idxs:
            if idx[2] >= arr.shape[2]:
                continue
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += h
            minus[idx] -= h
            args_p = {"q": (plus, k, v), "k": (q, plus, v), "v": (q, k, plus)}[name]
            args_m = {"q": (minus, k, v), "k": (q, minus, v), "v": (q, k, minus)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(grad[idx])), (name, idx, fd, grad[idx])


def test_bwd_closed_form_q_zero():
    B, S, Hq, D, block = 1, 64, 2, 4, 8
    kept = np.array([0, 2, 3, 6])
    pos = oracle.token_positions(kept, block)
    k, v, dout = _rand((B, S, Hq, D), 41), _rand((B, S, Hq, D), 42), _rand((B, S, Hq, D), 43)
    _, _, dv = oracle.attn_bwd(np.zeros((B, S, Hq, D)), k, v, kept, block, dout)
    for r, j in enumerate(pos):
        ref = sum(dout[0, pos[t]] / (t + 1) for t in range(r, len(pos)))
        np.testing.assert_allclose(dv[0, j], ref, atol=1e-12)


def test_sampled_helpers_match_full():
    B, S, Hq, Hkv, D, block = 1, 128, 4, 2, 8, 16
    kept = np.array([0, 2, 3, 5, 7])
    q, k, v = _rand((B, S, Hq, D), 51), _rand((B, S, Hkv, D), 52), _rand((B, S, Hkv, D), 53)
    dout = _rand((B, S, Hq, D), 54)
    pos = oracle.token_positions(kept, block)
    O, LSE = oracle.attn_fwd(q, k, v, kept, block)
    ranks = [0, 5, 17, 40, 79]
    for h in range(Hq):
        o, l = oracle.attn_fwd_rows(q, k, v, kept, block, 0, h, ranks)
        np.testing.assert_allclose(o, O[0, pos[ranks], h], atol=1e-12)
        np.testing.assert_allclose(l, LSE[0, h, pos[ranks]], rtol=1e-12)
    dq, dk, dv = oracle.attn_bwd(q, k, v, kept, block, dout)
    for g in range(Hkv):
        sk, sv, sq = oracle.attn_bwd_sampled(q, k, v, kept, block, dout, 0, g, ranks, ranks)
        np.testing.assert_allclose(sk, dk[0, pos[ranks], g], atol=1e-12)
        np.testing.assert_allclose(sv, dv[0, pos[ranks], g], atol=1e-12)
        for hh in range(Hq // Hkv):
            np.testing.assert_allclose(sq[hh], dq[0, pos[ranks], g * (Hq // Hkv) + hh], atol=1e-12)


def test_stack_all_eliminated_rows_bitwise_and_additive():
    B, S, Hq, D, block = 1, 64, 2, 8, 8
    x0 = _rand((B, S, Hq, D), 61).astype(np.float32)
    kepts = [np.array([0, 1, 4]), np.array([1, 2]), np.array([0, 4, 5])]
    layers = [(_rand((B, S, Hq, D), 70 + l), _rand((B, S, Hq, D), 80 + l),
               _rand((B, S, Hq, D), 90 + l), kepts[l]) for l in range(3)]
    x, outs = oracle.stack_forward(x0, layers, block)
    never = np.setdiff1d(np.arange(S), np.concatenate([oracle.token_positions(kk, block) for kk in kepts]))
    assert len(never) == 24          # blocks 3, 6, 7
    assert np.array_equal(x[:, never], x0[:, never].astype(np.float64))
    np.testing.assert_allclose(x, x0 + sum(outs), atol=1e-12)
