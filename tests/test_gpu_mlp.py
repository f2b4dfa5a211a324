"""GPU parity of token elimination in the MLP block ([summary] 4.2.4; [notes] 4.2) against the
oracle: the fused activation (gated SiLU and ReLU) with per-token and per-block
informativeness, the selection on those scores, and the down projection of the kept tokens
added into the residual in place (rows gathered from the full activation).

Tolerances: token and block scores 1e-5 relative (fp32 GEMM, then a sum of magnitudes);
the bf16 activation within one bf16 rounding of the oracle's value (2^-8 relative) plus
1e-5; the residual 2e-2 max-abs as for every bf16 product; selection bit-exact on the GPU's
own scores; eliminated residual rows bitwise unchanged."""
import numpy as np
import pytest

import oracle
from gpu_helpers import kept_tensor, max_abs, say

pytestmark = pytest.mark.gpu
TOL = 2e-2
SCORE_RTOL = 1e-5


@pytest.fixture(scope="module")
def J():
    import token_sparse_attention_jenga_amd as J
    return J


def _bf16(rng, shape, std=1.0):
    from synth.generate import to_bf16_bits_f32
    return to_bf16_bits_f32((rng.standard_normal(shape, dtype=np.float32) * std).astype(np.float32))


def _dev(a, bf16=True):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t.to(torch.bfloat16) if bf16 else t).cuda()


def _round_bf16(a):
    from synth.generate import to_bf16_bits_f32
    return to_bf16_bits_f32(np.asarray(a, dtype=np.float32))


def _check_act(got, ref):
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5)


def _kind_weights(rng, kind, F, K):
    w1 = _bf16(rng, (F, K), 1.0 / np.sqrt(K))
    wu = _bf16(rng, (F, K), 1.0 / np.sqrt(K)) if kind == oracle.MLP_SILU_GATED else None
    return w1, wu


CASES = [
    # kind, B, S, block, K, F   (S % 256 != 0 and F % 128 != 0 give ragged row / column tiles)
    (oracle.MLP_SILU_GATED, 2, 320, 64, 128, 192),
    (oracle.MLP_SILU_GATED, 1, 1024, 128, 256, 512),
    (oracle.MLP_SILU_GATED, 1, 768, 256, 64, 64),
    (oracle.MLP_RELU, 2, 320, 64, 128, 256),
    (oracle.MLP_RELU, 1, 1024, 128, 256, 384),
]


@pytest.mark.parametrize("kind,B,S,block,K,F", CASES)
def test_mlp_act_scores_match_oracle(J, kind, B, S, block, K, F):
    import torch
    rng = np.random.default_rng(1000 * kind + S + K + F)
    x = _bf16(rng, (B, S, K))
    w1, wu = _kind_weights(rng, kind, F, K)
    say(f"mlp act kind{kind} B{B} S{S} block{block} K{K} F{F}")
    act, tok, blk = J.mlp_act_scores(_dev(x), _dev(w1), _dev(wu) if wu is not None else None,
                                     kind, block)
    torch.cuda.synchronize()
    ref = oracle.mlp_activation(x, w1, wu, kind)
    _check_act(act.float().cpu().numpy(), ref)
    np.testing.assert_allclose(tok.cpu().numpy(), oracle.mlp_token_scores(ref), rtol=SCORE_RTOL)
    bs = blk.cpu().numpy()
    np.testing.assert_allclose(bs, oracle.mlp_block_scores(ref, block), rtol=SCORE_RTOL)
    # the block score is the largest of the GPU's own token scores, exactly
    assert np.array_equal(bs, tok.cpu().numpy().reshape(B, S // block, block).max(axis=2))
    # repeatable bit for bit
    act2, tok2, blk2 = J.mlp_act_scores(_dev(x), _dev(w1), _dev(wu) if wu is not None else None,
                                        kind, block)
    assert torch.equal(act, act2) and torch.equal(tok, tok2) and torch.equal(blk, blk2)


@pytest.mark.parametrize("mode,param", [(oracle.SELECT_TOPK, 0.5), (oracle.SELECT_THRESH_REL, 1.0)])
def test_sparse_mlp_forward_matches_oracle(J, mode, param):
    import torch
    B, S, block, K, F = 2, 1024, 64, 128, 320
    rng = np.random.default_rng(77 + mode)
    x = _bf16(rng, (B, S, K))
    wg, wu = _kind_weights(rng, oracle.MLP_SILU_GATED, F, K)
    wd = _bf16(rng, (K, F), 1.0 / np.sqrt(F))
    resid = rng.standard_normal((B, S, K), dtype=np.float32)
    rd = _dev(resid, bf16=False)
    say(f"sparse mlp forward mode{mode} param{param} B{B} S{S} block{block} K{K} F{F}")
    blk, kept, n_kept, mkb = J.sparse_mlp_forward(_dev(x), _dev(wg), _dev(wu), _dev(wd), rd,
                                                  block, mode, param)
    torch.cuda.synchronize()
    bs = blk.cpu().numpy()
    kg = kept.cpu().numpy()
    ng = n_kept.cpu().numpy()
    kept_list = []
    for b in range(B):
        want = oracle.select_blocks(bs[b], mode, param)        # the GPU's own scores: bit-exact
        assert list(kg[b, :ng[b]]) == list(want)
        kept_list.append(want)
    ref_out, ref_sc, ref_kept = oracle.mlp_sparse_forward(x, wg, wu, wd, resid, block, mode, param,
                                                          act_round=_round_bf16)
    np.testing.assert_allclose(bs, ref_sc, rtol=SCORE_RTOL)
    for b in range(B):
        assert list(ref_kept[b]) == list(kept_list[b])
    out = rd.cpu().numpy()
    for b in range(B):
        pos = oracle.token_positions(kept_list[b], block)
        elim = np.setdiff1d(np.arange(S), pos)
        assert np.array_equal(out[b, elim], resid[b, elim])    # bitwise untouched
        assert max_abs(out[b, pos], ref_out[b, pos]) <= TOL


def test_gather_scatter_add_ragged(J):
    """Down projection alone: kept lists of different lengths per batch row, max_kept_blocks
    above every count, rows gathered from a strided (non-contiguous) activation view."""
    import torch
    B, S, block, K, N = 2, 640, 64, 192, 256
    rng = np.random.default_rng(5)
    a_full = _bf16(rng, (B, S, K + 64))
    w = _bf16(rng, (N, K), 1.0 / np.sqrt(K))
    resid = rng.standard_normal((B, S, N), dtype=np.float32)
    kept = [[0, 3, 4, 9], [7]]
    kd, nd = kept_tensor(kept, S // block)
    ad = _dev(a_full)[:, :, :K]                                # row stride K + 64
    rd = _dev(resid, bf16=False)
    say(f"gather-scatter-add B{B} S{S} block{block} K{K} N{N} kept={kept}")
    J.proj_gather_scatter_add(ad, _dev(w), kd, nd, 5, block, rd)
    torch.cuda.synchronize()
    out = rd.cpu().numpy()
    ref = oracle.proj_gather_scatter_add(resid, a_full[:, :, :K], w, kept, block)
    for b in range(B):
        pos = oracle.token_positions(kept[b], block)
        elim = np.setdiff1d(np.arange(S), pos)
        assert np.array_equal(out[b, elim], resid[b, elim])
        assert max_abs(out[b, pos], ref[b, pos]) <= TOL


@pytest.mark.parametrize("kind,F", [(oracle.MLP_SILU_GATED, 11008), (oracle.MLP_RELU, 16384)])
def test_mlp_full_size(J, kind, F):
    """Llama-2-7B (gated SiLU, F = 11008) and OPT-6.7B (ReLU, F = 16384) MLP blocks at
    S = 32768, d = 4096, block 128, top-k 0.5: sampled activation rows and token scores,
    two whole blocks' scores, selection bit-exact on the GPU's scores, sampled residual rows,
    and every eliminated row bitwise unchanged."""
    import torch
    B, S, block, K = 1, 32768, 128, 4096
    gen = torch.Generator(device="cuda").manual_seed(4242 + kind)
    say(f"mlp full size kind{kind} S{S} K{K} F{F}")
    xd = torch.randn((B, S, K), generator=gen, device="cuda").to(torch.bfloat16)
    w1d = (torch.randn((F, K), generator=gen, device="cuda") / K ** 0.5).to(torch.bfloat16)
    wud = ((torch.randn((F, K), generator=gen, device="cuda") / K ** 0.5).to(torch.bfloat16)
           if kind == oracle.MLP_SILU_GATED else None)
    wdd = (torch.randn((K, F), generator=gen, device="cuda") / F ** 0.5).to(torch.bfloat16)
    resid0 = torch.randn((B, S, K), generator=gen, device="cuda")
    rd = resid0.clone()
    act, tok, blk = J.mlp_act_scores(xd, w1d, wud, kind, block)
    kept, n_kept = J.select_blocks(blk, block, S, J.JENGA_SELECT_TOPK, 0.5)
    mkb = J.topk_count(0.5, S // block)
    J.proj_gather_scatter_add(act, wdd, kept, n_kept, mkb, block, rd)
    torch.cuda.synchronize()

    w1 = w1d.float().cpu().numpy()
    wu = wud.float().cpu().numpy() if wud is not None else None
    wdn = wdd.float().cpu().numpy()
    rng = np.random.default_rng(9)
    rows = np.sort(rng.choice(S, 24, replace=False))
    xs = xd[0, rows].float().cpu().numpy()
    ref = oracle.mlp_activation(xs, w1, wu, kind)
    _check_act(act[0, rows].float().cpu().numpy(), ref)
    np.testing.assert_allclose(tok[0, rows].cpu().numpy(), oracle.mlp_token_scores(ref),
                               rtol=SCORE_RTOL)
    bs = blk.cpu().numpy()
    for n in (0, S // block - 1):
        xb = xd[0, n * block:(n + 1) * block].float().cpu().numpy()
        e = oracle.mlp_token_scores(oracle.mlp_activation(xb, w1, wu, kind))
        assert abs(bs[0, n] - e.max()) <= SCORE_RTOL * e.max()
    kg = kept.cpu().numpy()[0, :int(n_kept[0])]
    assert list(kg) == list(oracle.select_blocks(bs[0], oracle.SELECT_TOPK, 0.5))

    pos = oracle.token_positions(kg, block)
    keep_mask = torch.zeros(S, dtype=torch.bool, device="cuda")
    keep_mask[torch.from_numpy(pos).cuda()] = True
    assert torch.equal(rd[0, ~keep_mask], resid0[0, ~keep_mask])
    samp = np.sort(rng.choice(pos, 16, replace=False))
    a_s = act[0, samp].float().cpu().numpy()                   # the stored activation rows
    want = resid0[0, samp].cpu().numpy().astype(np.float64) + a_s.astype(np.float64) @ wdn.T.astype(np.float64)
    assert max_abs(rd[0, samp].cpu().numpy(), want) <= TOL
