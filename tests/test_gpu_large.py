"""GPU parity of the paths that only large problems reach.

- Selection over more than 1024 blocks: the selection workgroup compacts 1024 blocks per pass,
  so 1025, 4096 and 16384 blocks take two, four and sixteen passes.
- Scoring in several query chunks: the bf16 scorer stores the partial log2-sums of one chunk
  of 128 * ceil(2048 / (B * Hq)) queries at a time, so many heads and a few thousand tokens
  already need more than one chunk (and a ragged last one).
- Attention with more than 1024 kept blocks: the kernels resolve kept ranks through an LDS copy
  of the first 1024 kept-block indices and read the rest from the global list.
- Tile dispatch with several (batch, head) rows per XCD range in groups with a shorter last
  group, for two batch rows of different kept counts.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import BF16_TOL, kept_tensor, max_abs, random_inputs, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def J():
    import torch
    assert torch.cuda.is_available()
    import token_sparse_attention_jenga_amd as J
    return J


def _large_select_cases():
    rng = np.random.default_rng(2025)
    levels = np.float32([0.0, -0.0, 0.25, 0.5, 0.5, 1.0, np.nan, -1.0])
    cases = []
    for n in (1025, 4096, 16384):
        ties = rng.choice(levels, n).astype(np.float32)
        normal = rng.standard_normal(n).astype(np.float32)
        cases += [
            (ties, oracle.SELECT_TOPK, 0.5, True),
            (ties, oracle.SELECT_TOPK, 0.123, False),
            (normal, oracle.SELECT_TOPK, 0.35, True),
            (normal, oracle.SELECT_TOPK, 1.0, False),
            (ties, oracle.SELECT_THRESH_REL, 1.0, True),
            (normal, oracle.SELECT_THRESH_REL, 0.0, False),
            (normal, oracle.SELECT_THRESH_ABS, 0.7, False),
        ]
    return cases


def test_select_past_1024_blocks(J):
    import torch
    for i, (x, mode, param, ff) in enumerate(_large_select_cases()):
        n = len(x)
        say(f"select n={n} mode={mode} param={param} force={ff}")
        scores = torch.from_numpy(x[None].copy()).cuda()
        kept, nk = J.select_blocks(scores, 64, n * 64, mode, param, ff)
        torch.cuda.synchronize()
        ref = oracle.select_blocks(x, mode, param, ff)
        got_n = int(nk.cpu()[0])
        got = kept.cpu().numpy()[0]
        assert got_n == len(ref), (i, n, got_n, len(ref))
        assert np.array_equal(got[:got_n], ref), (i, n)
        assert np.all(got[got_n:] == -1), (i, n)


CHUNK_CASES = [
    # B, S, Hq, Hkv, D, block: B*Hq = 256 -> chunks of 1024 queries: 1024 + 512
    (4, 1536, 64, 8, 64, 64),
    # B*Hq = 512 -> chunks of 512 queries: 512 + 512 + 256, block 128
    (16, 1280, 32, 32, 128, 128),
]


@pytest.mark.parametrize("B,S,Hq,Hkv,D,block", CHUNK_CASES)
def test_scores_in_several_chunks(J, B, S, Hq, Hkv, D, block):
    import torch
    chunk = 128 * -(-2048 // (B * Hq))
    assert S > chunk                                   # the case really spans several chunks
    q, k, _, _, _ = random_inputs(B, S, Hq, Hkv, D, "bf16", seed=31 * S + Hq)
    say(f"chunked scores B{B} S{S} Hq{Hq} Hkv{Hkv} D{D} block{block} chunk{chunk}")
    got = J.score_blocks(to_device(q, "bf16"), to_device(k, "bf16"), block)
    torch.cuda.synchronize()
    ref = oracle.block_scores(q, k, block)
    rel = np.max(np.abs(got.cpu().numpy().astype(np.float64) - ref) / np.abs(ref))
    assert rel <= 1e-5, rel


def test_attention_past_1024_kept_blocks(J):
    """1056 of 1088 blocks of 64 kept (67584 kept tokens): ranks past 1024 blocks go through the
    global kept list in the forward, the dQ tiles and the dK/dV tiles.  Sampled rows against
    the oracle, the eliminated rows bitwise unchanged, two backward segments."""
    import torch
    B, S, Hq, Hkv, D, block = 1, 1088 * 64, 1, 1, 64, 64
    nkb = S // block
    rng = np.random.default_rng(77)
    dropped = rng.choice(nkb, 32, replace=False)
    kept = np.setdiff1d(np.arange(nkb), dropped).astype(np.int64)
    assert len(kept) == 1056
    q, k, v, x0, dout = random_inputs(B, S, Hq, Hkv, D, "bf16", seed=1088)
    kt, nk = kept_tensor([kept], nkb)
    maxk = len(kept)
    say(f"attention past 1024 kept blocks: S{S} kept {maxk} blocks of {block}")
    qd, kd, vd = to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16")
    resid = torch.from_numpy(x0.copy()).cuda()
    o_saved, lse = J.sparse_attn_fwd(qd, kd, vd, kt, nk, maxk, block, resid)
    dq, dk, dv = J.sparse_attn_bwd(qd, kd, vd, kt, nk, maxk, block, o_saved, lse,
                                   torch.from_numpy(dout).cuda(), n_segments=2)
    torch.cuda.synchronize()
    Nk = maxk * block
    pos = oracle.token_positions(kept, block)
    # ranks on both sides of the 1024-block table boundary, the last rank, and a spread
    ranks = np.unique(np.concatenate([np.arange(0, 32), np.arange(65536 - 48, 65536 + 80),
                                      np.arange(Nk - 32, Nk), rng.choice(Nk, 16, replace=False)]))
    O, LSE = oracle.attn_fwd_rows(q, k, v, kept, block, 0, 0, ranks)
    r = resid.cpu().numpy()
    assert max_abs(r[0, pos[ranks], 0] - x0[0, pos[ranks], 0], O) <= BF16_TOL
    assert max_abs(o_saved.float().cpu().numpy()[0, ranks, 0], O) <= BF16_TOL
    assert np.all(np.abs(lse.cpu().numpy()[0, 0, ranks] - LSE) <= 1e-4 * np.maximum(1.0, np.abs(LSE)))
    elim = np.setdiff1d(np.arange(S), pos)
    assert np.array_equal(r[0, elim], x0[0, elim])
    # backward: keys on both sides of the table boundary and at the end (each needs every later
    # query row, so they are taken late), queries anywhere (each needs only its own rows)
    kr = np.unique(np.concatenate([np.arange(65536 - 48, 65536 + 80), np.arange(Nk - 32, Nk)]))
    qr = np.unique(np.concatenate([np.arange(0, 32), np.arange(65536 - 48, 65536 + 80),
                                   np.arange(Nk - 32, Nk), rng.choice(Nk, 6, replace=False)]))
    rdk, rdv, rdq = oracle.attn_bwd_sampled(q, k, v, kept, block, dout, 0, 0, kr, qr)
    assert max_abs(dk.cpu().numpy()[0, pos[kr], 0], rdk) <= BF16_TOL
    assert max_abs(dv.cpu().numpy()[0, pos[kr], 0], rdv) <= BF16_TOL
    assert max_abs(dq.cpu().numpy()[0, pos[qr], 0], rdq[0]) <= BF16_TOL
    for g in (dq, dk, dv):
        assert np.all(g.cpu().numpy()[0, elim] == 0.0)


def test_weight_major_dispatch_two_batch_rows(J):
    """Two batch rows, 8 query heads, 80 kept blocks of 64 in one row and 72 in the other: the
    forward's XCD ranges then hold two (batch, head) rows each, visited in groups of 32 tiles with
    a shorter last group (40 tiles of 128 queries per row); the backward's light launches send
    their dK/dV tiles out weight-major.  Sampled rows of both batch rows against the oracle,
    eliminated rows bitwise unchanged."""
    import torch
    B, S, Hq, Hkv, D, block = 2, 8192, 8, 2, 128, 64
    nkb = S // block
    rng = np.random.default_rng(4040)
    kept = [np.sort(rng.choice(nkb, 80, replace=False)).astype(np.int64),
            np.sort(rng.choice(nkb, 72, replace=False)).astype(np.int64)]
    q, k, v, x0, dout = random_inputs(B, S, Hq, Hkv, D, "bf16", seed=4041)
    kt, nk = kept_tensor(kept, nkb)
    maxk = 80
    say(f"weight-major dispatch: B{B} S{S} Hq{Hq} Hkv{Hkv} kept 80/72 blocks of {block}, 3 segments")
    qd, kd, vd = to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16")
    resid = torch.from_numpy(x0.copy()).cuda()
    o_saved, lse = J.sparse_attn_fwd(qd, kd, vd, kt, nk, maxk, block, resid)
    dq, dk, dv = J.sparse_attn_bwd(qd, kd, vd, kt, nk, maxk, block, o_saved, lse,
                                   torch.from_numpy(dout).cuda(), n_segments=3)
    torch.cuda.synchronize()
    r = resid.cpu().numpy()
    for b in range(B):
        Nk = len(kept[b]) * block
        pos = oracle.token_positions(kept[b], block)
        ranks = np.unique(np.concatenate([np.arange(0, 8), rng.choice(Nk, 24, replace=False),
                                          np.arange(Nk - 8, Nk)]))
        for h in (0, 5):
            O, LSE = oracle.attn_fwd_rows(q, k, v, kept[b], block, b, h, ranks)
            assert max_abs(r[b, pos[ranks], h] - x0[b, pos[ranks], h], O) <= BF16_TOL, (b, h)
            assert max_abs(o_saved.float().cpu().numpy()[b, ranks, h], O) <= BF16_TOL, (b, h)
        elim = np.setdiff1d(np.arange(S), pos)
        assert np.array_equal(r[b, elim], x0[b, elim])
        # keys late in the kept order (a key needs every later query row), queries anywhere
        kr = np.unique(np.concatenate([np.arange(Nk - 6, Nk), Nk // 2 + rng.choice(Nk // 2, 4, replace=False)]))
        qr = np.unique(np.concatenate([rng.choice(Nk, 6, replace=False), np.arange(Nk - 4, Nk)]))
        for g in (0, 1):
            rdk, rdv, rdq = oracle.attn_bwd_sampled(q, k, v, kept[b], block, dout, b, g, kr, qr)
            assert max_abs(dk.cpu().numpy()[b, pos[kr], g], rdk) <= BF16_TOL, (b, g)
            assert max_abs(dv.cpu().numpy()[b, pos[kr], g], rdv) <= BF16_TOL, (b, g)
            G = Hq // Hkv
            for i, hh in enumerate(range(g * G, (g + 1) * G)):
                assert max_abs(dq.cpu().numpy()[b, pos[qr], hh], rdq[i]) <= BF16_TOL, (b, g, hh)
