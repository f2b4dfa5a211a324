"""GPU parity of the permutation-free projections ([notes] 4.4; [summary] 4.4.1) against the
oracle: the gathered input projection y = x[pos] W^T (compact bf16) and the in-place
scatter-add resid[pos] += y W^T (fp32).  Eliminated rows of the residual must stay bitwise
unchanged and compact rows past a batch row's kept count must not be written."""
import numpy as np
import pytest

import oracle
from gpu_helpers import kept_tensor, max_abs, say

pytestmark = pytest.mark.gpu
TOL = 2e-2


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


CASES = [
    # B, S, block, K, N, kept per batch row, max_kept_blocks
    (2, 512, 64, 256, 256, [[0, 2, 3, 7], [1, 5]], 4),
    (1, 1024, 256, 64, 128, [[0, 3]], 2),
    (1, 2048, 128, 512, 384, [[1, 2, 3, 4, 6, 9, 10, 15]], 8),
    (2, 640, 64, 128, 128, [[9], [0, 1, 2, 3, 4, 5, 6]], 7),
]


@pytest.mark.parametrize("B,S,block,K,N,kept,maxk", CASES)
def test_proj_gather_and_scatter(J, B, S, block, K, N, kept, maxk):
    import torch
    rng = np.random.default_rng(S + K + N)
    x = _bf16(rng, (B, S, K))
    w = _bf16(rng, (N, K), 1.0 / np.sqrt(K))
    kd, nd = kept_tensor(kept, S // block)
    say(f"proj gather B{B} S{S} block{block} K{K} N{N} kept={kept}")
    y = torch.full((B, maxk * block, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    p = J.make_proj_problem(_dev(x), _dev(w), y, block, S)
    xd, wd = _dev(x), _dev(w)
    assert J.lib.jenga_proj_gather(J.ctypes.byref(p), xd.data_ptr(), wd.data_ptr(), kd.data_ptr(),
                                   nd.data_ptr(), maxk, y.data_ptr(), None) == 0
    torch.cuda.synchronize()
    ref = oracle.proj_gather(x, w, kept, block)
    got = y.float().cpu().numpy()
    for b in range(B):
        nk = len(kept[b]) * block
        assert max_abs(got[b, :nk], ref[b, :nk]) <= TOL
        assert np.isnan(got[b, nk:]).all()                      # rows past the kept count untouched

    say(f"proj scatter-add B{B} S{S} block{block} K{K} N{N}")
    yin = _bf16(rng, (B, maxk * block, K))
    wo = _bf16(rng, (N, K), 1.0 / np.sqrt(K))
    resid = rng.standard_normal((B, S, N), dtype=np.float32)
    rd = _dev(resid, bf16=False)
    J.proj_scatter_add(_dev(yin), _dev(wo), kd, nd, maxk, block, rd)
    torch.cuda.synchronize()
    out = rd.cpu().numpy()
    ref = oracle.proj_scatter_add(resid, yin, wo, kept, block)
    for b in range(B):
        pos = oracle.token_positions(kept[b], block)
        elim = np.setdiff1d(np.arange(S), pos)
        assert np.array_equal(out[b, elim], resid[b, elim])    # bitwise untouched
        assert max_abs(out[b, pos], ref[b, pos]) <= TOL


def test_proj_full_size_llama_layer(J):
    """The Llama-2-7B projections at S = 32K with half the 128-token blocks kept (a scattered
    set): QKV (4096 -> 12288) gathered, O (4096 -> 4096) scattered into the residual; sampled
    rows against the oracle, every eliminated residual row bitwise unchanged."""
    import torch
    from synth.generate import random_kept_blocks
    B, S, block, d = 1, 32768, 128, 4096
    nkb = S // block
    kb = random_kept_blocks(nkb, nkb // 2, 6007)
    kd, nd = kept_tensor([kb], nkb)
    rng = np.random.default_rng(77)
    x = _bf16(rng, (B, S, d))
    wqkv = _bf16(rng, (3 * d, d), 1.0 / np.sqrt(d))
    say("proj full size: QKV gather 4096 -> 12288, S=32768, 128 of 256 blocks")
    y = J.proj_gather(_dev(x), _dev(wqkv), kd, nd, nkb // 2, block)
    torch.cuda.synchronize()
    ranks = np.sort(rng.choice(len(kb) * block, 48, replace=False))
    pos = oracle.token_positions(kb, block)
    ref = x[0, pos[ranks]].astype(np.float64) @ wqkv.astype(np.float64).T
    assert max_abs(y[0, ranks].float().cpu().numpy(), ref) <= TOL

    say("proj full size: O scatter-add 4096 -> 4096 into the fp32 residual")
    wo = _bf16(rng, (d, d), 1.0 / np.sqrt(d))
    yo = _bf16(rng, (B, len(kb) * block, d))
    resid0 = torch.from_numpy(rng.standard_normal((B, S, d), dtype=np.float32)).cuda()
    rd = resid0.clone()
    J.proj_scatter_add(_dev(yo), _dev(wo), kd, nd, nkb // 2, block, rd)
    torch.cuda.synchronize()
    elim = torch.from_numpy(np.setdiff1d(np.arange(S), pos)).cuda()
    assert torch.equal(rd[0, elim], resid0[0, elim])
    got = rd[0, torch.from_numpy(pos[ranks]).cuda()].cpu().numpy().astype(np.float64)
    want = resid0[0, torch.from_numpy(pos[ranks]).cuda()].cpu().numpy().astype(np.float64) + \
        yo[0, ranks].astype(np.float64) @ wo.astype(np.float64).T
    assert max_abs(got, want) <= TOL
