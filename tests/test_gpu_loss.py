"""GPU parity of the segmented language-model-head loss ([summary] 4.4.2, [notes] 4.4
segment-based peak cutting) against the oracle, and independence from the segment count."""
import numpy as np
import pytest

import oracle
from gpu_helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def J():
    import token_sparse_attention_jenga_amd as J
    return J


def _inputs(T, d, V, seed):
    import torch
    from synth.generate import to_bf16_bits_f32
    rng = np.random.default_rng(seed)
    h = to_bf16_bits_f32(rng.standard_normal((T, d), dtype=np.float32))
    w = to_bf16_bits_f32((rng.standard_normal((V, d), dtype=np.float32) / np.sqrt(d)).astype(np.float32))
    t = rng.integers(0, V, T).astype(np.int32)
    hd = torch.from_numpy(h).to(torch.bfloat16).cuda()
    wd = torch.from_numpy(w).to(torch.bfloat16).cuda()
    return h, w, t, hd, wd, wd.t().contiguous(), torch.from_numpy(t).cuda()


def _dh_bound(g, w):
    """Element-wise bound on |dh_gpu - dh| from the GPU's arithmetic: dh = G W with G the logit
    gradient rounded once to bf16 (relative 2^-9 per element) and fp32 accumulation; the fp32
    logits shift G by a relative 1e-4 or less.  So |error_tc| <= c * sum_v |G_tv| |W_vc| with
    c = 2^-9 (rounding) doubled for the logits and the accumulation order: 2^-8."""
    return 2.0 ** -8 * (np.abs(g) @ np.abs(np.asarray(w, dtype=np.float64))) + 1e-12


@pytest.mark.parametrize("T,d,V,nseg", [(256, 256, 1024, 1), (256, 256, 1024, 3), (512, 128, 2048, 4),
                                        (96, 384, 640, 2)])
def test_loss_matches_oracle(J, T, d, V, nseg):
    import torch
    h, w, t, hd, wd, wtd, td = _inputs(T, d, V, T + d + V)
    say(f"loss T{T} d{d} V{V} segments {nseg}")
    loss, rows, dh = J.lm_head_ce(hd, wd, wtd, td, nseg)
    torch.cuda.synchronize()
    rl, rr, rdh, rg = oracle.lm_head_ce(h, w, t, with_logit_grad=True)
    assert abs(loss.item() - rl) <= 1e-5 * abs(rl)
    assert np.max(np.abs(rows.cpu().numpy() - rr)) <= 1e-4
    err = np.abs(dh.cpu().numpy() - rdh)
    assert np.all(err <= _dh_bound(rg, w)), float(np.max(err / _dh_bound(rg, w)))


def test_loss_independent_of_segments(J):
    import torch
    T, d, V = 1024, 256, 4096
    _, _, _, hd, wd, wtd, td = _inputs(T, d, V, 5)
    say("loss segments 1 vs 8")
    a = J.lm_head_ce(hd, wd, wtd, td, 1)
    b = J.lm_head_ce(hd, wd, wtd, td, 8)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_loss_full_size_llama_head(J):
    """The Llama-2-7B head (d 4096, vocabulary 32000) over 32768 tokens in 8 segments; sampled
    rows against the oracle, the mean against the row losses."""
    import torch
    T, d, V = 32768, 4096, 32000
    h, w, t, hd, wd, wtd, td = _inputs(T, d, V, 11)
    say("loss full size T32768 d4096 V32000, 8 segments")
    loss, rows, dh = J.lm_head_ce(hd, wd, wtd, td, 8)
    torch.cuda.synchronize()
    idx = np.array([0, 1, 4095, 4096, 17000, 32767])
    _, rr, rdh, rg = oracle.lm_head_ce(h[idx], w, t[idx], with_logit_grad=True)
    assert np.max(np.abs(rows.cpu().numpy()[idx] - rr)) <= 1e-4
    rdh = rdh * len(idx) / T                      # the oracle's mean ran over len(idx) rows
    rg = rg * len(idx) / T
    err = np.abs(dh.cpu().numpy()[idx] - rdh)
    assert np.all(err <= _dh_bound(rg, w)), float(np.max(err / _dh_bound(rg, w)))
    assert abs(loss.item() - rows.double().mean().item()) <= 1e-6 * abs(loss.item())
