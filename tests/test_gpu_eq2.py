"""GPU parity of the Eq. 2 literal block scores ([summary] 4.2.2 Eq. 2, 4.2.3) against the
oracle: full comparisons at small shapes, sampled key blocks at the workloads' full shapes.
Scores must match within 1e-5 relative; the selection on them is checked bit-exact."""
import numpy as np
import pytest

import oracle
from gpu_helpers import random_inputs, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def J():
    import token_sparse_attention_jenga_amd as J
    return J


def _rel(got, ref):
    got = np.asarray(got, dtype=np.float64)
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-30)))


# (odd head counts and a single head: the kernel takes heads in pairs, and an odd count's last
# head finishes after the loop)
@pytest.mark.parametrize("B,S,Hq,Hkv,D,block", [(1, 512, 4, 2, 128, 64), (2, 768, 2, 2, 64, 128),
                                                (1, 1024, 8, 8, 128, 128), (1, 640, 4, 1, 64, 64),
                                                (1, 384, 3, 1, 128, 128), (1, 512, 5, 5, 64, 128),
                                                (1, 320, 1, 1, 64, 64), (1, 256, 1, 1, 128, 128)])
def test_eq2_scores_full(J, B, S, Hq, Hkv, D, block):
    import torch
    q, k, _, _, _ = random_inputs(B, S, Hq, Hkv, D, "bf16", seed=S + 7 * Hq)
    say(f"eq2 scores B{B} S{S} Hq{Hq} Hkv{Hkv} D{D} block{block}")
    got = J.score_blocks_eq2(to_device(q, "bf16"), to_device(k, "bf16"), block)
    torch.cuda.synchronize()
    ref = oracle.block_scores_eq2(q, k, block)
    assert _rel(got.cpu().numpy(), ref) <= 1e-5


def test_eq2_scores_deterministic_and_selection(J):
    import torch
    B, S, Hq, Hkv, D, block = 1, 2048, 4, 4, 128, 64
    q, k, _, _, _ = random_inputs(B, S, Hq, Hkv, D, "bf16", seed=31)
    qd, kd = to_device(q, "bf16"), to_device(k, "bf16")
    say("eq2 determinism + top-k on eq2 scores")
    a = J.score_blocks_eq2(qd, kd, block)
    b = J.score_blocks_eq2(qd, kd, block)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    kept, n = J.select_blocks(a, block, S, J.JENGA_SELECT_TOPK, 0.4)
    torch.cuda.synchronize()
    want = oracle.select_blocks(a.cpu().numpy()[0], oracle.SELECT_TOPK, 0.4)
    assert int(n[0]) == len(want)
    assert np.array_equal(kept.cpu().numpy()[0, :len(want)], want)


@pytest.mark.parametrize("name,key_blocks", [("c2", [0, 17, 62, 63]), ("c4", [1, 200, 254, 255]),
                                             ("c5", [120, 230, 254, 255])])
def test_eq2_full_size_sampled(J, name, key_blocks):
    """Whole-sequence Eq. 2 scores at the workloads' shapes; the oracle evaluates the listed key
    blocks exactly (every query block m >= n of each)."""
    import torch
    from synth import config_by_name
    from synth.generate import make_layer
    cfg = config_by_name(name)
    li = make_layer(cfg, 0)
    say(f"eq2 full size {name} S{cfg.seq_len} block{cfg.block}")
    got = J.score_blocks_eq2(to_device(li.q, "bf16"), to_device(li.k, "bf16"), cfg.block)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    ref = oracle.block_scores_eq2(li.q, li.k, cfg.block, key_blocks=key_blocks)
    assert _rel(got[0, key_blocks], ref[0, key_blocks]) <= 1e-5
    assert np.all(np.isfinite(got)) and np.all(got >= 0)
