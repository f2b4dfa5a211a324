"""Edge cases of the attention path against the oracle ([notes] 4.4 permutation-free token
movement, the segmented backward): a kept count above max_kept_blocks (only the first
max_kept_blocks blocks take part), large blocks, a batch row with nothing kept beside one with
blocks kept, segments past the kept count (empty), head counts whose tiles do not fill the
launch evenly, and bit-for-bit repeatable bf16 gradients."""
import numpy as np
import pytest

import oracle
from gpu_helpers import kept_tensor, max_abs, random_inputs, say, to_device, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def J():
    import token_sparse_attention_jenga_amd as J
    return J


def _run(J, q, k, v, x0, dout, kept_list, block, dtype, nseg, maxk):
    import torch
    S = q.shape[1]
    qd, kd, vd = to_device(q, dtype), to_device(k, dtype), to_device(v, dtype)
    kept_d, nk_d = kept_tensor(kept_list, S // block)
    resid = torch.from_numpy(x0.copy()).cuda()
    o_saved, lse = J.sparse_attn_fwd(qd, kd, vd, kept_d, nk_d, maxk, block, resid)
    dq, dk, dv = J.sparse_attn_bwd(qd, kd, vd, kept_d, nk_d, maxk, block, o_saved, lse,
                                   torch.from_numpy(dout).cuda(), nseg)
    torch.cuda.synchronize()
    return resid.cpu().numpy(), dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()


def _check(q, k, v, x0, dout, used, block, got, tol):
    """used: the kept blocks that take part, per batch row."""
    resid, dq, dk, dv = got
    S = q.shape[1]
    used_np = [np.array(u, dtype=np.int64) for u in used]
    O, _ = oracle.attn_fwd(q, k, v, used_np, block)
    rq, rk, rv = oracle.attn_bwd(q, k, v, used_np, block, dout)
    for b in range(q.shape[0]):
        pos = oracle.token_positions(used_np[b], block)
        elim = np.setdiff1d(np.arange(S), pos)
        assert np.array_equal(resid[b, elim], x0[b, elim])
        if len(pos):
            assert max_abs(resid[b, pos] - x0[b, pos], O[b, pos]) <= tol
        for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
            if len(pos):
                assert max_abs(g[b, pos], r[b, pos]) <= tol, name
            assert np.all(g[b, elim] == 0), name


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_kept_count_capped_by_max_kept_blocks(J, dtype):
    D = 128 if dtype == "bf16" else 64
    B, S, Hq, Hkv, block = 1, 1024, 4, 4, 64
    q, k, v, x0, dout = random_inputs(B, S, Hq, Hkv, D, dtype, seed=21)
    kept = [[0, 2, 3, 6, 9, 11, 14]]
    say(f"cap: n_kept 7, max_kept_blocks 4, {dtype}")
    got = _run(J, q, k, v, x0, dout, kept, block, dtype, 2, maxk=4)
    _check(q, k, v, x0, dout, [kept[0][:4]], block, got, tol_for(dtype))


@pytest.mark.parametrize("block", [256, 512])
def test_large_blocks(J, block):
    B, S, Hq, Hkv, D, dtype = 1, 2048, 2, 2, 128, "bf16"
    q, k, v, x0, dout = random_inputs(B, S, Hq, Hkv, D, dtype, seed=block)
    kept = [[0, 2, 3]] if block == 256 else [[1, 3]]
    say(f"large blocks: block {block} kept {kept}")
    got = _run(J, q, k, v, x0, dout, kept, block, dtype, 2, maxk=len(kept[0]))
    _check(q, k, v, x0, dout, kept, block, got, tol_for(dtype))


def test_batch_row_with_nothing_kept(J):
    B, S, Hq, Hkv, D, block, dtype = 3, 512, 2, 2, 128, 64, "bf16"
    q, k, v, x0, dout = random_inputs(B, S, Hq, Hkv, D, dtype, seed=23)
    kept = [[1, 4, 5], [], [0, 7]]
    say(f"batch rows {kept}")
    got = _run(J, q, k, v, x0, dout, kept, block, dtype, 2, maxk=3)
    _check(q, k, v, x0, dout, kept, block, got, tol_for(dtype))


def test_empty_segments(J):
    """Capacity for 8 kept blocks of 64 rows, 8 segments, but only 2 blocks kept: the segments
    past the kept count are empty.  One segment more than the capacity allows (64 rows each)
    is rejected as an invalid argument, as the header states."""
    import torch
    B, S, Hq, Hkv, D, block, dtype = 1, 512, 2, 2, 128, 64, "bf16"
    q, k, v, x0, dout = random_inputs(B, S, Hq, Hkv, D, dtype, seed=24)
    kept = [[2, 6]]
    say("8 segments, capacity 8 blocks, 2 kept")
    got = _run(J, q, k, v, x0, dout, kept, block, dtype, 8, maxk=8)
    _check(q, k, v, x0, dout, kept, block, got, tol_for(dtype))
    with pytest.raises(J.JengaError) as e:
        _run(J, q, k, v, x0, dout, kept, block, dtype, 9, maxk=8)
    assert e.value.status == J.JENGA_ERR_INVALID_ARG


def test_bf16_backward_repeatable(J):
    B, S, Hq, Hkv, D, block, dtype = 1, 2048, 4, 2, 128, 128, "bf16"
    q, k, v, x0, dout = random_inputs(B, S, Hq, Hkv, D, dtype, seed=25)
    kept = [[0, 1, 3, 4, 6, 9, 12, 15]]
    say("bf16 backward bitwise repeatable")
    a = _run(J, q, k, v, x0, dout, kept, block, dtype, 3, maxk=8)
    b = _run(J, q, k, v, x0, dout, kept, block, dtype, 3, maxk=8)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_odd_head_counts(J):
    """Grouped heads whose tile counts are not multiples of 8: the backward launch pads each
    of its two workgroup runs with idle workgroups, and every dQ and dK/dV tile must still be
    computed exactly once."""
    B, S, Hq, Hkv, D, block, dtype = 2, 768, 6, 3, 128, 64, "bf16"
    q, k, v, x0, dout = random_inputs(B, S, Hq, Hkv, D, dtype, seed=26)
    kept = [[0, 1, 4, 5, 7, 9, 10], [2, 3, 6, 11]]
    say(f"odd heads: Hq {Hq} Hkv {Hkv}, kept {kept}, 3 segments")
    got = _run(J, q, k, v, x0, dout, kept, block, dtype, 3, maxk=7)
    _check(q, k, v, x0, dout, kept, block, got, tol_for(dtype))
