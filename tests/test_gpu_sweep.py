"""A seeded sweep of small bf16 problems through score-free fwd + segmented bwd, against the oracle.

Each case draws its shape (batch rows, sequence length, query heads, query heads per KV head,
head_dim, block), a kept set per batch row (different counts, so rows end in different
segments and key tiles) and a segment count from one seeded generator.  Both backward
workspaces run: two sets of segment buffers (each launch also runs the next segment's prologue)
and one set; they must agree bit for bit, and with the oracle within the bf16 tolerance.  The
kept rows of the residual take the output, every other row stays bitwise untouched, and the
gradients are zero outside the kept rows.

Tolerance: the bf16 bound of 2e-2 max-abs, for values up to magnitude 1, and scaled by the
largest reference magnitude above that.  The bf16 rounding of the MFMA operands (P, dS, dO, Q)
is relative (2^-9 each), and with several query heads per KV head dK and dV add up that many
heads' terms: for a key that every later query attends to, four heads' dO rows of N(0, 1)
values give |dV| near 4 and rounding errors a little above 2e-2.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import kept_tensor, max_abs, random_inputs, say, to_device, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def J():
    import torch
    assert torch.cuda.is_available()
    import token_sparse_attention_jenga_amd as J
    return J


def _case(seed):
    rng = np.random.default_rng(seed)
    block = int(rng.choice([64, 128]))
    D = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4]))
    Hkv = int(rng.integers(1, 3))
    Hq = G * Hkv
    B = int(rng.integers(1, 3))
    nkb = int(rng.integers(4, 2048 // block + 1))           # up to 2048 tokens
    S = nkb * block
    counts = [int(rng.integers(1, nkb + 1)) for _ in range(B)]
    kept = [np.sort(rng.choice(nkb, c, replace=False)) for c in counts]
    maxk = max(counts)
    nseg = int(rng.integers(1, min(4, maxk * block // 64) + 1))
    return B, S, Hq, Hkv, D, block, kept, maxk, nseg


@pytest.mark.parametrize("seed", range(100, 124))
def test_fwd_bwd_sweep(J, seed):
    import torch
    B, S, Hq, Hkv, D, block, kept, maxk, nseg = _case(seed)
    nkb = S // block
    q, k, v, x0, dout = random_inputs(B, S, Hq, Hkv, D, "bf16", seed=seed)
    qd, kd, vd = to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16")
    kept_d, nk_d = kept_tensor(kept, nkb)
    say(f"sweep seed {seed}: B{B} S{S} Hq{Hq} Hkv{Hkv} D{D} block{block} "
        f"kept {[len(x) for x in kept]} of {nkb}, max {maxk}, N={nseg}")
    resid = torch.from_numpy(x0.copy()).cuda()
    o_saved, lse = J.sparse_attn_fwd(qd, kd, vd, kept_d, nk_d, maxk, block, resid)
    dd = torch.from_numpy(dout).cuda()
    got = [J.sparse_attn_bwd(qd, kd, vd, kept_d, nk_d, maxk, block, o_saved, lse, dd, n_segments=nseg,
                             min_workspace=lean) for lean in (False, True)]
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got[0], got[1]):
        assert torch.equal(a, b), name
    O, _ = oracle.attn_fwd(q, k, v, kept, block)
    rq, rk, rv = oracle.attn_bwd(q, k, v, kept, block, dout)
    res = resid.cpu().numpy()
    osv = o_saved.float().cpu().numpy()
    g = [x.cpu().numpy() for x in got[0]]
    tol = lambda ref: tol_for("bf16") * max(1.0, float(np.max(np.abs(ref))))
    for b in range(B):
        pos = oracle.token_positions(kept[b], block)
        elim = np.setdiff1d(np.arange(S), pos)
        assert np.array_equal(res[b, elim], x0[b, elim])
        assert max_abs(res[b, pos] - x0[b, pos], O[b, pos]) <= tol(O[b, pos])
        assert max_abs(osv[b, :len(pos)], O[b, pos]) <= tol(O[b, pos])
        for name, x, ref in (("dq", g[0], rq), ("dk", g[1], rk), ("dv", g[2], rv)):
            err = max_abs(x[b, pos], ref[b, pos])
            assert err <= tol(ref[b, pos]), (b, name, err)
            assert not x[b, elim].any(), (b, name)
