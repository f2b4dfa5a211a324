"""The backward entry point that allocates nothing, against the entry point with a workspace.

jenga_sparse_attn_bwd_segmented_noalloc runs the segmented backward's kernels with the
library's fixed per-GPU scratch array instead of a caller workspace.  Called through the C ABI
twice in a row -- the second time on a smaller problem, so the scratch holds the first call's
leftovers -- its gradients must match those of jenga_sparse_attn_bwd_segmented on the same
inputs within the parity tolerance (bf16 2e-2, fp32 1e-4 max-abs), and rows outside the kept
set must stay zero.
"""
import ctypes

import numpy as np
import pytest

from gpu_helpers import kept_tensor, max_abs, random_inputs, say, to_device, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def J():
    import torch
    assert torch.cuda.is_available()
    import token_sparse_attention_jenga_amd as J
    return J


# B, S, Hq, Hkv, D, block, dtype, kept blocks, segments -- each pair: larger, then smaller
CASES = [
    [(1, 4096, 8, 2, 128, 64, "bf16", 37, 3), (1, 1024, 4, 4, 128, 128, "bf16", 5, 2)],
    [(2, 2048, 4, 4, 64, 64, "f32", 21, 2), (1, 512, 2, 2, 64, 64, "f32", 6, 1)],
]


def _run_pair(J, pair, seed):
    import torch
    for i, (B, S, Hq, Hkv, D, block, dtype, nk, nseg) in enumerate(pair):
        nkb = S // block
        rng = np.random.default_rng(seed + i)
        kept = [np.sort(rng.choice(nkb, nk, replace=False)) for _ in range(B)]
        q, k, v, x0, dout = random_inputs(B, S, Hq, Hkv, D, dtype, seed=seed + 10 * i)
        qd, kd, vd = to_device(q, dtype), to_device(k, dtype), to_device(v, dtype)
        kt, nkt = kept_tensor(kept, nkb)
        resid = torch.from_numpy(x0.copy()).cuda()
        say(f"no-alloc backward call {i}: B{B} S{S} Hq{Hq} Hkv{Hkv} D{D} block{block} {dtype} "
            f"kept {nk} segments {nseg}")
        o_saved, lse = J.sparse_attn_fwd(qd, kd, vd, kt, nkt, nk, block, resid)
        dd = torch.from_numpy(dout).cuda()
        p = J.make_problem(qd, kd, vd, block)
        ref = J.sparse_attn_bwd(qd, kd, vd, kt, nkt, nk, block, o_saved, lse, dd, n_segments=nseg)
        got = (torch.zeros_like(ref[0]), torch.zeros_like(ref[1]), torch.zeros_like(ref[2]))
        need = J.workspace_bytes(p, J.JENGA_OP_BWD, nk, nseg)
        assert 0 < need <= J.NOALLOC_SCRATCH_BYTES
        torch.cuda.synchronize()
        st = J.lib.jenga_sparse_attn_bwd_segmented_noalloc(
            ctypes.byref(p), qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), kt.data_ptr(), nkt.data_ptr(),
            nk, o_saved.data_ptr(), lse.data_ptr(), dd.data_ptr(), got[0].data_ptr(), got[1].data_ptr(),
            got[2].data_ptr(), nseg, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == J.JENGA_OK, J.status_string(st)
        torch.cuda.synchronize()
        tol = tol_for(dtype)
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            err = max_abs(a.cpu().numpy(), b.cpu().numpy())
            assert err <= tol, (i, name, err)
        pos = [np.concatenate([np.arange(kb * block, (kb + 1) * block) for kb in kb_list]) for kb_list in kept]
        for b in range(B):
            elim = np.setdiff1d(np.arange(S), pos[b])
            for g in got:
                assert np.all(g.cpu().numpy()[b, elim] == 0.0)


@pytest.mark.parametrize("pair", range(len(CASES)))
def test_noalloc_backward_matches_workspace_backward(J, pair):
    _run_pair(J, CASES[pair], seed=900 + 17 * pair)
