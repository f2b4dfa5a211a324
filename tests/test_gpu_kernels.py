"""GPU parity of each entry point against the oracle at sizes the oracle finishes in seconds.

Shapes span several tiles and a ragged tail (odd kept-block counts against 128-row tiles),
both operand dtypes, head_dim 64 and 128, block 64 and 128, grouped-query attention,
scattered and empty kept sets, and 1 vs several backward segments.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import (kept_tensor, max_abs, random_inputs, say, to_device, tol_for)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def J():
    import torch
    assert torch.cuda.is_available()
    import token_sparse_attention_jenga_amd as J
    return J


# ----------------------------------------------------------------------------------------
# selection: bit-exact
# ----------------------------------------------------------------------------------------

def _select_cases():
    rng = np.random.default_rng(123)
    levels = np.float32([0.0, -0.0, 0.5, 1.0, 1.0, 2.0, np.nan, -3.0])
    cases = []
    for t in range(40):
        n = int(rng.integers(1, 700))
        if t % 3 == 0:
            x = rng.choice(levels, n).astype(np.float32)
        else:
            x = rng.standard_normal(n).astype(np.float32)
        mode = t % 3
        param = [float(rng.uniform(0.05, 1.0)), float(rng.uniform(0.2, 2.0)),
                 float(rng.standard_normal())][mode]
        cases.append((x, mode, param, bool(t % 2)))
    return cases


def test_select_bit_exact(J):
    import torch
    for i, (x, mode, param, ff) in enumerate(_select_cases()):
        say(f"select case {i} n={len(x)} mode={mode} param={param:.4f} force={ff}")
        n = len(x)
        S = n * 64
        scores = torch.from_numpy(x[None].copy()).cuda()
        kept, nk = J.select_blocks(scores, 64, S, mode, param, ff)
        torch.cuda.synchronize()
        ref = oracle.select_blocks(x, mode, param, ff)
        got_n = int(nk.cpu()[0])
        got = kept.cpu().numpy()[0]
        assert got_n == len(ref), (i, got_n, len(ref))
        assert np.array_equal(got[:got_n], ref), i
        assert np.all(got[got_n:] == -1)


def test_select_batched(J):
    import torch
    rng = np.random.default_rng(5)
    x = rng.choice(np.float32([0.1, 0.2, 0.3]), (3, 256)).astype(np.float32)
    say("select batched B=3 nkb=256")
    kept, nk = J.select_blocks(torch.from_numpy(x).cuda(), 128, 256 * 128, J.JENGA_SELECT_TOPK, 0.35,
                               True)
    torch.cuda.synchronize()
    for b in range(3):
        ref = oracle.select_blocks(x[b], oracle.SELECT_TOPK, 0.35, True)
        assert int(nk[b]) == len(ref) == 90
        assert np.array_equal(kept.cpu().numpy()[b, :90], ref)


# ----------------------------------------------------------------------------------------
# scores: relative 1e-5
# ----------------------------------------------------------------------------------------

SCORE_CASES = [
    # B, S, Hq, Hkv, D, block, dtype, input std (None: 1 for f32, 1/sqrt(D) for bf16)
    (1, 1024, 8, 8, 64, 64, "f32", None),
    (1, 512, 4, 4, 128, 64, "bf16", None),
    (2, 384, 4, 2, 128, 128, "bf16", None),
    (1, 448, 2, 1, 64, 64, "bf16", None),
    # a block of three 32-key steps, and the largest block (32 steps)
    (1, 576, 2, 2, 128, 192, "bf16", None),
    (1, 2048, 2, 1, 128, 1024, "bf16", None),
    # logits of standard deviation about 8 in log2 units: the running maximum of a query row
    # moves inside key blocks, so the block partial sums are rescaled on the way
    (1, 1024, 2, 2, 128, 64, "bf16", 2.0),
]


@pytest.mark.parametrize("B,S,Hq,Hkv,D,block,dtype,std", SCORE_CASES)
def test_scores(J, B, S, Hq, Hkv, D, block, dtype, std):
    import torch
    q, k, _, _, _ = random_inputs(B, S, Hq, Hkv, D, dtype, seed=S + Hq, std=std)
    say(f"scores B{B} S{S} Hq{Hq} Hkv{Hkv} D{D} block{block} {dtype} std{std}")
    got = J.score_blocks(to_device(q, dtype), to_device(k, dtype), block)
    torch.cuda.synchronize()
    ref = oracle.block_scores(q, k, block)
    got = got.cpu().numpy().astype(np.float64)
    rel = np.max(np.abs(got - ref) / np.abs(ref))
    assert rel <= 1e-5, rel


def test_scores_head_subset_view(J):
    """Strided head-subset views (the full-size score check uses them) match contiguous."""
    import torch
    B, S, Hq, Hkv, D, block = 1, 512, 8, 2, 128, 64
    q, k, _, _, _ = random_inputs(B, S, Hq, Hkv, D, "bf16", seed=77)
    qd, kd = to_device(q, "bf16"), to_device(k, "bf16")
    say("scores head-subset view")
    got = J.score_blocks(qd[:, :, 4:8], kd[:, :, 1:2], block)
    torch.cuda.synchronize()
    ref = oracle.block_scores(q[:, :, 4:8], k[:, :, 1:2], block)
    assert np.max(np.abs(got.cpu().numpy() - ref) / ref) <= 1e-5


# ----------------------------------------------------------------------------------------
# forward / backward
# ----------------------------------------------------------------------------------------

ATTN_CASES = [
    # B, S, Hq, Hkv, D, block, dtype, kept per batch, n_segments
    (1, 1024, 8, 8, 64, 64, "f32", [[0, 1, 3, 4, 6, 9, 10, 15]], 3),
    (1, 1024, 4, 4, 128, 64, "bf16", [[0, 2, 3, 5, 8, 9, 11, 12, 13]], 2),      # 9 blocks: ragged
    (2, 1024, 4, 2, 128, 128, "bf16", [[1, 2, 4, 7], [0, 3, 5, 6]], 3),        # GQA, per-batch sets
    (1, 768, 4, 1, 64, 64, "bf16", [list(range(12))], 4),                        # keep all, G=4
    (1, 512, 2, 2, 128, 64, "bf16", [[7]], 1),                                   # one block
    (1, 512, 2, 2, 64, 128, "f32", [[1, 3]], 2),
]


def _run_attn(J, q, k, v, x0, dout, kept_list, block, dtype, n_segments, maxk=None):
    import torch
    B, S = q.shape[0], q.shape[1]
    nkb = S // block
    maxk = max(max(len(x) for x in kept_list), 1) if maxk is None else maxk
    qd, kd, vd = to_device(q, dtype), to_device(k, dtype), to_device(v, dtype)
    kept_d, nk_d = kept_tensor(kept_list, nkb)
    resid = torch.from_numpy(x0.copy()).cuda()
    o_saved, lse = J.sparse_attn_fwd(qd, kd, vd, kept_d, nk_d, maxk, block, resid)
    dq, dk, dv = J.sparse_attn_bwd(qd, kd, vd, kept_d, nk_d, maxk, block, o_saved, lse,
                                   torch.from_numpy(dout).cuda(), n_segments)
    torch.cuda.synchronize()
    return (resid.cpu().numpy(), o_saved.float().cpu().numpy(), lse.cpu().numpy(),
            dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy())


@pytest.mark.parametrize("B,S,Hq,Hkv,D,block,dtype,kept,nseg", ATTN_CASES)
def test_fwd_bwd(J, B, S, Hq, Hkv, D, block, dtype, kept, nseg):
    q, k, v, x0, dout = random_inputs(B, S, Hq, Hkv, D, dtype, seed=S + D + len(kept[0]))
    say(f"fwd/bwd B{B} S{S} Hq{Hq} Hkv{Hkv} D{D} block{block} {dtype} kept={kept} N={nseg}")
    resid, o_saved, lse, dq, dk, dv = _run_attn(J, q, k, v, x0, dout, kept, block, dtype, nseg)
    tol = tol_for(dtype)
    kept_np = [np.array(x) for x in kept]
    O, LSE = oracle.attn_fwd(q, k, v, kept_np, block)
    rq, rk, rv = oracle.attn_bwd(q, k, v, kept_np, block, dout)
    for b in range(B):
        pos = oracle.token_positions(kept_np[b], block)
        elim = np.setdiff1d(np.arange(S), pos)
        assert np.array_equal(resid[b, elim], x0[b, elim])               # bitwise untouched
        assert max_abs(resid[b, pos] - x0[b, pos], O[b, pos]) <= tol
        assert max_abs(o_saved[b, :len(pos)], O[b, pos]) <= tol
        lr = lse[b][:, :len(pos)]
        assert np.max(np.abs(lr - LSE[b][:, pos]) / np.maximum(1.0, np.abs(LSE[b][:, pos]))) <= 1e-5
        for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
            err = max_abs(got[b, pos], ref[b, pos])
            assert err <= tol, (name, err)
            assert np.all(got[b, elim] == 0), name


def test_fwd_bwd_rescale_heavy(J):
    """Large logits whose scale grows along the sequence: Q times 64 and the keys of token t
    times 2^(t // 256) (powers of two, exact in bf16), so the logits reach a standard deviation
    of about 6 in log2 units late in the sequence and most rows move their running maximum
    many times.  The forward takes the row maximum only where a lane's exponentials sum past
    2^7, so this exercises its rescale path on most steps.  Gradients scale with Q and K here,
    so the bf16 bound is taken relative to the largest reference magnitude above 1."""
    B, S, Hq, Hkv, D, block, nseg = 1, 1024, 4, 2, 128, 64, 3
    q, k, v, x0, dout = random_inputs(B, S, Hq, Hkv, D, "bf16", seed=77)
    q = (q * 64.0).astype(np.float32)
    k = (k * (2.0 ** (np.arange(S) // 256)).astype(np.float32)[None, :, None, None]).astype(np.float32)
    kept = [[0, 2, 3, 5, 7, 8, 10, 12, 13, 15]]
    say(f"fwd/bwd rescale-heavy S{S} Hq{Hq} Hkv{Hkv} D{D} block{block} kept={kept} N={nseg}")
    resid, o_saved, lse, dq, dk, dv = _run_attn(J, q, k, v, x0, dout, kept, block, "bf16", nseg)
    kept_np = [np.array(x) for x in kept]
    O, LSE = oracle.attn_fwd(q, k, v, kept_np, block)
    rq, rk, rv = oracle.attn_bwd(q, k, v, kept_np, block, dout)
    pos = oracle.token_positions(kept_np[0], block)
    tol = tol_for("bf16")
    assert max_abs(o_saved[0, :len(pos)], O[0, pos]) <= tol
    lr = lse[0][:, :len(pos)]
    assert np.max(np.abs(lr - LSE[0][:, pos]) / np.maximum(1.0, np.abs(LSE[0][:, pos]))) <= 1e-5
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        scale = max(1.0, float(np.max(np.abs(ref[0, pos]))))
        err = max_abs(got[0, pos], ref[0, pos])
        assert err <= tol * scale, (name, err, scale)


# Forward over few kept tokens: a row's query tiles of more than 32 key steps run in parts
# merged by k_fwd_combine.  Row 0 below keeps 40 blocks of 64 (20 tiles of 128 queries: tiles
# 8..19 split, the last in 3 parts); row 1 keeps 9 blocks (5 tiles, none longer than a part);
# the D=64 case keeps 15 of 16 blocks of 128 with a capacity of 16 blocks; the last case keeps
# 37 blocks of 64, so its last tile holds 64 queries (two of its four waves idle) and runs 74
# steps in 3 parts, with two query heads on one KV head.
SPLIT_FWD_CASES = [
    # B, S, Hq, Hkv, D, block, kept counts, capacity (blocks)
    (2, 4096, 4, 2, 128, 64, (40, 9), 40),
    (1, 2048, 2, 2, 64, 128, (15,), 16),
    (1, 4096, 2, 1, 128, 64, (37,), 48),
]


@pytest.mark.parametrize("B,S,Hq,Hkv,D,block,counts,maxk", SPLIT_FWD_CASES)
def test_fwd_split_tiles(J, B, S, Hq, Hkv, D, block, counts, maxk):
    nkb = S // block
    rng = np.random.default_rng(sum(counts) + D)
    kept = [np.sort(rng.choice(nkb, c, replace=False)) for c in counts]
    q, k, v, x0, dout = random_inputs(B, S, Hq, Hkv, D, "bf16", seed=31 + D)
    say(f"split forward B{B} S{S} Hq{Hq} Hkv{Hkv} D{D} block{block} kept {counts} cap {maxk}")
    first = _run_attn(J, q, k, v, x0, dout, kept, block, "bf16", 2, maxk=maxk)
    again = _run_attn(J, q, k, v, x0, dout, kept, block, "bf16", 2, maxk=maxk)
    # parts merge in a fixed order: bitwise repeatable (o_saved and lse rows past a batch row's
    # kept count are not written)
    for i in (0, 3, 4, 5):
        assert np.array_equal(first[i], again[i])
    for b, c in enumerate(counts):
        n = c * block
        assert np.array_equal(first[1][b, :n], again[1][b, :n])
        assert np.array_equal(first[2][b, :, :n], again[2][b, :, :n])
    resid, o_saved, lse, dq, dk, dv = first
    tol = tol_for("bf16")
    O, LSE = oracle.attn_fwd(q, k, v, kept, block)
    rq, rk, rv = oracle.attn_bwd(q, k, v, kept, block, dout)
    for b in range(B):
        pos = oracle.token_positions(kept[b], block)
        elim = np.setdiff1d(np.arange(S), pos)
        assert np.array_equal(resid[b, elim], x0[b, elim])
        assert max_abs(resid[b, pos] - x0[b, pos], O[b, pos]) <= tol
        assert max_abs(o_saved[b, :len(pos)], O[b, pos]) <= tol
        lr = lse[b][:, :len(pos)]
        assert np.max(np.abs(lr - LSE[b][:, pos]) / np.maximum(1.0, np.abs(LSE[b][:, pos]))) <= 1e-5
        for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
            err = max_abs(got[b, pos], ref[b, pos])
            assert err <= tol * max(1.0, float(np.max(np.abs(ref[b, pos])))), (b, name, err)


def test_bwd_segments_equivalent(J):
    """N = 1 and N = 8 segments give the same gradients up to fp32 rounding."""
    B, S, Hq, Hkv, D, block, dtype = 1, 2048, 4, 4, 128, 128, "bf16"
    kept = [[0, 1, 2, 4, 5, 7, 8, 9, 11, 12, 15]]
    q, k, v, x0, dout = random_inputs(B, S, Hq, Hkv, D, dtype, seed=3)
    say("segments N=1 vs N=8")
    r1 = _run_attn(J, q, k, v, x0, dout, kept, block, dtype, 1)
    r8 = _run_attn(J, q, k, v, x0, dout, kept, block, dtype, 8)
    for a, b in zip(r1[3:], r8[3:]):
        scale = max(1.0, float(np.max(np.abs(a))))
        assert max_abs(a, b) <= 1e-5 * scale


# B, S, Hq, Hkv, D, block, kept blocks per batch row, max_kept_blocks, segments
SCHED_CASES = [
    (2, 4096, 4, 2, 128, 64, (40, 26), 40, 3),   # short last segment; row 1 ends in segment 1
    (1, 2048, 3, 1, 64, 128, (16,), 16, 4),       # grouped-query attention, head_dim 64
    (1, 1024, 1, 1, 128, 64, (8,), 8, 8),         # two prologue groups per segment: a workgroup
                                                  # of the fused launch with idle halves
    # grouped-query attention where long dK/dV key tiles run in parts (sums of parts 1.. added
    # after the launch): one segment, the first key tiles in five parts
    (1, 8192, 8, 2, 128, 64, (40,), 40, 1),
    # four query heads per KV head, head_dim 64: row 1 ends before the last key tiles, whose
    # parts then do not run
    (2, 4096, 4, 1, 64, 64, (30, 18), 30, 1),
    # split key tiles with two sets of segment buffers
    (1, 4096, 8, 2, 128, 64, (48,), 48, 2),
]


@pytest.mark.parametrize("B,S,Hq,Hkv,D,block,counts,maxk,nseg", SCHED_CASES)
def test_bwd_schedules_bitwise(J, B, S, Hq, Hkv, D, block, counts, maxk, nseg):
    """bf16 backward with two sets of segment buffers (each segment's launch also runs the next
    segment's prologue) and with one set (each prologue a launch of its own): the same bits, and
    within tolerance of the oracle."""
    import torch
    nkb = S // block
    rng = np.random.default_rng(S + nseg)
    kept = [np.sort(rng.choice(nkb, c, replace=False)) for c in counts]
    q, k, v, x0, dout = random_inputs(B, S, Hq, Hkv, D, "bf16", seed=S + 3 * nseg)
    qd, kd, vd = to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16")
    kept_d, nk_d = kept_tensor(kept, nkb)
    resid = torch.from_numpy(x0.copy()).cuda()
    say(f"backward schedules B{B} S{S} Hq{Hq} Hkv{Hkv} D{D} block{block} kept {counts} N={nseg}")
    o_saved, lse = J.sparse_attn_fwd(qd, kd, vd, kept_d, nk_d, maxk, block, resid)
    dd = torch.from_numpy(dout).cuda()
    p = J.make_problem(qd, kd, vd, block)
    one = J.workspace_bytes(p, J.JENGA_OP_BWD_MIN, maxk, nseg)
    assert (J.workspace_bytes(p, J.JENGA_OP_BWD, maxk, nseg) > one) == (nseg > 1)   # a second set
    got = [J.sparse_attn_bwd(qd, kd, vd, kept_d, nk_d, maxk, block, o_saved, lse, dd, n_segments=nseg,
                             min_workspace=lean) for lean in (False, True)]
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got[0], got[1]):
        assert torch.equal(a, b), name
    rq, rk, rv = oracle.attn_bwd(q, k, v, kept, block, dout)
    tol = tol_for("bf16")
    for b in range(B):
        pos = oracle.token_positions(kept[b], block)
        for name, g, ref in (("dq", got[0][0], rq), ("dk", got[0][1], rk), ("dv", got[0][2], rv)):
            err = max_abs(g[b].cpu().numpy()[pos], ref[b, pos])
            assert err <= tol, (b, name, err)


def test_noalloc_bwd_falls_back_to_one_buffer_set(J):
    """A problem whose two sets of segment buffers exceed the no-alloc scratch but one set fits:
    the entry point that allocates nothing runs each prologue on its own and gives the bits of
    the entry point with the larger workspace."""
    import ctypes
    import torch
    B, S, Hq, Hkv, D, block, maxk, nseg = 1, 16384, 32, 32, 128, 128, 64, 4
    nkb = S // block
    kept = [np.sort(np.random.default_rng(77).choice(nkb, maxk, replace=False))]
    g = torch.Generator(device="cuda").manual_seed(78)
    qd = (torch.randn((B, S, Hq, D), generator=g, device="cuda") / 4).to(torch.bfloat16)
    kd = (torch.randn((B, S, Hkv, D), generator=g, device="cuda") / 4).to(torch.bfloat16)
    vd = torch.randn((B, S, Hkv, D), generator=g, device="cuda").to(torch.bfloat16)
    dd = torch.randn((B, S, Hq, D), generator=g, device="cuda")
    kept_d, nk_d = kept_tensor(kept, nkb)
    p = J.make_problem(qd, kd, vd, block)
    one = J.workspace_bytes(p, J.JENGA_OP_BWD_MIN, maxk, nseg)
    assert one <= J.NOALLOC_SCRATCH_BYTES < J.workspace_bytes(p, J.JENGA_OP_BWD, maxk, nseg)
    say(f"no-alloc backward with one buffer set: S{S} Hq{Hq} Hkv{Hkv} kept {maxk} N={nseg}")
    resid = torch.zeros((B, S, Hq, D), device="cuda")
    o_saved, lse = J.sparse_attn_fwd(qd, kd, vd, kept_d, nk_d, maxk, block, resid)
    ref = J.sparse_attn_bwd(qd, kd, vd, kept_d, nk_d, maxk, block, o_saved, lse, dd, n_segments=nseg)
    got = [torch.zeros_like(x) for x in ref]
    st = J.lib.jenga_sparse_attn_bwd_segmented_noalloc(
        ctypes.byref(p), qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), kept_d.data_ptr(),
        nk_d.data_ptr(), maxk, o_saved.data_ptr(), lse.data_ptr(), dd.data_ptr(), got[0].data_ptr(),
        got[1].data_ptr(), got[2].data_ptr(), nseg, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == J.JENGA_OK, J.status_string(st)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a, b), name


def test_empty_kept_set_is_noop(J):
    import torch
    B, S, Hq, Hkv, D, block, dtype = 1, 512, 2, 2, 128, 64, "bf16"
    q, k, v, x0, dout = random_inputs(B, S, Hq, Hkv, D, dtype, seed=9)
    say("empty kept set")
    resid, _, _, dq, dk, dv = _run_attn(J, q, k, v, x0, dout, [[]], block, dtype, 2, maxk=4)
    assert np.array_equal(resid, x0)
    assert not dq.any() and not dk.any() and not dv.any()


def test_fwd_deterministic(J):
    B, S, Hq, Hkv, D, block, dtype = 1, 1024, 4, 4, 128, 64, "bf16"
    q, k, v, x0, dout = random_inputs(B, S, Hq, Hkv, D, dtype, seed=10)
    kept = [[0, 2, 4, 6, 8, 10, 12, 14]]
    say("determinism")
    a = _run_attn(J, q, k, v, x0, dout, kept, block, dtype, 1)
    b = _run_attn(J, q, k, v, x0, dout, kept, block, dtype, 1)
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x, y)
    assert np.array_equal(a[4], b[4]) and np.array_equal(a[5], b[5])   # dk, dv: no atomics
