"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every function
that include/jenga.h declares, and rejects bad arguments with the documented status before
any launch.  Also pins the host-side top-k count against the oracle."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def J():
    import token_sparse_attention_jenga_amd as J
    return J


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "jenga.h")).read()
    return sorted(set(re.findall(r"\b(jenga_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(J):
    names = _declared_functions()
    assert set(names) == set(J.EXPORTED), names
    for n in names:
        assert hasattr(J.lib, n), n
        getattr(J.lib, n)                 # resolves the symbol


def test_status_strings(J):
    for st in (0, -1, -2, -3, -4, -5):
        assert J.status_string(st) != "unknown status"
    assert J.status_string(7) == "unknown status"


@pytest.mark.parametrize("r,n", [(0.5, 16), (0.35, 256), (0.5, 256), (0.3, 10), (0.31, 10), (1.0, 5),
                                 (1e-9, 9), (0.25, 4), (0.999, 1000), (0.123, 4096)])
def test_topk_count_matches_oracle(J, r, n):
    assert J.topk_count(r, n) == oracle.keep_count(r, n)


def _problem(J, B=1, S=1024, Hq=8, Hkv=8, D=64, block=64, dtype=0, scale=0.0):
    p = J.JengaProblem()
    p.batch, p.seq_len, p.n_heads_q, p.n_heads_kv, p.head_dim, p.block = B, S, Hq, Hkv, D, block
    p.dtype, p.scale = dtype, scale
    for name, H in (("q_stride", Hq), ("k_stride", Hkv), ("v_stride", Hkv)):
        arr = getattr(p, name)
        arr[0], arr[1], arr[2] = S * H * D, H * D, D
    return p


FAKE = 0x10000  # a 64 KiB-aligned non-null address; never dereferenced (checks fail first)


def _score(J, p, ws_bytes=1 << 30, q=FAKE, ws=FAKE):
    return J.lib.jenga_score_blocks(ctypes.byref(p), q, FAKE, FAKE, ws, ws_bytes, None)


def test_score_validation(J):
    assert J.lib.jenga_score_blocks(None, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == J.JENGA_ERR_INVALID_ARG
    assert _score(J, _problem(J, D=96)) == J.JENGA_ERR_UNSUPPORTED
    assert _score(J, _problem(J, D=128, dtype=0)) == J.JENGA_ERR_UNSUPPORTED     # fp32 needs D=64
    assert _score(J, _problem(J, block=32)) == J.JENGA_ERR_UNSUPPORTED
    assert _score(J, _problem(J, S=1000)) == J.JENGA_ERR_UNSUPPORTED
    assert _score(J, _problem(J, Hq=6, Hkv=4)) == J.JENGA_ERR_INVALID_ARG
    assert _score(J, _problem(J, dtype=5)) == J.JENGA_ERR_UNSUPPORTED
    assert _score(J, _problem(J, B=0)) == J.JENGA_ERR_INVALID_ARG
    assert _score(J, _problem(J, scale=-1.0)) == J.JENGA_ERR_INVALID_ARG
    assert _score(J, _problem(J), q=0) == J.JENGA_ERR_INVALID_ARG
    assert _score(J, _problem(J), q=FAKE + 4) == J.JENGA_ERR_INVALID_ARG           # misaligned
    p = _problem(J)
    need = J.workspace_bytes(p, J.JENGA_OP_SCORE)
    assert need > 0
    assert _score(J, p, ws_bytes=need - 1) == J.JENGA_ERR_WORKSPACE
    assert _score(J, p, ws=0) == J.JENGA_ERR_WORKSPACE
    bad = _problem(J)
    bad.q_stride[1] = 8 * 64 + 2                                                     # row not 16-B aligned
    assert _score(J, bad) == J.JENGA_ERR_INVALID_ARG


def test_offsets_past_4gib_rejected(J):
    # the kernels address each batch row of q / k / v through 32-bit buffer offsets, and the
    # fp32 residual and gradient rows of a batch row with 32-bit offsets too: a problem whose
    # rows span 4 GiB or more is refused before any launch, in every entry point
    def calls(pp):
        # (a zero-byte workspace: a problem that passes the shape checks stops at the workspace
        # check, so nothing is ever launched on these fake pointers)
        return (J.lib.jenga_score_blocks(ctypes.byref(pp), FAKE, FAKE, FAKE, FAKE, 0, None),
                J.lib.jenga_sparse_attn_fwd(ctypes.byref(pp), FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE,
                                            FAKE, FAKE, FAKE, 0, None),
                J.lib.jenga_sparse_attn_bwd_segmented(ctypes.byref(pp), FAKE, FAKE, FAKE, FAKE, FAKE, 1,
                                                      FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE,
                                                      0, None))
    U = J.JENGA_ERR_UNSUPPORTED
    # 512K tokens of 32 x 128 bf16 heads: 4 GiB per batch row of q
    assert calls(_problem(J, S=1 << 19, Hq=32, Hkv=32, D=128, block=128, dtype=1)) == (U, U, U)
    # K as a view into a packed QKV tensor (3 * 32 * 128 bf16 per token, 24 KiB): 171K tokens
    # already span 4 GiB, though K alone would not
    packed = _problem(J, S=176128, Hq=32, Hkv=32, D=128, block=128, dtype=1)
    for name in ("q_stride", "k_stride", "v_stride"):
        getattr(packed, name)[1] = 3 * 32 * 128
    assert calls(packed) == (U, U, U)
    # the fp32 residual rows alone: 256K tokens of 32 x 128 heads is 4 GiB of fp32 per batch row,
    # even though the bf16 q / k / v rows are half that
    assert calls(_problem(J, S=1 << 18, Hq=32, Hkv=8, D=128, block=128, dtype=1)) == (U, U, U)
    # just below every limit the shape checks pass and the workspace check decides
    ok = _problem(J, S=(1 << 18) - 128, Hq=32, Hkv=8, D=128, block=128, dtype=1)
    W = J.JENGA_ERR_WORKSPACE
    assert calls(ok) == (W, W, W)


def test_select_validation(J):
    p = _problem(J)
    f = lambda mode=0, param=0.5, flags=0, s=FAKE: J.lib.jenga_select_blocks(
        ctypes.byref(p), s, mode, ctypes.c_float(param), flags, FAKE, FAKE, None)
    assert f(mode=3) == J.JENGA_ERR_INVALID_ARG
    assert f(param=0.0) == J.JENGA_ERR_INVALID_ARG
    assert f(param=float("nan")) == J.JENGA_ERR_INVALID_ARG
    assert f(flags=2) == J.JENGA_ERR_INVALID_ARG
    assert f(s=0) == J.JENGA_ERR_INVALID_ARG
    big = _problem(J, S=64 * 20000)
    assert J.lib.jenga_select_blocks(ctypes.byref(big), FAKE, 0, ctypes.c_float(0.5), 0, FAKE, FAKE,
                                     None) == J.JENGA_ERR_UNSUPPORTED


def test_fwd_bwd_validation(J):
    p = _problem(J)
    fwd = lambda maxk=8, resid=FAKE, ws=FAKE, wsb=1 << 30, pp=p: J.lib.jenga_sparse_attn_fwd(
        ctypes.byref(pp), FAKE, FAKE, FAKE, FAKE, FAKE, maxk, resid, FAKE, FAKE, ws, wsb, None)
    assert fwd(maxk=0) == J.JENGA_ERR_INVALID_ARG
    assert fwd(maxk=17) == J.JENGA_ERR_INVALID_ARG
    assert fwd(resid=0) == J.JENGA_ERR_INVALID_ARG
    assert fwd(resid=FAKE + 8) == J.JENGA_ERR_INVALID_ARG
    pb = _problem(J, D=128, dtype=1)                       # bf16 needs a forward workspace
    need_f = J.workspace_bytes(pb, J.JENGA_OP_FWD, 8)
    assert need_f > 0
    assert fwd(pp=pb, ws=0) == J.JENGA_ERR_WORKSPACE
    assert fwd(pp=pb, wsb=need_f - 1) == J.JENGA_ERR_WORKSPACE
    assert fwd(pp=pb, ws=FAKE + 16) == J.JENGA_ERR_WORKSPACE
    need = J.workspace_bytes(p, J.JENGA_OP_BWD, 8, 2)
    assert need > 0
    bwd = lambda nseg=2, ws_bytes=need, maxk=8: J.lib.jenga_sparse_attn_bwd_segmented(
        ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, maxk, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
        nseg, FAKE, ws_bytes, None)
    assert bwd(nseg=0) == J.JENGA_ERR_INVALID_ARG
    assert bwd(nseg=9) == J.JENGA_ERR_INVALID_ARG            # more segments than 64-row tiles
    assert bwd(ws_bytes=need - 1) == J.JENGA_ERR_WORKSPACE
    assert bwd(maxk=20) == J.JENGA_ERR_INVALID_ARG


def test_workspace_scales_with_segments_and_kept_blocks(J):
    p = _problem(J, S=32768, Hq=32, Hkv=32, D=128, block=128, dtype=1)
    w1 = J.workspace_bytes(p, J.JENGA_OP_BWD, 128, 1)
    w8 = J.workspace_bytes(p, J.JENGA_OP_BWD_MIN, 128, 8)
    w8_half = J.workspace_bytes(p, J.JENGA_OP_BWD_MIN, 64, 8)
    vtp = 32 * 128 * 128 * 128 * 2                # forward: transposed V tiles of all kept keys
    seg = lambda L: 2 * 32 * L * 4 + 3 * 32 * L * 128 * 2   # D, lse2, dOut, dOut^T and Q^T tiles
    assert w1 == seg(16384)                       # one segment: one set of buffers either way
    assert J.workspace_bytes(p, J.JENGA_OP_BWD_MIN, 128, 1) == w1
    assert w8 == seg(2048)                        # the backward workspace shrinks as 1/N
    assert abs(w8_half * 2 - w8) <= 4096          # and scales with the kept tokens
    # bf16 with two or more segments: the faster schedule takes two sets of segment buffers
    assert J.workspace_bytes(p, J.JENGA_OP_BWD, 128, 8) == 2 * w8
    assert J.workspace_bytes(p, J.JENGA_OP_BWD, 64, 8) == 2 * w8_half
    # grouped-query attention in one segment (32/8 heads, 90 kept blocks of 64): the long dK/dV
    # key tiles run in parts, whose sums need slots beyond the segment buffers
    pg = _problem(J, S=16384, Hq=32, Hkv=8, D=128, block=64, dtype=1)
    one_g = J.workspace_bytes(pg, J.JENGA_OP_BWD_MIN, 90, 1)
    assert one_g > seg(5760)
    assert (one_g - seg(5760)) % (2 * 256 * 128 * 4 * 8) == 0          # whole slots per KV head
    assert J.workspace_bytes(pg, J.JENGA_OP_BWD, 90, 1) == one_g         # one segment: one set
    p32 = _problem(J, S=4096, Hq=4, Hkv=4, D=64, block=64, dtype=0)
    assert J.workspace_bytes(p32, J.JENGA_OP_BWD, 32, 4) == J.workspace_bytes(p32, J.JENGA_OP_BWD_MIN, 32, 4)
    slot = 128 * (2 * 128 + 8)                    # a query tile's bf16 rows, fp32 max and sum
    assert J.workspace_bytes(p, J.JENGA_OP_FWD, 128) == vtp + 32 * 27 * slot
    assert J.workspace_bytes(_problem(J), J.JENGA_OP_FWD, 8) == 0       # fp32 path needs none


def test_fwd_workspace_part_slots(J):
    # A batch row of n 128-query tiles splits when (n + 1) * Hq * B < 768 (its longest tile, 4n
    # steps of 32 keys, is more than twice the mean 2n(n + 1) Hq B / 768 per workgroup slot);
    # parts are T = max(32, ceil(mean)) steps, and only tiles longer than T take slots.  The
    # workspace holds the worst row up to the capacity.
    slot = lambda D: 128 * (2 * D + 8)            # 128 unnormalised bf16 rows, fp32 max and sum
    vtp = lambda B, Hkv, ncap, D: B * Hkv * ncap * D * 2
    # 32 heads, capacity 16384: rows of n <= 22 tiles split; the most slots are at n = 20
    # (T = 26880 / 768 = 35): tiles 8..16 (36..68 steps) in 2 parts, 17..19 (72..80) in 3
    c5 = _problem(J, S=32768, Hq=32, Hkv=32, D=128, block=128, dtype=1)
    assert J.workspace_bytes(c5, J.JENGA_OP_FWD, 128) == vtp(1, 32, 16384, 128) + 32 * 27 * slot(128)
    # capacity 2048 (n <= 16, T = 32): tiles 8..15 (36..64 steps) in 2 parts
    c2 = _problem(J, S=4096, Hq=32, Hkv=32, D=128, block=64, dtype=1)
    assert J.workspace_bytes(c2, J.JENGA_OP_FWD, 32) == vtp(1, 32, 2048, 128) + 32 * 16 * slot(128)
    # capacity 1024: no tile is longer than 32 steps, nothing splits
    assert J.workspace_bytes(c2, J.JENGA_OP_FWD, 16) == vtp(1, 32, 1024, 128)
    # 64 heads x 2 rows: (n + 1) * 128 < 768 leaves n <= 4, tiles of at most 16 steps
    wide = _problem(J, B=2, S=4096, Hq=64, Hkv=8, D=64, block=64, dtype=1)
    assert J.workspace_bytes(wide, J.JENGA_OP_FWD, 64) == vtp(2, 8, 4096, 64)
    # whatever the shape, a (row, head) takes fewer than 1536 / (Hq B) slots
    for B, Hq, S, D in ((1, 1, 65536, 64), (1, 2, 32768, 128), (2, 4, 16384, 64), (1, 8, 16384, 128)):
        pr = _problem(J, B=B, S=S, Hq=Hq, Hkv=1, D=D, block=64, dtype=1)
        extra = J.workspace_bytes(pr, J.JENGA_OP_FWD, S // 64) - vtp(B, 1, S, D)
        assert extra % (B * Hq * slot(D)) == 0
        assert 0 < extra // (B * Hq * slot(D)) < 1536 // (B * Hq)


def test_score_workspace(J):
    # lse2 rows (fp32) and mass slots (fp64, one per 32 keys), each rounded to 256 bytes; the
    # bf16 path adds the partial log2-sums of one query chunk: chunk * nKB floats per (batch,
    # head), chunk = 128 * ceil(2048 / (B * Hq)) queries, at most S rounded up to 128
    up = lambda x: (x + 255) // 256 * 256
    for B, S, Hq, block in ((1, 32768, 32, 128), (2, 4096, 8, 64), (1, 576, 2, 192),
                            (1, 131072, 32, 128), (1, 16384, 32, 64)):
        nkb = S // block
        chunk = min(128 * -(-2048 // (B * Hq)), -(-S // 128) * 128)
        base = up(B * Hq * S * 4) + up(B * Hq * (S // 32) * 8)
        p16 = _problem(J, B=B, S=S, Hq=Hq, Hkv=Hq, D=128, block=block, dtype=1)
        assert J.workspace_bytes(p16, J.JENGA_OP_SCORE) == base + up(B * Hq * nkb * chunk * 4)
        p32 = _problem(J, B=B, S=S, Hq=Hq, Hkv=Hq, D=64, block=block, dtype=0)
        assert J.workspace_bytes(p32, J.JENGA_OP_SCORE) == base
    # 32K tokens, 32 heads, block 128: chunks of 8192 queries, 256 MiB of partial sums beside
    # 4.25 MiB of rows and slots (the whole causal triangle would be 514 MiB)
    c5 = _problem(J, S=32768, Hq=32, Hkv=32, D=128, block=128, dtype=1)
    assert J.workspace_bytes(c5, J.JENGA_OP_SCORE) == 4 * 2**20 + 2**18 + 256 * 2**20
    # linear in S: at four times the tokens the partial sums take four times the bytes
    c5x4 = _problem(J, S=131072, Hq=32, Hkv=32, D=128, block=128, dtype=1)
    rows = lambda S: S * 32 * 4 + S // 32 * 32 * 8
    assert (J.workspace_bytes(c5x4, J.JENGA_OP_SCORE) - rows(131072)
            == 4 * (J.workspace_bytes(c5, J.JENGA_OP_SCORE) - rows(32768)))


def test_timing_calls_without_gpu_work(J):
    assert J.lib.jenga_timing_enable(2) == J.JENGA_ERR_INVALID_ARG
    J.timing_enable(True)
    assert J.timing_query("k_bwd64") == (0, 0.0)           # nothing launched yet
    J.timing_enable(False)
    n = ctypes.c_int32(0)
    assert J.lib.jenga_timing_query(None, ctypes.byref(n), None) == J.JENGA_ERR_INVALID_ARG


def test_score_eq2_validation(J):
    p = _problem(J, D=128, dtype=1, block=64)
    need = J.workspace_bytes(p, J.JENGA_OP_SCORE_EQ2)
    assert need == 1 * 16 * 16 * 4 or need == 256        # B * nKB^2 fp32, 256-byte rounded
    f = lambda pp=p, ws=FAKE, wsb=need: J.lib.jenga_score_blocks_eq2(ctypes.byref(pp), FAKE, FAKE, FAKE,
                                                                    ws, wsb, None)
    assert f(pp=_problem(J, D=64, dtype=0)) == J.JENGA_ERR_UNSUPPORTED          # fp32
    assert f(pp=_problem(J, D=128, dtype=1, block=256)) == J.JENGA_ERR_UNSUPPORTED
    assert f(wsb=need - 1) == J.JENGA_ERR_WORKSPACE
    assert f(ws=0) == J.JENGA_ERR_WORKSPACE


def test_proj_validation(J):
    p = J.JengaProjProblem()
    p.batch, p.seq_len, p.block, p.in_features, p.out_features = 1, 1024, 64, 256, 256
    p.in_stride[0], p.in_stride[1] = 1024 * 256, 256
    p.out_stride[0], p.out_stride[1] = 16 * 64 * 256, 256
    g = lambda pp=p, maxk=4, x=FAKE: J.lib.jenga_proj_gather(ctypes.byref(pp), x, FAKE, FAKE, FAKE,
                                                            maxk, FAKE, None)
    assert g(maxk=0) == J.JENGA_ERR_INVALID_ARG
    assert g(maxk=17) == J.JENGA_ERR_INVALID_ARG
    assert g(x=0) == J.JENGA_ERR_INVALID_ARG
    assert g(x=FAKE + 2) == J.JENGA_ERR_INVALID_ARG
    bad = J.JengaProjProblem.from_buffer_copy(p)
    bad.out_features = 192                                       # not a multiple of 128
    assert g(pp=bad) == J.JENGA_ERR_UNSUPPORTED
    bad = J.JengaProjProblem.from_buffer_copy(p)
    bad.in_features = 96                                         # not a multiple of 64
    assert g(pp=bad) == J.JENGA_ERR_UNSUPPORTED
    bad = J.JengaProjProblem.from_buffer_copy(p)
    bad.block = 32
    assert g(pp=bad) == J.JENGA_ERR_UNSUPPORTED
    bad = J.JengaProjProblem.from_buffer_copy(p)
    bad.in_stride[1] = 257                                       # rows not 16-byte aligned
    assert g(pp=bad) == J.JENGA_ERR_INVALID_ARG
    assert J.lib.jenga_proj_scatter_add(None, FAKE, FAKE, FAKE, FAKE, 4, FAKE, None) == \
        J.JENGA_ERR_INVALID_ARG


def test_mlp_validation_and_workspace(J):
    p = J.JengaProjProblem()
    p.batch, p.seq_len, p.block, p.in_features, p.out_features = 1, 32768, 128, 4096, 11008
    p.in_stride[0], p.in_stride[1] = 32768 * 4096, 4096
    p.out_stride[0], p.out_stride[1] = 32768 * 11008, 11008
    gated, relu = J.JENGA_MLP_SILU_GATED, J.JENGA_MLP_RELU
    wsb = J.mlp_workspace_bytes(p, gated)
    assert wsb == 32768 * (11008 // 32) * 4                   # partial sums per 32 units
    assert J.mlp_workspace_bytes(p, relu) == wsb                # 11008 = 86 * 128
    p64 = J.JengaProjProblem.from_buffer_copy(p)
    p64.out_features = 11072                                    # a multiple of 64, not of 128
    assert J.mlp_workspace_bytes(p64, gated) > 0
    assert J.mlp_workspace_bytes(p64, relu) == 0                # ReLU tiles need F % 128 == 0
    assert J.mlp_workspace_bytes(p, 2) == 0                     # unknown kind
    f = lambda pp=p, kind=gated, x=FAKE, wu=FAKE, ws=FAKE, n=wsb: J.lib.jenga_mlp_act_scores(
        ctypes.byref(pp), kind, x, FAKE, wu, FAKE, FAKE, FAKE, ws, n, None)
    assert f(kind=5) == J.JENGA_ERR_INVALID_ARG
    assert f(x=0) == J.JENGA_ERR_INVALID_ARG
    assert f(wu=0) == J.JENGA_ERR_INVALID_ARG                  # gated needs the up projection
    assert f(x=FAKE + 2) == J.JENGA_ERR_INVALID_ARG
    assert f(n=wsb - 1) == J.JENGA_ERR_WORKSPACE
    assert f(ws=FAKE + 16) == J.JENGA_ERR_WORKSPACE             # not 256-byte aligned
    assert f(pp=p64, kind=relu) == J.JENGA_ERR_UNSUPPORTED
    bad = J.JengaProjProblem.from_buffer_copy(p)
    bad.block = 96
    assert f(pp=bad) == J.JENGA_ERR_UNSUPPORTED
    bad = J.JengaProjProblem.from_buffer_copy(p)
    bad.out_stride[1] = 11009                                  # act rows not 16-byte aligned
    assert f(pp=bad) == J.JENGA_ERR_INVALID_ARG
    assert J.lib.jenga_proj_gather_scatter_add(None, FAKE, FAKE, FAKE, FAKE, 4, FAKE, None) == \
        J.JENGA_ERR_INVALID_ARG


def test_loss_validation_and_workspace(J):
    p1 = J.loss_problem(32768, 4096, 32000, 1)
    p8 = J.loss_problem(32768, 4096, 32000, 8)
    w1, w8 = J.loss_workspace_bytes(p1), J.loss_workspace_bytes(p8)
    assert w1 == 32768 * 32000 * 6 and w8 == 4096 * 32000 * 6    # the transient scales as 1/N
    assert J.loss_workspace_bytes(J.loss_problem(100, 4096, 32000, 1)) == 0   # tokens % 32
    assert J.loss_workspace_bytes(J.loss_problem(64, 4096, 40000, 1)) == 0    # vocab > 32768
    f = lambda pp=p8, ws=FAKE, wsb=w8, h=FAKE: J.lib.jenga_lm_head_ce_segmented(
        ctypes.byref(pp), h, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, wsb, None)
    assert f(h=0) == J.JENGA_ERR_INVALID_ARG
    assert f(wsb=w8 - 1) == J.JENGA_ERR_WORKSPACE
    assert f(pp=J.loss_problem(64, 4096, 32000, 3)) == J.JENGA_ERR_INVALID_ARG   # > T/32 segments
    assert f(pp=J.loss_problem(64, 4000, 32000, 1)) == J.JENGA_ERR_UNSUPPORTED


def test_binding_refuses_views_dtypes_and_shapes(J):
    # the binding checks every dense argument before a pointer reaches the library: a view, a
    # wrong dtype or a wrong shape raises ValueError (CPU tensors: these checks come first)
    import torch
    B, S, Hq, Hkv, D, block, maxk = 1, 256, 4, 2, 64, 64, 2
    q = torch.zeros((B, S, Hq, D), dtype=torch.bfloat16)
    k = torch.zeros((B, S, Hkv, D), dtype=torch.bfloat16)
    p = J.make_problem(q, k, k, block)
    kept = torch.zeros((B, S // block), dtype=torch.int32)
    nk = torch.zeros((B,), dtype=torch.int32)
    resid = torch.zeros((B, S, Hq, D), dtype=torch.float32)
    o = torch.zeros((B, maxk * block, Hq, D), dtype=torch.bfloat16)
    lse = torch.zeros((B, Hq, maxk * block), dtype=torch.float32)
    fwd = lambda **kw: J.jenga_sparse_attn_fwd(p, q, k, k, kw.get("kept", kept), kw.get("nk", nk), maxk,
                                               kw.get("resid", resid), kw.get("o", o), kw.get("lse", lse))
    with pytest.raises(ValueError, match="resid: dtype"):
        fwd(resid=resid.to(torch.bfloat16))
    with pytest.raises(ValueError, match="resid: must be contiguous"):
        fwd(resid=torch.zeros((B, Hq, S, D)).transpose(1, 2))
    with pytest.raises(ValueError, match="o_saved: shape"):
        fwd(o=o[:, :block])
    with pytest.raises(ValueError, match="lse: shape"):
        fwd(lse=lse.transpose(1, 2))
    with pytest.raises(ValueError, match="kept_idx: dtype"):
        fwd(kept=kept.long())
    with pytest.raises(ValueError, match="n_kept: shape"):
        fwd(nk=torch.zeros((2,), dtype=torch.int32))
    g = torch.zeros((B, S, Hq, D), dtype=torch.float32)
    gk = torch.zeros((B, S, Hkv, D), dtype=torch.float32)
    bwd = lambda **kw: J.jenga_sparse_attn_bwd_segmented(
        p, q, k, k, kept, nk, maxk, o, lse, kw.get("dout", g), kw.get("dq", g), kw.get("dk", gk),
        kw.get("dv", gk), 1, torch.zeros(256, dtype=torch.uint8))
    with pytest.raises(ValueError, match="dk: shape"):
        bwd(dk=g)
    with pytest.raises(ValueError, match="dout: dtype"):
        bwd(dout=g.double())
    with pytest.raises(ValueError, match="dq: must be contiguous"):
        bwd(dq=torch.zeros((B, S, D, Hq)).transpose(2, 3))
    with pytest.raises(ValueError, match="block_scores: shape"):
        J.jenga_score_blocks(p, q, k, torch.zeros((B, 3)), torch.zeros(256, dtype=torch.uint8))
    with pytest.raises(ValueError, match="share one dtype"):
        J.make_problem(q, k.float(), k, block)
    with pytest.raises(ValueError, match="do not match"):
        J.make_problem(q, k[:, :128], k, block)
    with pytest.raises(ValueError, match="targets: dtype"):
        J.lm_head_ce(torch.zeros((64, 128), dtype=torch.bfloat16), torch.zeros((256, 128), dtype=torch.bfloat16),
                     torch.zeros((128, 256), dtype=torch.bfloat16), torch.zeros(64, dtype=torch.int64))


def test_noalloc_backward_refuses_past_its_scratch(J):
    # 32K tokens x 32 heads x 128 with 128 kept blocks of 128: one segment needs 388 MiB of
    # scratch, past the fixed 64 MiB, so the call returns JENGA_ERR_SCRATCH_LIMIT before
    # anything is launched; eight segments need 48.5 MiB (within the limit; their two-set
    # schedule, 97 MiB, is not, so that call runs each prologue as a launch of its own)
    p = _problem(J, S=32768, Hq=32, Hkv=32, D=128, block=128, dtype=1)
    assert J.workspace_bytes(p, J.JENGA_OP_BWD_MIN, 128, 1) > J.NOALLOC_SCRATCH_BYTES
    assert J.workspace_bytes(p, J.JENGA_OP_BWD_MIN, 128, 8) <= J.NOALLOC_SCRATCH_BYTES
    assert J.workspace_bytes(p, J.JENGA_OP_BWD, 128, 8) > J.NOALLOC_SCRATCH_BYTES
    st = J.lib.jenga_sparse_attn_bwd_segmented_noalloc(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 128,
                                                       FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None)
    assert st == J.JENGA_ERR_SCRATCH_LIMIT
    assert "n_segments" in J.status_string(st)
    # argument checks come first, as in the entry point with a workspace
    assert J.lib.jenga_sparse_attn_bwd_segmented_noalloc(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 0,
                                                         FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1,
                                                         None) == J.JENGA_ERR_INVALID_ARG
