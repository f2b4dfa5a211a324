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
    for st in (0, -1, -2, -3, -4):
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
    w8 = J.workspace_bytes(p, J.JENGA_OP_BWD, 128, 8)
    w8_half = J.workspace_bytes(p, J.JENGA_OP_BWD, 64, 8)
    vtp = 32 * 128 * 128 * 128 * 2                # forward: transposed V tiles of all kept keys
    seg = lambda L: 2 * 32 * L * 4 + 3 * 32 * L * 128 * 2   # D, lse2, dOut, dOut^T and Q^T tiles
    assert w1 == seg(16384)
    assert w8 == seg(2048)                        # the backward workspace shrinks as 1/N
    assert abs(w8_half * 2 - w8) <= 4096          # and scales with the kept tokens
    assert J.workspace_bytes(p, J.JENGA_OP_FWD, 128) == vtp
    assert J.workspace_bytes(_problem(J), J.JENGA_OP_FWD, 8) == 0       # fp32 path needs none


def test_score_workspace(J):
    # lse2 rows (fp32) and mass slots (fp64, one per 32 keys), each rounded to 256 bytes; the
    # bf16 path adds, per (batch, head), the causal triangle of key-block partial log2-sums:
    # row n holds the queries n*block .. S-1, S*nKB - block*nKB*(nKB-1)/2 floats in all
    up = lambda x: (x + 255) // 256 * 256
    for B, S, Hq, block in ((1, 32768, 32, 128), (2, 4096, 8, 64), (1, 576, 2, 192)):
        nkb = S // block
        tri = S * nkb - block * nkb * (nkb - 1) // 2
        base = up(B * Hq * S * 4) + up(B * Hq * (S // 32) * 8)
        p16 = _problem(J, B=B, S=S, Hq=Hq, Hkv=Hq, D=128, block=block, dtype=1)
        assert J.workspace_bytes(p16, J.JENGA_OP_SCORE) == base + up(B * Hq * tri * 4)
        p32 = _problem(J, B=B, S=S, Hq=Hq, Hkv=Hq, D=64, block=block, dtype=0)
        assert J.workspace_bytes(p32, J.JENGA_OP_SCORE) == base
    # 32K tokens, 32 heads, block 128: 514 MiB of partial sums beside 4.25 MiB of rows and slots
    c5 = _problem(J, S=32768, Hq=32, Hkv=32, D=128, block=128, dtype=1)
    assert J.workspace_bytes(c5, J.JENGA_OP_SCORE) == 4 * 2**20 + 2**18 + 32 * 4210688 * 4


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
