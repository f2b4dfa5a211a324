"""Python binding of libjenga.so, the gfx950 token-sparse attention hot path.

Argument marshalling only: every step runs in the library's HIP kernels.  PyTorch supplies
device memory and the current stream.  Importing this package loads the library and fails
loudly if it has not been built (python -m token_sparse_attention_jenga_amd.build).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libjenga.so")

JENGA_OK = 0
JENGA_ERR_INVALID_ARG = -1
JENGA_ERR_UNSUPPORTED = -2
JENGA_ERR_WORKSPACE = -3
JENGA_ERR_LAUNCH = -4
JENGA_ERR_SCRATCH_LIMIT = -5
NOALLOC_SCRATCH_BYTES = 64 << 20
JENGA_DTYPE_F32 = 0
JENGA_DTYPE_BF16 = 1
JENGA_SELECT_TOPK = 0
JENGA_SELECT_THRESH_REL = 1
JENGA_SELECT_THRESH_ABS = 2
JENGA_MLP_RELU = 0
JENGA_MLP_SILU_GATED = 1
JENGA_FORCE_FIRST_BLOCK = 1
JENGA_OP_SCORE = 0
JENGA_OP_FWD = 1
JENGA_OP_BWD = 2
JENGA_OP_SCORE_EQ2 = 3
JENGA_OP_BWD_MIN = 4

EXPORTED = ["jenga_status_string", "jenga_topk_count", "jenga_workspace_bytes",
            "jenga_score_blocks", "jenga_score_blocks_eq2", "jenga_select_blocks",
            "jenga_sparse_attn_fwd", "jenga_sparse_attn_bwd_segmented",
            "jenga_sparse_attn_bwd_segmented_noalloc", "jenga_proj_gather",
            "jenga_proj_scatter_add", "jenga_proj_gather_scatter_add", "jenga_mlp_workspace_bytes",
            "jenga_mlp_act_scores", "jenga_loss_workspace_bytes", "jenga_lm_head_ce_segmented",
            "jenga_timing_enable", "jenga_timing_query"]


class JengaProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("n_heads_q", ctypes.c_int32), ("n_heads_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
                ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
                ("v_stride", ctypes.c_int64 * 3)]


class JengaProjProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32), ("block", ctypes.c_int32),
                ("in_features", ctypes.c_int32), ("out_features", ctypes.c_int32),
                ("in_stride", ctypes.c_int64 * 2), ("out_stride", ctypes.c_int64 * 2)]


class JengaLossProblem(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int32), ("d_model", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("n_segments", ctypes.c_int32)]


class JengaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({status_string(status)})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          f"`python -m token_sparse_attention_jenga_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    P = ctypes.POINTER(JengaProblem)
    lib.jenga_status_string.argtypes = [i32]
    lib.jenga_status_string.restype = ctypes.c_char_p
    lib.jenga_topk_count.argtypes = [ctypes.c_float, i32]
    lib.jenga_topk_count.restype = i32
    lib.jenga_workspace_bytes.argtypes = [P, i32, i32, i32]
    lib.jenga_workspace_bytes.restype = sz
    lib.jenga_score_blocks.argtypes = [P, vp, vp, vp, vp, sz, vp]
    lib.jenga_score_blocks.restype = i32
    lib.jenga_score_blocks_eq2.argtypes = [P, vp, vp, vp, vp, sz, vp]
    lib.jenga_score_blocks_eq2.restype = i32
    lib.jenga_select_blocks.argtypes = [P, vp, i32, ctypes.c_float, ctypes.c_uint, vp, vp, vp]
    lib.jenga_select_blocks.restype = i32
    lib.jenga_sparse_attn_fwd.argtypes = [P, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, sz, vp]
    lib.jenga_sparse_attn_fwd.restype = i32
    lib.jenga_sparse_attn_bwd_segmented.argtypes = [P, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp,
                                                    vp, i32, vp, sz, vp]
    lib.jenga_sparse_attn_bwd_segmented.restype = i32
    lib.jenga_sparse_attn_bwd_segmented_noalloc.argtypes = [P, vp, vp, vp, vp, vp, i32, vp, vp, vp,
                                                            vp, vp, vp, i32, vp]
    lib.jenga_sparse_attn_bwd_segmented_noalloc.restype = i32
    PP = ctypes.POINTER(JengaProjProblem)
    lib.jenga_proj_gather.argtypes = [PP, vp, vp, vp, vp, i32, vp, vp]
    lib.jenga_proj_gather.restype = i32
    lib.jenga_proj_scatter_add.argtypes = [PP, vp, vp, vp, vp, i32, vp, vp]
    lib.jenga_proj_scatter_add.restype = i32
    lib.jenga_proj_gather_scatter_add.argtypes = [PP, vp, vp, vp, vp, i32, vp, vp]
    lib.jenga_proj_gather_scatter_add.restype = i32
    lib.jenga_mlp_workspace_bytes.argtypes = [PP, i32]
    lib.jenga_mlp_workspace_bytes.restype = sz
    lib.jenga_mlp_act_scores.argtypes = [PP, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.jenga_mlp_act_scores.restype = i32
    LP = ctypes.POINTER(JengaLossProblem)
    lib.jenga_loss_workspace_bytes.argtypes = [LP]
    lib.jenga_loss_workspace_bytes.restype = sz
    lib.jenga_lm_head_ce_segmented.argtypes = [LP, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.jenga_lm_head_ce_segmented.restype = i32
    lib.jenga_timing_enable.argtypes = [i32]
    lib.jenga_timing_enable.restype = i32
    lib.jenga_timing_query.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_int32),
                                       ctypes.POINTER(ctypes.c_double)]
    lib.jenga_timing_query.restype = i32
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.jenga_status_string(int(status)).decode()


def topk_count(keep_ratio: float, n_blocks: int) -> int:
    return int(lib.jenga_topk_count(ctypes.c_float(keep_ratio), int(n_blocks)))


def timing_enable(enable: bool) -> None:
    """Start (clearing earlier records) or stop per-kernel HIP-event timing in the library."""
    st = lib.jenga_timing_enable(1 if enable else 0)
    if st != JENGA_OK:
        raise JengaError("jenga_timing_enable", st)


def timing_query(kernel: str):
    """(launches, total_ms) recorded for one kernel name since the last timing_enable(True)."""
    n, t = ctypes.c_int32(0), ctypes.c_double(0.0)
    st = lib.jenga_timing_query(kernel.encode(), ctypes.byref(n), ctypes.byref(t))
    if st != JENGA_OK:
        raise JengaError("jenga_timing_query", st)
    return int(n.value), float(t.value)


# ------------------------------------------------------------------------------------------
# torch-facing helpers (torch is imported lazily: the library itself needs no torch)
# ------------------------------------------------------------------------------------------

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return JENGA_DTYPE_BF16
    if t.dtype == torch.float32:
        return JENGA_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dense(name: str, t, shape, dtype=None) -> None:
    """The library indexes this argument as a dense tensor of exactly this shape: refuse views,
    other dtypes and other shapes here, before a pointer reaches a kernel."""
    if t is None:
        raise ValueError(f"{name}: missing")
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _on_device(**ts) -> None:
    """Every tensor argument lives in device memory (checked after shapes and dtypes)."""
    for name, t in ts.items():
        if t is not None and t.numel() and t.device.type != "cuda":
            raise ValueError(f"{name}: must be a device tensor")


def _f32():
    import torch
    return torch.float32


def _i32():
    import torch
    return torch.int32


def _ws_check(workspace) -> None:
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace: must be contiguous")


def make_problem(q, k, v=None, block: int = 64, scale: float = 0.0) -> JengaProblem:
    """Problem descriptor from BSHD tensors (views allowed: strides are passed through)."""
    if q.dim() != 4 or k.dim() != 4 or (v is not None and v.dim() != 4):
        raise ValueError("q, k, v: expected [batch, tokens, heads, head_dim] tensors")
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, S, Hkv, D) or (v is not None and tuple(v.shape) != (B, S, Hkv, D)):
        raise ValueError(f"k, v: shapes {tuple(k.shape)}, {None if v is None else tuple(v.shape)} "
                         f"do not match q {tuple(q.shape)}")
    if k.dtype != q.dtype or (v is not None and v.dtype != q.dtype):
        raise ValueError("q, k, v: must share one dtype")
    p = JengaProblem()
    p.batch, p.seq_len, p.n_heads_q, p.n_heads_kv, p.head_dim, p.block = B, S, Hq, Hkv, D, block
    p.dtype = _dtype_code(q)
    p.scale = float(scale)
    for name, t in (("q_stride", q), ("k_stride", k), ("v_stride", v if v is not None else k)):
        if t.stride(3) != 1:
            raise ValueError(f"{name}: head_dim must be contiguous")
        arr = getattr(p, name)
        arr[0], arr[1], arr[2] = t.stride(0), t.stride(1), t.stride(2)
    return p


def _stream(stream=None) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check(fn: str, st: int):
    if st != JENGA_OK:
        raise JengaError(fn, st)


def workspace_bytes(p: JengaProblem, op: int, max_kept_blocks: int = 0, n_segments: int = 1) -> int:
    return int(lib.jenga_workspace_bytes(ctypes.byref(p), op, max_kept_blocks, n_segments))


def alloc_workspace(nbytes: int, device):
    import torch
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def _nkb(p: JengaProblem) -> int:
    return p.seq_len // p.block if p.block > 0 else 0


def jenga_score_blocks(p: JengaProblem, q, k, block_scores, workspace, stream=None) -> None:
    _dense("block_scores", block_scores, (p.batch, _nkb(p)), _f32())
    _ws_check(workspace)
    _on_device(q=q, k=k, block_scores=block_scores, workspace=workspace)
    st = lib.jenga_score_blocks(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(block_scores),
                                _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream(stream))
    _check("jenga_score_blocks", st)


def jenga_score_blocks_eq2(p: JengaProblem, q, k, block_scores, workspace, stream=None) -> None:
    _dense("block_scores", block_scores, (p.batch, _nkb(p)), _f32())
    _ws_check(workspace)
    _on_device(q=q, k=k, block_scores=block_scores, workspace=workspace)
    st = lib.jenga_score_blocks_eq2(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(block_scores),
                                    _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(stream))
    _check("jenga_score_blocks_eq2", st)


def jenga_select_blocks(p: JengaProblem, block_scores, mode: int, param: float, flags: int,
                        kept_idx, n_kept, stream=None) -> None:
    _dense("block_scores", block_scores, (p.batch, _nkb(p)), _f32())
    _dense("kept_idx", kept_idx, (p.batch, _nkb(p)), _i32())
    _dense("n_kept", n_kept, (p.batch,), _i32())
    _on_device(block_scores=block_scores, kept_idx=kept_idx, n_kept=n_kept)
    st = lib.jenga_select_blocks(ctypes.byref(p), _ptr(block_scores), int(mode),
                                 ctypes.c_float(param), int(flags), _ptr(kept_idx), _ptr(n_kept),
                                 _stream(stream))
    _check("jenga_select_blocks", st)


def jenga_sparse_attn_fwd(p: JengaProblem, q, k, v, kept_idx, n_kept, max_kept_blocks: int,
                          resid, o_saved, lse, workspace=None, stream=None) -> None:
    B, S, Hq, D, Hkv = p.batch, p.seq_len, p.n_heads_q, p.head_dim, p.n_heads_kv
    ncap = int(max_kept_blocks) * p.block
    _dense("kept_idx", kept_idx, (B, _nkb(p)), _i32())
    _dense("n_kept", n_kept, (B,), _i32())
    _dense("resid", resid, (B, S, Hq, D), _f32())
    _dense("o_saved", o_saved, (B, ncap, Hq, D), q.dtype)
    _dense("lse", lse, (B, Hq, ncap), _f32())
    _ws_check(workspace)
    _on_device(q=q, k=k, v=v, kept_idx=kept_idx, n_kept=n_kept, resid=resid, o_saved=o_saved,
               lse=lse, workspace=workspace)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.jenga_sparse_attn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(kept_idx),
                                   _ptr(n_kept), int(max_kept_blocks), _ptr(resid), _ptr(o_saved),
                                   _ptr(lse), _ptr(workspace), nbytes, _stream(stream))
    _check("jenga_sparse_attn_fwd", st)


def jenga_sparse_attn_bwd_segmented(p: JengaProblem, q, k, v, kept_idx, n_kept,
                                    max_kept_blocks: int, o_saved, lse, dout, dq, dk, dv,
                                    n_segments: int, workspace, stream=None) -> None:
    B, S, Hq, D, Hkv = p.batch, p.seq_len, p.n_heads_q, p.head_dim, p.n_heads_kv
    ncap = int(max_kept_blocks) * p.block
    _dense("kept_idx", kept_idx, (B, _nkb(p)), _i32())
    _dense("n_kept", n_kept, (B,), _i32())
    _dense("o_saved", o_saved, (B, ncap, Hq, D), q.dtype)
    _dense("lse", lse, (B, Hq, ncap), _f32())
    _dense("dout", dout, (B, S, Hq, D), _f32())
    _dense("dq", dq, (B, S, Hq, D), _f32())
    _dense("dk", dk, (B, S, Hkv, D), _f32())
    _dense("dv", dv, (B, S, Hkv, D), _f32())
    _ws_check(workspace)
    _on_device(q=q, k=k, v=v, kept_idx=kept_idx, n_kept=n_kept, o_saved=o_saved, lse=lse,
               dout=dout, dq=dq, dk=dk, dv=dv, workspace=workspace)
    st = lib.jenga_sparse_attn_bwd_segmented(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(kept_idx), _ptr(n_kept),
        int(max_kept_blocks), _ptr(o_saved), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
        int(n_segments), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check("jenga_sparse_attn_bwd_segmented", st)


def jenga_sparse_attn_bwd_segmented_noalloc(p: JengaProblem, q, k, v, kept_idx, n_kept,
                                            max_kept_blocks: int, o_saved, lse, dout, dq, dk, dv,
                                            n_segments: int, stream=None) -> None:
    """The segmented backward with the library's fixed per-GPU scratch instead of a workspace
    (no allocation anywhere; calls on one GPU must not overlap)."""
    B, S, Hq, D, Hkv = p.batch, p.seq_len, p.n_heads_q, p.head_dim, p.n_heads_kv
    ncap = int(max_kept_blocks) * p.block
    _dense("kept_idx", kept_idx, (B, _nkb(p)), _i32())
    _dense("n_kept", n_kept, (B,), _i32())
    _dense("o_saved", o_saved, (B, ncap, Hq, D), q.dtype)
    _dense("lse", lse, (B, Hq, ncap), _f32())
    _dense("dout", dout, (B, S, Hq, D), _f32())
    _dense("dq", dq, (B, S, Hq, D), _f32())
    _dense("dk", dk, (B, S, Hkv, D), _f32())
    _dense("dv", dv, (B, S, Hkv, D), _f32())
    _on_device(q=q, k=k, v=v, kept_idx=kept_idx, n_kept=n_kept, o_saved=o_saved, lse=lse,
               dout=dout, dq=dq, dk=dk, dv=dv)
    st = lib.jenga_sparse_attn_bwd_segmented_noalloc(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(kept_idx), _ptr(n_kept),
        int(max_kept_blocks), _ptr(o_saved), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
        int(n_segments), _stream(stream))
    _check("jenga_sparse_attn_bwd_segmented_noalloc", st)


# ------------------------------------------------------------------------------------------
# Convenience layer: allocate outputs with torch and call the entry points above
# ------------------------------------------------------------------------------------------

def score_blocks(q, k, block: int, scale: float = 0.0):
    import torch
    p = make_problem(q, k, None, block, scale)
    out = torch.empty((q.shape[0], q.shape[1] // block), dtype=torch.float32, device=q.device)
    ws = alloc_workspace(workspace_bytes(p, JENGA_OP_SCORE), q.device)
    jenga_score_blocks(p, q, k, out, ws)
    return out


def score_blocks_eq2(q, k, block: int, scale: float = 0.0):
    """Eq. 2 literal block scores (positive head-mean, score-block maximum, sum over m >= n)."""
    import torch
    p = make_problem(q, k, None, block, scale)
    out = torch.empty((q.shape[0], q.shape[1] // block), dtype=torch.float32, device=q.device)
    ws = alloc_workspace(workspace_bytes(p, JENGA_OP_SCORE_EQ2), q.device)
    jenga_score_blocks_eq2(p, q, k, out, ws)
    return out


def select_blocks(scores, block: int, seq_len: int, mode: int, param: float,
                  force_first: bool = False) -> Tuple[object, object]:
    import torch
    B, nkb = scores.shape
    p = JengaProblem()
    p.batch, p.seq_len, p.block = B, seq_len, block
    kept = torch.empty((B, nkb), dtype=torch.int32, device=scores.device)
    n_kept = torch.empty((B,), dtype=torch.int32, device=scores.device)
    jenga_select_blocks(p, scores, mode, param, JENGA_FORCE_FIRST_BLOCK if force_first else 0,
                        kept, n_kept)
    return kept, n_kept


def sparse_attn_fwd(q, k, v, kept_idx, n_kept, max_kept_blocks: int, block: int, resid,
                    scale: float = 0.0):
    """resid is updated in place; returns (o_saved, lse) sized by max_kept_blocks."""
    import torch
    p = make_problem(q, k, v, block, scale)
    B, S, Hq, D = q.shape
    ncap = max_kept_blocks * block
    o_saved = torch.empty((B, ncap, Hq, D), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, Hq, ncap), dtype=torch.float32, device=q.device)
    ws = alloc_workspace(workspace_bytes(p, JENGA_OP_FWD, max_kept_blocks), q.device)
    jenga_sparse_attn_fwd(p, q, k, v, kept_idx, n_kept, max_kept_blocks, resid, o_saved, lse, ws)
    return o_saved, lse


def sparse_attn_bwd(q, k, v, kept_idx, n_kept, max_kept_blocks: int, block: int, o_saved, lse,
                    dout, n_segments: int = 1, scale: float = 0.0, grads=None,
                    min_workspace: bool = False):
    """Returns (dq, dk, dv) fp32; accumulates into `grads` when given.  min_workspace: one set of
    segment buffers (JENGA_OP_BWD_MIN) instead of the two of the faster schedule."""
    import torch
    p = make_problem(q, k, v, block, scale)
    if grads is None:
        dq = torch.zeros(q.shape, dtype=torch.float32, device=q.device)
        dk = torch.zeros(k.shape, dtype=torch.float32, device=q.device)
        dv = torch.zeros(v.shape, dtype=torch.float32, device=q.device)
    else:
        dq, dk, dv = grads
    op = JENGA_OP_BWD_MIN if min_workspace else JENGA_OP_BWD
    ws = alloc_workspace(workspace_bytes(p, op, max_kept_blocks, n_segments), q.device)
    jenga_sparse_attn_bwd_segmented(p, q, k, v, kept_idx, n_kept, max_kept_blocks, o_saved, lse,
                                    dout, dq, dk, dv, n_segments, ws)
    return dq, dk, dv


# ------------------------------------------------------------------------------------------
# permutation-free projections
# ------------------------------------------------------------------------------------------

def make_proj_problem(inp, w, out, block: int, seq_len: int) -> JengaProjProblem:
    """inp: [B, rows, K] bf16 (rows = S for the gathered input, Ncap for compact rows);
    w: [N, K] bf16; out: [B, rows_out, N] (bf16 compact or fp32 residual)."""
    import torch
    if inp.dim() != 3 or out.dim() != 3 or w.dim() != 2:
        raise ValueError("projection: inp [B, rows, K], w [N, K] and out [B, rows, N] expected")
    if inp.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise ValueError("projection: inp and w must be bf16")
    _dense("w", w, (w.shape[0], inp.shape[2]), torch.bfloat16)
    if out.shape[0] != inp.shape[0] or out.shape[2] != w.shape[0]:
        raise ValueError(f"projection: out {tuple(out.shape)} does not match inp {tuple(inp.shape)} "
                         f"and w {tuple(w.shape)}")
    if inp.stride(2) != 1 or out.stride(2) != 1:
        raise ValueError("projection: the feature dimension of inp and out must be contiguous")
    p = JengaProjProblem()
    p.batch, p.seq_len, p.block = inp.shape[0], int(seq_len), int(block)
    p.in_features, p.out_features = inp.shape[2], w.shape[0]
    p.in_stride[0], p.in_stride[1] = inp.stride(0), inp.stride(1)
    p.out_stride[0], p.out_stride[1] = out.stride(0), out.stride(1)
    return p


def proj_gather(x, w, kept_idx, n_kept, max_kept_blocks: int, block: int, stream=None):
    """y[b, r] = x[b, pos(r)] @ w^T over the kept ranks (compact bf16 [B, Ncap, N])."""
    import torch
    B, S, _ = x.shape
    y = torch.empty((B, max_kept_blocks * block, w.shape[0]), dtype=torch.bfloat16, device=x.device)
    p = make_proj_problem(x, w, y, block, S)
    _kept_check(kept_idx, n_kept, B, S // block)
    st = lib.jenga_proj_gather(ctypes.byref(p), _ptr(x), _ptr(w), _ptr(kept_idx), _ptr(n_kept),
                               int(max_kept_blocks), _ptr(y), _stream(stream))
    _check("jenga_proj_gather", st)
    return y


def _kept_check(kept_idx, n_kept, B: int, nkb: int) -> None:
    _dense("kept_idx", kept_idx, (B, nkb), _i32())
    _dense("n_kept", n_kept, (B,), _i32())
    _on_device(kept_idx=kept_idx, n_kept=n_kept)


def proj_scatter_add(y, w, kept_idx, n_kept, max_kept_blocks: int, block: int, resid,
                     stream=None) -> None:
    """resid[b, pos(r)] += y[b, r] @ w^T at the kept rows (resid fp32 [B, S, N], in place)."""
    if resid.dtype != _f32():
        raise ValueError("resid: must be float32")
    p = make_proj_problem(y, w, resid, block, resid.shape[1])
    _kept_check(kept_idx, n_kept, p.batch, resid.shape[1] // block)
    if y.shape[1] < max_kept_blocks * block:
        raise ValueError("y: fewer rows than max_kept_blocks * block")
    st = lib.jenga_proj_scatter_add(ctypes.byref(p), _ptr(y), _ptr(w), _ptr(kept_idx), _ptr(n_kept),
                                    int(max_kept_blocks), _ptr(resid), _stream(stream))
    _check("jenga_proj_scatter_add", st)


def proj_gather_scatter_add(a, w, kept_idx, n_kept, max_kept_blocks: int, block: int, resid,
                            stream=None) -> None:
    """resid[b, pos(r)] += a[b, pos(r)] @ w^T at the kept rows (a bf16 [B, S, K] full rows,
    resid fp32 [B, S, N], in place)."""
    if resid.dtype != _f32():
        raise ValueError("resid: must be float32")
    p = make_proj_problem(a, w, resid, block, resid.shape[1])
    _kept_check(kept_idx, n_kept, p.batch, resid.shape[1] // block)
    if a.shape[1] != resid.shape[1]:
        raise ValueError("a: one row per token of resid expected")
    st = lib.jenga_proj_gather_scatter_add(ctypes.byref(p), _ptr(a), _ptr(w), _ptr(kept_idx),
                                           _ptr(n_kept), int(max_kept_blocks), _ptr(resid),
                                           _stream(stream))
    _check("jenga_proj_gather_scatter_add", st)


# ------------------------------------------------------------------------------------------
# token elimination in the MLP block
# ------------------------------------------------------------------------------------------

def mlp_workspace_bytes(p: JengaProjProblem, kind: int) -> int:
    return int(lib.jenga_mlp_workspace_bytes(ctypes.byref(p), int(kind)))


def mlp_act_scores(x, w1, w_up, kind: int, block: int, workspace=None, stream=None):
    """(act bf16 [B, S, F], token_scores fp32 [B, S], block_scores fp32 [B, S / block]).
    x bf16 [B, S, K]; w1 (gate or first layer) and w_up bf16 [F, K] (w_up None for ReLU)."""
    import torch
    B, S, _ = x.shape
    F = w1.shape[0]
    if w_up is not None:
        _dense("w_up", w_up, tuple(w1.shape), torch.bfloat16)
    _ws_check(workspace)
    act = torch.empty((B, S, F), dtype=torch.bfloat16, device=x.device)
    tok = torch.empty((B, S), dtype=torch.float32, device=x.device)
    blk = torch.empty((B, S // block), dtype=torch.float32, device=x.device)
    p = make_proj_problem(x, w1, act, block, S)
    ws = workspace if workspace is not None else alloc_workspace(mlp_workspace_bytes(p, kind), x.device)
    st = lib.jenga_mlp_act_scores(ctypes.byref(p), int(kind), _ptr(x), _ptr(w1),
                                  _ptr(w_up) if w_up is not None else None, _ptr(act), _ptr(tok),
                                  _ptr(blk), _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(stream))
    _check("jenga_mlp_act_scores", st)
    return act, tok, blk


def sparse_mlp_forward(x, w1, w_up, w_down, resid, block: int, mode: int, param: float,
                       kind: int = JENGA_MLP_SILU_GATED, workspace=None):
    """One MLP block with token elimination: activation and scores for every token, block
    selection, then the down projection of the kept tokens added into resid (fp32, in place).
    Returns (block_scores, kept_idx, n_kept, max_kept_blocks)."""
    act, _, blk = mlp_act_scores(x, w1, w_up, kind, block, workspace)
    nkb = blk.shape[1]
    kept, n_kept = select_blocks(blk, block, x.shape[1], mode, param)
    mkb = topk_count(param, nkb) if mode == JENGA_SELECT_TOPK else nkb
    proj_gather_scatter_add(act, w_down, kept, n_kept, mkb, block, resid)
    return blk, kept, n_kept, mkb


# ------------------------------------------------------------------------------------------
# segmented language-model-head loss
# ------------------------------------------------------------------------------------------

def loss_problem(tokens: int, d_model: int, vocab: int, n_segments: int) -> JengaLossProblem:
    p = JengaLossProblem()
    p.tokens, p.d_model, p.vocab, p.n_segments = tokens, d_model, vocab, n_segments
    return p


def loss_workspace_bytes(p: JengaLossProblem) -> int:
    return int(lib.jenga_loss_workspace_bytes(ctypes.byref(p)))


def lm_head_ce(h, w, wt, targets, n_segments: int = 1, workspace=None, stream=None):
    """(loss [1] fp32, row_loss [T] fp32, dh [T, d] fp32) of the head logits h w^T, computed
    n_segments rows-segments at a time.  wt is w transposed ([d, V], contiguous)."""
    import torch
    T, d = h.shape
    V = w.shape[0]
    _dense("h", h, (T, d), torch.bfloat16)
    _dense("w", w, (V, d), torch.bfloat16)
    _dense("wt", wt, (d, V), torch.bfloat16)
    _dense("targets", targets, (T,), torch.int32)
    _ws_check(workspace)
    _on_device(h=h, w=w, wt=wt, targets=targets, workspace=workspace)
    p = loss_problem(T, d, V, n_segments)
    ws = workspace if workspace is not None else alloc_workspace(loss_workspace_bytes(p), h.device)
    row_loss = torch.empty((T,), dtype=torch.float32, device=h.device)
    loss = torch.empty((1,), dtype=torch.float32, device=h.device)
    dh = torch.empty((T, d), dtype=torch.float32, device=h.device)
    st = lib.jenga_lm_head_ce_segmented(ctypes.byref(p), _ptr(h), _ptr(w), _ptr(wt), _ptr(targets),
                                        _ptr(row_loss), _ptr(loss), _ptr(dh), _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream(stream))
    _check("jenga_lm_head_ce_segmented", st)
    return loss, row_loss, dh
