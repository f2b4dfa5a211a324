"""The hot path on a stream of the caller's choosing, and replayed from a HIP graph.

Every entry point launches its kernels on the stream it is given and makes no allocation,
memset or synchronising call of its own (the backward without a workspace looks up its scratch
array once per device, on its first call).  So the path runs on any stream and can be captured
in a graph.  bf16 results come from a fixed schedule, so the checks are bitwise:
- score -> select -> forward -> backward on a side stream gives the bits it gives on the current
  stream;
- a graph captured from the same four calls (outputs spoiled and accumulators reset by eager
  work between replays) reproduces the eager results on every replay, and so does a graph of
  the backward entry point that allocates nothing, and one whose backward runs long dK/dV key
  tiles in parts and whose forward runs long query tiles in parts (its graph also holds the
  launches that add and merge the parts).
"""
import numpy as np
import pytest

from gpu_helpers import random_inputs, say, to_device

pytestmark = pytest.mark.gpu

B, S, HQ, HKV, D, BLOCK, KEEP, NSEG = 2, 2048, 8, 2, 128, 64, 0.5, 3
# one segment of a longer grouped-query problem: its first dK/dV key tiles run in parts, so the
# captured backward also holds the launch that adds the parts' sums
SPLIT_SHAPE = dict(B=1, S=8192, HQ=8, HKV=2, KEEP=0.3125, NSEG=1)


@pytest.fixture(scope="module")
def J():
    import torch
    assert torch.cuda.is_available()
    import token_sparse_attention_jenga_amd as J
    return J


class Path:
    """Inputs, preallocated outputs and workspaces of one score/select/fwd/bwd pass."""

    def __init__(self, J, seed, B=B, S=S, HQ=HQ, HKV=HKV, KEEP=KEEP, NSEG=NSEG):
        import torch
        self.KEEP, self.NSEG = KEEP, NSEG
        q, k, v, x0, dout = random_inputs(B, S, HQ, HKV, D, "bf16", seed=seed)
        self.q, self.k, self.v = (to_device(a, "bf16") for a in (q, k, v))
        self.x0 = torch.from_numpy(x0).cuda()
        self.dout = torch.from_numpy(dout).cuda()
        self.p = J.make_problem(self.q, self.k, self.v, BLOCK)
        nkb = S // BLOCK
        self.mk = J.topk_count(KEEP, nkb)
        ncap = self.mk * BLOCK
        dev = self.q.device
        self.scores = torch.empty((B, nkb), dtype=torch.float32, device=dev)
        self.kept = torch.empty((B, nkb), dtype=torch.int32, device=dev)
        self.n_kept = torch.empty((B,), dtype=torch.int32, device=dev)
        self.resid = self.x0.clone()
        self.o_saved = torch.empty((B, ncap, HQ, D), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B, HQ, ncap), dtype=torch.float32, device=dev)
        self.dq = torch.zeros((B, S, HQ, D), dtype=torch.float32, device=dev)
        self.dk = torch.zeros((B, S, HKV, D), dtype=torch.float32, device=dev)
        self.dv = torch.zeros((B, S, HKV, D), dtype=torch.float32, device=dev)
        self.ws_score = J.alloc_workspace(J.workspace_bytes(self.p, J.JENGA_OP_SCORE), dev)
        self.ws_fwd = J.alloc_workspace(J.workspace_bytes(self.p, J.JENGA_OP_FWD, self.mk), dev)
        self.ws_bwd = J.alloc_workspace(J.workspace_bytes(self.p, J.JENGA_OP_BWD, self.mk, NSEG), dev)

    def reset(self):
        """Eager work between runs: spoil every output, restore the accumulated ones."""
        self.scores.fill_(float("nan"))
        self.kept.fill_(-7)
        self.n_kept.fill_(-7)
        self.o_saved.fill_(float("nan"))
        self.lse.fill_(float("nan"))
        self.resid.copy_(self.x0)
        self.dq.zero_()
        self.dk.zero_()
        self.dv.zero_()

    def forward_path(self, J, stream=None):
        J.jenga_score_blocks(self.p, self.q, self.k, self.scores, self.ws_score, stream)
        J.jenga_select_blocks(self.p, self.scores, J.JENGA_SELECT_TOPK, self.KEEP, 0, self.kept,
                              self.n_kept, stream)
        J.jenga_sparse_attn_fwd(self.p, self.q, self.k, self.v, self.kept, self.n_kept, self.mk,
                                self.resid, self.o_saved, self.lse, self.ws_fwd, stream)

    def backward(self, J, stream=None, noalloc=False):
        args = (self.p, self.q, self.k, self.v, self.kept, self.n_kept, self.mk, self.o_saved,
                self.lse, self.dout, self.dq, self.dk, self.dv, self.NSEG)
        if noalloc:
            J.jenga_sparse_attn_bwd_segmented_noalloc(*args, stream=stream)
        else:
            J.jenga_sparse_attn_bwd_segmented(*args, self.ws_bwd, stream)

    def outputs(self):
        return [t.clone() for t in (self.scores, self.kept, self.n_kept, self.resid, self.o_saved,
                                    self.lse, self.dq, self.dk, self.dv)]


NAMES = ("scores", "kept", "n_kept", "resid", "o_saved", "lse", "dq", "dk", "dv")


def _same(got, ref, what):
    import torch
    for name, a, b in zip(NAMES, got, ref):
        assert torch.equal(a, b), f"{what}: {name} differs"


def test_path_on_side_stream(J):
    import torch
    path = Path(J, seed=404)
    say(f"path on the current stream: B{B} S{S} Hq{HQ} Hkv{HKV} D{D} block{BLOCK} keep {KEEP}")
    path.reset()
    path.forward_path(J)
    path.backward(J)
    torch.cuda.synchronize()
    ref = path.outputs()
    assert int(ref[2].min()) == path.mk and bool(torch.isfinite(ref[6]).all())

    side = torch.cuda.Stream()
    say("path on a side stream")
    path.reset()
    side.wait_stream(torch.cuda.current_stream())       # the resets above run on the current one
    with torch.cuda.stream(side):
        path.forward_path(J, side)
        path.backward(J, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    _same(path.outputs(), ref, "side stream")


@pytest.mark.parametrize("noalloc,shape", [(False, None), (True, None), (False, "split")])
def test_graph_replays_match_eager(J, noalloc, shape):
    import torch
    path = Path(J, seed=505) if shape is None else Path(J, seed=606, **SPLIT_SHAPE)
    if shape == "split":
        # one segment of 2560 kept tokens, four query heads per KV head: the first key tiles
        # run 320 steps, more than the launch's load per compute unit, so they run in parts
        # and the workspace holds slots beyond the one set of segment buffers
        L = path.mk * BLOCK
        one_set = 2 * SPLIT_SHAPE["B"] * SPLIT_SHAPE["HQ"] * L * 4 + 3 * SPLIT_SHAPE["B"] * SPLIT_SHAPE["HQ"] * L * D * 2
        assert J.workspace_bytes(path.p, J.JENGA_OP_BWD_MIN, path.mk, 1) > one_set
    say(f"eager path (backward {'without' if noalloc else 'with'} a workspace)")
    path.reset()
    path.forward_path(J)
    path.backward(J, noalloc=noalloc)          # also places the scratch array before capture
    torch.cuda.synchronize()
    ref = path.outputs()

    say("capturing the path in a graph")
    path.reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        path.forward_path(J)
        path.backward(J, noalloc=noalloc)
    torch.cuda.synchronize()
    for rep in range(3):
        say(f"graph replay {rep}")
        path.reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(path.outputs(), ref, f"replay {rep}")
        # eager work of the program's own between replays
        path.forward_path(J)
        torch.cuda.synchronize()
    del g
