"""CPU oracle for the Jenga token-sparse attention hot path.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the cpu_baseline
leg of bench.py may import or run anything in this package; the library and its Python
binding never do.  It shares no code, tables or helpers with the HIP path.

Plain float64 NumPy written from the definitions on the pages, without blocking or
fusion beyond what the definitions state (query rows are processed in chunks only to
bound host memory; every row's softmax is complete inside its chunk).  Inputs are the
stored values (bf16 inputs arrive as the float32 values of their bits) upcast exactly.

Page keys used in the citations below:
  [summary] "JENGA: Enhancing LLM Long-Context Fine-tuning with Contextual Token Sparsity",
            the aipaper.cc structured summary of the ATC'25 paper.
  [notes]   "Jenga: Enhancing LLM Long-Context Fine-tuning with Contextual Token Sparsity",
            the papercache.org deep-notes page on the same paper.

Readings taken where the pages leave a step open:
  * score = received attention-probability mass: for every key token j, the sum over
    queries i != j of the causal softmax probability P_ij ([summary] 4.2.1 Eq. 1 sums the
    interaction a token *receives* from all other tokens, self excluded), summed over the
    b tokens of a key block and over the query heads, divided by the number of query heads
    ([summary] 4.2.2 Eq. 2 scales by N_head; 4.2.3 aggregates score blocks over the
    query-block index for each key block).
  * softmax scale 1/sqrt(d_head) ([summary] 3.1 attention formula); causal mask.
  * keep iff score >= threshold ([notes] 4.2, layer-specific threshold; Algorithm 1 step 1
    initialises the threshold from the average block score); top-k keeps
    ceil(r * nKB - 1e-6) blocks, clamped to [1, nKB]; ties go to the lower block index;
    NaN scores are never kept and sort last.
  * eliminated tokens take no part in the layer, neither as queries nor as keys
    ([notes] 4.4 permutation-free token movement: kept tokens are the attention input,
    the output is zero-padded and added to the residual).
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

SELECT_TOPK = 0
SELECT_THRESH_REL = 1
SELECT_THRESH_ABS = 2

_ROW_CHUNK = 512


def default_scale(head_dim: int) -> float:
    """1/sqrt(d_k) of the scaled dot-product attention formula ([summary] 3.1)."""
    return 1.0 / math.sqrt(head_dim)


def kv_head_of(h: int, n_heads_q: int, n_heads_kv: int) -> int:
    """Grouped-query attention: query head h reads KV head floor(h / (Hq/Hkv))."""
    return h // (n_heads_q // n_heads_kv)


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def token_positions(kept_blocks: Sequence[int], block: int) -> np.ndarray:
    """Original token positions of the kept blocks, in ascending kept-rank order."""
    kb = np.asarray(kept_blocks, dtype=np.int64)
    return (kb[:, None] * block + np.arange(block, dtype=np.int64)[None, :]).reshape(-1)


# ----------------------------------------------------------------------------------------
# Scoring: per-key-block received probability mass ([summary] 4.2.1 Eq. 1, 4.2.2, 4.2.3)
# ----------------------------------------------------------------------------------------

def _causal_probs(q_rows: np.ndarray, k_keys: np.ndarray, row_pos: np.ndarray, scale: float):
    """Causal softmax rows: P[r, j] over keys j <= row_pos[r]; returns (P, LSE)."""
    z = scale * (q_rows @ k_keys.T)
    z[np.arange(k_keys.shape[0])[None, :] > row_pos[:, None]] = -np.inf
    zmax = z.max(axis=1, keepdims=True)
    e = np.exp(z - zmax)
    ssum = e.sum(axis=1, keepdims=True)
    return e / ssum, zmax[:, 0] + np.log(ssum[:, 0])


def received_mass(q_h: np.ndarray, k_g: np.ndarray, scale: float) -> np.ndarray:
    """M(j) = sum_{i != j} P_ij for one head, with P the causal softmax over all S tokens.

    Eq. 1 of [summary] 4.2.1 sums over every token i except j itself; with a causal
    softmax P_ij = 0 for i < j, so only later queries contribute.
    """
    S = q_h.shape[0]
    M = np.zeros(S)
    for i0 in range(0, S, _ROW_CHUNK):
        i1 = min(S, i0 + _ROW_CHUNK)
        rows = np.arange(i0, i1)
        P, _ = _causal_probs(q_h[i0:i1], k_g[:i1], rows, scale)
        P[np.arange(i1 - i0), rows] = 0.0          # self term excluded (i != j)
        M[:i1] += P.sum(axis=0)
    return M


def block_scores(q, k, block: int, scale: float = None) -> np.ndarray:
    """Token-block scores s[b, n] = (1/Hq) * sum_h sum_{j in block n} M_h(j).

    q: [B,S,Hq,D], k: [B,S,Hkv,D].  Returns float64 [B, S/block].
    Head mean as in Eq. 2 ([summary] 4.2.2, division by N_head); the per-key-block
    aggregation over all query blocks as in [summary] 4.2.3 (B^T_n = sum_m B^S_mn).
    """
    q, k = _f64(q), _f64(k)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if scale is None:
        scale = default_scale(D)
    nkb = S // block
    out = np.zeros((B, nkb))
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            M = received_mass(q[b, :, h, :], k[b, :, g, :], scale)
            out[b] += M.reshape(nkb, block).sum(axis=1)
        out[b] /= Hq
    return out


# ----------------------------------------------------------------------------------------
# Eq. 2 literal scoring ([summary] 4.2.2 Eq. 2, 4.2.3): informativeness of a score block is the
# maximum, over its elements, of the head-averaged *positive* attention scores; a key block's
# score sums its score blocks over the query blocks.
# ----------------------------------------------------------------------------------------

def eq2_tile_max(q, k, block: int, b: int, m: int, n: int, scale: float = None) -> float:
    """I(B^S) of the score block with query block m and key block n (m >= n) of batch row b.

    Per element (i, j): e_ij = (1/Hq) * sum over heads of max(scale * q_i . k_j, 0) -- only
    positive scores enter the head aggregation -- then the maximum over the block's elements
    with j <= i (causal; on the diagonal block the masked upper triangle does not take part).
    """
    q, k = _f64(q), _f64(k)
    _, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if scale is None:
        scale = default_scale(D)
    qi = np.arange(m * block, (m + 1) * block)
    kj = np.arange(n * block, (n + 1) * block)
    e = np.zeros((block, block))
    for h in range(Hq):
        g = kv_head_of(h, Hq, Hkv)
        sc = scale * (q[b, qi, h, :] @ k[b, kj, g, :].T)
        e += np.maximum(sc, 0.0)
    e /= Hq
    allowed = kj[None, :] <= qi[:, None]
    return float(e[allowed].max())


def block_scores_eq2(q, k, block: int, scale: float = None, key_blocks=None) -> np.ndarray:
    """s[b, n] = sum over query blocks m >= n of eq2_tile_max(m, n)  ([summary] 4.2.3: the
    token-block score aggregates its score blocks; the causal mask leaves only m >= n).
    key_blocks restricts the computation to those n (other entries are NaN)."""
    B, S = q.shape[0], q.shape[1]
    nkb = S // block
    ns = range(nkb) if key_blocks is None else key_blocks
    out = np.full((B, nkb), np.nan)
    for b in range(B):
        for n in ns:
            out[b, n] = sum(eq2_tile_max(q, k, block, b, m, n, scale) for m in range(n, nkb))
    return out


# ----------------------------------------------------------------------------------------
# Permutation-free token movement around the projections ([notes] 4.4; [summary] 4.4.1):
# the input projection reads only the kept rows of the hidden states, and the output
# projection's result is added into the residual stream at the kept rows only.
# ----------------------------------------------------------------------------------------

def proj_gather(x, w, kept, block: int) -> np.ndarray:
    """y[b, r] = x[b, pos(r)] @ w^T for the kept ranks r of each batch row (compact output).

    x: [B, S, K]; w: [N, K] (a linear layer's weight, out_features x in_features).
    Returns float64 [B, max_r, N]; rows past a batch row's own kept count stay 0."""
    x, w = _f64(x), _f64(w)
    B = x.shape[0]
    keptb = _per_batch(kept, B)
    nmax = max(len(kb) for kb in keptb) * block
    y = np.zeros((B, nmax, w.shape[0]))
    for b in range(B):
        pos = token_positions(keptb[b], block)
        if len(pos):
            y[b, :len(pos)] = x[b, pos] @ w.T
    return y


def proj_scatter_add(resid, y, w, kept, block: int) -> np.ndarray:
    """resid[b, pos(r)] + y[b, r] @ w^T at the kept positions; every other row unchanged.

    resid: [B, S, N]; y: [B, >= Nk, K] compact by kept rank; w: [N, K]."""
    out = _f64(resid).copy()
    y, w = _f64(y), _f64(w)
    keptb = _per_batch(kept, out.shape[0])
    for b in range(out.shape[0]):
        pos = token_positions(keptb[b], block)
        if len(pos):
            out[b, pos] += y[b, :len(pos)] @ w.T
    return out


# ----------------------------------------------------------------------------------------
# Loss of the language-model head, the step that segment-based peak cutting targets
# ([summary] 4.4.2; [notes] 4.4): cross-entropy of softmax(h W^T) against the next tokens.
# ----------------------------------------------------------------------------------------

def lm_head_ce(h, w, targets, with_logit_grad: bool = False):
    """Mean cross-entropy over the T rows of h and its gradient with respect to h.

    h: [T, d]; w: [V, d] (the head's weight); targets: [T] ints in [0, V).
    logits = h w^T; row_loss_t = logsumexp(logits_t) - logits_t[target_t];
    loss = mean_t row_loss_t; dh = g w with the logit gradient g = (softmax(logits) -
    onehot(targets)) / T.
    Returns (loss, row_loss [T], dh [T, d]) in float64, and g [T, V] when with_logit_grad."""
    h, w = _f64(h), _f64(w)
    T = h.shape[0]
    logits = h @ w.T
    mx = logits.max(axis=1, keepdims=True)
    lse = (mx + np.log(np.exp(logits - mx).sum(axis=1, keepdims=True)))[:, 0]
    t = np.asarray(targets, dtype=np.int64)
    row_loss = lse - logits[np.arange(T), t]
    g = np.exp(logits - lse[:, None])
    g[np.arange(T), t] -= 1.0
    g /= T
    dh = g @ w
    if with_logit_grad:
        return float(row_loss.mean()), row_loss, dh, g
    return float(row_loss.mean()), row_loss, dh


# ----------------------------------------------------------------------------------------
# Token elimination in the MLP block ([summary] 4.2.4; [notes] 4.2 "extend to MLP block"):
# a token's informativeness comes from the block's intermediate activation -- the ReLU
# output for ReLU MLPs, SiLU(gate) * up for gated SiLU MLPs.  Readings: a token's score is
# the mean activation magnitude over the F intermediate units (the units stand where the
# heads stand in Eq. 2; for ReLU every activation is >= 0, so this is Eq. 2's positive-part
# mean); a token block's score is the maximum over its tokens (Eq. 2's block maximum); the
# kept blocks then run the down projection, added into the residual in place.
# ----------------------------------------------------------------------------------------

MLP_RELU = 0
MLP_SILU_GATED = 1


def mlp_activation(x, w1, w_up=None, kind: int = MLP_SILU_GATED) -> np.ndarray:
    """Intermediate activation of an MLP block.

    x: [..., K]; w1: [F, K] (ReLU MLPs: the first linear layer; gated MLPs: the gate
    projection); w_up: [F, K], the up projection of gated MLPs (unused for ReLU).
    ReLU:       a = max(x w1^T, 0)
    SiLU gated: a = silu(x w1^T) * (x w_up^T), silu(z) = z / (1 + exp(-z))."""
    x, w1 = _f64(x), _f64(w1)
    z = x @ w1.T
    if kind == MLP_RELU:
        return np.maximum(z, 0.0)
    u = x @ _f64(w_up).T
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z)) * u


def mlp_token_scores(act) -> np.ndarray:
    """Per-token informativeness: mean over the F units of |a| (last axis)."""
    act = _f64(act)
    return np.abs(act).sum(axis=-1) / act.shape[-1]


def mlp_block_scores(act, block: int) -> np.ndarray:
    """Per-token-block informativeness: the maximum token score in each block of b tokens.

    act: [B, S, F] -> [B, S / b]."""
    e = mlp_token_scores(act)
    B, S = e.shape
    return e.reshape(B, S // block, block).max(axis=2)


def proj_gather_scatter_add(resid, a, w, kept, block: int) -> np.ndarray:
    """resid[b, pos(r)] + a[b, pos(r)] @ w^T at the kept positions; every other row unchanged.

    resid: [B, S, N]; a: [B, S, K] (full rows, read only where kept); w: [N, K]."""
    out = _f64(resid).copy()
    a, w = _f64(a), _f64(w)
    keptb = _per_batch(kept, out.shape[0])
    for b in range(out.shape[0]):
        pos = token_positions(keptb[b], block)
        if len(pos):
            out[b, pos] += a[b, pos] @ w.T
    return out


def mlp_sparse_forward(x, w1, w_up, w_down, resid, block: int, mode: int, param,
                       kind: int = MLP_SILU_GATED, act_round=None):
    """One MLP block with token elimination: activation for every token, block scores,
    selection (the same rule as for attention), then the down projection of the kept
    tokens only, added into the residual in place.

    act_round: optional function applied to the activation before the down projection
    (the stored precision of the activation, e.g. a bf16 rounding); the scores always come
    from the unrounded activation.  Returns (resid_out, block_scores, kept per batch row)."""
    act = mlp_activation(x, w1, w_up, kind)
    sc = mlp_block_scores(act, block)
    kept = [select_blocks(sc[b].astype(np.float32), mode, param) for b in range(sc.shape[0])]
    a_down = act if act_round is None else _f64(act_round(act))
    return proj_gather_scatter_add(resid, a_down, w_down, kept, block), sc, kept


# ----------------------------------------------------------------------------------------
# Selection ([notes] 4.2 layer-specific threshold, Algorithm 1 step 1; top-k by keep ratio)
# ----------------------------------------------------------------------------------------

def keep_count(keep_ratio, n_blocks: int) -> int:
    """Number of blocks kept by top-k: ceil(r * nKB - 1e-6), clamped to [1, nKB].

    r is the float32 value the caller passes, widened to double.
    """
    r = float(np.float32(keep_ratio))
    k = math.ceil(r * n_blocks - 1e-6)
    return int(min(n_blocks, max(1, k)))


def threshold_value(scores_f32, mode: int, param) -> float:
    """The layer threshold T in double precision.

    THRESH_REL: T = alpha * mean(scores), the mean summed left to right in double
    ([notes] Algorithm 1 step 1 initialises T_i to the average token-block score).
    THRESH_ABS: T = param.
    """
    x = [float(v) for v in np.asarray(scores_f32, dtype=np.float32)]
    p = float(np.float32(param))
    if mode == SELECT_THRESH_ABS:
        return p
    total = 0.0
    for val in x:
        total += val
    mean = total / len(x)
    return p * mean


def select_blocks(scores_f32, mode: int, param, force_first: bool = False) -> np.ndarray:
    """Kept block indices (ascending int32) for one batch row of fp32 block scores.

    TOPK: the keep_count(param) best blocks under the order (score descending, index
    ascending), NaN last; with force_first block 0 plus the best keep_count-1 others.
    THRESH_*: every block whose score (as double) is >= T; NaN never kept; with
    force_first block 0 is added.
    """
    x = [float(v) for v in np.asarray(scores_f32, dtype=np.float32)]
    n = len(x)
    if mode == SELECT_TOPK:
        kcount = keep_count(param, n)

        def key(m):
            if math.isnan(x[m]):
                return (1, 0.0, m)
            return (0, -x[m], m)

        cand = list(range(1, n)) if force_first else list(range(n))
        order = sorted(cand, key=key)
        kept = ([0] + order[:kcount - 1]) if force_first else order[:kcount]
    elif mode in (SELECT_THRESH_REL, SELECT_THRESH_ABS):
        T = threshold_value(x, mode, param)
        kept = [m for m in range(n) if x[m] >= T]     # NaN >= T is False
        if force_first and 0 not in kept:
            kept = [0] + kept
    else:
        raise ValueError(f"unknown selection mode {mode}")
    return np.asarray(sorted(kept), dtype=np.int32)


# ----------------------------------------------------------------------------------------
# Token-sparse causal attention ([notes] 4.4 permutation-free token movement;
# [summary] 3.1 attention formula)
# ----------------------------------------------------------------------------------------

def _masked_attention(qh, kh, vh, allowed, scale):
    """O_i = sum_j softmax_{allowed j}(scale q_i.k_j) v_j; rows with no allowed key give
    O_i = 0 and LSE_i = -inf.  Returns (O, LSE, P)."""
    z = scale * (qh @ kh.T)
    z = np.where(allowed, z, -np.inf)
    has = allowed.any(axis=1)
    zmax = np.where(has, np.max(np.where(allowed, z, -np.inf), axis=1, initial=-np.inf), 0.0)
    e = np.where(allowed, np.exp(z - zmax[:, None]), 0.0)
    ssum = e.sum(axis=1)
    P = np.where(has[:, None], e / np.where(has, ssum, 1.0)[:, None], 0.0)
    O = P @ vh
    lse = np.where(has, zmax + np.log(np.where(has, ssum, 1.0)), -np.inf)
    return O, lse, P


def _masked_attention_bwd(qh, kh, vh, allowed, scale, do):
    """Softmax-attention backward for one head under an explicit mask.

    D_i = dO_i . O_i;  dP = dO V^T;  dS = P * (dP - D);  dQ = scale dS K;
    dK = scale dS^T Q;  dV = P^T dO.
    """
    O, _, P = _masked_attention(qh, kh, vh, allowed, scale)
    Dv = (do * O).sum(axis=1)
    dP = do @ vh.T
    dS = P * (dP - Dv[:, None])
    return scale * (dS @ kh), scale * (dS.T @ qh), P.T @ do


def _kept_token_mask(S: int, kept_blocks, block: int) -> np.ndarray:
    m = np.zeros(S, dtype=bool)
    m[token_positions(kept_blocks, block)] = True
    return m


def _per_batch(kept, B):
    if isinstance(kept, np.ndarray) and kept.ndim == 1:
        return [kept] * B
    if isinstance(kept, (list, tuple)) and len(kept) and np.ndim(kept[0]) == 0:
        return [np.asarray(kept)] * B
    return [np.asarray(x) for x in kept]


def attn_fwd_masked(q, k, v, kept, block: int, scale: float = None):
    """Explicit-mask definition over all S tokens.

    mask_ij = [i kept] and [j kept] and [j <= i].  Returns O [B,S,Hq,D] (zero at
    eliminated rows) and LSE [B,Hq,S] (natural log, -inf at eliminated rows).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if scale is None:
        scale = default_scale(D)
    keptb = _per_batch(kept, B)
    O = np.zeros((B, S, Hq, D))
    LSE = np.full((B, Hq, S), -np.inf)
    causal = np.tril(np.ones((S, S), dtype=bool))
    for b in range(B):
        tm = _kept_token_mask(S, keptb[b], block)
        allowed = causal & tm[:, None] & tm[None, :]
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            o, lse, _ = _masked_attention(q[b, :, h], k[b, :, g], v[b, :, g], allowed, scale)
            O[b, :, h] = o
            LSE[b, h] = lse
    return O, LSE


def attn_fwd_compact(q, k, v, kept, block: int, scale: float = None):
    """Gather kept tokens -> dense causal attention over the Nk kept tokens -> scatter.

    The naive token movement of [notes] 4.4 (Fig. 9): same result as attn_fwd_masked.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if scale is None:
        scale = default_scale(D)
    keptb = _per_batch(kept, B)
    O = np.zeros((B, S, Hq, D))
    LSE = np.full((B, Hq, S), -np.inf)
    for b in range(B):
        pos = token_positions(keptb[b], block)
        nk = len(pos)
        if nk == 0:
            continue
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            Qc, Kc, Vc = q[b, pos, h], k[b, pos, g], v[b, pos, g]
            for r0 in range(0, nk, _ROW_CHUNK):
                r1 = min(nk, r0 + _ROW_CHUNK)
                allowed = np.arange(r1)[None, :] <= np.arange(r0, r1)[:, None]
                o, lse, _ = _masked_attention(Qc[r0:r1], Kc[:r1], Vc[:r1], allowed, scale)
                O[b, pos[r0:r1], h] = o
                LSE[b, h, pos[r0:r1]] = lse
    return O, LSE


def attn_fwd(q, k, v, kept, block: int, scale: float = None):
    """Token-sparse attention output; explicit-mask form up to S=2048, compact above."""
    if np.shape(q)[1] <= 2048:
        return attn_fwd_masked(q, k, v, kept, block, scale)
    return attn_fwd_compact(q, k, v, kept, block, scale)


def residual_add(resid, O, kept, block: int) -> np.ndarray:
    """In-place residual semantics ([notes] 4.4): resid[t] + O_t at kept tokens,
    resid[t] untouched elsewhere.  Returns a float64 copy."""
    out = _f64(resid).copy()
    B = out.shape[0]
    for b, kb in enumerate(_per_batch(kept, B)):
        pos = token_positions(kb, block)
        out[b, pos] += O[b, pos]
    return out


def attn_bwd_masked(q, k, v, kept, block: int, dout, scale: float = None):
    """Gradients of L = <dout, O> under the explicit mask.

    Returns dq [B,S,Hq,D], dk and dv [B,S,Hkv,D] (float64, zero at eliminated tokens;
    GQA sums the gradients of the query heads that share a KV head).  The selection is
    a constant input: no gradient flows through it.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if scale is None:
        scale = default_scale(D)
    keptb = _per_batch(kept, B)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    causal = np.tril(np.ones((S, S), dtype=bool))
    for b in range(B):
        tm = _kept_token_mask(S, keptb[b], block)
        allowed = causal & tm[:, None] & tm[None, :]
        do_b = np.where(tm[:, None, None], dout[b], 0.0)
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            a, c, e = _masked_attention_bwd(q[b, :, h], k[b, :, g], v[b, :, g], allowed, scale,
                                            do_b[:, h])
            dq[b, :, h] = a
            dk[b, :, g] += c
            dv[b, :, g] += e
    return dq, dk, dv


def attn_bwd_compact(q, k, v, kept, block: int, dout, scale: float = None):
    """Same gradients via gather -> dense causal backward over kept tokens -> scatter."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if scale is None:
        scale = default_scale(D)
    keptb = _per_batch(kept, B)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        pos = token_positions(keptb[b], block)
        nk = len(pos)
        if nk == 0:
            continue
        allowed = np.tril(np.ones((nk, nk), dtype=bool))
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            a, c, e = _masked_attention_bwd(q[b, pos, h], k[b, pos, g], v[b, pos, g], allowed,
                                            scale, dout[b, pos, h])
            dq[b, pos, h] = a
            dk[b, pos, g] += c
            dv[b, pos, g] += e
    return dq, dk, dv


def attn_bwd(q, k, v, kept, block: int, dout, scale: float = None):
    if np.shape(q)[1] <= 2048:
        return attn_bwd_masked(q, k, v, kept, block, dout, scale)
    return attn_bwd_compact(q, k, v, kept, block, dout, scale)


# ----------------------------------------------------------------------------------------
# Sampled outputs for full-size workloads (same definitions, restricted to a few heads
# and a few rows so that the oracle finishes in seconds)
# ----------------------------------------------------------------------------------------

def attn_fwd_rows(q, k, v, kept_blocks, block: int, b: int, h: int, ranks, scale: float = None):
    """O and LSE of head h at the kept ranks `ranks` of batch row b (keys: kept, <= row)."""
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    Hq, D = q.shape[2], q.shape[3]
    Hkv = k.shape[2]
    if scale is None:
        scale = default_scale(D)
    g = kv_head_of(h, Hq, Hkv)
    pos = token_positions(kept_blocks, block)
    ranks = np.asarray(ranks, dtype=np.int64)
    O = np.zeros((len(ranks), D))
    LSE = np.zeros(len(ranks))
    for t, r in enumerate(ranks):
        keys = pos[:r + 1]
        qi = _f64(q[b, pos[r], h])
        z = scale * (_f64(k[b, keys, g]) @ qi)
        zmax = z.max()
        e = np.exp(z - zmax)
        O[t] = (e / e.sum()) @ _f64(v[b, keys, g])
        LSE[t] = zmax + np.log(e.sum())
    return O, LSE


def attn_bwd_sampled(q, k, v, kept_blocks, block: int, dout, b: int, g: int,
                     key_ranks, query_ranks, scale: float = None):
    """dK, dV of KV head g at kept ranks key_ranks, and dQ of every query head of the group
    at kept ranks query_ranks.  Streams over row chunks of the full compact problem.

    Returns dk [len(key_ranks), D], dv [len(key_ranks), D], dq [G, len(query_ranks), D].
    """
    q, k, v, dout = np.asarray(q), np.asarray(k), np.asarray(v), np.asarray(dout)
    Hq, D = q.shape[2], q.shape[3]
    Hkv = k.shape[2]
    G = Hq // Hkv
    if scale is None:
        scale = default_scale(D)
    pos = token_positions(kept_blocks, block)
    nk = len(pos)
    key_ranks = np.asarray(key_ranks, dtype=np.int64)
    query_ranks = np.asarray(query_ranks, dtype=np.int64)
    Kc, Vc = _f64(k[b, pos, g]), _f64(v[b, pos, g])
    dk = np.zeros((len(key_ranks), D))
    dv = np.zeros((len(key_ranks), D))
    dq = np.zeros((G, len(query_ranks), D))
    for hh in range(G):
        h = g * G + hh
        Qc, dOc = _f64(q[b, pos, h]), _f64(dout[b, pos, h])
        for r0 in range(0, nk, 1024):
            r1 = min(nk, r0 + 1024)
            # rows r0..r1-1 reach a sampled key only if it is at or before them (causal), and
            # a sampled query only if it is one of them: otherwise they add nothing here
            if not np.any(key_ranks < r1) and not np.any((query_ranks >= r0) & (query_ranks < r1)):
                continue
            allowed = np.arange(r1)[None, :] <= np.arange(r0, r1)[:, None]
            O, _, P = _masked_attention(Qc[r0:r1], Kc[:r1], Vc[:r1], allowed, scale)
            Dv = (dOc[r0:r1] * O).sum(axis=1)
            sel = key_ranks < r1
            kr = key_ranks[sel]
            if len(kr):
                Pj = P[:, kr]                                   # [R, nsel]
                dPj = dOc[r0:r1] @ Vc[kr].T
                dSj = Pj * (dPj - Dv[:, None])
                dk[sel] += scale * (dSj.T @ Qc[r0:r1])
                dv[sel] += Pj.T @ dOc[r0:r1]
            inq = (query_ranks >= r0) & (query_ranks < r1)
            for t in np.nonzero(inq)[0]:
                rr = query_ranks[t] - r0
                dP = Vc[:r1] @ dOc[r0 + rr]
                dS = P[rr] * (dP - Dv[rr])
                dq[hh, t] = scale * (dS @ Kc[:r1])
    return dk, dv, dq


# ----------------------------------------------------------------------------------------
# Layer stack (each layer selects its own kept set; [notes] 4.4: different layers use
# different token subsets and the output is added to the residual in place)
# ----------------------------------------------------------------------------------------

def stack_forward(x0, layers: List[Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]],
                  block: int, scale: float = None):
    """x_{l+1} = x_l + scatter(O_l) for layers given as (q, k, v, kept).  Returns
    (x_final float64, [O_l])."""
    x = _f64(x0).copy()
    outs = []
    for (q, k, v, kept) in layers:
        O, _ = attn_fwd(q, k, v, kept, block, scale)
        x = residual_add(x, O, kept, block)
        outs.append(O)
    return x, outs
