/*
 * jenga.h — C ABI of the MI355X (gfx950) token-sparse attention hot path of Jenga's
 * contextual token sparsity.
 *
 * Citations name the pages the operations are defined on:
 *   [summary] "JENGA: Enhancing LLM Long-Context Fine-tuning with Contextual Token Sparsity",
 *             the aipaper.cc structured summary of the ATC'25 paper;
 *   [notes]   the papercache.org deep-notes page of the same title.
 *
 * Conventions shared by every call
 *   - Tensors are BSHD: [batch][token][head][head_dim] with head_dim contiguous.  q, k, v may
 *     be strided views (strides in elements for batch, token and head); every other tensor
 *     is dense as stated at its argument.
 *   - All pointers are device pointers unless stated otherwise; the caller owns and frees
 *     every buffer, including the workspace.  The library allocates nothing.  Apart from the
 *     per-GPU scratch array of jenga_sparse_attn_bwd_segmented_noalloc and the optional
 *     per-kernel timing records it keeps no state between calls, so calls on different
 *     streams may run concurrently as long as they do not share output buffers.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call only enqueues kernels on
 *     it and returns: no memset, copy or host synchronisation.  The kept-block count stays on
 *     the device.  A sequence of calls can therefore be captured in a HIP graph and replayed
 *     (jenga_sparse_attn_bwd_segmented_noalloc must first have run once on the device, which
 *     places its scratch array; per-kernel timing must be off during capture).
 *   - Errors: every argument check happens before anything is launched; a negative status
 *     means nothing was enqueued.  JENGA_ERR_LAUNCH reports a failed launch (from
 *     hipGetLastError).  Faults inside a kernel surface at the caller's next synchronisation.
 *   - Supported shapes: head_dim in {64, 128}; block a multiple of 64 (at most 1024) that
 *     divides seq_len; n_heads_q a multiple of n_heads_kv; q/k/v rows 16-byte aligned.
 */
#ifndef JENGA_H
#define JENGA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { JENGA_DTYPE_F32 = 0, JENGA_DTYPE_BF16 = 1 } jenga_dtype;

typedef enum {
  JENGA_OK = 0,
  JENGA_ERR_INVALID_ARG = -1,  /* null pointer, non-positive size, bad stride or alignment */
  JENGA_ERR_UNSUPPORTED = -2,  /* valid but unsupported shape (head_dim, block, dtype)      */
  JENGA_ERR_WORKSPACE = -3,    /* workspace missing or smaller than jenga_workspace_bytes   */
  JENGA_ERR_LAUNCH = -4,       /* a kernel launch failed                                    */
  JENGA_ERR_SCRATCH_LIMIT = -5 /* needs more than the no-alloc entry point's fixed scratch  */
} jenga_status;

typedef enum {
  JENGA_SELECT_TOPK = 0,        /* param = keep ratio r: keep jenga_topk_count(r, nKB) blocks  */
  JENGA_SELECT_THRESH_REL = 1,  /* param = alpha: keep blocks with score >= alpha * mean score */
  JENGA_SELECT_THRESH_ABS = 2   /* param = absolute per-layer threshold T                      */
} jenga_select_mode;

#define JENGA_FORCE_FIRST_BLOCK 1u  /* flag: block 0 is always kept */

typedef enum {
  JENGA_OP_SCORE = 0,
  JENGA_OP_FWD = 1,
  JENGA_OP_BWD = 2,      /* the backward's workspace for its fastest schedule                  */
  JENGA_OP_SCORE_EQ2 = 3,
  JENGA_OP_BWD_MIN = 4   /* the least workspace the backward accepts (one segment's buffers)   */
} jenga_op;

/* Problem shape, shared by every call of one layer. */
typedef struct jenga_problem {
  int32_t batch;
  int32_t seq_len;      /* S, tokens per sequence                                       */
  int32_t n_heads_q;    /* Hq                                                           */
  int32_t n_heads_kv;   /* Hkv (grouped-query attention when Hkv < Hq)                  */
  int32_t head_dim;     /* D                                                            */
  int32_t block;        /* b, tokens per token block (the unit of elimination)          */
  int32_t dtype;        /* jenga_dtype of q, k, v and o_saved (MFMA operand type)       */
  float scale;          /* softmax scale; 0 selects 1/sqrt(head_dim)                    */
  int64_t q_stride[3];  /* batch, token, head strides of q, in elements                 */
  int64_t k_stride[3];  /* batch, token, head strides of k, in elements                 */
  int64_t v_stride[3];  /* batch, token, head strides of v, in elements                 */
} jenga_problem;

/* Status code -> static English string. */
const char* jenga_status_string(int status);

/* Number of blocks kept by top-k selection: ceil(r * n_blocks - 1e-6) clamped to
 * [1, n_blocks] (r widened to double).  Host-side; returns -1 if n_blocks < 1. */
int jenga_topk_count(float keep_ratio, int n_blocks);

/* Workspace bytes needed by `op` (a jenga_op) for this problem.  max_kept_blocks matters for
 * _FWD and _BWD*, n_segments for _BWD*.  Returns 0 for an invalid problem (and for ops that
 * need no workspace). */
size_t jenga_workspace_bytes(const jenga_problem* p, int op, int max_kept_blocks, int n_segments);

/*
 * jenga_score_blocks — block-level token informativeness ([summary] 4.2.1 Eq. 1;
 * 4.2.2 Eq. 2 head averaging; 4.2.3 aggregation of score blocks per key block).
 *
 * For every batch row and key block n:
 *   block_scores[b][n] = (1/Hq) * sum_h sum_{j in block n} sum_{i > j} P^h_ij,
 * where P^h is the causal softmax of scale * q_i . k_j over all S tokens of head h (KV head
 * h / (Hq/Hkv)); the self term i = j is excluded as in Eq. 1.  No S x S matrix is stored.
 * bf16: one streamed pass over the causal scores yields each row's log-sum-exp and, per query
 * and key block, the log2 of the block's partial sum; a memory-bound pass turns these into the
 * mass per key block.  The queries go through both passes in chunks (segment-based peak
 * cutting, [summary] 4.4.2), so the workspace holds the partial sums of one chunk only:
 * chunk * S/block floats per (batch, head), chunk = 128 * ceil(2048 / (B * Hq)) queries
 * (at most S rounded up to 128) -- linear in S.  fp32: two streamed passes (row log-sum-exp,
 * then received mass per key).  The result is deterministic: sums are fp64 and reduced in a
 * fixed order.
 * Returns JENGA_ERR_UNSUPPORTED when a batch row of q or k spans 4 GiB or more.
 *
 *   q            [B][S][Hq][D] (dtype, strided per q_stride)
 *   k            [B][S][Hkv][D] (dtype, strided per k_stride)
 *   block_scores [B][S/block] fp32, dense, written
 *   workspace    >= jenga_workspace_bytes(p, JENGA_OP_SCORE, 0, 1) bytes, 256-byte aligned
 */
int jenga_score_blocks(const jenga_problem* p, const void* q, const void* k, float* block_scores,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * jenga_score_blocks_eq2 — the literal form of [summary] 4.2.2 Eq. 2 and 4.2.3: a score block's
 * informativeness is the maximum over its elements of the head-averaged positive attention
 * scores, and a key block's score sums its score blocks over the query blocks.
 *
 * For every batch row and key block n, with query block m >= n (causal):
 *   e_ij = (1/Hq) sum_h max(scale * q_i^h . k_j^(h/(Hq/Hkv)), 0)
 *   B(m, n) = max over i in block m, j in block n, j <= i of e_ij
 *   block_scores[b][n] = sum_{m >= n} B(m, n)
 * One pass over the causal score blocks without exponentials; deterministic (the sum over m
 * is fp64 in ascending m).  bf16 only, block 64 or 128, head_dim 64 or 128.
 *
 *   q, k         as for jenga_score_blocks
 *   block_scores [B][S/block] fp32, dense, written
 *   workspace    >= jenga_workspace_bytes(p, JENGA_OP_SCORE_EQ2, 0, 1) = B * nKB^2 * 4 bytes
 *                (rounded up), 256-byte aligned
 * Errors: UNSUPPORTED for fp32 or another block size; otherwise as jenga_score_blocks.
 */
int jenga_score_blocks_eq2(const jenga_problem* p, const void* q, const void* k,
                           float* block_scores, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * jenga_select_blocks — token-block elimination against a per-layer threshold or a keep
 * ratio ([notes] 4.2 layer-specific threshold; [summary] 4.2.3 Algorithm 1, step 1 sets the
 * threshold from the average token-block score).
 *
 *   TOPK:       keep the jenga_topk_count(param, nKB) best blocks, ordered by score
 *               descending then index ascending; NaN scores sort last.
 *   THRESH_REL: T = (double)param * mean, the mean summed left to right in double;
 *               keep blocks with (double)score >= T.
 *   THRESH_ABS: the same with T = (double)param.
 *   flags & JENGA_FORCE_FIRST_BLOCK: block 0 is kept (top-k then keeps block 0 plus the
 *               best count-1 of the others).
 *
 *   block_scores [B][S/block] fp32, dense, read
 *   kept_idx     [B][S/block] int32, dense, written: kept block indices ascending in the
 *                first n_kept[b] entries; the rest is set to -1
 *   n_kept       [B] int32, written (device memory)
 * Only p->batch, p->seq_len and p->block are used.  Selection is exact and deterministic.
 */
int jenga_select_blocks(const jenga_problem* p, const float* block_scores, int mode, float param,
                        unsigned flags, int32_t* kept_idx, int32_t* n_kept, void* stream);

/*
 * jenga_sparse_attn_fwd — permutation-free token-sparse causal attention forward
 * ([notes] 4.4: kept tokens are loaded straight from the original tensors through the
 * index list, and the attention output is added to the original input in place, which
 * pads and residual-adds in one step; [summary] 3.1 attention formula).
 *
 * With T_k the tokens of the kept blocks of batch row b (kept rank r = position of the token
 * among kept tokens in ascending order):
 *   O_i = softmax_{j in T_k, j <= i}(scale * q_i . k_j) v_j   for i in T_k
 *   resid[b][i][h][:] += O_i                                   for i in T_k
 * Rows of eliminated tokens are never read as queries or keys and resid there is not
 * written (bitwise unchanged).
 *
 * bf16: when a batch row holds few kept tokens for the launch (its longest 128-query tile,
 * which sees every kept key, would hold more than twice the mean work per workgroup slot), the
 * row's long query tiles run in parts over ranges of their keys, and a second launch merges
 * each tile's parts in a fixed order (the online-softmax merge).  The decision follows n_kept
 * on the device.  Results are deterministic; the partial rows are held in bf16, so a split
 * tile rounds differently from a single pass, within the bf16 tolerance.
 *
 *   kept_idx, n_kept   output of jenga_select_blocks (device)
 *   max_kept_blocks    host upper bound on n_kept[b] (1 <= .. <= S/block); sizes the grids
 *                      and the compact outputs; kept blocks beyond it are ignored
 *   resid              [B][S][Hq][D] fp32, dense, read-modify-write
 *   o_saved            [B][max_kept_blocks*block][Hq][D] dtype, dense, written by kept rank
 *                      (the saved attention output used by the backward)
 *   lse                [B][Hq][max_kept_blocks*block] fp32, dense, written by kept rank:
 *                      natural-log softmax normaliser of each kept query
 *   workspace          >= jenga_workspace_bytes(p, JENGA_OP_FWD, max_kept_blocks, 1) bytes,
 *                      256-byte aligned (bf16: a transposed copy of the kept V rows, then the
 *                      part slots of split query tiles, sized for the worst n_kept up to
 *                      max_kept_blocks; fp32 needs none and may pass NULL)
 */
int jenga_sparse_attn_fwd(const jenga_problem* p, const void* q, const void* k, const void* v,
                          const int32_t* kept_idx, const int32_t* n_kept, int max_kept_blocks,
                          float* resid, void* o_saved, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * jenga_sparse_attn_bwd_segmented — backward of jenga_sparse_attn_fwd, computed over
 * n_segments contiguous ranges of kept query ranks one after the other so that the
 * transient buffers (the per-query dot(dO, O) terms and the operand copies of dOut and Q)
 * scale with the segment, not the sequence ([notes] 4.4 segment-based peak cutting: process
 * segments independently, aggregate their gradients, discard each segment's activations).
 *
 * With P the forward's probabilities and dO_i = dout[b][i][h] for i in T_k:
 *   D_i = dO_i . O_i;  dS_ij = P_ij (dO_i . v_j - D_i)
 *   dq_i += scale sum_j dS_ij k_j;  dk_j += scale sum_{h in group} sum_i dS_ij q_i;
 *   dv_j += sum_{h in group} sum_i P_ij dO_i
 * The gradient through resid is the identity (dout itself) and needs no call.  The result
 * does not depend on n_segments beyond fp32 rounding.
 *
 *   o_saved, lse      outputs of jenga_sparse_attn_fwd for the same inputs and kept set
 *   dout              [B][S][Hq][D] fp32, dense, read at kept rows only
 *   dq                [B][S][Hq][D] fp32, dense, accumulated (+=) at kept rows only
 *   dk, dv            [B][S][Hkv][D] fp32, dense, accumulated (+=) at kept rows only
 *   n_segments        1 <= n_segments <= max_kept_blocks*block/64
 *   workspace         >= jenga_workspace_bytes(p, JENGA_OP_BWD_MIN, max_kept_blocks, n_segments)
 *                     bytes, 256-byte aligned: one set of segment buffers, plus (bf16) slots
 *                     for the parts of long dK/dV key tiles (below).  bf16 with two or more
 *                     segments: jenga_workspace_bytes(p, JENGA_OP_BWD, ...) adds a second set,
 *                     and each segment's launch then also runs the next segment's prologue;
 *                     with less, every prologue is a launch of its own.  Both schedules give
 *                     the same bits.
 * bf16: a dK/dV key tile (256 kept keys of one KV head) loops over the segment's queries of
 * every query head of its group.  When that loop is longer than the launch's average load per
 * compute unit (grouped-query attention in few segments), the tile runs in parts; the first
 * adds into dk/dv, the others' sums are added after the launch in part order.
 * bf16: every gradient is accumulated by a fixed schedule, so results repeat bit for bit.
 * fp32: dq receives fp32 atomic additions, so its low bits may differ run to run.
 */
int jenga_sparse_attn_bwd_segmented(const jenga_problem* p, const void* q, const void* k,
                                    const void* v, const int32_t* kept_idx, const int32_t* n_kept,
                                    int max_kept_blocks, const void* o_saved, const float* lse,
                                    const float* dout, float* dq, float* dk, float* dv,
                                    int n_segments, void* workspace, size_t workspace_bytes,
                                    void* stream);

/*
 * jenga_sparse_attn_bwd_segmented_noalloc — jenga_sparse_attn_bwd_segmented for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  It takes no workspace argument and allocates nothing: its scratch is
 * a fixed device array of JENGA_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU,
 * located on the first call on each device and held until the process ends.  The caller
 * still passes every input and output, with the meanings, layouts and results of
 * jenga_sparse_attn_bwd_segmented (the same kernels run).
 *
 * Returns JENGA_ERR_SCRATCH_LIMIT, launching nothing, when
 * jenga_workspace_bytes(p, JENGA_OP_BWD_MIN, max_kept_blocks, n_segments) exceeds
 * JENGA_NOALLOC_SCRATCH_BYTES; the backward's scratch shrinks as 1/n_segments, so a larger
 * n_segments makes a bigger problem fit (32K tokens x 32 heads x 128, half the blocks kept:
 * 8 segments need 48.5 MiB).  When the scratch holds JENGA_OP_BWD's two sets of segment
 * buffers, the faster schedule runs.  Every call on one GPU shares that GPU's scratch: calls that
 * overlap in time on one GPU (different streams, or host threads) race and must be ordered
 * by the caller.  The scratch keeps the last call's contents; nothing in it needs to start
 * at zero.
 */
#define JENGA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int jenga_sparse_attn_bwd_segmented_noalloc(const jenga_problem* p, const void* q, const void* k,
                                            const void* v, const int32_t* kept_idx,
                                            const int32_t* n_kept, int max_kept_blocks,
                                            const void* o_saved, const float* lse,
                                            const float* dout, float* dq, float* dk, float* dv,
                                            int n_segments, void* stream);

/*
 * Permutation-free token movement around the projections ([notes] §4.4; [summary] 4.4.1: the
 * kept tokens are loaded straight from the full hidden-state tensor by the layer that consumes
 * them, and the result is added into the residual stream in place -- no gathered copy, padding
 * or separate residual pass).  bf16 inputs and weights, fp32 accumulation.
 *
 *   in_features   K, a multiple of 64;  out_features  N, a multiple of 128
 *   in_stride     (batch, row) element strides of the input rows (16-byte aligned rows)
 *   out_stride    (batch, row) element strides of the output rows
 *   block         kept-block size (multiple of 64, <= 1024); seq_len % block == 0
 */
typedef struct {
  int32_t batch, seq_len, block, in_features, out_features;
  int64_t in_stride[2];
  int64_t out_stride[2];
} jenga_proj_problem;

/*
 * jenga_proj_gather — y[b][r][:] = x[b][pos(r)][:] . w^T for every kept rank r < Nk_b, where
 * pos(r) = kept_idx[b][r / block] * block + r % block and Nk_b = min(n_kept[b],
 * max_kept_blocks) * block.  Rows of y at or past Nk_b are not written.
 *   x  [B][S][K] bf16 (full sequence; only kept rows are read)
 *   w  [N][K] bf16, contiguous (a linear layer's weight)
 *   y  [B][max_kept_blocks*block][N] bf16 (compact, by kept rank), written
 * Errors: INVALID_ARG for null / misaligned pointers, bad strides or max_kept_blocks outside
 * [1, nKB]; UNSUPPORTED for sizes outside the limits above or a row extent over 4 GiB.
 */
int jenga_proj_gather(const jenga_proj_problem* p, const void* x, const void* w,
                      const int32_t* kept_idx, const int32_t* n_kept, int max_kept_blocks,
                      void* y, void* stream);

/*
 * jenga_proj_scatter_add — resid[b][pos(r)][:] += y[b][r][:] . w^T for every kept rank r;
 * rows of eliminated tokens are not touched.
 *   y      [B][max_kept_blocks*block][K] bf16 (compact, by kept rank)
 *   w      [N][K] bf16, contiguous
 *   resid  [B][S][N] fp32, updated in place
 * Errors as jenga_proj_gather.
 */
int jenga_proj_scatter_add(const jenga_proj_problem* p, const void* y, const void* w,
                           const int32_t* kept_idx, const int32_t* n_kept, int max_kept_blocks,
                           float* resid, void* stream);

/*
 * jenga_proj_gather_scatter_add — resid[b][pos(r)][:] += a[b][pos(r)][:] . w^T for every kept
 * rank r; rows of eliminated tokens are neither read nor written.  The down projection of an
 * MLP block with token elimination (aipaper summary §4.2.4 with the permutation-free movement
 * of papercache notes §4.4).
 *   a      [B][S][K] bf16 (full sequence, in_stride; only kept rows are read)
 *   w      [N][K] bf16, contiguous
 *   resid  [B][S][N] fp32 (out_stride), updated in place
 * Errors as jenga_proj_gather.
 */
int jenga_proj_gather_scatter_add(const jenga_proj_problem* p, const void* a, const void* w,
                                  const int32_t* kept_idx, const int32_t* n_kept,
                                  int max_kept_blocks, float* resid, void* stream);

/*
 * Token elimination in the MLP block (aipaper summary §4.2.4; papercache notes §4.2): a token's
 * informativeness comes from the block's intermediate activation.
 *   JENGA_MLP_RELU        act = max(x w1^T, 0)                      (ReLU MLPs)
 *   JENGA_MLP_SILU_GATED  act = silu(x w1^T) * (x w_up^T)           (gated SiLU MLPs; w1 = gate)
 * Token score e[b][t] = mean over the F units of |act[b][t][:]| (from the fp32 activation,
 * before its rounding to bf16); block score = max of e over the block's tokens.  Selection then
 * uses jenga_select_blocks on the block scores; jenga_proj_gather_scatter_add runs the down
 * projection of the kept tokens.
 * The problem is a jenga_proj_problem: in_features = K (model width, multiple of 64),
 * out_features = F (units: multiple of 64 gated, of 128 ReLU), in_stride for x, out_stride for
 * act (both bf16 element strides).
 */
#define JENGA_MLP_RELU 0
#define JENGA_MLP_SILU_GATED 1

/* Workspace: B * (F / 32) * S * 4 bytes (partial |act| sums), rounded up to 256; 0 for an
 * invalid problem or kind. */
size_t jenga_mlp_workspace_bytes(const jenga_proj_problem* p, int kind);

/*
 * jenga_mlp_act_scores — activation and informativeness of every token.
 *   x             [B][S][K] bf16        w1, w_up  [F][K] bf16 contiguous (w_up unused for ReLU)
 *   act           [B][S][F] bf16, written        token_scores [B][S] fp32, written
 *   block_scores  [B][S / block] fp32, written   workspace >= jenga_mlp_workspace_bytes, 256-aligned
 * Token scores sum the per-unit magnitudes in a fixed order (fp32 groups of 32, then fp64),
 * so results repeat bit for bit.  Errors: INVALID_ARG (null / misaligned pointers, bad
 * strides, unknown kind), UNSUPPORTED (sizes outside the limits or a row extent over 4 GiB),
 * WORKSPACE, LAUNCH.
 */
int jenga_mlp_act_scores(const jenga_proj_problem* p, int kind, const void* x, const void* w1,
                         const void* w_up, void* act, float* token_scores, float* block_scores,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Segment-based peak cutting of the language-model-head loss ([summary] 4.4.2; [notes] §4.4:
 * the loss step's transient -- logits over the whole vocabulary for every token -- is split
 * into segments processed one after another, each segment's activations discarded before the
 * next, so the transient peak follows tokens / n_segments).
 *
 *   tokens      T, a multiple of 32;   d_model  d, a multiple of 128
 *   vocab       V, a multiple of 128, at most 32768;   n_segments in [1, T / 32]
 * Segment rows L = ceil(T / n_segments) rounded up to 32 (the last segment may be shorter).
 */
typedef struct {
  int32_t tokens, d_model, vocab, n_segments;
} jenga_loss_problem;

/* Workspace for one segment: L * V * (4 + 2) bytes (fp32 logits, bf16 logit gradient), rounded
 * up to 256; 0 for an invalid problem.  This is the transient that segmenting bounds. */
size_t jenga_loss_workspace_bytes(const jenga_loss_problem* p);

/*
 * jenga_lm_head_ce_segmented — mean next-token cross-entropy of the head logits = h w^T and its
 * gradient with respect to h, one segment of L rows at a time:
 *   row_loss[t] = logsumexp(logits_t) - logits_t[targets[t]]      (fp32, from fp32 logits)
 *   loss[0]     = mean_t row_loss[t]                               (fp64 sum, fixed order)
 *   dh[t][:]    = ((softmax(logits_t) - onehot(targets[t])) / T) w   (the factor in bf16)
 *   h        [T][d] bf16 row-major        w  [V][d] bf16 (the head's weight)
 *   wt       [d][V] bf16 (the same weight transposed, prepared once: the head is frozen)
 *   targets  [T] int32 in [0, V)           row_loss [T] fp32, loss [1] fp32, dh [T][d] fp32
 *   workspace >= jenga_loss_workspace_bytes(p), 256-byte aligned
 * The results do not depend on n_segments.  Errors: INVALID_ARG (null / misaligned pointers),
 * UNSUPPORTED (sizes outside the limits), WORKSPACE, LAUNCH.
 */
int jenga_lm_head_ce_segmented(const jenga_loss_problem* p, const void* h, const void* w,
                               const void* wt, const int32_t* targets, float* row_loss,
                               float* loss, float* dh, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * Kernel timing (instrumentation; not part of the method).
 *
 * jenga_timing_enable(1) discards earlier records and, from then on, brackets every kernel
 * launched by the entry points above with two HIP events recorded on that call's stream;
 * jenga_timing_enable(0) stops recording (the records stay readable).  Kernel names:
 * k_slse64, k_sblock_mass (bf16 scoring), k_eq2_tiles, k_eq2_reduce (Eq. 2 scoring), k_select,
 * k_pack_tp, k_fwd64, k_prep64, k_bwd64 (bf16 attention; k_bwd64 is one launch per backward
 * segment, with the dK/dV and dQ tiles), k_proj_gather, k_proj_scatter, k_proj_gather_scatter,
 * k_mlp_act_gated, k_mlp_act_relu, k_mlp_block (MLP elimination), k_proj_logits, k_ce_rows,
 * k_proj_dh (loss).  The fp32 kernels are not bracketed.
 *
 * jenga_timing_query(kernel, launches, total_ms) waits for the recorded events of that name
 * and returns how many launches were recorded and the sum of their event-to-event times.
 * Errors: INVALID_ARG for a null pointer or enable not in {0, 1}; LAUNCH if an event query
 * fails.  Not thread-safe; one process-wide record list.
 */
int jenga_timing_enable(int enable);
int jenga_timing_query(const char* kernel, int32_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* JENGA_H */
