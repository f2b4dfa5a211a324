// C ABI of the token-sparse attention hot path: argument validation, workspace sizing,
// launch geometry and the segment loop.  Every check happens before the first launch.
#include <math.h>
#include <algorithm>
#include <mutex>
#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/jenga.h"
#include "kernels.h"

namespace {

constexpr int kMaxBlocks = 16384;      // selection keeps one 32-bit key per block in LDS
constexpr size_t kAlign = 256;
constexpr double kOffsetLimit = 4294967296.0;   // 32-bit buffer-resource offsets

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Scratch of jenga_sparse_attn_bwd_segmented_noalloc: a fixed device array, one copy per GPU,
// held until the process ends.  Host code never uses the array's name as an address (on the
// host it is only a stand-in for the symbol): each GPU's copy is located once, with that GPU
// current, through hipGetSymbolAddress, and that pointer is what the kernels receive.
constexpr size_t kNoAllocScratchBytes = JENGA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) static unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return JENGA_ERR_LAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return JENGA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return JENGA_ERR_LAUNCH;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return JENGA_OK;
}

int check_problem(const jenga_problem* p, bool need_qkv_strides) {
  if (!p) return JENGA_ERR_INVALID_ARG;
  if (p->batch <= 0 || p->seq_len <= 0 || p->n_heads_q <= 0 || p->n_heads_kv <= 0 ||
      p->head_dim <= 0 || p->block <= 0)
    return JENGA_ERR_INVALID_ARG;
  if (p->n_heads_q % p->n_heads_kv != 0) return JENGA_ERR_INVALID_ARG;
  if (!(p->scale >= 0.f) || isinf(p->scale)) return JENGA_ERR_INVALID_ARG;
  if (p->block % 64 != 0 || p->block > 1024) return JENGA_ERR_UNSUPPORTED;
  if (p->seq_len % p->block != 0) return JENGA_ERR_UNSUPPORTED;
  if (p->seq_len / p->block > kMaxBlocks) return JENGA_ERR_UNSUPPORTED;
  if (p->dtype != JENGA_DTYPE_F32 && p->dtype != JENGA_DTYPE_BF16) return JENGA_ERR_UNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 128) return JENGA_ERR_UNSUPPORTED;
  if (p->dtype == JENGA_DTYPE_F32 && p->head_dim != 64) return JENGA_ERR_UNSUPPORTED;
  if (need_qkv_strides) {
    const int es = p->dtype == JENGA_DTYPE_BF16 ? 2 : 4;
    const int64_t* st[3] = {p->q_stride, p->k_stride, p->v_stride};
    for (int t = 0; t < 3; ++t)
      for (int i = 0; i < 3; ++i)
        if (st[t][i] < 0 || (st[t][i] * es) % 16 != 0) return JENGA_ERR_INVALID_ARG;
    // The kernels address Q, K and V through buffer resources whose base is a batch row and
    // whose per-lane offsets are 32-bit: every byte of a batch row they can touch (any token,
    // any head) must lie below 4 GiB from that row's start.
    for (int t = 0; t < 3; ++t) {
      const double heads = t == 0 ? p->n_heads_q : p->n_heads_kv;
      const double extent = ((double)(p->seq_len - 1) * (double)st[t][1] +
                             (heads - 1.0) * (double)st[t][2] + (double)p->head_dim) * es;
      if (extent >= kOffsetLimit) return JENGA_ERR_UNSUPPORTED;
    }
  }
  // fp32 residual and gradient rows of one batch row, and the per-head score workspace, are
  // indexed with the same 32-bit offsets
  if ((double)p->seq_len * p->n_heads_q * p->head_dim * 4.0 >= kOffsetLimit) return JENGA_ERR_UNSUPPORTED;
  return JENGA_OK;
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

float scale_of(const jenga_problem* p) {
  return p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->head_dim);
}

void copy_strides(int64_t dst[3], const int64_t src[3]) {
  for (int i = 0; i < 3; ++i) dst[i] = src[i];
}

// Segment length in kept ranks: ceil(Nk_cap / N) rounded up to the 64-query tile.
int seg_len_of(int ncap, int n_segments) {
  int L = (ncap + n_segments - 1) / n_segments;
  return (L + 63) / 64 * 64;
}

struct BwdLayout {
  size_t d, l2, dO, qtp, dotp, total;
};

BwdLayout bwd_layout(const jenga_problem* p, int max_kept_blocks, int n_segments) {
  const int ncap = max_kept_blocks * p->block;
  const int L = seg_len_of(ncap, n_segments);
  const size_t es = p->dtype == JENGA_DTYPE_BF16 ? 2 : 4;
  const size_t B = p->batch, Hq = p->n_heads_q, D = p->head_dim;
  BwdLayout o;
  o.d = 0;
  o.l2 = o.d + align_up(B * Hq * L * sizeof(float));
  o.dO = o.l2 + (p->dtype == JENGA_DTYPE_BF16 ? align_up(B * Hq * L * sizeof(float)) : 0);
  size_t end = o.dO + align_up(B * L * Hq * D * es);
  o.qtp = o.dotp = end;
  if (p->dtype == JENGA_DTYPE_BF16) {            // transposed operand tiles of the bf16 path
    o.qtp = end;
    o.dotp = o.qtp + align_up(B * Hq * (size_t)L * D * 2);
    end = o.dotp + align_up(B * Hq * (size_t)L * D * 2);
  }
  o.total = end;
  return o;
}

// Segments the backward runs: the capacity max_kept_blocks * block cut into seg_len pieces.
int bwd_segments_run(const jenga_problem* p, int max_kept_blocks, int n_segments) {
  const int ncap = max_kept_blocks * p->block;
  const int L = seg_len_of(ncap, n_segments);
  return (ncap + L - 1) / L;
}

// Slots for the parts of split dK/dV tiles (bf16): the most any segment needs, since the
// segments run one after another and each one's slots are added up before the next starts.
size_t bwd_kv_slot_bytes(const jenga_problem* p, int max_kept_blocks, int n_segments) {
  if (p->dtype != JENGA_DTYPE_BF16) return 0;
  const int ncap = max_kept_blocks * p->block;
  const int L = seg_len_of(ncap, n_segments);
  const int G = p->n_heads_q / p->n_heads_kv;
  int most = 0;
  for (int s = 0; s < bwd_segments_run(p, max_kept_blocks, n_segments); ++s) {
    const int qs = s * L, cap = std::min(L, ncap - qs);
    const int target = jenga::kv_split_target(qs, cap, G, p->n_heads_q, p->n_heads_kv, p->batch);
    most = std::max(most, jenga::kv_split_extra(qs, cap, G, target));
  }
  return align_up((size_t)p->batch * p->n_heads_kv * most * 2 * jenga::kKvKeys * p->head_dim * sizeof(float));
}

// The bf16 path with two or more segments takes two sets of one segment's buffers: the
// prologue of segment s + 1 then runs inside the launch of segment s, writing the other set.
// One set (bwd_ws_min_bytes) also works, with each prologue launched on its own.  The slots of
// split dK/dV tiles follow the sets.
size_t bwd_ws_min_bytes(const jenga_problem* p, int max_kept_blocks, int n_segments) {
  return bwd_layout(p, max_kept_blocks, n_segments).total + bwd_kv_slot_bytes(p, max_kept_blocks, n_segments);
}

size_t bwd_ws_bytes(const jenga_problem* p, int max_kept_blocks, int n_segments) {
  const size_t one = bwd_layout(p, max_kept_blocks, n_segments).total;
  const bool two = p->dtype == JENGA_DTYPE_BF16 && bwd_segments_run(p, max_kept_blocks, n_segments) >= 2;
  return (two ? 2 * one : one) + bwd_kv_slot_bytes(p, max_kept_blocks, n_segments);
}

// bf16 forward: the TP tiles of the kept V rows, then the part slots of split query tiles
size_t fwd_vtp_bytes(const jenga_problem* p, int max_kept_blocks) {
  return align_up((size_t)p->batch * p->n_heads_kv * max_kept_blocks * p->block * p->head_dim * 2);
}

struct FwdPlan {
  int items, slots, split_tiles;
};

FwdPlan fwd_plan(const jenga_problem* p, int max_kept_blocks) {
  FwdPlan f;
  jenga::fwd_split_bounds(max_kept_blocks * p->block, p->n_heads_q, p->batch, &f.items, &f.slots,
                          &f.split_tiles);
  return f;
}

size_t fwd_ws_bytes(const jenga_problem* p, int max_kept_blocks, const FwdPlan& f) {
  if (p->dtype != JENGA_DTYPE_BF16) return 0;
  const size_t slot = (size_t)jenga::kFwdRows * (2 * p->head_dim + 8);   // bf16 rows, fp32 m, l
  return fwd_vtp_bytes(p, max_kept_blocks) + align_up((size_t)p->batch * p->n_heads_q * f.slots * slot);
}

size_t score_eq2_ws_bytes(const jenga_problem* p) {
  const size_t nkb = p->seq_len / p->block;
  return align_up((size_t)p->batch * nkb * nkb * sizeof(float));
}

// bf16 scoring runs in chunks of queries; each chunk's partial log2-sums (one per query and key
// block) are turned into mass before the next chunk.  A chunk holds enough 128-query tiles for
// at least 2048 workgroups (two rounds of four per compute unit: the heaviest-first order then
// pairs long tiles with short ones; one round lasts as long as its longest tile), or S rounded
// up to the tile if that is less, so the stored partials are chunk x S/block floats per
// (batch, head): linear in S.
constexpr int kScoreTile = 128;
constexpr int kScoreMinWorkgroups = 2048;

int score_chunk(const jenga_problem* p) {
  const int64_t heads = (int64_t)p->batch * p->n_heads_q;
  const int64_t tiles = (kScoreMinWorkgroups + heads - 1) / heads;
  const int64_t s_up = ((int64_t)p->seq_len + kScoreTile - 1) / kScoreTile * kScoreTile;
  return (int)std::min<int64_t>(tiles * kScoreTile, s_up);
}

size_t score_part_elems(const jenga_problem* p) {        // per (batch, head)
  return (size_t)(p->seq_len / p->block) * score_chunk(p);
}

size_t score_ws_bytes(const jenga_problem* p) {
  const size_t lse = (size_t)p->batch * p->n_heads_q * p->seq_len * sizeof(float);
  const size_t mass = (size_t)p->batch * p->n_heads_q * (p->seq_len / 32) * sizeof(double);
  const size_t part = p->dtype == JENGA_DTYPE_BF16
                          ? (size_t)p->batch * p->n_heads_q * score_part_elems(p) * sizeof(float)
                          : 0;
  return align_up(lse) + align_up(mass) + align_up(part);
}

int check_proj(const jenga_proj_problem* p, const void* in, const void* w, const int32_t* kept,
               const int32_t* n_kept, int max_kept_blocks, const void* out, int out_es) {
  if (!p || !in || !w || !kept || !n_kept || !out) return JENGA_ERR_INVALID_ARG;
  if (p->batch <= 0 || p->seq_len <= 0 || p->block <= 0 || p->in_features <= 0 ||
      p->out_features <= 0)
    return JENGA_ERR_INVALID_ARG;
  if (p->block % 64 != 0 || p->block > 1024 || p->seq_len % p->block != 0) return JENGA_ERR_UNSUPPORTED;
  const int nkb = p->seq_len / p->block;
  if (nkb > kMaxBlocks) return JENGA_ERR_UNSUPPORTED;
  if (p->in_features % 64 != 0 || p->out_features % 128 != 0) return JENGA_ERR_UNSUPPORTED;
  if (max_kept_blocks < 1 || max_kept_blocks > nkb) return JENGA_ERR_INVALID_ARG;
  for (int i = 0; i < 2; ++i) {
    if (p->in_stride[i] < 0 || (p->in_stride[i] * 2) % 16 != 0) return JENGA_ERR_INVALID_ARG;
    if (p->out_stride[i] < 0 || (p->out_stride[i] * out_es) % 16 != 0) return JENGA_ERR_INVALID_ARG;
  }
  if (!aligned16(in) || !aligned16(w) || !aligned16(out)) return JENGA_ERR_INVALID_ARG;
  // buffer-resource offsets are 32-bit: every per-batch-row extent stays below 4 GiB
  const double lim = 4294967296.0;
  if ((double)p->seq_len * (double)p->in_stride[1] * 2.0 >= lim) return JENGA_ERR_UNSUPPORTED;
  if ((double)p->out_features * (double)p->in_features * 2.0 >= lim) return JENGA_ERR_UNSUPPORTED;
  return JENGA_OK;
}

jenga::ProjParams proj_params(const jenga_proj_problem* p, const void* in, const void* w,
                              const int32_t* kept, const int32_t* n_kept, int max_kept_blocks,
                              void* out) {
  jenga::ProjParams pp;
  pp.a = in;
  pp.as0 = p->in_stride[0];
  pp.as1 = p->in_stride[1];
  pp.w = w;
  pp.out = out;
  pp.os0 = p->out_stride[0];
  pp.os1 = p->out_stride[1];
  pp.kept = kept;
  pp.n_kept = n_kept;
  pp.B = p->batch;
  pp.S = p->seq_len;
  pp.K = p->in_features;
  pp.N = p->out_features;
  pp.block = p->block;
  pp.nkb = p->seq_len / p->block;
  pp.max_kept_blocks = max_kept_blocks;
  pp.ncap = max_kept_blocks * p->block;
  pp.rows = 0;
  return pp;
}


int loss_rows(const jenga_loss_problem* p) {
  int L = (p->tokens + p->n_segments - 1) / p->n_segments;
  return (L + 31) / 32 * 32;
}

int check_loss(const jenga_loss_problem* p) {
  if (!p) return JENGA_ERR_INVALID_ARG;
  if (p->tokens <= 0 || p->d_model <= 0 || p->vocab <= 0 || p->n_segments <= 0)
    return JENGA_ERR_INVALID_ARG;
  if (p->tokens % 32 != 0 || p->d_model % 128 != 0 || p->vocab % 128 != 0 || p->vocab > 32768)
    return JENGA_ERR_UNSUPPORTED;
  if (p->n_segments > p->tokens / 32) return JENGA_ERR_INVALID_ARG;
  const double lim = 4294967296.0;
  if ((double)p->tokens * p->d_model * 2.0 >= lim || (double)p->vocab * p->d_model * 2.0 >= lim ||
      (double)loss_rows(p) * p->vocab * 2.0 >= lim)
    return JENGA_ERR_UNSUPPORTED;
  return JENGA_OK;
}

size_t loss_ws_bytes(const jenga_loss_problem* p) {
  const size_t L = loss_rows(p), V = p->vocab;
  return align_up(L * V * sizeof(float)) + align_up(L * V * 2);
}

int check_mlp(const jenga_proj_problem* p, int kind) {
  if (!p || (kind != JENGA_MLP_RELU && kind != JENGA_MLP_SILU_GATED)) return JENGA_ERR_INVALID_ARG;
  if (p->batch <= 0 || p->seq_len <= 0 || p->block <= 0 || p->in_features <= 0 ||
      p->out_features <= 0)
    return JENGA_ERR_INVALID_ARG;
  if (p->block % 64 != 0 || p->block > 1024 || p->seq_len % p->block != 0) return JENGA_ERR_UNSUPPORTED;
  if (p->seq_len / p->block > kMaxBlocks) return JENGA_ERR_UNSUPPORTED;
  if (p->in_features % 64 != 0) return JENGA_ERR_UNSUPPORTED;
  if (p->out_features % (kind == JENGA_MLP_SILU_GATED ? 64 : 128) != 0) return JENGA_ERR_UNSUPPORTED;
  for (int i = 0; i < 2; ++i)
    if (p->in_stride[i] < 0 || p->out_stride[i] < 0 || (p->in_stride[i] * 2) % 16 != 0 ||
        (p->out_stride[i] * 2) % 16 != 0)
      return JENGA_ERR_INVALID_ARG;
  const double lim = 4294967296.0;
  if ((double)p->seq_len * (double)p->in_stride[1] * 2.0 >= lim) return JENGA_ERR_UNSUPPORTED;
  if ((double)p->out_features * (double)p->in_features * 2.0 >= lim) return JENGA_ERR_UNSUPPORTED;
  return JENGA_OK;
}

size_t mlp_ws_bytes(const jenga_proj_problem* p) {
  return align_up((size_t)p->batch * (p->out_features / 32) * (size_t)p->seq_len * sizeof(float));
}

}  // namespace

extern "C" {

const char* jenga_status_string(int status) {
  switch (status) {
    case JENGA_OK: return "ok";
    case JENGA_ERR_INVALID_ARG: return "invalid argument";
    case JENGA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case JENGA_ERR_WORKSPACE: return "workspace missing or too small";
    case JENGA_ERR_LAUNCH: return "kernel launch failed";
    case JENGA_ERR_SCRATCH_LIMIT:
      return "the problem needs more scratch than the no-alloc entry point's fixed buffer holds "
             "(raise n_segments: the backward's scratch shrinks as 1/n_segments)";
    default: return "unknown status";
  }
}

int jenga_topk_count(float keep_ratio, int n_blocks) {
  if (n_blocks < 1) return -1;
  const double r = (double)keep_ratio;
  if (!(r == r)) return 1;
  double k = ceil(r * (double)n_blocks - 1e-6);
  if (k < 1.0) k = 1.0;
  if (k > (double)n_blocks) k = (double)n_blocks;
  return (int)k;
}

size_t jenga_workspace_bytes(const jenga_problem* p, int op, int max_kept_blocks, int n_segments) {
  if (check_problem(p, false) != JENGA_OK) return 0;
  if (op == JENGA_OP_SCORE) return score_ws_bytes(p);
  if (op == JENGA_OP_SCORE_EQ2) return score_eq2_ws_bytes(p);
  if (op == JENGA_OP_FWD) {
    const int nkb = p->seq_len / p->block;
    if (max_kept_blocks < 1 || max_kept_blocks > nkb) return 0;
    return fwd_ws_bytes(p, max_kept_blocks, fwd_plan(p, max_kept_blocks));
  }
  if (op == JENGA_OP_BWD || op == JENGA_OP_BWD_MIN) {
    const int nkb = p->seq_len / p->block;
    if (max_kept_blocks < 1 || max_kept_blocks > nkb || n_segments < 1) return 0;
    if (n_segments > max_kept_blocks * p->block / 64) return 0;
    return op == JENGA_OP_BWD ? bwd_ws_bytes(p, max_kept_blocks, n_segments)
                              : bwd_ws_min_bytes(p, max_kept_blocks, n_segments);
  }
  return 0;
}

int jenga_score_blocks(const jenga_problem* p, const void* q, const void* k, float* block_scores,
                       void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_problem(p, true);
  if (st != JENGA_OK) return st;
  if (!q || !k || !block_scores) return JENGA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k)) return JENGA_ERR_INVALID_ARG;
  const size_t need = score_ws_bytes(p);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace % kAlign) != 0)
    return JENGA_ERR_WORKSPACE;
  jenga::ScoreParams sp;
  sp.q = q;
  sp.k = k;
  copy_strides(sp.qs, p->q_stride);
  copy_strides(sp.ks, p->k_stride);
  sp.B = p->batch;
  sp.S = p->seq_len;
  sp.Hq = p->n_heads_q;
  sp.Hkv = p->n_heads_kv;
  sp.block = p->block;
  sp.scale_log2 = scale_of(p) * 1.4426950408889634f;
  sp.lse2 = (float*)workspace;
  sp.mass32 = (double*)((char*)workspace +
                        align_up((size_t)p->batch * p->n_heads_q * p->seq_len * sizeof(float)));
  sp.lpart = (float*)((char*)sp.mass32 +
                      align_up((size_t)p->batch * p->n_heads_q * (p->seq_len / 32) * sizeof(double)));
  sp.chunk = score_chunk(p);
  sp.q_begin = 0;
  sp.q_end = p->seq_len;
  sp.mass_gpb = 0;
  sp.scores = block_scores;
  if (jenga::launch_score(sp, p->dtype, p->head_dim, (hipStream_t)stream) != hipSuccess)
    return JENGA_ERR_LAUNCH;
  return JENGA_OK;
}

int jenga_score_blocks_eq2(const jenga_problem* p, const void* q, const void* k,
                           float* block_scores, void* workspace, size_t workspace_bytes,
                           void* stream) {
  int st = check_problem(p, true);
  if (st != JENGA_OK) return st;
  if (p->dtype != JENGA_DTYPE_BF16) return JENGA_ERR_UNSUPPORTED;
  if (p->block != 64 && p->block != 128) return JENGA_ERR_UNSUPPORTED;
  if (!q || !k || !block_scores) return JENGA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k)) return JENGA_ERR_INVALID_ARG;
  const size_t need = score_eq2_ws_bytes(p);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace % kAlign) != 0)
    return JENGA_ERR_WORKSPACE;
  jenga::Eq2Params ep;
  ep.q = q;
  ep.k = k;
  copy_strides(ep.qs, p->q_stride);
  copy_strides(ep.ks, p->k_stride);
  ep.B = p->batch;
  ep.S = p->seq_len;
  ep.Hq = p->n_heads_q;
  ep.Hkv = p->n_heads_kv;
  ep.block = p->block;
  ep.nkb = p->seq_len / p->block;
  ep.scale = scale_of(p);
  ep.tilemax = (float*)workspace;
  ep.scores = block_scores;
  if (jenga::launch_score_eq2(ep, p->head_dim, p->block, (hipStream_t)stream) != hipSuccess)
    return JENGA_ERR_LAUNCH;
  return JENGA_OK;
}

int jenga_select_blocks(const jenga_problem* p, const float* block_scores, int mode, float param,
                        unsigned flags, int32_t* kept_idx, int32_t* n_kept, void* stream) {
  if (!p) return JENGA_ERR_INVALID_ARG;
  if (p->batch <= 0 || p->seq_len <= 0 || p->block <= 0) return JENGA_ERR_INVALID_ARG;
  if (p->seq_len % p->block != 0) return JENGA_ERR_UNSUPPORTED;
  const int nkb = p->seq_len / p->block;
  if (nkb > kMaxBlocks) return JENGA_ERR_UNSUPPORTED;
  if (!block_scores || !kept_idx || !n_kept) return JENGA_ERR_INVALID_ARG;
  if (mode != JENGA_SELECT_TOPK && mode != JENGA_SELECT_THRESH_REL && mode != JENGA_SELECT_THRESH_ABS)
    return JENGA_ERR_INVALID_ARG;
  if ((flags & ~JENGA_FORCE_FIRST_BLOCK) != 0) return JENGA_ERR_INVALID_ARG;
  if (mode == JENGA_SELECT_TOPK && !(param > 0.f)) return JENGA_ERR_INVALID_ARG;
  jenga::SelectParams sp;
  sp.scores = block_scores;
  sp.B = p->batch;
  sp.nkb = nkb;
  sp.mode = mode;
  sp.kcount = mode == JENGA_SELECT_TOPK ? jenga_topk_count(param, nkb) : 0;
  sp.param = param;
  sp.flags = flags;
  sp.kept_idx = kept_idx;
  sp.n_kept = n_kept;
  if (jenga::launch_select(sp, (hipStream_t)stream) != hipSuccess) return JENGA_ERR_LAUNCH;
  return JENGA_OK;
}

int jenga_sparse_attn_fwd(const jenga_problem* p, const void* q, const void* k, const void* v,
                          const int32_t* kept_idx, const int32_t* n_kept, int max_kept_blocks,
                          float* resid, void* o_saved, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream) {
  int st = check_problem(p, true);
  if (st != JENGA_OK) return st;
  const int nkb = p->seq_len / p->block;
  if (!q || !k || !v || !kept_idx || !n_kept || !resid || !o_saved || !lse)
    return JENGA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(resid) || !aligned16(o_saved))
    return JENGA_ERR_INVALID_ARG;
  if (max_kept_blocks < 1 || max_kept_blocks > nkb) return JENGA_ERR_INVALID_ARG;
  const FwdPlan plan = fwd_plan(p, max_kept_blocks);
  const size_t need = fwd_ws_bytes(p, max_kept_blocks, plan);
  if (need > 0 && (!workspace || workspace_bytes < need || ((uintptr_t)workspace % kAlign) != 0))
    return JENGA_ERR_WORKSPACE;
  jenga::FwdParams fp;
  fp.q = q;
  fp.k = k;
  fp.v = v;
  copy_strides(fp.qs, p->q_stride);
  copy_strides(fp.ks, p->k_stride);
  copy_strides(fp.vs, p->v_stride);
  fp.kept = kept_idx;
  fp.n_kept = n_kept;
  fp.resid = resid;
  fp.o_saved = o_saved;
  fp.lse = lse;
  fp.B = p->batch;
  fp.S = p->seq_len;
  fp.Hq = p->n_heads_q;
  fp.Hkv = p->n_heads_kv;
  fp.block = p->block;
  fp.nkb = nkb;
  fp.max_kept_blocks = max_kept_blocks;
  fp.ncap = max_kept_blocks * p->block;
  fp.scale_log2 = scale_of(p) * 1.4426950408889634f;
  fp.vtp = workspace;
  fp.wsPart = nullptr;
  fp.fs_items = plan.items;
  fp.fs_slots = 0;
  fp.fs_split_tiles = plan.split_tiles;
  if (p->dtype == JENGA_DTYPE_BF16) {
    fp.wsPart = (char*)workspace + fwd_vtp_bytes(p, max_kept_blocks);
    fp.fs_slots = plan.slots;
  }
  const hipError_t e = p->dtype == JENGA_DTYPE_BF16
                           ? jenga::launch_fwd64(fp, p->head_dim, (hipStream_t)stream)
                           : jenga::launch_fwd_f32(fp, (hipStream_t)stream);
  if (e != hipSuccess) return JENGA_ERR_LAUNCH;
  return JENGA_OK;
}

}  // extern "C"

namespace {

// The segmented backward behind both entry points.  With noalloc set, the workspace is this
// GPU's fixed scratch array, fetched only after every argument check has passed.
int bwd_segmented(const jenga_problem* p, const void* q, const void* k, const void* v,
                  const int32_t* kept_idx, const int32_t* n_kept, int max_kept_blocks,
                  const void* o_saved, const float* lse, const float* dout, float* dq, float* dk,
                  float* dv, int n_segments, void* workspace, size_t workspace_bytes, bool noalloc,
                  void* stream) {
  int st = check_problem(p, true);
  if (st != JENGA_OK) return st;
  const int nkb = p->seq_len / p->block;
  if (!q || !k || !v || !kept_idx || !n_kept || !o_saved || !lse || !dout || !dq || !dk || !dv)
    return JENGA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o_saved) || !aligned16(dout))
    return JENGA_ERR_INVALID_ARG;
  if (max_kept_blocks < 1 || max_kept_blocks > nkb) return JENGA_ERR_INVALID_ARG;
  const int ncap = max_kept_blocks * p->block;
  if (n_segments < 1 || n_segments > ncap / 64) return JENGA_ERR_INVALID_ARG;
  const size_t need = bwd_ws_min_bytes(p, max_kept_blocks, n_segments);
  const size_t need2 = bwd_ws_bytes(p, max_kept_blocks, n_segments);
  if (noalloc) {
    if (need > kNoAllocScratchBytes) return JENGA_ERR_SCRATCH_LIMIT;
    const int st2 = scratch_of_current_device(&workspace);
    if (st2 != JENGA_OK) return st2;
    workspace_bytes = kNoAllocScratchBytes;
  }
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace % kAlign) != 0)
    return JENGA_ERR_WORKSPACE;
  // two sets of segment buffers: each segment's launch also runs the next segment's prologue
  const bool overlap = need2 > need && workspace_bytes >= need2;
  const int L = seg_len_of(ncap, n_segments);
  const BwdLayout lay = bwd_layout(p, max_kept_blocks, n_segments);
  const size_t set_bytes = lay.total;              // one set of segment buffers
  jenga::BwdParams bp;
  bp.q = q;
  bp.k = k;
  bp.v = v;
  copy_strides(bp.qs, p->q_stride);
  copy_strides(bp.ks, p->k_stride);
  copy_strides(bp.vs, p->v_stride);
  bp.kept = kept_idx;
  bp.n_kept = n_kept;
  bp.o_saved = o_saved;
  bp.lse = lse;
  bp.dout = dout;
  bp.dq = dq;
  bp.dk = dk;
  bp.dv = dv;
  bp.wsD = (float*)((char*)workspace + lay.d);
  bp.wsL2 = (float*)((char*)workspace + lay.l2);
  bp.wsdO = (char*)workspace + lay.dO;
  bp.qtp = (char*)workspace + lay.qtp;
  bp.dotp = (char*)workspace + lay.dotp;
  bp.wsKv = (float*)((char*)workspace + (overlap ? 2 : 1) * set_bytes);
  bp.B = p->batch;
  bp.S = p->seq_len;
  bp.Hq = p->n_heads_q;
  bp.Hkv = p->n_heads_kv;
  bp.block = p->block;
  bp.nkb = nkb;
  bp.max_kept_blocks = max_kept_blocks;
  bp.ncap = ncap;
  bp.seg_len = L;
  bp.scale = scale_of(p);
  bp.scale_log2 = bp.scale * 1.4426950408889634f;
  const bool fast = p->dtype == JENGA_DTYPE_BF16;
  const int nrun = bwd_segments_run(p, max_kept_blocks, n_segments);
  const hipStream_t hs = (hipStream_t)stream;
  if (overlap) {
    // segment s reads buffer set s % 2; its launch fills set (s + 1) % 2 for segment s + 1
    auto seg_params = [&](int s) {
      jenga::BwdParams x = bp;
      const size_t off = (s % 2) ? set_bytes : 0;
      x.wsD = (float*)((char*)bp.wsD + off);
      x.wsL2 = (float*)((char*)bp.wsL2 + off);
      x.wsdO = (char*)bp.wsdO + off;
      x.qtp = (char*)bp.qtp + off;
      x.dotp = (char*)bp.dotp + off;
      x.seg = s;
      return x;
    };
    jenga::BwdParams cur = seg_params(0);
    if (jenga::launch_prep64(cur, p->head_dim, hs) != hipSuccess) return JENGA_ERR_LAUNCH;
    for (int s = 0; s < nrun; ++s) {
      const jenga::BwdParams nxt = seg_params(s + 1);
      if (jenga::launch_bwd64_main(cur, s + 1 < nrun ? &nxt : nullptr, p->head_dim, hs) != hipSuccess)
        return JENGA_ERR_LAUNCH;
      cur = nxt;
    }
    return JENGA_OK;
  }
  for (int s = 0; s < nrun; ++s) {
    bp.seg = s;
    hipError_t e;
    if (fast) {
      e = jenga::launch_prep64(bp, p->head_dim, hs);
      if (e == hipSuccess) e = jenga::launch_bwd64_main(bp, nullptr, p->head_dim, hs);
    } else {
      e = jenga::launch_bwd_segment_f32(bp, hs);
    }
    if (e != hipSuccess) return JENGA_ERR_LAUNCH;
  }
  return JENGA_OK;
}

}  // namespace

extern "C" {

int jenga_sparse_attn_bwd_segmented(const jenga_problem* p, const void* q, const void* k,
                                    const void* v, const int32_t* kept_idx, const int32_t* n_kept,
                                    int max_kept_blocks, const void* o_saved, const float* lse,
                                    const float* dout, float* dq, float* dk, float* dv,
                                    int n_segments, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  return bwd_segmented(p, q, k, v, kept_idx, n_kept, max_kept_blocks, o_saved, lse, dout, dq, dk,
                       dv, n_segments, workspace, workspace_bytes, false, stream);
}

int jenga_sparse_attn_bwd_segmented_noalloc(const jenga_problem* p, const void* q, const void* k,
                                            const void* v, const int32_t* kept_idx,
                                            const int32_t* n_kept, int max_kept_blocks,
                                            const void* o_saved, const float* lse,
                                            const float* dout, float* dq, float* dk, float* dv,
                                            int n_segments, void* stream) {
  return bwd_segmented(p, q, k, v, kept_idx, n_kept, max_kept_blocks, o_saved, lse, dout, dq, dk,
                       dv, n_segments, nullptr, 0, true, stream);
}


int jenga_proj_gather(const jenga_proj_problem* p, const void* x, const void* w,
                      const int32_t* kept_idx, const int32_t* n_kept, int max_kept_blocks,
                      void* y, void* stream) {
  const int st = check_proj(p, x, w, kept_idx, n_kept, max_kept_blocks, y, 2);
  if (st != JENGA_OK) return st;
  const jenga::ProjParams pp = proj_params(p, x, w, kept_idx, n_kept, max_kept_blocks, y);
  return jenga::launch_proj(pp, jenga::kGather, "k_proj_gather", (hipStream_t)stream) == hipSuccess
             ? JENGA_OK : JENGA_ERR_LAUNCH;
}

int jenga_proj_scatter_add(const jenga_proj_problem* p, const void* y, const void* w,
                           const int32_t* kept_idx, const int32_t* n_kept, int max_kept_blocks,
                           float* resid, void* stream) {
  const int st = check_proj(p, y, w, kept_idx, n_kept, max_kept_blocks, resid, 4);
  if (st != JENGA_OK) return st;
  const jenga::ProjParams pp = proj_params(p, y, w, kept_idx, n_kept, max_kept_blocks, resid);
  return jenga::launch_proj(pp, jenga::kScatter, "k_proj_scatter", (hipStream_t)stream) == hipSuccess
             ? JENGA_OK : JENGA_ERR_LAUNCH;
}

int jenga_proj_gather_scatter_add(const jenga_proj_problem* p, const void* a, const void* w,
                                  const int32_t* kept_idx, const int32_t* n_kept,
                                  int max_kept_blocks, float* resid, void* stream) {
  const int st = check_proj(p, a, w, kept_idx, n_kept, max_kept_blocks, resid, 4);
  if (st != JENGA_OK) return st;
  const jenga::ProjParams pp = proj_params(p, a, w, kept_idx, n_kept, max_kept_blocks, resid);
  return jenga::launch_proj(pp, jenga::kGatherScatter, "k_proj_gather_scatter",
                            (hipStream_t)stream) == hipSuccess
             ? JENGA_OK : JENGA_ERR_LAUNCH;
}

size_t jenga_mlp_workspace_bytes(const jenga_proj_problem* p, int kind) {
  if (check_mlp(p, kind) != JENGA_OK) return 0;
  return mlp_ws_bytes(p);
}

int jenga_mlp_act_scores(const jenga_proj_problem* p, int kind, const void* x, const void* w1,
                         const void* w_up, void* act, float* token_scores, float* block_scores,
                         void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_mlp(p, kind);
  if (st != JENGA_OK) return st;
  if (!x || !w1 || !act || !token_scores || !block_scores) return JENGA_ERR_INVALID_ARG;
  if (kind == JENGA_MLP_SILU_GATED && (!w_up || !aligned16(w_up))) return JENGA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w1) || !aligned16(act)) return JENGA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < mlp_ws_bytes(p) || ((uintptr_t)workspace % kAlign) != 0)
    return JENGA_ERR_WORKSPACE;
  const hipStream_t s = (hipStream_t)stream;
  jenga::ProjParams pp{};
  pp.a = x;
  pp.as0 = p->in_stride[0];
  pp.as1 = p->in_stride[1];
  pp.w = w1;
  pp.w2 = w_up;
  pp.out = act;
  pp.os0 = p->out_stride[0];
  pp.os1 = p->out_stride[1];
  pp.B = p->batch;
  pp.S = p->seq_len;
  pp.K = p->in_features;
  pp.N = p->out_features;
  pp.block = p->block;
  pp.nkb = p->seq_len / p->block;
  pp.rows = p->seq_len;
  pp.part = (float*)workspace;
  const int mode = kind == JENGA_MLP_SILU_GATED ? jenga::kMlpGated : jenga::kMlpRelu;
  if (jenga::launch_proj(pp, mode, kind == JENGA_MLP_SILU_GATED ? "k_mlp_act_gated" : "k_mlp_act_relu",
                         s) != hipSuccess)
    return JENGA_ERR_LAUNCH;
  jenga::MlpBlockParams bp;
  bp.part = pp.part;
  bp.B = p->batch;
  bp.S = p->seq_len;
  bp.ncg = p->out_features / 32;
  bp.F = p->out_features;
  bp.block = p->block;
  bp.nkb = pp.nkb;
  bp.token_scores = token_scores;
  bp.block_scores = block_scores;
  return jenga::launch_mlp_block(bp, s) == hipSuccess ? JENGA_OK : JENGA_ERR_LAUNCH;
}

size_t jenga_loss_workspace_bytes(const jenga_loss_problem* p) {
  if (check_loss(p) != JENGA_OK) return 0;
  return loss_ws_bytes(p);
}

int jenga_lm_head_ce_segmented(const jenga_loss_problem* p, const void* h, const void* w,
                               const void* wt, const int32_t* targets, float* row_loss,
                               float* loss, float* dh, void* workspace, size_t workspace_bytes,
                               void* stream) {
  const int st0 = check_loss(p);
  if (st0 != JENGA_OK) return st0;
  if (!h || !w || !wt || !targets || !row_loss || !loss || !dh) return JENGA_ERR_INVALID_ARG;
  if (!aligned16(h) || !aligned16(w) || !aligned16(wt) || !aligned16(dh)) return JENGA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < loss_ws_bytes(p) || ((uintptr_t)workspace % kAlign) != 0)
    return JENGA_ERR_WORKSPACE;
  const hipStream_t s = (hipStream_t)stream;
  const int T = p->tokens, d = p->d_model, V = p->vocab, L = loss_rows(p);
  float* logits = (float*)workspace;
  void* glog = (char*)workspace + align_up((size_t)L * V * sizeof(float));
  for (int seg = 0; seg < p->n_segments; ++seg) {
    const int r0 = seg * L;
    const int rows = r0 < T ? (T - r0 < L ? T - r0 : L) : 0;
    if (rows <= 0) break;
    jenga::ProjParams g1{};                                   // logits = h_seg w^T
    g1.a = (const char*)h + (size_t)r0 * d * 2;
    g1.as1 = d;
    g1.w = w;
    g1.out = logits;
    g1.os1 = V;
    g1.B = 1;
    g1.K = d;
    g1.N = V;
    g1.rows = rows;
    if (jenga::launch_proj(g1, jenga::kPlain, "k_proj_logits", s) != hipSuccess) return JENGA_ERR_LAUNCH;
    jenga::CeParams ce;
    ce.logits = logits;
    ce.targets = targets + r0;
    ce.row_loss = row_loss + r0;
    ce.dlogits = glog;
    ce.rows = rows;
    ce.V = V;
    ce.grad_scale = 1.0f / (float)T;
    if (jenga::launch_ce_rows(ce, s) != hipSuccess) return JENGA_ERR_LAUNCH;
    jenga::ProjParams g2{};                                   // dh_seg = g w  (w^T rows)
    g2.a = glog;
    g2.as1 = V;
    g2.w = wt;
    g2.out = dh + (size_t)r0 * d;
    g2.os1 = d;
    g2.B = 1;
    g2.K = V;
    g2.N = d;
    g2.rows = rows;
    if (jenga::launch_proj(g2, jenga::kPlain, "k_proj_dh", s) != hipSuccess) return JENGA_ERR_LAUNCH;
  }
  if (jenga::launch_loss_mean(row_loss, T, loss, s) != hipSuccess) return JENGA_ERR_LAUNCH;
  return JENGA_OK;
}

int jenga_timing_enable(int enable) {
  if (enable != 0 && enable != 1) return JENGA_ERR_INVALID_ARG;
  jenga::timing_set(enable == 1);
  return JENGA_OK;
}

int jenga_timing_query(const char* kernel, int32_t* launches, double* total_ms) {
  if (!kernel || !launches || !total_ms) return JENGA_ERR_INVALID_ARG;
  int n = 0;
  double t = 0.0;
  if (jenga::timing_query(kernel, &n, &t) != hipSuccess) return JENGA_ERR_LAUNCH;
  *launches = n;
  *total_ms = t;
  return JENGA_OK;
}

}  // extern "C"
