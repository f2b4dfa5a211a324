// Launch interface between the C ABI layer (api.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jenga {

struct ScoreParams {
  const void* q;
  const void* k;
  int64_t qs[3], ks[3];
  int B, S, Hq, Hkv, block;
  float scale_log2;   // softmax scale * log2(e)
  float* lse2;        // workspace [B][Hq][S]: log2-domain row normaliser
  double* mass32;     // workspace [B][Hq][S/32]: received mass per group of keys
  float* lpart;       // workspace, bf16 path: per (batch, head) the causal triangle of partial
                      // log2-sums, row n (key block n) holding queries n*block .. S-1
  int mass_gpb;       // mass32 groups per key block (set by launch_score)
  float* scores;      // [B][S/block]
};

struct Eq2Params {
  const void* q;
  const void* k;
  int64_t qs[3], ks[3];
  int B, S, Hq, Hkv, block, nkb;
  float scale;        // softmax scale
  float* tilemax;     // workspace [B][nkb][nkb]: score-block maxima (query block, key block)
  float* scores;      // [B][nkb]
};

enum ProjMode { kGather = 0, kScatter = 1, kPlain = 2, kGatherScatter = 3, kMlpGated = 4, kMlpRelu = 5 };

struct ProjParams {
  const void* a;        // bf16 input rows: gathered x [B][S][K] or compact y [B][Ncap][K]
  int64_t as0, as1;     // element strides of a: batch, row
  const void* w;        // bf16 [N][K], contiguous
  void* out;            // bf16 compact [B][Ncap][N] (gather) or fp32 resid [B][S][N] (scatter)
  int64_t os0, os1;     // element strides of out: batch, row
  const int32_t* kept;
  const int32_t* n_kept;
  int B, S, K, N, block, nkb, max_kept_blocks, ncap;
  int rows;             // plain and MLP modes: rows of a per batch row (a multiple of 32)
  const void* w2;       // MLP gated mode: the up projection [N][K] (w is the gate projection)
  float* part;          // MLP modes: [B][N/32][rows] sums of |activation| per 32 units
};

struct MlpBlockParams {
  const float* part;    // [B][ncg][S]
  int B, S, ncg, F, block, nkb;
  float* token_scores;  // [B][S]
  float* block_scores;  // [B][nkb]
};

struct CeParams {
  const float* logits;  // [rows][V] fp32
  const int32_t* targets;  // [rows]
  float* row_loss;      // [rows]
  void* dlogits;        // bf16 [rows][V]: (softmax - onehot) * grad_scale
  int rows, V;
  float grad_scale;     // 1 / total rows of the mean
};

struct SelectParams {
  const float* scores;
  int B, nkb, mode, kcount;
  float param;
  unsigned flags;
  int32_t* kept_idx;
  int32_t* n_kept;
};

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  int64_t qs[3], ks[3], vs[3];
  const int32_t* kept;
  const int32_t* n_kept;
  float* resid;
  void* o_saved;
  float* lse;
  void* vtp;     // bf16 path: workspace [B][Hkv][ncap/32] TP tiles of the kept V rows
  int B, S, Hq, Hkv, block, nkb, max_kept_blocks, ncap;
  float scale_log2;
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  int64_t qs[3], ks[3], vs[3];
  const int32_t* kept;
  const int32_t* n_kept;
  const void* o_saved;
  const float* lse;
  const float* dout;
  float* dq;
  float* dk;
  float* dv;
  float* wsD;    // [B][Hq][L]   dot(dO, O) of the segment's queries
  float* wsL2;   // bf16 path: [B][Hq][L] lse of the segment's queries in the log2 domain
  void* wsdO;    // [B][L][Hq][D] dOut rows of the segment in operand dtype, by kept rank
  void* qtp;     // bf16 path: [B][Hq][L/32] TP tiles of the segment's Q rows
  void* dotp;    // bf16 path: [B][Hq][L/32] TP tiles of the segment's dOut rows (bf16)
  int B, S, Hq, Hkv, block, nkb, max_kept_blocks, ncap, seg_len, seg;
  float scale, scale_log2;
};

// Workgroup runs of the fused backward launch of one segment (computed on the host): the dQ
// tiles, then the dK/dV key tiles; o_kv is the launch offset of the second run (a multiple of 8).
struct BwdGrid {
  int nqt, nkt;                // dQ tiles per query head; dK/dV key tiles per KV head
  int n_dq, n_kv;              // workgroups of each run (all heads and batch rows)
  int o_kv;
};


// dtype: 0 = fp32 operands, 1 = bf16 operands.  Each returns hipGetLastError().
hipError_t launch_score(const ScoreParams& p, int dtype, int D, hipStream_t st);
hipError_t launch_select(const SelectParams& p, hipStream_t st);
hipError_t launch_fwd(const FwdParams& p, int dtype, int D, hipStream_t st);
hipError_t launch_bwd_segment(const BwdParams& p, int dtype, int D, hipStream_t st);

// bf16 scoring with async LDS staging (score64.hip)
hipError_t launch_score64(const ScoreParams& p, int D, hipStream_t st);

// projections (proj.hip): gathered input rows, scatter-add into resid, or plain rows
hipError_t launch_proj(const ProjParams& p, int mode, const char* name, hipStream_t st);

hipError_t launch_mlp_block(const MlpBlockParams& p, hipStream_t st);

// language-model-head loss (loss.hip)
hipError_t launch_ce_rows(const CeParams& p, hipStream_t st);
hipError_t launch_loss_mean(const float* row_loss, int rows, float* loss, hipStream_t st);

// bf16 Eq. 2 literal scoring (eq2.hip): block 64 or 128
hipError_t launch_score_eq2(const Eq2Params& p, int D, int block, hipStream_t st);

// Per-kernel event timing (timing.cpp).  A TimedLaunch placed around a launch records a start
// event on construction and a stop event on destruction when timing is enabled.
class TimedLaunch {
 public:
  TimedLaunch(const char* name, hipStream_t st);
  ~TimedLaunch();
  TimedLaunch(const TimedLaunch&) = delete;
  TimedLaunch& operator=(const TimedLaunch&) = delete;

 private:
  hipStream_t st_;
  long idx_;
};
bool timing_enabled();
void timing_set(bool on);
hipError_t timing_query(const char* name, int* launches, double* total_ms);

// bf16 attention kernels (attn64.hip)
hipError_t launch_fwd64(const FwdParams& p, int D, hipStream_t st);
hipError_t launch_bwd64_segment(const BwdParams& p, int D, hipStream_t st);

}  // namespace jenga
