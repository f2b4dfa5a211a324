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
  float* lpart;       // workspace, bf16 path: [B][Hq][S/block][chunk] partial log2-sums of the
                      // queries of one query chunk, row n (key block n), column i - q_begin
  int chunk;          // bf16 path: queries per scoring chunk (a multiple of 128)
  int q_begin, q_end; // bf16 path: the query chunk of one launch pair (set by launch_score64)
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
  char* wsPart;  // bf16 path: [B][Hq][fs_slots] slots of split query tiles' parts (FwdSlot)
  int B, S, Hq, Hkv, block, nkb, max_kept_blocks, ncap;
  float scale_log2;
  // the split plan's bounds (fwd_split_bounds) for ncap, Hq, B
  int fs_items;        // workgroups per (batch row, query head) of the forward launch
  int fs_slots;        // part slots per (batch row, query head); 0: no query tile is split
  int fs_split_tiles;  // split tiles per (batch row, query head)
};

// A causal forward over few kept tokens lasts as long as its longest query tile, the last one,
// whose queries see every kept key.  When a batch row's longest tile holds more than twice the
// mean work per workgroup slot of the launch, the row's tiles longer than a part run in parts
// over equal ranges of their key steps.  Each part writes its unnormalised output rows and their
// running max and sum to a slot; k_fwd_combine merges a tile's parts in part order (a fixed
// order) and writes the residual, o_saved and lse as the whole tile would.  The plan follows each
// row's own kept count (read on the device), so no host synchronisation is needed; the host
// sizes the grid and the slots for the worst count up to the capacity.  A query tile is 128
// kept queries, a step 32 kept keys; three workgroups share a compute unit.
constexpr int kFwdRows = 128;
constexpr int kFwdWgPerCu = 3;
constexpr int kFwdMinPartSteps = 32;

// key steps of query tile t of a batch row with nk kept ranks (nk > t * kFwdRows)
__host__ __device__ inline int fwd_tile_steps(int t, int nk) {
  const int end = (t + 1) * kFwdRows < nk ? (t + 1) * kFwdRows : nk;
  return (end - 1) / 32 + 1;
}
// Whether a row of ntiles query tiles splits, with HqB = query heads x batch rows workgroups per
// tile index (every row taken to be alike).  Its tiles hold 2 ntiles (ntiles + 1) steps, so the
// mean per workgroup slot is 2 ntiles (ntiles + 1) HqB / (256 kFwdWgPerCu); the longest tile,
// 4 ntiles steps, exceeds twice that exactly when (ntiles + 1) HqB < 256 kFwdWgPerCu.
__host__ __device__ inline bool fwd_row_splits(int ntiles, int HqB) {
  return (long long)(ntiles + 1) * HqB < 256 * kFwdWgPerCu;
}
// Steps per part: that mean, and no fewer than kFwdMinPartSteps.  Since a tile longer than a part
// of T steps makes ceil(s / T) <= 2 s / T parts, a row's slots stay below 4 ntiles (ntiles + 1) / T
// <= 2 * 256 kFwdWgPerCu / HqB, whatever the shape.
__host__ __device__ inline int fwd_part_steps(int ntiles, int HqB) {
  const long long slots = 256 * kFwdWgPerCu;
  const long long mean = (2LL * ntiles * (ntiles + 1) * HqB + slots - 1) / slots;
  return mean > kFwdMinPartSteps ? (int)mean : kFwdMinPartSteps;
}
__host__ __device__ inline int fwd_tile_parts(int steps, int part_steps) {
  return (steps + part_steps - 1) / part_steps;
}
// A part's slot: its 128 unnormalised output rows in bf16 (D values each), then the rows'
// running maxima and sums in fp32.  bf16 rows halve the slot traffic, which a merge pays on top
// of the unsplit tile's; they round as the P operand of the P V product already did.
template <int D>
struct FwdSlot {
  static constexpr int64_t O_BYTES = (int64_t)kFwdRows * D * 2;
  static constexpr int64_t BYTES = O_BYTES + (int64_t)kFwdRows * 8;
};
// Worst case over the kept counts up to ncap: workgroups per (batch row, query head) of the
// forward launch, part slots and split tiles per (batch row, query head).
void fwd_split_bounds(int ncap, int Hq, int B, int* items, int* slots, int* split_tiles);

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
  float* wsKv;   // bf16 path: [B][Hkv][extra parts][2][256][D] sums of split dK/dV tiles
  int B, S, Hq, Hkv, block, nkb, max_kept_blocks, ncap, seg_len, seg;
  float scale, scale_log2;
};

// Workgroup runs of the fused backward launch of one segment (computed on the host): the dQ
// tiles, then the dK/dV key tiles, then (when the next segment's prologue rides along) its
// 32-rank groups, two per workgroup; o_kv and o_prep are the launch offsets of the second and
// third runs (multiples of 8).
struct BwdGrid {
  int nqt, nkt;                // dQ tiles per query head; dK/dV key tiles per KV head
  int n_dq, n_kv;              // workgroups of the first two runs (all heads and batch rows)
  int o_dq, o_kv, o_prep;
  int ng;                      // prologue groups per (batch row, head) of the next segment
  int seg_end;                 // end of the segment's ranks at full capacity
  int kv_target;               // steps per part of a split dK/dV tile (0: no tile is split)
  int nki, n_extra;            // dK/dV workgroups and extra parts per (batch row, KV head)
};

// Long dK/dV key tiles of the bf16 backward run in parts.  A key tile's steps are the query
// rows of the segment at or after its keys (32 per step) times the query heads of its KV
// group; at full capacity its step count follows from the segment alone.  When a tile would
// have more steps than the launch's average load per compute unit (grouped-query attention
// with one segment: the first key tiles take every query of four heads), it runs as parts over
// consecutive ranges of its steps.  Part 0 adds into dk/dv as a whole tile does;
// parts 1.. write their sums to slots, which k_kv_reduce adds after the launch in part order --
// a fixed order, so results still repeat bit for bit.
constexpr int kKvKeys = 256;           // keys per dK/dV tile (8 waves x 32)
constexpr int kKvMaxParts = 8;
constexpr int kComputeUnits = 256;     // MI355X

__host__ __device__ inline int kv_tile_steps(int tx, int qs, int seg_end, int G) {
  const int from = qs > kKvKeys * tx ? qs : kKvKeys * tx;
  return from < seg_end ? G * ((seg_end - from) / 32) : 0;
}
__host__ __device__ inline int kv_tile_parts(int steps, int target) {
  if (target <= 0) return 1;
  const int n = (steps + target - 1) / target;
  return n < 1 ? 1 : (n > kKvMaxParts ? kKvMaxParts : n);
}
// Steps per part for the segment of ranks [qs, qs + seg_cap) (0: no split), and the extra
// parts per (batch row, KV head) it makes.
int kv_split_target(int qs, int seg_cap, int G, int Hq, int Hkv, int B);
int kv_split_extra(int qs, int seg_cap, int G, int target);


// dtype: 0 = fp32 operands, 1 = bf16 operands.  Each returns hipGetLastError().
hipError_t launch_score(const ScoreParams& p, int dtype, int D, hipStream_t st);
hipError_t launch_select(const SelectParams& p, hipStream_t st);
// fp32 attention, head_dim 64 (attn_fwd.hip, attn_bwd.hip)
hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t st);
hipError_t launch_bwd_segment_f32(const BwdParams& p, hipStream_t st);

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
// One segment's backward: the prologue of segment p.seg (launch_prep64), then its dQ and dK/dV
// tiles (launch_bwd64_main).  With `next` given, the main launch also runs the prologue of
// segment next->seg, which must write a workspace other than p's.
hipError_t launch_prep64(const BwdParams& p, int D, hipStream_t st);
hipError_t launch_bwd64_main(const BwdParams& p, const BwdParams* next, int D, hipStream_t st);

}  // namespace jenga
