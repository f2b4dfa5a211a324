// bf16 token-sparse attention forward and segmented backward for gfx950.
//
// Jenga (papercache notes, §4.4): kept rows are addressed in place through the kept-block
// list (permutation-free token movement), the forward adds its output into the residual in
// place, and the backward runs segment by segment (segment-based peak cutting).
//
// Every wave owns 32 rows (one 32x32 MFMA block); waves of a workgroup share K / V / Q / dO
// tiles that direct-to-LDS loads stage through a ring of LDS buffers while earlier tiles are
// consumed.  Operands that reduce over head_dim are 16-byte reads of natural tiles.  Operands
// that reduce over rows are 16-byte reads of TP tiles prepared in global memory (V in the
// forward, Q and dO in the dK/dV tiles), or, in the dQ tiles, two transposing 8-byte reads of
// the natural K tile (see tiles64.h).
//
//   k_pack_tp   kept rows of V (head h) -> TP tiles [D][32] in a workspace (forward)
//   k_fwd64     forward:   S^T = K Q^T, online softmax per query (lane-local), O^T += V^T P^T;
//               rows with few kept tokens run their long query tiles in parts over key ranges
//   k_fwd_combine  after a forward with split tiles: merges each tile's parts in part order
//   k_prep64    backward prologue per segment: D_i = dO_i.O_i, dOut -> bf16 natural + TP,
//               the segment's Q rows -> TP
//   k_bwd64     one launch per segment with two kinds of workgroup tiles (no atomics):
//                 dK/dV, key-major:   S = Q K^T, dP = dO V^T, dV += P^T dO, dK += dS^T Q
//                 dQ, query-major:    S^T = K Q^T, dP^T = V dO^T, dQ += dS K
//               and, when two sets of segment buffers are given, the next segment's prologue
//   k_kv_reduce after a launch whose long dK/dV tiles ran in parts: adds the parts' sums
#include "common.h"
#include "kernels.h"
#include "tiles64.h"

namespace jenga {

struct PackArgs {
  const void* src;
  int64_t s0, s1, s2;        // element strides of src: batch, token, head
  const int32_t* kept;
  const int32_t* n_kept;
  int block, nkb, max_kept_blocks;
  int rank0, rank_count;     // tiles cover kept ranks [rank0, rank0 + rank_count)
  int tiles_per_head, H;
  void* dst;                 // [B][H][tiles_per_head][D][32] bf16
};

// ------------------------------------------------------------------------------------------
// Write a 32-row natural tile staged in LDS (row pitch D + 8 elements) as its TP tile [D][32]
// at dst; 256 threads (index tid) write 16 bytes each per pass.
template <int D>
__device__ __forceinline__ void write_tp_tile(const bf16* tile, char* dst, int tid) {
  constexpr int PITCH = D + 8;
  for (int idx = tid; idx < D * 4; idx += 256) {
    const int d = idx >> 2, c = idx & 3;
    uint16_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = __builtin_bit_cast(uint16_t, tile[pi16(8 * c + e) * PITCH + d]);
    u32x4 wv;
    wv[0] = v[0] | ((uint32_t)v[1] << 16);
    wv[1] = v[2] | ((uint32_t)v[3] << 16);
    wv[2] = v[4] | ((uint32_t)v[5] << 16);
    wv[3] = v[6] | ((uint32_t)v[7] << 16);
    *(u32x4*)(dst + d * 64 + c * 16) = wv;
  }
}

template <int D>
__global__ __launch_bounds__(256) void k_pack_tp(PackArgs a) {
  constexpr int PITCH = D + 8;                        // elements; breaks bank aliasing
  __shared__ bf16 tile[32 * PITCH];
  const int b = blockIdx.z, h = blockIdx.y, t = blockIdx.x, tid = threadIdx.x;
  const int32_t* kept = a.kept + (int64_t)b * a.nkb;
  const int Nk = min(a.n_kept[b], a.max_kept_blocks) * a.block;
  const int r0 = a.rank0 + 32 * t;
  const int rend = min(a.rank0 + a.rank_count, Nk);
  if (r0 >= rend) return;
  const int pos0 = rank_to_pos(kept, a.block, r0);
  const bf16* src = (const bf16*)a.src + b * a.s0 + h * a.s2;
  constexpr int CPR = D / 8;
  for (int idx = tid; idx < 32 * CPR; idx += 256) {
    const int row = idx / CPR, c = idx % CPR;
    *(u32x4*)(tile + row * PITCH + c * 8) = ld16(src + (int64_t)(pos0 + row) * a.s1 + c * 8);
  }
  __syncthreads();
  write_tp_tile<D>(tile, (char*)a.dst + ((((int64_t)b * a.H + h) * a.tiles_per_head + t) * D) * 64, tid);
}

template <int D>
static hipError_t pack_tp(const PackArgs& a, int B, hipStream_t st) {
  const int ntiles = (a.rank_count + 31) / 32;
  if (ntiles <= 0) return hipSuccess;
  TimedLaunch tl("k_pack_tp", st);
  k_pack_tp<D><<<dim3(ntiles, a.H, B), 256, 0, st>>>(a);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Forward
// ------------------------------------------------------------------------------------------
// Rescaling of the running output is deferred while the running max grows by less than
// kLazyRescale (log2 units): exp2(z - m) then stays below 2^kLazyRescale, far inside fp32 and
// bf16 range, and the final normalisation uses the same stale max, so the result is exact.
constexpr float kLazyRescale = 8.f;
constexpr float kLazyCheck = 128.f;    // 2^7: a lane sum above it may need the rule

// SPLIT: the instance for launches where some batch row's long query tiles run in parts (see
// fwd_row_splits); workgroup x of a (head, batch row) then takes the row's tiles heaviest first
// and each tile as its parts.  Without it, workgroup x takes tile nqt - 1 - x.
// Three waves per SIMD, the occupancy the three-buffer ring's LDS allows anyway: the bound keeps
// the compiler within that occupancy's 168 registers.
template <int D, int NB, int NW, bool SPLIT>
__global__ __launch_bounds__(64 * NW, NB == 1 ? 3 : 1) void k_fwd64(FwdParams p) {
  constexpr int RW = 32 * NB, RG = RW * NW;                // rows per wave / per workgroup
  using C = T64<D>;
  constexpr int OFF_V = C::NAT32;
  constexpr int STAGE = C::NAT32 + C::TP32;
  using DC = DmaCount<D, NW>;
  constexpr int PER = DC::NAT_W + DC::TP_W;     // direct-to-LDS instructions per wave per step
  __shared__ __attribute__((aligned(1024))) char sA[STAGE];
  __shared__ __attribute__((aligned(1024))) char sB[STAGE];
  __shared__ __attribute__((aligned(1024))) char sC[STAGE];
  __shared__ int ktab[kKeptTab];

  const Tile3 tl = xcd_tile_weight_major();
  const int b = tl.z, h = tl.y;
  const int g = h / (p.Hq / p.Hkv);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, hl = l >> 5, lc = l & 31;
  const int32_t* kept = p.kept + (int64_t)b * p.nkb;
  const int Nk = min(p.n_kept[b], p.max_kept_blocks) * p.block;
  const int nqt = (Nk + RG - 1) / RG;
  int tile, part = 0, nparts = 1, sbase = 0;             // slots of the row's earlier split tiles
  if (SPLIT && fwd_row_splits(nqt, p.Hq * p.B)) {
    static_assert(!SPLIT || RG == kFwdRows, "the split plan counts 128-query tiles");
    const int T = fwd_part_steps(nqt, p.Hq * p.B);
    int rem = tl.x;
    for (tile = nqt - 1;; --tile) {                      // heaviest tiles first, each as its parts
      if (tile < 0) return;
      nparts = fwd_tile_parts(fwd_tile_steps(tile, Nk), T);
      if (rem < nparts) break;
      rem -= nparts;
    }
    part = rem;
    if (nparts > 1)
      for (int u = 0; u < tile; ++u) {
        const int k = fwd_tile_parts(fwd_tile_steps(u, Nk), T);
        if (k > 1) sbase += k;
      }
  } else {
    if (tl.x >= nqt) return;
    tile = nqt - 1 - tl.x;                               // heaviest tiles first
  }
  const int q0 = tile * RG;
  const int qw0 = q0 + RW * w;
  const bool active = qw0 < Nk;                          // Nk is a multiple of 64 >= RW
  const int qlast = min(q0 + RG, Nk) - 1;
  const int tsteps = qlast / 32 + 1;
  // this part's key steps: an equal share of the tile's (the whole tile when not split)
  const int s0 = part * tsteps / nparts;
  const int nsteps = (part + 1) * tsteps / nparts - s0;
  stage_kept(ktab, kept, qlast / p.block + 1);
  __syncthreads();
  const KeptTab kt{(const LDS_AS int*)ktab, kept, p.block};

  bf16x8 qf[NB][C::NS];
  int qpos[NB];
  if (active) {
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
      qpos[qb] = kt.pos(qw0 + 32 * qb + lc);
      const char* qrow = (const char*)((const bf16*)p.q + b * p.qs[0] + (int64_t)qpos[qb] * p.qs[1] +
                                       h * p.qs[2]);
#pragma unroll
      for (int s = 0; s < C::NS; ++s) qf[qb][s] = *(const bf16x8*)(qrow + (16 * s + 8 * hl) * 2);
    }
  }
  // retire the register operand loads now: a load still pending when the staged loop starts
  // would make the compiler wait for all vector memory, prefetched tiles included, at its first
  // use in every iteration
  wait_all_mem();
  f32x16 o[NB][C::NDB];
#pragma unroll
  for (int qb = 0; qb < NB; ++qb)
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) o[qb][db] = zero16();
  float m_run[NB], l_run[NB];                               // log2 domain
#pragma unroll
  for (int qb = 0; qb < NB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
  }

  const char* kbase = (const char*)((const bf16*)p.k + b * p.ks[0] + g * p.ks[2]);
  const int64_t kstride = p.ks[1] * 2;
  const char* vtp = (const char*)p.vtp + (((int64_t)b * p.Hkv + g) * (p.ncap / 32)) * C::TP32;
  const float c2 = p.scale_log2;
  NatPlan<D, NW> kplan;
  kplan.init(kstride);
  TpPlan<D, NW> vplan;
  vplan.init();
  ReadPlan<D> rp;
  rp.init();

  const rsrc_t rk = make_rsrc(kbase), rv = make_rsrc(vtp);
  // steps are issued in order s0, s0 + 1, ..., then the last one again (reloads past the end)
  StepPos sp;
  sp.init(32 * s0, p.block);
  auto issue = [&](int step, char* buf) {
    kplan.issue(buf, rk, (uint32_t)(sp.pos(kt) * kstride));
    vplan.issue(buf + OFF_V, rv, (uint32_t)(step * C::TP32));
    if (step < s0 + nsteps - 1) sp.advance(p.block);
  };

  auto compute = [&](int step, const char* buf) {
    const int kr0 = step * 32;
    if (!active || kr0 > qw0 + RW - 1) return;
    const char* Kl = buf;
    const char* Vl = buf + OFF_V;
    f32x16 st[NB];
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) st[qb] = zero16();
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
      const bf16x8 a = ldo(Kl, rp.nat[s]);
#pragma unroll
      for (int qb = 0; qb < NB; ++qb) st[qb] = Mfma<bf16>::mma(a, qf[qb][s], st[qb]);
    }
    SCHED_READS_AHEAD(C::NS, 1, NB, 0);
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
      if (kr0 + 31 > qw0 + 32 * qb) {                      // diagonal step: causal mask
        // key kr0 + 8(r/4) + 4hl + r%4 > query qw0 + 32qb + lc  <=>  8(r/4) + r%4 > lim
        const int lim = qw0 + 32 * qb + lc - kr0 - 4 * hl;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (8 * (r >> 2) + (r & 3) > lim) st[qb][r] = -INFINITY;
      }
      // P against the current reference max, and its lane sum (no addition of 0 to start)
      f32x16 pe;
      float rs;
      auto exps = [&]() {
        const float m = m_run[qb];
#pragma unroll
        for (int r = 0; r < 16; ++r) pe[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[qb][r], c2, -m));
        rs = pe[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) rs += pe[r];
      };
      exps();
      // Lazy rescale: the reference max moves only when the row max grows by kLazyRescale or
      // more.  Then the lane holding that max has an exponential above 2^7.8 (while
      // |m_run| < 2^20, m_run + 8 and max * c2 each round within 2^-4 and the fma once), so
      // a wave whose lane sums all stay at or below 2^7 cannot need the rescale and skips the
      // row max; where the rule is checked the values are those of taking the max first, and
      // a moved reference forms P again.  (The first step, against -inf, always checks: a lane
      // with a masked key sums to NaN there, but the wave's last query sees its whole first
      // step, so its lanes sum to +inf.  Past 2^20 a missed check leaves every value of P below
      // 2^7: the reference lags, still exact.)
      if (__builtin_amdgcn_ballot_w64(rs > kLazyCheck) != 0) {
        const float mx = half_pair_max(max16(st[qb])) * c2;  // row max in the log2 domain
        if (__builtin_amdgcn_ballot_w64(mx > m_run[qb] + kLazyRescale) != 0) {
          const float m_new = fmaxf(m_run[qb], mx);
          float dm = m_run[qb] - m_new;
          // keep the rescale factor's exponential inside the branch: left alone, the compiler
          // computes it on every step, one quarter-rate instruction per step for nothing
          asm volatile("" : "+v"(dm));
          const float alpha = __builtin_amdgcn_exp2f(dm);
          l_run[qb] *= alpha;
          m_run[qb] = m_new;
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) o[qb][db] *= alpha;
          exps();
        }
      }
      st[qb] = pe;
      l_run[qb] += rs;                                    // lane partial; halves summed at the end
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      bf16x8 pf[NB];
#pragma unroll
      for (int qb = 0; qb < NB; ++qb) pf[qb] = frag_from_acc(st[qb], j);
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        const bf16x8 va = ldo(Vl + db * 2048, rp.tp[j]);
#pragma unroll
        for (int qb = 0; qb < NB; ++qb) o[qb][db] = Mfma<bf16>::mma(va, pf[qb], o[qb][db]);
      }
    }
    SCHED_READS_AHEAD(2 * C::NDB, 1, NB, 1);
  };

  // three-buffer ring: the tiles of step t+2 load while step t computes
  auto stage = [&](int t, const char* cur, char* nxt) {
    // every step issues one tile (past the end, a reload of the last one that nobody reads), so
    // exactly one tile's loads may still be in flight when tile t is needed
    if (!DC::EXACT) wait_all_mem();
    else wait_vm<PER>();
    stage_barrier();
    issue(s0 + min(t + 2, nsteps - 1), nxt);
    compute(s0 + t, cur);
  };
  issue(s0, sA);
  issue(s0 + min(1, nsteps - 1), sB);
  ring3_loop(nsteps, sA, sB, sC, stage);
  wait_all_mem();                                        // drain the trailing reloads

  if (!active) return;
  if (SPLIT && nparts > 1) {
    // a part of a split tile: its unnormalised rows, running max (the reference the rows were
    // scaled by) and sum go to its slot; a wave whose rows precede the part's keys writes zero
    // rows, max -inf and sum 0, which the merge weights by exp2(-inf) = 0
    char* so = p.wsPart + (((int64_t)b * p.Hq + h) * p.fs_slots + sbase + part) * FwdSlot<D>::BYTES;
    float* sml = (float*)(so + FwdSlot<D>::O_BYTES);
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
      const int r = RW * w + 32 * qb + lc;               // row within the tile
      const float lsum = half_pair_sum(l_run[qb]);
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          u32x2 pw;
          pw[0] = pack_bf16x2(o[qb][db][4 * rg + 0], o[qb][db][4 * rg + 1]);
          pw[1] = pack_bf16x2(o[qb][db][4 * rg + 2], o[qb][db][4 * rg + 3]);
          *(u32x2*)(so + (r * D + db * 32 + 8 * rg + 4 * hl) * 2) = pw;
        }
      if (hl == 0) {
        sml[r] = m_run[qb];
        sml[RG + r] = lsum;
      }
    }
    return;
  }
#pragma unroll
  for (int qb = 0; qb < NB; ++qb) {
    const int qr = qw0 + 32 * qb + lc;
    const float lsum = half_pair_sum(l_run[qb]);
    const float inv = 1.f / lsum;
    float* rrow = p.resid + (((int64_t)b * p.S + qpos[qb]) * p.Hq + h) * D;
    char* orow = (char*)p.o_saved + ((((int64_t)b * p.ncap + qr) * p.Hq + h) * D) * 2;
    f32x4 x[C::NDB][4];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) x[db][rg] = *(const f32x4*)(rrow + db * 32 + 8 * rg + 4 * hl);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = db * 32 + 8 * rg + 4 * hl;
        const float v0 = o[qb][db][4 * rg + 0] * inv, v1 = o[qb][db][4 * rg + 1] * inv;
        const float v2 = o[qb][db][4 * rg + 2] * inv, v3 = o[qb][db][4 * rg + 3] * inv;
        f32x4 y = x[db][rg];
        y[0] += v0;
        y[1] += v1;
        y[2] += v2;
        y[3] += v3;
        *(f32x4*)(rrow + d0) = y;
        u32x2 pw;
        pw[0] = pack_bf16x2(v0, v1);
        pw[1] = pack_bf16x2(v2, v3);
        *(u32x2*)(orow + d0 * 2) = pw;
      }
    }
    if (hl == 0) p.lse[((int64_t)b * p.Hq + h) * p.ncap + qr] = (m_run[qb] + log2f(lsum)) * kLn2;
  }
}

// Merge of a split query tile's parts.  Workgroup x of a (head, batch row) takes 32 rows of the
// row's split tile x / 4 (split tiles counted from the first); a thread takes 4 columns of
// 32 / ROWS of those rows, ROWS apart.  A row's parts, with running maxima m_p, sums l_p and
// unnormalised rows O_p, combine as
//   M = max_p m_p,  w_p = exp2(m_p - M),  L = sum_p w_p l_p,  O = (sum_p w_p O_p) / L,
// the online-softmax merge, added in part order.  The row then goes out as the whole tile's
// epilogue writes it: resid += O, o_saved = bf16(O), lse = (M + log2 L) ln 2.  A thread's loads
// for all its rows go out together (rows past the kept count load row 0 of the tile and store
// nothing), four parts at a time; the merge is latency-bound, not bandwidth-bound.
template <int D>
struct Combine {
  static constexpr int C4 = D / 4;                  // 4-column chunks per row
  static constexpr int ROWS = 256 / C4;             // rows a workgroup covers at once
  static constexpr int PER = 32 / ROWS;             // rows per thread
};

template <int D>
__global__ __launch_bounds__(256) void k_fwd_combine(FwdParams p) {
  constexpr int RG = kFwdRows, C4 = Combine<D>::C4, ROWS = Combine<D>::ROWS, PER = Combine<D>::PER;
  constexpr int64_t SLOT = FwdSlot<D>::BYTES, OB = FwdSlot<D>::O_BYTES;
  const int b = blockIdx.z, h = blockIdx.y;
  const int Nk = min(p.n_kept[b], p.max_kept_blocks) * p.block;
  const int nqt = (Nk + RG - 1) / RG;
  if (!fwd_row_splits(nqt, p.Hq * p.B)) return;
  const int T = fwd_part_steps(nqt, p.Hq * p.B);
  int tile = 0, sbase = 0, nparts = 1;
  for (int j = blockIdx.x >> 2;; ++tile) {
    if (tile >= nqt) return;
    nparts = fwd_tile_parts(fwd_tile_steps(tile, Nk), T);
    if (nparts > 1) {
      if (j == 0) break;
      --j;
      sbase += nparts;
    }
  }
  const int q0 = tile * RG;
  const int c = (int)threadIdx.x % C4;
  int r[PER];
  bool valid[PER];
  int kb[PER];
  const int32_t* kept = p.kept + (int64_t)b * p.nkb;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int rr = (blockIdx.x & 3) * 32 + (int)threadIdx.x / C4 + ROWS * i;
    valid[i] = q0 + rr < Nk;
    r[i] = valid[i] ? rr : 0;
    kb[i] = kept[(q0 + r[i]) / p.block];
  }
  const char* sl = p.wsPart + (((int64_t)b * p.Hq + h) * p.fs_slots + sbase) * SLOT;
  float M[PER], L[PER];
  f32x4 acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    M[i] = -INFINITY;
    L[i] = 0.f;
    acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // four parts at a time; across groups of four the sums are rescaled to the new maximum as in
  // the online softmax (one group for up to four parts)
  for (int k0 = 0; k0 < nparts; k0 += 4) {
    const int nk = min(4, nparts - k0);
    float m[PER][4], l[PER][4];
    u32x2 o[PER][4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const char* pk = sl + (k0 + min(k, nk - 1)) * SLOT;   // absent parts reload the last
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        m[i][k] = ((const float*)(pk + OB))[r[i]];
        l[i][k] = ((const float*)(pk + OB))[RG + r[i]];
        o[i][k] = *(const u32x2*)(pk + (r[i] * D + 4 * c) * 2);
      }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      float Mn = M[i];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (k < nk) Mn = fmaxf(Mn, m[i][k]);
      const float sc = __builtin_amdgcn_exp2f(M[i] - Mn);   // 0 for the first group (M = -inf)
      L[i] *= sc;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][e] *= sc;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (k < nk) {
          const float wk = __builtin_amdgcn_exp2f(m[i][k] - Mn);
          L[i] += wk * l[i][k];
          acc[i][0] += wk * bf16_lo(o[i][k][0]);
          acc[i][1] += wk * bf16_hi(o[i][k][0]);
          acc[i][2] += wk * bf16_lo(o[i][k][1]);
          acc[i][3] += wk * bf16_hi(o[i][k][1]);
        }
      }
      M[i] = Mn;
    }
  }
  float* rrow[PER];
  f32x4 x[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int qr = q0 + r[i];
    const int pos = kb[i] * p.block + (qr - (qr / p.block) * p.block);
    rrow[i] = p.resid + (((int64_t)b * p.S + pos) * p.Hq + h) * D + 4 * c;
    x[i] = *(const f32x4*)rrow[i];
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (!valid[i]) continue;
    const int qr = q0 + r[i];
    const float inv = 1.f / L[i];
    const float v0 = acc[i][0] * inv, v1 = acc[i][1] * inv, v2 = acc[i][2] * inv, v3 = acc[i][3] * inv;
    f32x4 y = x[i];
    y[0] += v0;
    y[1] += v1;
    y[2] += v2;
    y[3] += v3;
    *(f32x4*)rrow[i] = y;
    u32x2 pw;
    pw[0] = pack_bf16x2(v0, v1);
    pw[1] = pack_bf16x2(v2, v3);
    *(u32x2*)((char*)p.o_saved + ((((int64_t)b * p.ncap + qr) * p.Hq + h) * D + 4 * c) * 2) = pw;
    if (c == 0) p.lse[((int64_t)b * p.Hq + h) * p.ncap + qr] = (M[i] + log2f(L[i])) * kLn2;
  }
}

// ------------------------------------------------------------------------------------------
// Backward prologue (one segment): D_i, dOut -> bf16 natural rows and TP tiles, and the TP
// tiles of the same ranks' Q rows.  One group = 32 ranks of one head, run by 256 threads.
// ------------------------------------------------------------------------------------------
constexpr int kPrepThreads = 256;
constexpr int kPrepIters = 2;   // a workgroup of the fused backward launch runs 2 x this many groups

template <int D>
struct PrepLds {
  static constexpr int PITCH = D + 8;                      // elements; breaks bank aliasing
  static constexpr int TILE = 32 * PITCH * 2;              // bytes of one staged 32-row tile
};

// Group t of head h, batch row b (ranks seg * seg_len + 32 t ..), by the threads tid = 0..255
// of a workgroup; tile and qtile are LDS arrays of PrepLds<D>::TILE bytes.  A thread with
// `valid` false (or whose group lies past the segment's kept ranks) only takes part in the
// barrier, which every thread of the workgroup reaches.
template <int D>
__device__ __forceinline__ void prep_group(const BwdParams& p, int t, int h, int b, int tid,
                                           bf16* tile, bf16* qtile, bool valid) {
  constexpr int E = D / 8;                    // elements per thread (8 threads per row)
  constexpr int PITCH = PrepLds<D>::PITCH;
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int QC = 32 * CPR / kPrepThreads; // Q chunks per thread
  const int qs = p.seg * p.seg_len;
  const int r0 = qs + 32 * t;
  if (valid) {                                // (b may be past the last batch row when not)
    const int Nk = min(p.n_kept[b], p.max_kept_blocks) * p.block;
    valid = r0 < min(qs + p.seg_len, Nk);     // the kept ranks end on a multiple of 64
  }
  if (valid) {
    const int32_t* kept = p.kept + (int64_t)b * p.nkb;
    const int pos0 = rank_to_pos(kept, p.block, r0);
    // the Q rows' loads go out first; they land while dO . O is formed
    const bf16* qsrc = (const bf16*)p.q + b * p.qs[0] + h * p.qs[2];
    u32x4 qv[QC];
#pragma unroll
    for (int i = 0; i < QC; ++i) {
      const int idx = tid + kPrepThreads * i, qr = idx / CPR, c = idx % CPR;
      qv[i] = ld16(qsrc + (int64_t)(pos0 + qr) * p.qs[1] + c * 8);
    }
    const int row = tid >> 3, part = tid & 7;
    const float* drow = p.dout + (((int64_t)b * p.S + pos0 + row) * p.Hq + h) * D + part * E;
    const char* orow = (const char*)p.o_saved + ((((int64_t)b * p.ncap + r0 + row) * p.Hq + h) * D + part * E) * 2;
    float dot = 0.f;
    uint32_t packed[E / 2];
#pragma unroll
    for (int c = 0; c < E / 8; ++c) {
      const u32x4 ow = *(const u32x4*)(orow + c * 16);
      const f32x4 d0 = *(const f32x4*)(drow + c * 8);
      const f32x4 d1 = *(const f32x4*)(drow + c * 8 + 4);
      dot += d0[0] * bf16_lo(ow[0]) + d0[1] * bf16_hi(ow[0]) + d0[2] * bf16_lo(ow[1]) +
             d0[3] * bf16_hi(ow[1]) + d1[0] * bf16_lo(ow[2]) + d1[1] * bf16_hi(ow[2]) +
             d1[2] * bf16_lo(ow[3]) + d1[3] * bf16_hi(ow[3]);
      packed[4 * c + 0] = pack_bf16x2(d0[0], d0[1]);
      packed[4 * c + 1] = pack_bf16x2(d0[2], d0[3]);
      packed[4 * c + 2] = pack_bf16x2(d1[0], d1[1]);
      packed[4 * c + 3] = pack_bf16x2(d1[2], d1[3]);
    }
    dot += __shfl_xor(dot, 4, 64);
    dot += __shfl_xor(dot, 2, 64);
    dot += __shfl_xor(dot, 1, 64);
    const int rl = r0 - qs + row;
    if (part == 0) {
      p.wsD[((int64_t)b * p.Hq + h) * p.seg_len + rl] = dot;
      p.wsL2[((int64_t)b * p.Hq + h) * p.seg_len + rl] = p.lse[((int64_t)b * p.Hq + h) * p.ncap + r0 + row] * kLog2e;
    }
    char* wrow = (char*)p.wsdO + ((((int64_t)b * p.seg_len + rl) * p.Hq + h) * D + part * E) * 2;
#pragma unroll
    for (int c = 0; c < E / 8; ++c) {
      u32x4 v = {packed[4 * c], packed[4 * c + 1], packed[4 * c + 2], packed[4 * c + 3]};
      *(u32x4*)(wrow + c * 16) = v;
      *(u32x4*)(tile + row * PITCH + part * E + c * 8) = v;
    }
#pragma unroll
    for (int i = 0; i < QC; ++i) {
      const int idx = tid + kPrepThreads * i, qr = idx / CPR, c = idx % CPR;
      *(u32x4*)(qtile + qr * PITCH + c * 8) = qv[i];
    }
  }
  __syncthreads();
  if (valid) {
    const int64_t tp_tile = ((int64_t)b * p.Hq + h) * (p.seg_len / 32) + (r0 - qs) / 32;
    write_tp_tile<D>(tile, (char*)p.dotp + tp_tile * D * 64, tid);
    write_tp_tile<D>(qtile, (char*)p.qtp + tp_tile * D * 64, tid);
  }
}

template <int D>
__global__ __launch_bounds__(kPrepThreads) void k_prep64(BwdParams p) {
  __shared__ __attribute__((aligned(16))) char tile[PrepLds<D>::TILE];
  __shared__ __attribute__((aligned(16))) char qtile[PrepLds<D>::TILE];
  prep_group<D>(p, blockIdx.x, blockIdx.y, blockIdx.z, threadIdx.x, (bf16*)tile, (bf16*)qtile, true);
}

// ------------------------------------------------------------------------------------------
// dK, dV: key-major.  Workgroup = NW waves x 32 kept keys of one KV head.  V is held in
// registers (B operand of dP = dO V^T) and K in an LDS tile shared by the workgroup (B operand
// of S = Q K^T), so a wave stays within 256 registers and two waves share each SIMD.
// ------------------------------------------------------------------------------------------
template <int D, int NW>
struct DkdvLds {
  using C = T64<D>;
  static constexpr int OFF_Q = 0, OFF_DO = C::NAT32, OFF_QT = 2 * C::NAT32, OFF_DOT = 2 * C::NAT32 + C::TP32;
  static constexpr int OFF_LD = 2 * C::NAT32 + 2 * C::TP32;     // lse2[32], D[32] (fp32)
  static constexpr int STAGE = OFF_LD + 256;
  static constexpr int KROWS = NW * C::NAT32;                   // the workgroup's K rows
};

// key tile tx (32 * NW kept keys) of KV head g, batch row b; part `part` of `nparts` runs the
// steps [part * n / nparts, (part + 1) * n / nparts) of the tile's n steps and adds into dk/dv
// (part 0, slot null) or writes its sums to `slot` ([2][32 NW][D]: dK scaled, then dV)
template <int D, int NW>
__device__ __forceinline__ void dkdv_tile(const BwdParams& p, char* sA, char* sB, char* sK, int* ktab,
                                          int tx, int g, int b, int part, int nparts, float* slot) {
  using C = T64<D>;
  using LY = DkdvLds<D, NW>;
  constexpr int KEYS = 32 * NW;
  constexpr int OFF_Q = LY::OFF_Q, OFF_DO = LY::OFF_DO, OFF_QT = LY::OFF_QT, OFF_DOT = LY::OFF_DOT;
  constexpr int OFF_LD = LY::OFF_LD;

  const int G = p.Hq / p.Hkv;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, hl = l >> 5, lc = l & 31;
  const int32_t* kept = p.kept + (int64_t)b * p.nkb;
  const int Nk = min(p.n_kept[b], p.max_kept_blocks) * p.block;
  const int qs = p.seg * p.seg_len;
  const int qe = min(qs + p.seg_len, Nk);
  const int k0 = tx * KEYS;
  if (qs >= qe || k0 >= qe) return;
  const int kw0 = k0 + 32 * w;
  const bool key_valid = kw0 < Nk;                               // Nk is a multiple of 64
  stage_kept(ktab, kept, (max(qe, min(k0 + KEYS, Nk)) - 1) / p.block + 1);
  __syncthreads();
  const KeptTab kt{(const LDS_AS int*)ktab, kept, p.block};

  const int64_t kstride = p.ks[1] * 2, qstride = p.qs[1] * 2;
  const int64_t dostride = (int64_t)p.Hq * D * 2;
  {
    NatPlan<D, NW> kp;
    kp.init(kstride);
    const rsrc_t rkk = make_rsrc((const bf16*)p.k + b * p.ks[0] + g * p.ks[2]);
#pragma unroll
    for (int t = 0; t < NW; ++t)
      if (k0 + 32 * t < Nk) kp.issue(sK + t * C::NAT32, rkk, (uint32_t)(kt.pos_u(k0 + 32 * t) * kstride));
  }
  bf16x8 vf[C::NS];
  if (key_valid) {
    const int pos = kt.pos(kw0 + lc);
    const char* vr = (const char*)((const bf16*)p.v + b * p.vs[0] + (int64_t)pos * p.vs[1] + g * p.vs[2]);
#pragma unroll
    for (int s = 0; s < C::NS; ++s) vf[s] = *(const bf16x8*)(vr + (16 * s + 8 * hl) * 2);
  }
  // retire the register operand loads now: a load still pending when the staged loop starts
  // would make the compiler wait for all vector memory, prefetched tiles included, at its first
  // use in every iteration
  wait_all_mem();
  f32x16 dk[C::NDB], dv[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
    dk[db] = zero16();
    dv[db] = zero16();
  }

  const int qstart = max(qs, k0);
  const int nq = (qe - qstart) / 32;
  const int nsteps = nq * G;
  NatPlan<D, NW> qplan, dplan;
  qplan.init(qstride);
  dplan.init(dostride);
  TpPlan<D, NW> tplan;
  tplan.init();
  ReadPlan<D> rp;
  rp.init();
  // lse2 / D rows of a step: 256 bytes = 16 chunks, LDC per wave
  constexpr int LDC = 16 / NW;
  static_assert(16 % NW == 0, "lse/D chunks must split evenly over the waves");
  const int ld_chunk = LDC * w + l;
  // LDS offset of this wave's lse2/D chunks, from the wave index taken through readfirstlane:
  // derived from the plain index it sits in a vector register, which the compiler spilled and
  // reloaded in the loop -- a scratch load whose wait drained the tile loads just issued
  const int ld_lds = 16 * LDC * __builtin_amdgcn_readfirstlane(w);

  const rsrc_t rq = make_rsrc((const bf16*)p.q + b * p.qs[0]);
  const rsrc_t rdo = make_rsrc((const char*)p.wsdO + (int64_t)b * p.seg_len * p.Hq * D * 2);
  const rsrc_t rqt = make_rsrc((const char*)p.qtp + (int64_t)b * p.Hq * (p.seg_len / 32) * C::TP32);
  const rsrc_t rdot = make_rsrc((const char*)p.dotp + (int64_t)b * p.Hq * (p.seg_len / 32) * C::TP32);
  // lse2 and D rows of a step, one 16-byte chunk per lane l < LDC: lse2 chunks 0..7, D 8..15,
  // both addressed from the D array of batch row b (the lse2 array follows it in the workspace)
  const rsrc_t rld = make_rsrc(p.wsD + (int64_t)b * p.Hq * p.seg_len);
  const uint32_t ld_voff = ld_chunk < 8 ? (uint32_t)((const char*)p.wsL2 - (const char*)p.wsD) + 16u * ld_chunk
                                        : 16u * (ld_chunk - 8);

  // A step's head within the group and query block: the steps run the segment's query blocks
  // of head g * G, then those of the next head of the group, ...  The loop below walks them one
  // step at a time (a division per step cost the wave's scalar unit 20 instructions).
  struct Cur {
    int hh, qi;
  };
  auto next = [&](Cur c) { return ++c.qi == nq ? Cur{c.hh + 1, 0} : c; };
  auto issue = [&](Cur c, char* buf) {
    const int q0 = qstart + c.qi * 32;
    const int h = g * G + c.hh;
    qplan.issue(buf + OFF_Q, rq, (uint32_t)((h * p.qs[2] + (int64_t)kt.pos_u(q0) * p.qs[1]) * 2));
    dplan.issue(buf + OFF_DO, rdo, (uint32_t)(((int64_t)(q0 - qs) * p.Hq + h) * D * 2));
    const uint32_t tile = (uint32_t)((h * (p.seg_len / 32) + (q0 - qs) / 32) * C::TP32);
    tplan.issue(buf + OFF_QT, rqt, tile);
    tplan.issue(buf + OFF_DOT, rdot, tile);
    if (l < LDC)
      dma16b(rld, ld_voff, (uint32_t)((h * p.seg_len + (q0 - qs)) * 4), buf + OFF_LD + ld_lds);
  };

  auto compute = [&](Cur c, const char* buf) {
    const int q0 = qstart + c.qi * 32;
    if (!key_valid || q0 + 31 < kw0) return;
    const char* Ql = buf + OFF_Q;
    const char* dOl = buf + OFF_DO;
    const char* QTl = buf + OFF_QT;
    const char* dOTl = buf + OFF_DOT;
    const float* lsel = (const float*)(buf + OFF_LD);
    const float* Dl = lsel + 32;
    f32x16 sacc = zero16(), pacc = zero16();
    const char* Kw = sK + w * C::NAT32;                          // this wave's 32 key rows
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
      sacc = Mfma<bf16>::mma(ldo(Ql, rp.nat[s]), ldo(Kw, rp.nat[s]), sacc);
      pacc = Mfma<bf16>::mma(ldo(dOl, rp.nat[s]), vf[s], pacc);
    }
    SCHED_READS_AHEAD(C::NS, 3, 2, 0);
    // lane = key kw0 + lc; register r = query q0 + 8(r/4) + 4hl + r%4
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const f32x4 lq = *(const f32x4*)(lsel + 8 * rg + 4 * hl);
      const f32x4 dd = *(const f32x4*)(Dl + 8 * rg + 4 * hl);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * rg + i;
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], p.scale_log2, -lq[i]));
        sacc[r] = pv;
        pacc[r] = pv * (pacc[r] - dd[i]);
      }
    }
    if (q0 < kw0 + 31) {                                          // diagonal step: causal mask
      // query q0 + 8(r/4) + 4hl + r%4 < key kw0 + lc  <=>  8(r/4) + r%4 < kw0 + lc - q0 - 4hl
      const int lim = kw0 + lc - q0 - 4 * hl;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + (r & 3) < lim) {
          sacc[r] = 0.f;
          pacc[r] = 0.f;
        }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bf16x8 pf = frag_from_acc(sacc, j), sf = frag_from_acc(pacc, j);
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        dv[db] = Mfma<bf16>::mma(pf, ldo(dOTl + db * 2048, rp.tp[j]), dv[db]);
        dk[db] = Mfma<bf16>::mma(sf, ldo(QTl + db * 2048, rp.tp[j]), dk[db]);
      }
    }
    SCHED_READS_AHEAD(2 * C::NDB, 2, 2, 1);
  };

  const int s0 = part * nsteps / nparts, s1 = (part + 1) * nsteps / nparts;
  if (s1 > s0) {
    Cur ci{s0 / nq, s0 % nq};                    // the step issued next
    Cur cc = ci;                                 // the step computed next
    issue(ci, sA);
    ci = next(ci);
    wait_all_mem();
    __syncthreads();
    for (int step = s0; step < s1; step += 2) {
      if (step + 1 < s1) {
        issue(ci, sB);
        ci = next(ci);
      }
      compute(cc, sA);
      cc = next(cc);
      wait_all_mem();
      stage_barrier();
      if (step + 1 >= s1) break;
      if (step + 2 < s1) {
        issue(ci, sA);
        ci = next(ci);
      }
      compute(cc, sB);
      cc = next(cc);
      wait_all_mem();
      stage_barrier();
    }
  }

  if (!key_valid) return;
  if (slot) {
    // row w * 32 + 8(r/4) + 4hl + r%4 of the tile, column db*32 + lc
    float* const sk = slot + (w * 32 + 4 * hl) * D + lc;
    float* const sv = sk + KEYS * D;
#pragma unroll
    for (int rg = 0; rg < 4; ++rg)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          sk[(8 * rg + i) * D + db * 32] = p.scale * dk[db][4 * rg + i];
          sv[(8 * rg + i) * D + db * 32] = dv[db][4 * rg + i];
        }
    return;
  }
  // dK (scaled), dV += accumulators; lane holds head_dim column db*32 + lc of keys
  // kw0 + 8(r/4) + 4hl + r%4.  Reads are issued in two batches of 8 rows.  The wave's 32 kept
  // ranks lie in one kept block (blocks are multiples of 64 rows), so one lookup places them
  // all: a lookup per row waited for every read issued before it.
  const int kpos0 = kt.pos_u(kw0);
  const int64_t rstride = (int64_t)p.Hkv * D;                     // elements per token row
  float* const dk0 = p.dk + (((int64_t)b * p.S + kpos0 + 4 * hl) * p.Hkv + g) * D + lc;
  float* const dv0 = p.dv + (((int64_t)b * p.S + kpos0 + 4 * hl) * p.Hkv + g) * D + lc;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    float xk[8][C::NDB], xv[8][C::NDB];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int rg = 2 * half + (k >> 2), i = k & 3;
      const int64_t off = (8 * rg + i) * rstride;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        xk[k][db] = dk0[off + db * 32];
        xv[k][db] = dv0[off + db * 32];
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int rg = 2 * half + (k >> 2), i = k & 3;
      const int64_t off = (8 * rg + i) * rstride;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        dk0[off + db * 32] = xk[k][db] + p.scale * dk[db][4 * rg + i];
        dv0[off + db * 32] = xv[k][db] + dv[db][4 * rg + i];
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// dQ: query-major.  Workgroup = NW waves x 32 kept queries of one query head (NW = 8: the K, V
// and K-transposed tiles of a step serve 256 queries; two waves per SIMD either way).
// ------------------------------------------------------------------------------------------
template <int D>
struct DqLds {
  using C = T64<D>;
  static constexpr int OFF_K = 0, OFF_V = C::NAT32;
  static constexpr int STAGE = 2 * C::NAT32;
};

// query tile tx (32 * NB * NW kept queries of the segment, counted from its end) of query
// head h, batch row b
template <int D, int NB, int NW>
__device__ __forceinline__ void dq_tile(const BwdParams& p, char* sA, char* sB, char* sC, int* ktab,
                                        int tx, int h, int b) {
  constexpr int RW = 32 * NB, RG = RW * NW;
  using C = T64<D>;
  constexpr int OFF_K = DqLds<D>::OFF_K, OFF_V = DqLds<D>::OFF_V;
  using DC = DmaCount<D, NW>;
  constexpr int PER = 2 * DC::NAT_W;             // direct-to-LDS instructions per wave per step

  const int g = h / (p.Hq / p.Hkv);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, hl = l >> 5, lc = l & 31;
  const int32_t* kept = p.kept + (int64_t)b * p.nkb;
  const int Nk = min(p.n_kept[b], p.max_kept_blocks) * p.block;
  const int qs = p.seg * p.seg_len;
  const int qe = min(qs + p.seg_len, Nk);
  const int nqt = (qe - qs + RG - 1) / RG;
  if (qs >= qe || tx >= nqt) return;
  const int q0 = qs + (nqt - 1 - tx) * RG;                      // heaviest tiles first
  const int qw0 = q0 + RW * w;
  const bool active = qw0 < qe;                                  // qe - qs multiple of 64
  const int qlast = min(q0 + RG, qe) - 1;
  const int nsteps = qlast / 32 + 1;
  stage_kept(ktab, kept, qlast / p.block + 1);
  __syncthreads();
  const KeptTab kt{(const LDS_AS int*)ktab, kept, p.block};

  bf16x8 qf[NB][C::NS], df[NB][C::NS];
  float lse2[NB], Dv[NB];
  if (active) {
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
      const int qr = qw0 + 32 * qb + lc;
      const int qpos = kt.pos(qr);
      const char* qrow = (const char*)((const bf16*)p.q + b * p.qs[0] + (int64_t)qpos * p.qs[1] + h * p.qs[2]);
      const char* drow = (const char*)p.wsdO + ((((int64_t)b * p.seg_len + (qr - qs)) * p.Hq + h) * D) * 2;
#pragma unroll
      for (int s = 0; s < C::NS; ++s) {
        qf[qb][s] = *(const bf16x8*)(qrow + (16 * s + 8 * hl) * 2);
        df[qb][s] = *(const bf16x8*)(drow + (16 * s + 8 * hl) * 2);
      }
      lse2[qb] = p.wsL2[((int64_t)b * p.Hq + h) * p.seg_len + (qr - qs)];
      Dv[qb] = p.wsD[((int64_t)b * p.Hq + h) * p.seg_len + (qr - qs)];
    }
  }
  // retire the register operand loads now: a load still pending when the staged loop starts
  // would make the compiler wait for all vector memory, prefetched tiles included, at its first
  // use in every iteration
  wait_all_mem();
  f32x16 acc[NB][C::NDB];
#pragma unroll
  for (int qb = 0; qb < NB; ++qb)
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) acc[qb][db] = zero16();

  const char* kbase = (const char*)((const bf16*)p.k + b * p.ks[0] + g * p.ks[2]);
  const char* vbase = (const char*)((const bf16*)p.v + b * p.vs[0] + g * p.vs[2]);
  const int64_t kstride = p.ks[1] * 2, vstride = p.vs[1] * 2;
  NatPlan<D, NW> kplan, vplan;
  kplan.init(kstride);
  vplan.init(vstride);
  ReadPlan<D> rp;
  rp.init();
  TrPlan<D> tp;
  tp.init();

  const rsrc_t rk = make_rsrc(kbase), rv = make_rsrc(vbase);
  // steps are issued in order 0, 1, ..., then the last one again (reloads past the end)
  StepPos sp;
  sp.init(0, p.block);
  auto issue = [&](int step, char* buf) {
    const int pos0 = sp.pos(kt);
    kplan.issue(buf + OFF_K, rk, (uint32_t)(pos0 * kstride));
    vplan.issue(buf + OFF_V, rv, (uint32_t)(pos0 * vstride));
    if (step < nsteps - 1) sp.advance(p.block);
  };

  auto compute = [&](int step, const char* buf) {
    const int kr0 = step * 32;
    if (!active || kr0 > qw0 + RW - 1) return;
    const char* Kl = buf + OFF_K;
    const char* Vl = buf + OFF_V;
    f32x16 st[NB], dp[NB];
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
      st[qb] = zero16();
      dp[qb] = zero16();
    }
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
      const bf16x8 ak = ldo(Kl, rp.nat[s]), av = ldo(Vl, rp.nat[s]);
#pragma unroll
      for (int qb = 0; qb < NB; ++qb) {
        st[qb] = Mfma<bf16>::mma(ak, qf[qb][s], st[qb]);
        dp[qb] = Mfma<bf16>::mma(av, df[qb][s], dp[qb]);
      }
    }
    SCHED_READS_AHEAD(C::NS, 2, 2 * NB, 0);
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(st[qb][r], p.scale_log2, -lse2[qb]));
        st[qb][r] = pv * (dp[qb][r] - Dv[qb]);
      }
      if (kr0 + 31 > qw0 + 32 * qb) {                            // diagonal step: causal mask
        const int lim = qw0 + 32 * qb + lc - kr0 - 4 * hl;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (8 * (r >> 2) + (r & 3) > lim) st[qb][r] = 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      bf16x8 af[NB];
#pragma unroll
      for (int qb = 0; qb < NB; ++qb) af[qb] = frag_from_acc(st[qb], j);
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        const bf16x8 bk = ldtr(Kl + j * 16 * C::ROWB, tp.off[0][db], tp.off[1][db]);
#pragma unroll
        for (int qb = 0; qb < NB; ++qb) acc[qb][db] = Mfma<bf16>::mma(af[qb], bk, acc[qb][db]);
      }
    }
    SCHED_READS_AHEAD(2 * C::NDB, 2, NB, 1);
  };

  auto stage = [&](int t, const char* cur, char* nxt) {
    // every step issues one tile (past the end, a reload of the last one that nobody reads), so
    // exactly one tile's loads may still be in flight when tile t is needed
    if (!DC::EXACT) wait_all_mem();
    else wait_vm<PER>();
    stage_barrier();
    issue(min(t + 2, nsteps - 1), nxt);
    compute(t, cur);
  };
  issue(0, sA);
  issue(min(1, nsteps - 1), sB);
  ring3_loop(nsteps, sA, sB, sC, stage);
  wait_all_mem();                                        // drain the trailing reloads

  if (!active) return;
  // dQ accumulator: lane holds head_dim column db*32 + lc of queries 8(r/4)+4hl+r%4.  Each
  // 32-rank group lies in one kept block: one lookup per group (see the dK/dV tile).
  const int64_t rstride = (int64_t)p.Hq * D;                      // elements per token row
#pragma unroll
  for (int qb = 0; qb < NB; ++qb) {
    const int qpos0 = kt.pos_u(qw0 + 32 * qb);
    float* const dq0 = p.dq + (((int64_t)b * p.S + qpos0 + 4 * hl) * p.Hq + h) * D + lc;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float x[8][C::NDB];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int64_t off = (8 * (2 * half + (k >> 2)) + (k & 3)) * rstride;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) x[k][db] = dq0[off + db * 32];
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int rg = 2 * half + (k >> 2), i = k & 3;
        const int64_t off = (8 * rg + i) * rstride;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) dq0[off + db * 32] = x[k][db] + p.scale * acc[qb][db][4 * rg + i];
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// Shapes: *_NB 32-row blocks per wave, *_NW waves per workgroup.
constexpr int FWD_NB = 1, FWD_NW = 4;
constexpr int DKDV_NW = 8;
constexpr int DQ_NB = 1, DQ_NW = 8;
constexpr int kKvWeightOrderMax = 128;   // dK/dV tiles per XCD up to which they go weight-major
static_assert(DKDV_NW == DQ_NW, "the fused backward launch runs both tile kinds in one workgroup shape");
static_assert(32 * DKDV_NW == kKvKeys, "the split plan counts 256-key dK/dV tiles");

// ------------------------------------------------------------------------------------------
// One segment's dQ tiles and dK/dV tiles in one launch.  Each kind alone fills the GPU with
// one workgroup per compute unit, so a launch lasts as long as its heaviest tile (the causal
// tiles vary up to 8x in work); run together, short tiles fill in behind long ones.
//
// The launch is two runs of workgroups, each a multiple of 8 long (idle workgroups pad them):
// the dQ tiles, heaviest first (their queries see every earlier key), then the dK/dV tiles.
// Within a run, XCD x (launch index mod 8) takes a contiguous range of tiles in launch order,
// so the tiles of one head share an L2, as in xcd_tile().
//
// In a light launch (the first segments: at most kKvWeightOrderMax dK/dV tiles per XCD) each
// compute unit runs one dQ tile and then one or two dK/dV tiles, and the launch lasts as long
// as the busiest unit.  There the XCD's dK/dV tiles go out weight-major -- the heaviest tile of
// every head of its range, then the next heaviest, and so on -- so that the units freed first,
// by the lightest dQ tiles, take the heaviest dK/dV tiles.  (Head-major order sent heavy dK/dV
// tiles of later heads behind heavy dQ tiles: 209 against 176 us for the first segment of a
// 32K-token layer.)  Heavier launches keep head-major order, whose units share one head's
// Q and dO tiles in L2.
//
// The LDS buffers are separate arrays, shared by the two kinds (dQ: A, B, C; dK/dV: A, B and
// the K rows): as distinct objects the compiler can tell that a direct-to-LDS load into one
// buffer does not write another, and waits only for the loads of the buffer it reads.
//
// A third run may follow: the prologue of the next segment (pn, writing the other half of a
// double workspace), two 32-rank groups per workgroup.  Dispatched last, these workgroups take
// the compute units that the unequal tiles leave idle at the end of the launch, instead of a
// launch of their own between the segments.
// ------------------------------------------------------------------------------------------
// SPLIT: some dK/dV tiles run in parts (then the dK/dV run goes first).  A launch without
// split tiles runs the instance compiled without that code, whose loops carry nothing for it.
template <int D, bool SPLIT>
__global__ __launch_bounds__(64 * DQ_NW, 2) void k_bwd64(BwdParams pq, BwdParams pk, BwdGrid gr,
                                                         BwdParams pn) {
  using KL = DkdvLds<D, DKDV_NW>;
  using QL = DqLds<D>;
  constexpr int AB = KL::STAGE > QL::STAGE ? KL::STAGE : QL::STAGE;
  __shared__ __attribute__((aligned(1024))) char bufA[AB];
  __shared__ __attribute__((aligned(1024))) char bufB[AB];
  __shared__ __attribute__((aligned(1024))) char bufC[QL::STAGE];
  __shared__ __attribute__((aligned(1024))) char bufK[KL::KROWS];
  __shared__ int ktab[kKeptTab];
  // pq and pk are the same parameters, one copy per tile kind: a field that both kinds read
  // would otherwise be loaded once before the branch and held in scalar registers through
  // either body, more than the two bodies need on their own
  const int lin = blockIdx.x;
  // run [o, o + n rounded up to 8): XCD i & 7 takes tiles (i & 7) * q .. + q - 1, q = pad / 8
  auto tile_of = [&](int o, int n) {
    const int i = lin - o, q = ((n + 7) >> 3);
    return (i & 7) * q + (i >> 3);
  };
  if (lin >= gr.o_prep) {
    static_assert(64 * DQ_NW == 2 * kPrepThreads && PrepLds<D>::TILE * 2 <= AB,
                  "two prologue groups at a time, staged in buffers A and B");
    const int half = threadIdx.x / kPrepThreads;
    char* st = half ? bufB : bufA;
    for (int it = 0; it < kPrepIters; ++it) {
      if (it > 0) __syncthreads();                         // the staged tiles have been read
      const int grp = 2 * (kPrepIters * (lin - gr.o_prep) + it) + half;   // (b Hq + h) ng + t
      const int t = grp % gr.ng, h = (grp / gr.ng) % pn.Hq, b = grp / (gr.ng * pn.Hq);
      prep_group<D>(pn, t, h, b, threadIdx.x - half * kPrepThreads, (bf16*)st,
                    (bf16*)(st + PrepLds<D>::TILE), b < pn.B);
    }
    return;
  }
  if (SPLIT ? lin >= ((gr.n_kv + 7) & ~7) : lin < gr.o_kv) {
    const int L = SPLIT ? tile_of(gr.o_dq, gr.n_dq) : tile_of(0, gr.n_dq);
    if (L >= gr.n_dq) return;
    dq_tile<D, DQ_NB, DQ_NW>(pq, bufA, bufB, bufC, ktab, L % gr.nqt, (L / gr.nqt) % pq.Hq,
                             L / (gr.nqt * pq.Hq));
  } else {
    const int i = lin - gr.o_kv, q = (gr.n_kv + 7) >> 3, x = i & 7, j = i >> 3;
    int L;
    if (q <= kKvWeightOrderMax && q % gr.nki == 0) {
      const int rows = q / gr.nki;               // (batch, head) rows of XCD x's range
      L = (x * rows + j % rows) * gr.nki + j / rows;
    } else {
      L = x * q + j;                             // = tile_of(gr.o_kv, gr.n_kv)
    }
    if (L >= gr.n_kv) return;
    // item of its (batch row, KV head): the parts of key tile 0, then of tile 1, ...
    const int item = L % gr.nki, g = (L / gr.nki) % pk.Hkv, b = L / (gr.nki * pk.Hkv);
    int tx = item, part = 0, nparts = 1;
    float* slot = nullptr;
    if constexpr (SPLIT) {
      const int qs = pk.seg * pk.seg_len, G = pk.Hq / pk.Hkv;
      int first = 0, extra = 0;
      for (tx = 0;; ++tx) {
        nparts = kv_tile_parts(kv_tile_steps(tx, qs, gr.seg_end, G), gr.kv_target);
        if (item < first + nparts) break;
        first += nparts;
        extra += nparts - 1;
      }
      part = item - first;
      if (part > 0)
        slot = pk.wsKv + (((int64_t)b * pk.Hkv + g) * gr.n_extra + extra + part - 1) * (2 * kKvKeys * D);
    }
    dkdv_tile<D, DKDV_NW>(pk, bufA, bufB, bufK, ktab, tx, g, b, part, nparts, slot);
  }
}

// Adds the slots of the split dK/dV tiles of one segment into dk/dv, parts 1.. in order, after
// the launch in which part 0 added its own sums.  One workgroup per 32 rows of a key tile (tiles
// run in one part exit at once); each thread takes four runs of 4 floats, all loads issued
// before the sums are formed (16-byte loads from the slots; dk and dv, which need only 4-byte
// alignment, by the float).
constexpr int kKvReduceRows = 32;

template <int D>
__global__ __launch_bounds__(256) void k_kv_reduce(BwdParams p, BwdGrid gr) {
  constexpr int PIECES = kKvReduceRows * D / 4;             // float4 pieces per workgroup
  constexpr int PER = PIECES / 256;                         // per thread (4 at D = 128)
  static_assert(PER * 256 == PIECES, "whole pieces per thread");
  const int tx = blockIdx.x / (kKvKeys / kKvReduceRows), rg = blockIdx.x % (kKvKeys / kKvReduceRows);
  const int g = blockIdx.y, b = blockIdx.z;
  const int qs = p.seg * p.seg_len, G = p.Hq / p.Hkv;
  int extra = 0;
  for (int t = 0; t < tx; ++t) extra += kv_tile_parts(kv_tile_steps(t, qs, gr.seg_end, G), gr.kv_target) - 1;
  const int P = kv_tile_parts(kv_tile_steps(tx, qs, gr.seg_end, G), gr.kv_target);
  if (P <= 1) return;
  const int Nk = min(p.n_kept[b], p.max_kept_blocks) * p.block;
  const int qe = min(qs + p.seg_len, Nk);
  const int k0 = tx * kKvKeys, r0 = rg * kKvReduceRows;
  if (qs >= qe || k0 >= qe || k0 + r0 >= Nk) return;        // the tile's parts did not run
  // (kept keys of a tile end on a multiple of 64, so these 32 rows are all kept)
  const float* const s0 = p.wsKv + (((int64_t)b * p.Hkv + g) * gr.n_extra + extra) * (2 * kKvKeys * D);
  const int32_t* kept = p.kept + (int64_t)b * p.nkb;
  f32x4 xk[PER], xv[PER];
  int64_t off[PER];
  int so[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = threadIdx.x + 256 * i, r = r0 + c / (D / 4), d = 4 * (c % (D / 4));
    const int rank = k0 + r;
    const int pos = kept[rank / p.block] * p.block + rank % p.block;
    off[i] = (((int64_t)b * p.S + pos) * p.Hkv + g) * D + d;
    so[i] = r * D + d;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xk[i][e] = p.dk[off[i] + e];
      xv[i][e] = p.dv[off[i] + e];
    }
  }
  for (int q = 0; q < P - 1; ++q) {
    const float* sl = s0 + (int64_t)q * (2 * kKvKeys * D);
    f32x4 ak[PER], av[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      ak[i] = *(const f32x4*)(sl + so[i]);
      av[i] = *(const f32x4*)(sl + kKvKeys * D + so[i]);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      xk[i] += ak[i];
      xv[i] += av[i];
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p.dk[off[i] + e] = xk[i][e];
      p.dv[off[i] + e] = xv[i][e];
    }
}

int kv_split_target(int qs, int seg_cap, int G, int Hq, int Hkv, int B) {
  const int seg_end = qs + seg_cap;
  int64_t kv = 0, dq = 0;
  int longest = 0;
  for (int tx = 0; tx * kKvKeys < seg_end; ++tx) {
    const int st = kv_tile_steps(tx, qs, seg_end, G);
    kv += st;
    longest = max(longest, st);
  }
  for (int q0 = qs; q0 < seg_end; q0 += 32 * DQ_NB * DQ_NW) dq += (min(q0 + 32 * DQ_NB * DQ_NW, seg_end) - 1) / 32 + 1;
  // load per compute unit in dK/dV steps (a dQ step runs 24 MFMAs per wave, a dK/dV step 32)
  const double per_cu = ((double)kv * Hkv * B + 0.75 * (double)dq * Hq * B) / kComputeUnits;
  // only a tile longer than that load sets the launch's length; its parts, at most half the
  // load, let the launch pack its work evenly (128 steps or more each, so that light launches
  // do not spend much workspace on many small parts)
  if (longest <= per_cu) return 0;
  const int target = max(128, (int)(per_cu / 2));
  return longest > target ? target : 0;
}

int kv_split_extra(int qs, int seg_cap, int G, int target) {
  if (target <= 0) return 0;
  const int seg_end = qs + seg_cap;
  int extra = 0;
  for (int tx = 0; tx * kKvKeys < seg_end; ++tx) extra += kv_tile_parts(kv_tile_steps(tx, qs, seg_end, G), target) - 1;
  return extra;
}

template <int D>
static hipError_t launch_fwd64_t(const FwdParams& p, hipStream_t st) {
  PackArgs a{p.v, p.vs[0], p.vs[1], p.vs[2], p.kept, p.n_kept, p.block, p.nkb, p.max_kept_blocks,
             0, p.ncap, p.ncap / 32, p.Hkv, p.vtp};
  hipError_t e = pack_tp<D>(a, p.B, st);
  if (e != hipSuccess) return e;
  static_assert(32 * FWD_NB * FWD_NW == kFwdRows, "forward query tiles are 128 rows");
  if (p.fs_slots == 0) {
    TimedLaunch tl("k_fwd64", st);
    k_fwd64<D, FWD_NB, FWD_NW, false><<<dim3((p.ncap + kFwdRows - 1) / kFwdRows, p.Hq, p.B),
                                         64 * FWD_NW, 0, st>>>(p);
    return hipGetLastError();
  }
  {
    TimedLaunch tl("k_fwd64", st);
    k_fwd64<D, FWD_NB, FWD_NW, true><<<dim3(p.fs_items, p.Hq, p.B), 64 * FWD_NW, 0, st>>>(p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  TimedLaunch tl("k_fwd_combine", st);
  k_fwd_combine<D><<<dim3(4 * p.fs_split_tiles, p.Hq, p.B), 256, 0, st>>>(p);
  return hipGetLastError();
}

void fwd_split_bounds(int ncap, int Hq, int B, int* items, int* slots, int* split_tiles) {
  const int ntc = (ncap + kFwdRows - 1) / kFwdRows;
  int it_max = ntc, sl_max = 0, st_max = 0;
  // A row of n tiles (its last one possibly short) needs no more than a row of n full tiles,
  // whose tile j = 1..n holds 4j steps and makes k = ceil(4j / T) parts; the tiles of one k are
  // those with (k - 1) T < 4j <= k T, counted at once.  Rows that split are those of few tiles,
  // so the loop over n ends early.
  for (int n = 1; n <= ntc && fwd_row_splits(n, Hq * B); ++n) {
    const int T = fwd_part_steps(n, Hq * B);
    int it = 0, sl = 0, st = 0;
    for (int k = 1; (k - 1) * T < 4 * n; ++k) {
      const int jlo = (k - 1) * T / 4 + 1, jhi = min(n, k * T / 4);
      const int c = max(0, jhi - jlo + 1);
      it += k * c;
      if (k > 1) {
        sl += k * c;
        st += c;
      }
    }
    it_max = max(it_max, it);
    sl_max = max(sl_max, sl);
    st_max = max(st_max, st);
  }
  *items = it_max;
  *slots = sl_max;
  *split_tiles = st_max;
}

hipError_t launch_fwd64(const FwdParams& p, int D, hipStream_t st) {
  return D == 64 ? launch_fwd64_t<64>(p, st) : launch_fwd64_t<128>(p, st);
}

// ranks of segment p.seg (capacity: max_kept_blocks * block, cut into seg_len pieces)
static int seg_cap_of(const BwdParams& p) { return min(p.seg_len, p.ncap - p.seg * p.seg_len); }

template <int D>
static hipError_t prep64_t(const BwdParams& p, hipStream_t st) {
  const int seg_cap = seg_cap_of(p);
  if (seg_cap <= 0) return hipSuccess;
  TimedLaunch tl("k_prep64", st);
  k_prep64<D><<<dim3((seg_cap + 31) / 32, p.Hq, p.B), kPrepThreads, 0, st>>>(p);
  return hipGetLastError();
}

template <int D>
static hipError_t bwd64_main_t(const BwdParams& p, const BwdParams* next, hipStream_t st) {
  const int L = p.seg_len;
  const int seg_cap = seg_cap_of(p);
  if (seg_cap <= 0) return hipSuccess;
  const int seg_end = p.seg * L + seg_cap;
  constexpr int KG = 32 * DKDV_NW, QG = 32 * DQ_NB * DQ_NW;
  auto pad8 = [](int n) { return (n + 7) & ~7; };
  BwdGrid gr;
  gr.nqt = (seg_cap + QG - 1) / QG;
  gr.nkt = (seg_end + KG - 1) / KG;
  gr.n_dq = gr.nqt * p.Hq * p.B;
  gr.seg_end = seg_end;
  const int G = p.Hq / p.Hkv;
  gr.kv_target = kv_split_target(p.seg * L, seg_cap, G, p.Hq, p.Hkv, p.B);
  gr.n_extra = kv_split_extra(p.seg * L, seg_cap, G, gr.kv_target);
  gr.nki = gr.nkt + gr.n_extra;
  gr.n_kv = gr.nki * p.Hkv * p.B;
  // dQ tiles first, heaviest first; but when dK/dV tiles run in parts, those parts are the
  // longest work of the launch and go first (16K-token GQA layer, one segment: 1.44 -> 1.26 ms
  // against dQ first, both split)
  const bool split = gr.n_extra > 0;
  gr.o_kv = split ? 0 : pad8(gr.n_dq);
  gr.o_dq = split ? pad8(gr.n_kv) : 0;
  gr.o_prep = pad8(gr.n_dq) + pad8(gr.n_kv);
  gr.ng = 0;
  int n_prep = 0;
  const int next_cap = next ? seg_cap_of(*next) : 0;
  if (next_cap > 0) {
    gr.ng = (next_cap + 31) / 32;
    constexpr int per_wg = 2 * kPrepIters;                 // groups per workgroup
    n_prep = (gr.ng * next->Hq * next->B + per_wg - 1) / per_wg;
  }
  {
    TimedLaunch tl("k_bwd64", st);
    const dim3 grid(gr.o_prep + n_prep);
    if (split)
      k_bwd64<D, true><<<grid, 64 * DQ_NW, 0, st>>>(p, p, gr, next_cap > 0 ? *next : p);
    else
      k_bwd64<D, false><<<grid, 64 * DQ_NW, 0, st>>>(p, p, gr, next_cap > 0 ? *next : p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || gr.n_extra == 0) return e;
  }
  TimedLaunch tl("k_kv_reduce", st);
  k_kv_reduce<D><<<dim3(gr.nkt * (kKvKeys / kKvReduceRows), p.Hkv, p.B), 256, 0, st>>>(p, gr);
  return hipGetLastError();
}

hipError_t launch_prep64(const BwdParams& p, int D, hipStream_t st) {
  return D == 64 ? prep64_t<64>(p, st) : prep64_t<128>(p, st);
}

hipError_t launch_bwd64_main(const BwdParams& p, const BwdParams* next, int D, hipStream_t st) {
  return D == 64 ? bwd64_main_t<64>(p, next, st) : bwd64_main_t<128>(p, next, st);
}

}  // namespace jenga
