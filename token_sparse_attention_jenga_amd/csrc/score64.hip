// bf16 block scoring for gfx950 with async LDS staging (same tile plumbing as attn64.hip).
//
// Jenga (aipaper summary, §4.2.1 Eq. 1: informativeness of token j sums the interaction it
// receives from all other tokens; §4.2.2 Eq. 2: averaged over heads; §4.2.3: aggregated per key
// block over the query blocks).  The interaction is the causal softmax probability.
//
// The received mass of key block n sums p_ij = 2^(c q_i.k_j - lse2_i) over its keys j and the
// queries i > j.  Grouped by query, that is sum_i 2^(L_in - lse2_i) with the partial log2-sum
// L_in = log2 sum_{j in n, j < i} 2^(c q_i.k_j): the exponentials that make lse2_i also make
// every L_in, so one pass over the causal scores suffices.
//
// L_in can only be turned into mass once lse2_i is known, at the end of the query's pass, so
// the queries are scored in chunks (the same idea as segment-based peak cutting): the L_in of
// one chunk of queries are stored, turned into mass and added up before the next chunk is
// scored.  The stored partials are chunk x S/block floats per head, linear in S.
//
//   k_slse64       query-major, 32 queries per wave, S^T = K Q^T per 32-key step, running max
//                  (lazily moved): lse2_i with an fp64 running sum, and L_in per key block
//                  (fp32 block sum, stored as a log2 when the block ends).  VALU-bound: one
//                  exponential per score; the MFMA work is half of it or less.
//   k_sblock_mass  per (batch, head, key block): sum_i 2^(L_in - lse2_i) over the chunk's queries
//                  of the block's row, fp32 groups of 4 added into fp64, fixed order; the first
//                  chunk stores, later chunks add in chunk order.  Memory-bound.
#include "common.h"
#include "kernels.h"
#include "tiles64.h"

namespace jenga {

constexpr float kScoreLazy = 8.f;
constexpr float kScoreCheck = 128.f;   // 2^7: see the lazy rule in k_slse64

template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 2) void k_slse64(ScoreParams p) {
  using C = T64<D>;
  using DC = DmaCount<D, NW>;
  constexpr int PER = DC::NAT_W;
  constexpr int RG = 32 * NW;
  __shared__ __attribute__((aligned(1024))) char sA[C::NAT32];
  __shared__ __attribute__((aligned(1024))) char sB[C::NAT32];
  __shared__ __attribute__((aligned(1024))) char sC[C::NAT32];

  const Tile3 tl = xcd_tile_weight_major();
  const int b = tl.z, h = tl.y;
  const int g = h / (p.Hq / p.Hkv);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, hl = l >> 5, lc = l & 31;
  const int nqt = (p.q_end - p.q_begin + RG - 1) / RG;
  const int q0 = p.q_begin + (nqt - 1 - tl.x) * RG;      // heaviest tiles first
  const int qw0 = q0 + 32 * w;
  const bool active = qw0 < p.q_end;                     // q_end is a multiple of 64
  const int qi = qw0 + lc;
  const int nsteps = (min(q0 + RG, p.q_end) - 1) / 32 + 1;

  bf16x8 qf[C::NS];
  if (active) {
    const char* qrow = (const char*)((const bf16*)p.q + b * p.qs[0] + (int64_t)qi * p.qs[1] + h * p.qs[2]);
#pragma unroll
    for (int s = 0; s < C::NS; ++s) qf[s] = *(const bf16x8*)(qrow + (16 * s + 8 * hl) * 2);
  }
  // retire the register operand loads now: a load still pending when the staged loop starts
  // would make the compiler wait for all vector memory, prefetched tiles included, at its first
  // use in every iteration
  wait_all_mem();
  const char* kbase = (const char*)((const bf16*)p.k + b * p.ks[0] + g * p.ks[2]);
  const int64_t kstride = p.ks[1] * 2;
  NatPlan<D, NW> kplan;
  kplan.init(kstride);
  ReadPlan<D> rp;
  rp.init();
  const float c2 = p.scale_log2;
  float m_run = -INFINITY;
  double l_run = 0.0;
  // key-block partial sum (relative to m_run) of the scores of keys before the query
  float bsum = 0.f;
  const int tpb = p.block / 32;                          // key steps per block
  int in_blk = 0, blk = 0;                               // wave-uniform block position
  // this (batch, head)'s partials of the chunk: row n (key block n), column qi - q_begin
  const int nkb = p.S / p.block;
  float* const lp = p.lpart + ((int64_t)b * p.Hq + h) * nkb * p.chunk + (qi - p.q_begin);
  // a finished block's value is stored at the start of the next step, after that step's wait
  // and before its tile loads are issued: stored right away, it would sit behind those loads
  // and the next step's wait would have to take it along
  bool pend = false;
  float pend_v = 0.f;
  int64_t pend_i = 0;

  const rsrc_t rk = make_rsrc_u(kbase);
  auto issue = [&](int t, char* buf) { kplan.issue(buf, rk, (uint32_t)(32 * t * kstride)); };
  auto compute = [&](int t, const char* Kl) {
    const int kr0 = 32 * t;
    if (!active || kr0 > qw0 + 31) return;
    f32x16 st = zero16();
#pragma unroll
    for (int s = 0; s < C::NS; ++s) st = Mfma<bf16>::mma(ldo(Kl, rp.nat[s]), qf[s], st);
    SCHED_READS_AHEAD(C::NS, 1, 1, 0);
    const bool diag = kr0 == qw0;                        // the wave's last step
    if (diag) {                                          // causal mask
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kr0 + 8 * (r >> 2) + 4 * hl + (r & 3) > qi) st[r] = -INFINITY;
    }
    // Exponentials against the current reference max, and their sum.  (The sum starts from its
    // first term: starting from 0 costs an addition per step.)
    f32x16 ex;
    float rs;
    auto exps = [&]() {
#pragma unroll
      for (int r = 0; r < 16; ++r) ex[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[r], c2, -m_run));
      rs = ex[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) rs += ex[r];
    };
    exps();
    // The lazy rule moves the reference max when some lane's tile max exceeds it by kScoreLazy.
    // The lane holding that max then has an exponential above 2^7.8 (while |m_run| < 2^20 the
    // rule's rounded m_run + 8 and max * c2 each lie within 2^-4 of the exact values, and the
    // fma above rounds once), so its sum exceeds 2^7: a wave whose sums all stay at or below
    // 2^7 cannot need the rule and skips the tile max.  Where the rule is checked the values
    // are those of taking the max first; where it moves the reference, the exponentials are
    // formed again.  (The first step, against m_run = -inf, always checks: a lane with a masked
    // key sums to NaN there, but the wave's last query sees the whole first step, so its lanes
    // sum to +inf.  Past 2^20 a missed check leaves every exponential below 2^7, so the sums stay
    // exact in range, only their reference differs.)
    if (__builtin_amdgcn_ballot_w64(rs > kScoreCheck) != 0) {
      const float mx = half_pair_max(max16(st)) * c2;
      if (__builtin_amdgcn_ballot_w64(mx > m_run + kScoreLazy) != 0) {
        const float m_new = fmaxf(m_run, mx);
        float dm = m_run - m_new;
        // keep the rescale factor's exponential inside the branch: left alone, the compiler
        // computes it on every step, one quarter-rate instruction per step for nothing
        asm volatile("" : "+v"(dm));
        const float f = __builtin_amdgcn_exp2f(dm);
        l_run *= (double)f;
        bsum *= f;
        m_run = m_new;
        exps();
      }
    }
    l_run += (double)rs;
    if (!diag) {
      bsum += rs;
    } else {                                             // the mass leaves out the key i = j
      float rm = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) rm += (kr0 + 8 * (r >> 2) + 4 * hl + (r & 3) < qi) ? ex[r] : 0.f;
      bsum += rm;
    }
    if (++in_blk == tpb || diag) {                       // block ends here for these queries
      const float tot = half_pair_sum(bsum);             // lanes l, l^32: the two key halves
      pend_v = m_run + __builtin_amdgcn_logf(tot);       // log2; of 0, -inf: no key before i
      pend_i = (int64_t)blk * p.chunk;
      pend = true;
      bsum = 0.f;
      in_blk = 0;
      ++blk;
    }
  };
  auto flush = [&]() {
    if (pend && hl == 0) lp[pend_i] = pend_v;
    pend = false;
  };
  auto stage = [&](int t, const char* cur, char* nxt) {
    // every step issues one tile (past the end, a reload of the last one that nobody reads), so
    // exactly one tile's loads may still be in flight when tile t is needed
    if (!DC::EXACT) wait_all_mem();
    else wait_vm<PER>();
    stage_barrier();
    flush();
    issue(min(t + 2, nsteps - 1), nxt);
    compute(t, cur);
  };
  issue(0, sA);
  issue(min(1, nsteps - 1), sB);
  ring3_loop(nsteps, sA, sB, sC, stage);
  flush();
  wait_all_mem();                                        // drain the trailing reloads
  if (!active) return;
  const double lsum = l_run + __shfl_xor(l_run, 32, 64);
  if (hl == 0) p.lse2[((int64_t)b * p.Hq + h) * p.S + qi] = (float)((double)m_run + log2(lsum));
}

// Received mass of key block n for one (batch, head) from the queries of one chunk: the sum over
// the queries i >= n*block of the chunk of 2^(L_in - lse2_i).  One workgroup per row; each
// thread adds groups of four terms (fp32) into an fp64 sum, then a fixed-order reduction over
// the workgroup.  The chunk starting at query 0 stores the sum (0 for rows it does not reach),
// later chunks add theirs, one launch after another.
constexpr int kMassThreads = 256;

__global__ __launch_bounds__(kMassThreads) void k_sblock_mass(ScoreParams p) {
  const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int nkb = p.S / p.block;
  const int start = max(p.q_begin, n * p.block);         // a multiple of 64
  const int len = max(p.q_end - start, 0);               // a multiple of 64
  const float* lrow = p.lpart + (((int64_t)b * p.Hq + h) * nkb + n) * p.chunk + (start - p.q_begin);
  const float* lse = p.lse2 + ((int64_t)b * p.Hq + h) * p.S + start;
  double acc = 0.0;
  constexpr int U = 4;                                   // groups whose loads are issued together
  int i = 4 * threadIdx.x;
  for (; i + 4 * kMassThreads * (U - 1) < len; i += 4 * kMassThreads * U) {
    f32x4 a[U], c[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      a[u] = *(const f32x4*)(lrow + i + 4 * kMassThreads * u);
      c[u] = *(const f32x4*)(lse + i + 4 * kMassThreads * u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      acc += (double)((__builtin_amdgcn_exp2f(a[u][0] - c[u][0]) + __builtin_amdgcn_exp2f(a[u][1] - c[u][1])) +
                      (__builtin_amdgcn_exp2f(a[u][2] - c[u][2]) + __builtin_amdgcn_exp2f(a[u][3] - c[u][3])));
  }
  for (; i < len; i += 4 * kMassThreads) {
    const f32x4 a = *(const f32x4*)(lrow + i), c = *(const f32x4*)(lse + i);
    acc += (double)((__builtin_amdgcn_exp2f(a[0] - c[0]) + __builtin_amdgcn_exp2f(a[1] - c[1])) +
                    (__builtin_amdgcn_exp2f(a[2] - c[2]) + __builtin_amdgcn_exp2f(a[3] - c[3])));
  }
  __shared__ double part[kMassThreads / 64];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = part[0];
#pragma unroll
    for (int w = 1; w < kMassThreads / 64; ++w) t += part[w];
    double* m = p.mass32 + ((int64_t)b * p.Hq + h) * nkb + n;
    if (p.q_begin == 0) *m = t;
    else if (len > 0) *m += t;
  }
}

constexpr int SCORE_NW = 4;

template <int D>
static hipError_t launch_score64_t(const ScoreParams& p0, hipStream_t st) {
  constexpr int RG = 32 * SCORE_NW;
  ScoreParams p = p0;
  for (int c0 = 0; c0 < p.S; c0 += p.chunk) {
    p.q_begin = c0;
    p.q_end = min(p.S, c0 + p.chunk);
    hipError_t e;
    {
      TimedLaunch tl("k_slse64", st);
      k_slse64<D, SCORE_NW><<<dim3((p.q_end - p.q_begin + RG - 1) / RG, p.Hq, p.B), 64 * SCORE_NW, 0, st>>>(p);
      e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    TimedLaunch tl("k_sblock_mass", st);
    k_sblock_mass<<<dim3(p.S / p.block, p.Hq, p.B), kMassThreads, 0, st>>>(p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_score64(const ScoreParams& p, int D, hipStream_t st) {
  return D == 64 ? launch_score64_t<64>(p, st) : launch_score64_t<128>(p, st);
}

}  // namespace jenga
