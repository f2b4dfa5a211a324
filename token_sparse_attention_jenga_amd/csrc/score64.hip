// bf16 block scoring for gfx950 with async LDS staging (same tile plumbing as attn64.hip).
//
// Jenga (aipaper summary, §4.2.1 Eq. 1: informativeness of token j sums the interaction it
// receives from all other tokens; §4.2.2 Eq. 2: averaged over heads; §4.2.3: aggregated per key
// block over the query blocks).  The interaction is the causal softmax probability.
//
//   k_slse64   query-major, 32 queries per wave: lse2_i = log2 sum_{j<=i} 2^(c q_i.k_j);
//              S^T = K Q^T per 32-key step, running max (lazily moved) and an fp64 running sum.
//   k_smass64  key-major, 32 keys per wave (K in registers): per 32-query step
//              S = Q K^T, p = 2^(c S - lse2_i) for i > j, per-key fp32 partial sums added into
//              fp64; finally a fixed-order fp64 reduction to 32-key groups.
// Both are VALU-bound (one exp per score); the MFMA work is half of it or less.
#include "common.h"
#include "kernels.h"
#include "tiles64.h"

namespace jenga {

constexpr float kScoreLazy = 8.f;

template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 2) void k_slse64(ScoreParams p) {
  using C = T64<D>;
  using DC = DmaCount<D, NW>;
  constexpr int PER = DC::NAT_W;
  constexpr int RG = 32 * NW;
  __shared__ __attribute__((aligned(1024))) char sA[C::NAT32];
  __shared__ __attribute__((aligned(1024))) char sB[C::NAT32];
  __shared__ __attribute__((aligned(1024))) char sC[C::NAT32];

  const Tile3 tl = xcd_tile();
  const int b = tl.z, h = tl.y;
  const int g = h / (p.Hq / p.Hkv);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, hl = l >> 5, lc = l & 31;
  const int nqt = (p.S + RG - 1) / RG;
  const int q0 = (nqt - 1 - tl.x) * RG;                  // heaviest tiles first
  const int qw0 = q0 + 32 * w;
  const bool active = qw0 < p.S;                         // S is a multiple of 64
  const int qi = qw0 + lc;
  const int nsteps = (min(q0 + RG, p.S) - 1) / 32 + 1;

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

  const rsrc_t rk = make_rsrc_u(kbase);
  auto issue = [&](int t, char* buf) { kplan.issue(buf, rk, (uint32_t)(32 * t * kstride)); };
  auto compute = [&](int t, const char* Kl) {
    const int kr0 = 32 * t;
    if (!active || kr0 > qw0 + 31) return;
    f32x16 st = zero16();
#pragma unroll
    for (int s = 0; s < C::NS; ++s) st = Mfma<bf16>::mma(ldo(Kl, rp.nat[s]), qf[s], st);
    SCHED_READS_AHEAD(C::NS, 1, 1, 0);
    if (kr0 + 31 > qw0) {                                // diagonal step: causal mask
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kr0 + 8 * (r >> 2) + 4 * hl + (r & 3) > qi) st[r] = -INFINITY;
    }
    const float mx = half_pair_max(max16(st)) * c2;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kScoreLazy) != 0) {
      const float m_new = fmaxf(m_run, mx);
      float dm = m_run - m_new;
      // keep the rescale factor's exponential inside the branch: left alone, the compiler
      // computes it on every step, one quarter-rate instruction per step for nothing
      asm volatile("" : "+v"(dm));
      l_run *= (double)__builtin_amdgcn_exp2f(dm);
      m_run = m_new;
    }
    // (the sum starts from its first term: starting from 0 costs an addition per step)
    float rs = __builtin_amdgcn_exp2f(__builtin_fmaf(st[0], c2, -m_run));
#pragma unroll
    for (int r = 1; r < 16; ++r) rs += __builtin_amdgcn_exp2f(__builtin_fmaf(st[r], c2, -m_run));
    l_run += (double)rs;
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
  const double lsum = l_run + __shfl_xor(l_run, 32, 64);
  if (hl == 0) p.lse2[((int64_t)b * p.Hq + h) * p.S + qi] = (float)((double)m_run + log2(lsum));
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 2) void k_smass64(ScoreParams p) {
  using C = T64<D>;
  using DC = DmaCount<D, NW>;
  constexpr int LDC = 8 / NW;                      // 16-byte chunks of the 32 lse2 values per wave
  static_assert(8 % NW == 0, "lse2 chunks must split evenly over the waves");
  constexpr int PER = DC::NAT_W + 1;
  constexpr int KG = 32 * NW;
  constexpr int STAGE = C::NAT32 + 128;
  __shared__ __attribute__((aligned(1024))) char sA[STAGE];
  __shared__ __attribute__((aligned(1024))) char sB[STAGE];
  __shared__ __attribute__((aligned(1024))) char sC[STAGE];

  const Tile3 tl = xcd_tile();
  const int b = tl.z, h = tl.y;
  const int g = h / (p.Hq / p.Hkv);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, hl = l >> 5, lc = l & 31;
  const int k0 = tl.x * KG;
  const int kw0 = k0 + 32 * w;
  const bool active = kw0 < p.S;
  const int kj = kw0 + lc;
  const int nsteps = (p.S - k0) / 32;              // query steps k0, k0+32, ..., S-32

  bf16x8 kf[C::NS];
  if (active) {
    const char* krow = (const char*)((const bf16*)p.k + b * p.ks[0] + (int64_t)kj * p.ks[1] + g * p.ks[2]);
#pragma unroll
    for (int s = 0; s < C::NS; ++s) kf[s] = *(const bf16x8*)(krow + (16 * s + 8 * hl) * 2);
  }
  // retire the register operand loads now: a load still pending when the staged loop starts
  // would make the compiler wait for all vector memory, prefetched tiles included, at its first
  // use in every iteration
  wait_all_mem();
  const char* qbase = (const char*)((const bf16*)p.q + b * p.qs[0] + h * p.qs[2]);
  const int64_t qstride = p.qs[1] * 2;
  const float* lrow = p.lse2 + ((int64_t)b * p.Hq + h) * p.S;
  NatPlan<D, NW> qplan;
  qplan.init(qstride);
  ReadPlan<D> rp;
  rp.init();
  const float c2 = p.scale_log2;
  double acc = 0.0;

  const rsrc_t rq = make_rsrc_u(qbase), rl = make_rsrc_u(lrow);
  const uint32_t lvoff = 16u * (LDC * w + l);
  auto issue = [&](int t, char* buf) {
    const int q0 = k0 + 32 * t;
    qplan.issue(buf, rq, (uint32_t)(q0 * qstride));
    if (l < LDC) dma16b(rl, lvoff, (uint32_t)q0 * 4u, buf + C::NAT32 + 16 * LDC * w);
  };
  auto compute = [&](int t, const char* buf) {
    const int q0 = k0 + 32 * t;
    if (!active || q0 + 31 <= kw0) return;         // no query of the step follows a key
    f32x16 st = zero16();
#pragma unroll
    for (int s = 0; s < C::NS; ++s) st = Mfma<bf16>::mma(ldo(buf, rp.nat[s]), kf[s], st);
    SCHED_READS_AHEAD(C::NS, 1, 1, 0);
    const float* ls = (const float*)(buf + C::NAT32);
    float colsum = 0.f;
    if (q0 <= kw0 + 31) {                          // diagonal step: only queries after the key
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const f32x4 lq = *(const f32x4*)(ls + 8 * rg + 4 * hl);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(st[4 * rg + i], c2, -lq[i]));
          colsum += (q0 + 8 * rg + 4 * hl + i > kj) ? e : 0.f;
        }
      }
    } else {
      // (the sum starts from its first term: starting from 0 costs an addition per step)
      const f32x4 lq0 = *(const f32x4*)(ls + 4 * hl);
      colsum = __builtin_amdgcn_exp2f(__builtin_fmaf(st[0], c2, -lq0[0]));
#pragma unroll
      for (int i = 1; i < 4; ++i) colsum += __builtin_amdgcn_exp2f(__builtin_fmaf(st[i], c2, -lq0[i]));
#pragma unroll
      for (int rg = 1; rg < 4; ++rg) {
        const f32x4 lq = *(const f32x4*)(ls + 8 * rg + 4 * hl);
#pragma unroll
        for (int i = 0; i < 4; ++i) colsum += __builtin_amdgcn_exp2f(__builtin_fmaf(st[4 * rg + i], c2, -lq[i]));
      }
    }
    acc += (double)colsum;
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
  if (nsteps > 0) {
    issue(0, sA);
    issue(min(1, nsteps - 1), sB);
    ring3_loop(nsteps, sA, sB, sC, stage);
  }
  wait_all_mem();                                        // drain the trailing reloads
  // lanes l and l^32 hold the same key; then a fixed butterfly over the wave's 32 keys
  acc += __shfl_xor(acc, 32, 64);
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (active && l == 0) p.mass32[((int64_t)b * p.Hq + h) * (p.S / 32) + kw0 / 32] = acc;
}

constexpr int SCORE_NW = 4;

template <int D>
static hipError_t launch_score64_t(const ScoreParams& p, hipStream_t st) {
  constexpr int RG = 32 * SCORE_NW;
  hipError_t e;
  {
    TimedLaunch tl("k_slse64", st);
    k_slse64<D, SCORE_NW><<<dim3((p.S + RG - 1) / RG, p.Hq, p.B), 64 * SCORE_NW, 0, st>>>(p);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  TimedLaunch tl("k_smass64", st);
  k_smass64<D, SCORE_NW><<<dim3((p.S + RG - 1) / RG, p.Hq, p.B), 64 * SCORE_NW, 0, st>>>(p);
  return hipGetLastError();
}

hipError_t launch_score64(const ScoreParams& p, int D, hipStream_t st) {
  return D == 64 ? launch_score64_t<64>(p, st) : launch_score64_t<128>(p, st);
}

}  // namespace jenga
