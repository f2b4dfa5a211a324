// Block-level token informativeness on gfx950: received attention-probability mass per key
// block, without ever storing an S x S matrix.  This file holds the fp32-operand path, streamed
// in two passes, the launcher of both paths and the reduction over heads they share (the bf16
// path is score64.hip).
//
// Jenga (aipaper summary, §4.2.1 Eq. 1: a token's informativeness sums the interaction it
// receives from every other token, self excluded; §4.2.2 Eq. 2: per-head values are averaged
// over the heads; §4.2.3: score blocks are aggregated over the query-block index for each
// key block).  The interaction used here is the causal softmax probability.
//
//   pass 1 (k_score_lse):  per query i and head h, lse2_i = log2 sum_{j<=i} 2^(c q_i.k_j),
//                          c = scale*log2(e); online max/sum, the running sum in fp64.
//   pass 2 (k_score_mass): key-major; per key j, M(j) = sum_{i>j} 2^(c q_i.k_j - lse2_i),
//                          summed per 32-key group in fp64, in a fixed order.
//   reduce (k_score_reduce): s[b][n] = (1/Hq) sum_h sum_{groups of block n}, fp64 -> fp32
//                          (block/32 groups per block here; the bf16 path leaves one).
#include "common.h"
#include "kernels.h"

namespace jenga {

template <typename T>
__device__ inline typename Mfma<T>::frag ld_frag_s(const char* p) {
  return *(const float*)p;
}

template <typename T, int D>
struct ScoreCfg {
  static constexpr int ES = sizeof(T);
  static constexpr int ROWB = D * ES;
  static constexpr int LD = ROWB + 16;
  static constexpr int CPR = ROWB / 16;
  static constexpr int NS = D / Mfma<T>::KSTEP;
  // pass 1: 128 queries per workgroup, 64-key LDS tiles
  static constexpr int P1_BC = 64;
  static constexpr int P1_CPT = P1_BC * CPR / 256;
  // pass 2: 128 keys per workgroup, 64-query LDS tiles
  static constexpr int P2_BQ = 64;
  static constexpr int P2_CPT = P2_BQ * CPR / 256;
};

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void k_score_lse(ScoreParams p) {
  using M = Mfma<T>;
  using frag = typename M::frag;
  using C = ScoreCfg<T, D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::P1_BC * C::LD];

  const int b = blockIdx.z, h = blockIdx.y;
  const int g = h / (p.Hq / p.Hkv);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, hl = l >> 5, lc = l & 31;
  const int nqt = (p.S + 127) / 128;
  const int q0 = (nqt - 1 - (int)blockIdx.x) * 128;
  const int qw0 = q0 + 32 * w;
  const bool wave_active = qw0 < p.S;        // S is a multiple of 64
  const int qi = qw0 + lc;
  const int n_kt = (min(q0 + 128, p.S) - 1) / C::P1_BC + 1;

  frag qf[C::NS];
  if (wave_active) {
    const char* qrow = (const char*)((const T*)p.q + b * p.qs[0] + (int64_t)qi * p.qs[1] + h * p.qs[2]);
#pragma unroll
    for (int s = 0; s < C::NS; ++s) qf[s] = ld_frag_s<T>(qrow + (s * M::KSTEP + hl * M::KPL) * C::ES);
  }
  const char* kbase = (const char*)((const T*)p.k + b * p.ks[0] + g * p.ks[2]);
  u32x4 pk[C::P1_CPT];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < C::P1_CPT; ++i) {
      const int c = tid + 256 * i, row = c / C::CPR, col = c % C::CPR;
      pk[i] = ld16(kbase + ((int64_t)(kt * C::P1_BC + row) * p.ks[1]) * C::ES + col * 16);
    }
  };
  auto lstore = [&](int buf) {
    char* kl = smem + buf * C::P1_BC * C::LD;
#pragma unroll
    for (int i = 0; i < C::P1_CPT; ++i) {
      const int c = tid + 256 * i, row = c / C::CPR, col = c % C::CPR;
      *(u32x4*)(kl + row * C::LD + col * 16) = pk[i];
    }
  };

  float m_run = -INFINITY;
  double l_run = 0.0;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < n_kt; ++kt) {
    if (kt + 1 < n_kt) gload(kt + 1);
    const int kr0 = kt * C::P1_BC;
    if (wave_active && kr0 <= qw0 + 31) {
      const char* kl = smem + (kt & 1) * C::P1_BC * C::LD;
      f32x16 st[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        st[kb] = zero16();
        const char* krow = kl + (kb * 32 + lc) * C::LD + hl * M::KPL * C::ES;
#pragma unroll
        for (int s = 0; s < C::NS; ++s)
          st[kb] = M::mma(ld_frag_s<T>(krow + s * M::KSTEP * C::ES), qf[s], st[kb]);
      }
      const bool need_mask = kr0 + C::P1_BC - 1 > qw0;
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float z = st[kb][r] * p.scale_log2;
          if (need_mask) {
            const int kj = kr0 + kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
            if (kj > qi) z = -INFINITY;
          }
          st[kb][r] = z;
          mx = fmaxf(mx, z);
        }
      }
      mx = fmaxf(mx, wave_xor32(mx));
      const float m_new = fmaxf(m_run, mx);
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) rs += exp2f(st[kb][r] - m_new);
      rs += wave_xor32(rs);
      l_run = l_run * (double)exp2f(m_run - m_new) + (double)rs;
      m_run = m_new;
    }
    if (kt + 1 < n_kt) lstore((kt + 1) & 1);
    __syncthreads();
  }
  if (wave_active && hl == 0)
    p.lse2[((int64_t)b * p.Hq + h) * p.S + qi] = (float)((double)m_run + log2(l_run));
}

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void k_score_mass(ScoreParams p) {
  using M = Mfma<T>;
  using frag = typename M::frag;
  using C = ScoreCfg<T, D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::P2_BQ * C::LD];
  __shared__ float lse_s[2][C::P2_BQ];

  const int b = blockIdx.z, h = blockIdx.y;
  const int g = h / (p.Hq / p.Hkv);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, hl = l >> 5, lc = l & 31;
  const int k0 = blockIdx.x * 128;
  const int kw0 = k0 + 32 * w;
  const int kj = kw0 + lc;
  const bool wave_active = kw0 < p.S;        // S is a multiple of 64

  // K operand of S = Q K^T (B[k = d][n = key]) for this lane's key.
  frag kf[C::NS];
  if (wave_active) {
    const char* krow = (const char*)((const T*)p.k + b * p.ks[0] + (int64_t)kj * p.ks[1] + g * p.ks[2]);
#pragma unroll
    for (int s = 0; s < C::NS; ++s) kf[s] = ld_frag_s<T>(krow + (s * M::KSTEP + hl * M::KPL) * C::ES);
  }
  const char* qbase = (const char*)((const T*)p.q + b * p.qs[0] + h * p.qs[2]);
  const float* lse_row = p.lse2 + ((int64_t)b * p.Hq + h) * p.S;
  u32x4 pq[C::P2_CPT];
  float plse = 0.f;
  auto gload = [&](int qt0) {
#pragma unroll
    for (int i = 0; i < C::P2_CPT; ++i) {
      const int c = tid + 256 * i, row = c / C::CPR, col = c % C::CPR;
      pq[i] = ld16(qbase + ((int64_t)(qt0 + row) * p.qs[1]) * C::ES + col * 16);
    }
    if (tid < C::P2_BQ) plse = lse_row[qt0 + tid];
  };
  auto lstore = [&](int buf) {
    char* ql = smem + buf * C::P2_BQ * C::LD;
#pragma unroll
    for (int i = 0; i < C::P2_CPT; ++i) {
      const int c = tid + 256 * i, row = c / C::CPR, col = c % C::CPR;
      *(u32x4*)(ql + row * C::LD + col * 16) = pq[i];
    }
    if (tid < C::P2_BQ) lse_s[buf][tid] = plse;
  };

  double acc = 0.0;
  const int nq = (p.S - k0) / C::P2_BQ;     // query tiles k0, k0+64, ..., S-64
  gload(k0);
  lstore(0);
  __syncthreads();
  for (int it = 0; it < nq; ++it) {
    const int qt0 = k0 + it * C::P2_BQ;
    if (it + 1 < nq) gload(qt0 + C::P2_BQ);
    if (wave_active && qt0 + C::P2_BQ - 1 > kw0) {   // some query of the tile follows a key
      const char* ql = smem + (it & 1) * C::P2_BQ * C::LD;
      const float* ls = lse_s[it & 1];
      float colsum = 0.f;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        f32x16 st = zero16();
        const char* qrow = ql + (qb * 32 + lc) * C::LD + hl * M::KPL * C::ES;
#pragma unroll
        for (int s = 0; s < C::NS; ++s) st = M::mma(ld_frag_s<T>(qrow + s * M::KSTEP * C::ES), kf[s], st);
        const bool need_mask = qt0 + qb * 32 <= kw0 + 31;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qloc = qb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
          float e = exp2f(st[r] * p.scale_log2 - ls[qloc]);
          if (need_mask && qt0 + qloc <= kj) e = 0.f;     // only later queries, self excluded
          colsum += e;
        }
      }
      acc += (double)colsum;
    }
    if (it + 1 < nq) lstore((it + 1) & 1);
    __syncthreads();
  }
  // lanes l and l^32 hold the same key; then a fixed butterfly over the wave's 32 keys
  acc += __shfl_xor(acc, 32, 64);
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (wave_active && l == 0) p.mass32[((int64_t)b * p.Hq + h) * (p.S / 32) + kw0 / 32] = acc;
}

__global__ void k_score_reduce(ScoreParams p) {
  const int b = blockIdx.y;
  const int nkb = p.S / p.block;
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= nkb) return;
  const int gpb = p.mass_gpb, ng = nkb * gpb;
  const double* base = p.mass32 + (int64_t)b * p.Hq * ng + n * gpb;
  // terms k = h * gpb + c summed in ascending k; the reads of 16 terms are issued before they
  // are added, so the loop waits once per 16 terms instead of once per term
  constexpr int U = 16;
  const int K = p.Hq * gpb;
  double s = 0.0;
  int k = 0;
  for (; k + U <= K; k += U) {
    double t[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int h = (k + i) / gpb, c = k + i - h * gpb;
      t[i] = base[(int64_t)h * ng + c];
    }
#pragma unroll
    for (int i = 0; i < U; ++i) s += t[i];
  }
  for (; k < K; ++k) {
    const int h = k / gpb, c = k - h * gpb;
    s += base[(int64_t)h * ng + c];
  }
  p.scores[(int64_t)b * nkb + n] = (float)(s / p.Hq);
}

template <typename T, int D>
static hipError_t launch_score_t(const ScoreParams& p, hipStream_t st) {
  k_score_lse<T, D><<<dim3((p.S + 127) / 128, p.Hq, p.B), 256, 0, st>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_score_mass<T, D><<<dim3((p.S + 127) / 128, p.Hq, p.B), 256, 0, st>>>(p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nkb = p.S / p.block;
  k_score_reduce<<<dim3((nkb + 255) / 256, p.B), 256, 0, st>>>(p);
  return hipGetLastError();
}

hipError_t launch_score(const ScoreParams& p0, int dtype, int D, hipStream_t st) {
  ScoreParams p = p0;
  if (dtype == 1) {                      // bf16: one pass of score64.hip, mass per key block
    p.mass_gpb = 1;
    hipError_t e = launch_score64(p, D, st);
    if (e != hipSuccess) return e;
    const int nkb = p.S / p.block;
    k_score_reduce<<<dim3((nkb + 255) / 256, p.B), 256, 0, st>>>(p);
    return hipGetLastError();
  }
  p.mass_gpb = p.block / 32;             // fp32: mass per 32-key group
  return launch_score_t<float, 64>(p, st);    // fp32 operands: head_dim 64 only
}
}  // namespace jenga
