// Permutation-free token-sparse causal attention forward for gfx950, fp32 operands
// (head_dim 64, fp32 MFMA); the bf16 forward is attn64.hip.
//
// Jenga (papercache notes, §4.4, permutation-free token movement; Fig. 9): kept tokens are
// read straight from the full-length Q/K/V through the kept-block index list (no gathered
// copy), the attention output is added into the full-length residual in place (padding and
// residual add in one step), and eliminated rows are never touched.
//
// One workgroup = 4 waves = 128 kept query ranks of one query head.  Each wave owns 32
// queries and computes S^T = K Q^T (keys x queries) so that every lane holds one query's
// column: the online-softmax row statistics are lane-local plus one exchange with lane
// l^32.  O^T = V^T P^T accumulates in registers: each fp32 MFMA takes one key's P^T value
// straight from the S^T accumulator and that key's V values from the row-major LDS tile.
// K/V tiles of 64 kept keys are double-buffered in LDS; a tile is one contiguous run of
// token positions because blocks are multiples of 64 tokens.
#include "common.h"
#include "kernels.h"

namespace jenga {

template <typename T>
__device__ inline typename Mfma<T>::frag ld_frag(const char* p) {
  return *(const float*)p;
}

template <typename T, int D>
struct FwdCfg {
  static constexpr int BR = 128;                          // query ranks per workgroup
  static constexpr int BC = 64;                           // keys per LDS tile
  static constexpr int ES = sizeof(T);
  static constexpr int ROWB = D * ES;                     // bytes of one head row
  static constexpr int LDK = ROWB + 16;                   // K tile pitch (row reads)
  static constexpr int LDV = ROWB + (ES == 2 ? 64 : 16);  // V tile pitch (transpose reads)
  static constexpr int KT_BYTES = BC * LDK;
  static constexpr int VT_BYTES = BC * LDV;
  static constexpr int STAGE = KT_BYTES + VT_BYTES;
  static constexpr int CPR = ROWB / 16;                   // 16-byte chunks per row
  static constexpr int CPT = BC * CPR / 256;              // chunks per thread per tile
  static constexpr int NS = D / Mfma<T>::KSTEP;           // MFMA k-steps over head_dim
  static constexpr int NDB = D / 32;                      // 32-wide head_dim blocks
};

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void k_attn_fwd(FwdParams p) {
  using M = Mfma<T>;
  using frag = typename M::frag;
  using C = FwdCfg<T, D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE];

  const int b = blockIdx.z, h = blockIdx.y;
  const int g = h / (p.Hq / p.Hkv);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, hl = l >> 5, lc = l & 31;
  const int32_t* kept = p.kept + (int64_t)b * p.nkb;
  const int nkb_kept = min(p.n_kept[b], p.max_kept_blocks);
  const int Nk = nkb_kept * p.block;
  const int nqt = (Nk + C::BR - 1) / C::BR;
  if ((int)blockIdx.x >= nqt) return;
  const int q0 = (nqt - 1 - (int)blockIdx.x) * C::BR;     // heaviest (latest) tiles first
  const int qw0 = q0 + 32 * w;
  const bool wave_active = qw0 < Nk;                       // Nk is a multiple of 64
  const int qr = qw0 + lc;
  const int qlast = min(q0 + C::BR, Nk) - 1;
  const int n_kt = qlast / C::BC + 1;

  // Q operand of S^T = K Q^T for this lane's query, straight from global memory.
  frag qf[C::NS];
  int qpos = 0;
  if (wave_active) {
    qpos = rank_to_pos(kept, p.block, qr);
    const char* qrow = (const char*)((const T*)p.q + b * p.qs[0] + (int64_t)qpos * p.qs[1] +
                                     h * p.qs[2]);
#pragma unroll
    for (int s = 0; s < C::NS; ++s) qf[s] = ld_frag<T>(qrow + (s * M::KSTEP + hl * M::KPL) * C::ES);
  }

  f32x16 o[C::NDB];
#pragma unroll
  for (int i = 0; i < C::NDB; ++i) o[i] = zero16();
  float m_run = -INFINITY, l_run = 0.f;

  const char* kbase = (const char*)((const T*)p.k + b * p.ks[0] + g * p.ks[2]);
  const char* vbase = (const char*)((const T*)p.v + b * p.vs[0] + g * p.vs[2]);
  u32x4 pk[C::CPT], pv[C::CPT];

  auto gload = [&](int kt) {
    const int kpos0 = rank_to_pos(kept, p.block, kt * C::BC);
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int c = tid + 256 * i, row = c / C::CPR, col = c % C::CPR;
      pk[i] = ld16(kbase + ((int64_t)(kpos0 + row) * p.ks[1]) * C::ES + col * 16);
      pv[i] = ld16(vbase + ((int64_t)(kpos0 + row) * p.vs[1]) * C::ES + col * 16);
    }
  };
  auto lstore = [&](int buf) {
    char* kl = smem + buf * C::STAGE;
    char* vl = kl + C::KT_BYTES;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int c = tid + 256 * i, row = c / C::CPR, col = c % C::CPR;
      *(u32x4*)(kl + row * C::LDK + col * 16) = pk[i];
      *(u32x4*)(vl + row * C::LDV + col * 16) = pv[i];
    }
  };

  gload(0);
  lstore(0);
  __syncthreads();

  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_kt) gload(kt + 1);
    const int kr0 = kt * C::BC;
    if (wave_active && kr0 <= qw0 + 31) {
      const char* kl = smem + buf * C::STAGE;
      const char* vl = kl + C::KT_BYTES;
      f32x16 st[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        st[kb] = zero16();
        const char* krow = kl + (kb * 32 + lc) * C::LDK + hl * M::KPL * C::ES;
#pragma unroll
        for (int s = 0; s < C::NS; ++s)
          st[kb] = M::mma(ld_frag<T>(krow + s * M::KSTEP * C::ES), qf[s], st[kb]);
      }
      // scale into the log2 domain, causal mask in kept-rank space, row max
      const bool need_mask = kr0 + C::BC - 1 > qw0;
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float z = st[kb][r] * p.scale_log2;
          if (need_mask) {
            const int kr = kr0 + kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
            if (kr > qr) z = -INFINITY;
          }
          st[kb][r] = z;
          mx = fmaxf(mx, z);
        }
      }
      mx = fmaxf(mx, wave_xor32(mx));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2f(m_run - m_new);
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = exp2f(st[kb][r] - m_new);
          st[kb][r] = e;
          rs += e;
        }
      }
      rs += wave_xor32(rs);
      l_run = l_run * alpha + rs;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) o[db] *= alpha;

      // O^T += V^T P^T
      const LDS_AS char* vls = (const LDS_AS char*)vl;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int key = kb * 32 + 8 * (t >> 2) + 4 * hl + (t & 3);
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) {
            const float va = *(const float*)(vl + key * C::LDV + (db * 32 + lc) * 4);
            o[db] = M::mma(va, st[kb][t], o[db]);
          }
        }
      }
    }
    if (kt + 1 < n_kt) lstore((kt + 1) & 1);
    __syncthreads();
  }

  if (!wave_active) return;
  // Epilogue: normalise, add into the residual at the token's own row, save O and LSE
  // compactly by kept rank for the backward.
  const float inv = 1.f / l_run;
  float* rrow = p.resid + (((int64_t)b * p.S + qpos) * p.Hq + h) * D;
  char* orow = (char*)p.o_saved + ((((int64_t)b * p.ncap + qr) * p.Hq + h) * D) * C::ES;
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d0 = db * 32 + 8 * rg + 4 * hl;
      const float v0 = o[db][4 * rg + 0] * inv, v1 = o[db][4 * rg + 1] * inv;
      const float v2 = o[db][4 * rg + 2] * inv, v3 = o[db][4 * rg + 3] * inv;
      f32x4 x = *(f32x4*)(rrow + d0);
      x[0] += v0;
      x[1] += v1;
      x[2] += v2;
      x[3] += v3;
      *(f32x4*)(rrow + d0) = x;
      f32x4 y;
      y[0] = v0;
      y[1] = v1;
      y[2] = v2;
      y[3] = v3;
      *(f32x4*)(orow + d0 * 4) = y;
    }
  }
  if (hl == 0) p.lse[((int64_t)b * p.Hq + h) * p.ncap + qr] = (m_run + log2f(l_run)) * kLn2;
}

template <typename T, int D>
static hipError_t launch_fwd_t(const FwdParams& p, hipStream_t st) {
  const int ntiles = (p.max_kept_blocks * p.block + 127) / 128;
  dim3 grid(ntiles, p.Hq, p.B);
  k_attn_fwd<T, D><<<grid, 256, 0, st>>>(p);
  return hipGetLastError();
}

// fp32 operands, head_dim 64 (the bf16 forward is attn64.hip)
hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t st) { return launch_fwd_t<float, 64>(p, st); }
}  // namespace jenga
