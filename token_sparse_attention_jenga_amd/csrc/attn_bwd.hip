// Segmented backward of the token-sparse attention for gfx950, fp32 operands (head_dim 64,
// fp32 MFMA); the bf16 backward is attn64.hip.
//
// Jenga (papercache notes, §4.4, segment-based peak cutting: the sequence is processed as N
// segments one after the other, each segment's transient activations are discarded once its
// gradients are aggregated, so the transient peak falls to about 1/N).  Here a segment is a
// contiguous range of kept query ranks; its transients are the dot(dO, O) terms and an
// operand-dtype copy of its dOut rows.  Kept rows are addressed in place through the kept
// block list (§4.4 permutation-free token movement), and eliminated rows are never touched.
//
//   k_bwd_prep: D_i = dOut_i . O_i for the segment's queries, and dOut -> operand dtype,
//               both stored compactly by kept rank.
//   k_bwd_main: key-major.  A workgroup owns 128 kept keys of one KV head and walks the
//               segment's 64-query tiles for every query head of the group.  Per wave (32
//               keys):  S = Q K^T and dP = dO V^T (lanes hold one key's column),
//               P = 2^(c S - lse2), dS = P (dP - D), dV += P^T dO, dK += dS^T Q with the
//               accumulators in registers; dS^T goes to LDS and the four waves then compute
//               dQ = dS K for the tile and add it to dq with fp32 atomics.  dK/dV are added
//               to global memory once per segment.
#include "common.h"
#include "kernels.h"

namespace jenga {

template <typename T>
__device__ inline typename Mfma<T>::frag ld_frag_b(const char* p) {
  return *(const float*)p;
}

// ---------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void k_bwd_prep(BwdParams p) {
  constexpr int TPR = D / 4;               // threads per (rank, head) row
  constexpr int RPB = 256 / TPR;           // rows per block
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int row = blockIdx.x * RPB + tid / TPR;
  const int d0 = (tid % TPR) * 4;
  const int Nk = min(p.n_kept[b], p.max_kept_blocks) * p.block;
  const int qs = p.seg * p.seg_len;
  const int qe = min(qs + p.seg_len, Nk);
  const int rl = row / p.Hq, h = row % p.Hq;
  const int r = qs + rl;
  const bool valid = r < qe;
  float dot = 0.f;
  if (valid) {
    const int32_t* kept = p.kept + (int64_t)b * p.nkb;
    const int pos = rank_to_pos(kept, p.block, r);
    const f32x4 dov = *(const f32x4*)(p.dout + (((int64_t)b * p.S + pos) * p.Hq + h) * D + d0);
    const int64_t oidx = (((int64_t)b * p.ncap + r) * p.Hq + h) * D + d0;
    const int64_t widx = (((int64_t)b * p.seg_len + rl) * p.Hq + h) * D + d0;
    const f32x4 ov = *(const f32x4*)((const char*)p.o_saved + oidx * 4);
    dot = dov[0] * ov[0] + dov[1] * ov[1] + dov[2] * ov[2] + dov[3] * ov[3];
    *(f32x4*)((char*)p.wsdO + widx * 4) = dov;
  }
#pragma unroll
  for (int off = TPR / 2; off >= 1; off >>= 1) dot += __shfl_xor(dot, off, 64);
  if (valid && (tid % TPR) == 0) p.wsD[((int64_t)b * p.Hq + h) * p.seg_len + rl] = dot;
}

// ---------------------------------------------------------------------------------------
template <typename T, int D>
struct BwdCfg {
  static constexpr int BKC = 128;          // kept keys per workgroup (4 waves x 32)
  static constexpr int BQ = 64;            // queries per tile
  static constexpr int ES = sizeof(T);
  static constexpr int ROWB = D * ES;
  static constexpr int LDK = ROWB + 16;    // K tile pitch
  static constexpr int LDQ = ROWB + 16;    // Q / dO tile pitch
  static constexpr int LDS_ = BQ * ES + 16;  // dS^T tile pitch (rows = keys, cols = queries)
  static constexpr int K_OFF = 0;
  static constexpr int Q_OFF = K_OFF + BKC * LDK;
  static constexpr int DO_OFF = Q_OFF + BQ * LDQ;
  static constexpr int DS_OFF = DO_OFF + BQ * LDQ;
  static constexpr int V_OFF = Q_OFF;      // V staging reuses the Q/dO region at start
  static constexpr int BYTES = DS_OFF + BKC * LDS_;
  static constexpr int CPR = ROWB / 16;
  static constexpr int NS = D / Mfma<T>::KSTEP;
  static constexpr int NDB = D / 32;
};

template <typename T, int D>
__global__ __launch_bounds__(256, 1) void k_bwd_main(BwdParams p) {
  using M = Mfma<T>;
  using frag = typename M::frag;
  using C = BwdCfg<T, D>;
  static_assert(C::BKC * C::LDK <= 2 * C::BQ * C::LDQ + C::BKC * C::LDS_, "V staging must fit");
  __shared__ __attribute__((aligned(16))) char smem[C::BYTES];
  __shared__ float lse_s[C::BQ];
  __shared__ float dv_s[C::BQ];

  const int b = blockIdx.z, g = blockIdx.y;
  const int G = p.Hq / p.Hkv;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, hl = l >> 5, lc = l & 31;
  const int32_t* kept = p.kept + (int64_t)b * p.nkb;
  const int Nk = min(p.n_kept[b], p.max_kept_blocks) * p.block;
  const int qs = p.seg * p.seg_len;
  const int qe = min(qs + p.seg_len, Nk);
  const int k0 = blockIdx.x * C::BKC;
  if (qs >= qe || k0 >= qe) return;
  const int kw0 = k0 + 32 * w;
  const bool key_valid = kw0 < Nk;        // Nk is a multiple of 64: uniform per wave
  const int kr = kw0 + lc;

  // ---- stage K (kept for dQ) and V (only to build register operands) in LDS ----
  {
    const char* kbase = (const char*)((const T*)p.k + b * p.ks[0] + g * p.ks[2]);
    const char* vbase = (const char*)((const T*)p.v + b * p.vs[0] + g * p.vs[2]);
    for (int c = tid; c < C::BKC * C::CPR; c += 256) {
      const int row = c / C::CPR, col = c % C::CPR;
      const int rk = k0 + row;
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (rk < Nk) {
        const int pos = rank_to_pos(kept, p.block, rk);
        kv = ld16(kbase + ((int64_t)pos * p.ks[1]) * C::ES + col * 16);
        vv = ld16(vbase + ((int64_t)pos * p.vs[1]) * C::ES + col * 16);
      }
      *(u32x4*)(smem + C::K_OFF + row * C::LDK + col * 16) = kv;
      *(u32x4*)(smem + C::V_OFF + row * C::LDK + col * 16) = vv;
    }
  }
  __syncthreads();
  frag kf[C::NS], vf[C::NS];
  {
    const char* krow = smem + C::K_OFF + (32 * w + lc) * C::LDK + hl * M::KPL * C::ES;
    const char* vrow = smem + C::V_OFF + (32 * w + lc) * C::LDK + hl * M::KPL * C::ES;
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
      kf[s] = ld_frag_b<T>(krow + s * M::KSTEP * C::ES);
      vf[s] = ld_frag_b<T>(vrow + s * M::KSTEP * C::ES);
    }
  }
  f32x16 dka[C::NDB], dva[C::NDB];
#pragma unroll
  for (int i = 0; i < C::NDB; ++i) {
    dka[i] = zero16();
    dva[i] = zero16();
  }

  char* Ql = smem + C::Q_OFF;
  char* dOl = smem + C::DO_OFF;
  char* dSl = smem + C::DS_OFF;
  const LDS_AS char* Qls = (const LDS_AS char*)Ql;
  const LDS_AS char* dOls = (const LDS_AS char*)dOl;
  const LDS_AS char* dSls = (const LDS_AS char*)dSl;
  const LDS_AS char* Kls = (const LDS_AS char*)(smem + C::K_OFF);

  const int qfirst = max(qs, k0);
  for (int q0 = qfirst; q0 < qe; q0 += C::BQ) {
    const int qpos0 = rank_to_pos(kept, p.block, q0);      // 64 ranks = one position run
    for (int hh = 0; hh < G; ++hh) {
      const int h = g * G + hh;
      __syncthreads();                                        // previous tile fully consumed
      {
        const char* qbase = (const char*)((const T*)p.q + b * p.qs[0] + h * p.qs[2]);
        const char* dobase = (const char*)p.wsdO +
                             ((((int64_t)b * p.seg_len + (q0 - qs)) * p.Hq + h) * D) * C::ES;
        for (int c = tid; c < C::BQ * C::CPR; c += 256) {
          const int row = c / C::CPR, col = c % C::CPR;
          *(u32x4*)(Ql + row * C::LDQ + col * 16) =
              ld16(qbase + ((int64_t)(qpos0 + row) * p.qs[1]) * C::ES + col * 16);
          *(u32x4*)(dOl + row * C::LDQ + col * 16) =
              ld16(dobase + ((int64_t)row * p.Hq * D) * C::ES + col * 16);
        }
        if (tid < C::BQ) {
          lse_s[tid] = p.lse[((int64_t)b * p.Hq + h) * p.ncap + q0 + tid] * kLog2e;
          dv_s[tid] = p.wsD[((int64_t)b * p.Hq + h) * p.seg_len + (q0 - qs) + tid];
        }
      }
      __syncthreads();

      if (key_valid && q0 + C::BQ - 1 >= kw0) {
        f32x16 sacc[2], pacc[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          sacc[qb] = zero16();
          pacc[qb] = zero16();
          const char* qrow = Ql + (qb * 32 + lc) * C::LDQ + hl * M::KPL * C::ES;
          const char* drow = dOl + (qb * 32 + lc) * C::LDQ + hl * M::KPL * C::ES;
#pragma unroll
          for (int s = 0; s < C::NS; ++s) {
            sacc[qb] = M::mma(ld_frag_b<T>(qrow + s * M::KSTEP * C::ES), kf[s], sacc[qb]);
            pacc[qb] = M::mma(ld_frag_b<T>(drow + s * M::KSTEP * C::ES), vf[s], pacc[qb]);
          }
        }
        // P and dS; lane = key kr, register r = query qb*32 + 8(r/4) + 4hl + r%4
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ql = qb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
            float pv = exp2f(sacc[qb][r] * p.scale_log2 - lse_s[ql]);
            if (q0 + ql < kr) pv = 0.f;
            sacc[qb][r] = pv;
            pacc[qb][r] = pv * (pacc[qb][r] - dv_s[ql]);
          }
        }
        // dV += P^T dO, dK += dS^T Q  (M = keys, N = head_dim, reduction over queries)
#pragma unroll
        for (int t = 0; t < 32; ++t) {
          const int qb = t >> 4, r = t & 15;
          const int ql = qb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) {
            const float bdo = *(const float*)(dOl + ql * C::LDQ + (db * 32 + lc) * 4);
            const float bq = *(const float*)(Ql + ql * C::LDQ + (db * 32 + lc) * 4);
            dva[db] = M::mma(sacc[qb][r], bdo, dva[db]);
            dka[db] = M::mma(pacc[qb][r], bq, dka[db]);
          }
        }
        // dS^T -> LDS: row = key (32w + lc), 4 consecutive queries per store
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const int qcol = qb * 32 + 8 * rg + 4 * hl;
            char* dst = dSl + (32 * w + lc) * C::LDS_ + qcol * C::ES;
            f32x4 y;
            y[0] = pacc[qb][4 * rg + 0];
            y[1] = pacc[qb][4 * rg + 1];
            y[2] = pacc[qb][4 * rg + 2];
            y[3] = pacc[qb][4 * rg + 3];
            *(f32x4*)dst = y;
          }
        }
      } else {
        // no contribution from this wave's keys: zero its dS^T rows
        for (int c = l; c < 32 * C::BQ * C::ES / 16; c += 64) {
          const int row = c / (C::BQ * C::ES / 16), col = c % (C::BQ * C::ES / 16);
          *(u32x4*)(dSl + (32 * w + row) * C::LDS_ + col * 16) = u32x4{0u, 0u, 0u, 0u};
        }
      }
      __syncthreads();

      // dQ[q][d] = scale * sum_key dS[q][key] K[key][d] over this workgroup's 128 keys
      for (int item = w; item < 2 * C::NDB; item += 4) {
        const int qb = item / C::NDB, db = item % C::NDB;
        f32x16 acc = zero16();
#pragma unroll 8
        for (int ks = 0; ks < C::BKC / 2; ++ks) {
          const int key = 2 * ks + hl;
          const float a = *(const float*)(dSl + key * C::LDS_ + (qb * 32 + lc) * 4);
          const float bk = *(const float*)(smem + C::K_OFF + key * C::LDK + (db * 32 + lc) * 4);
          acc = M::mma(a, bk, acc);
        }

        float* dqb = p.dq + (((int64_t)b * p.S + qpos0) * p.Hq + h) * D + db * 32 + lc;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ql = qb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
          unsafeAtomicAdd(dqb + (int64_t)ql * p.Hq * D, p.scale * acc[r]);
        }
      }
    }
  }

  if (!key_valid) return;
  // dK, dV: lane holds head_dim column db*32 + lc for keys 8(r/4) + 4hl + r%4 of the wave
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int kl = 8 * (r >> 2) + 4 * hl + (r & 3);
    const int pos = rank_to_pos(kept, p.block, kw0 + kl);
    float* dkr = p.dk + (((int64_t)b * p.S + pos) * p.Hkv + g) * D + lc;
    float* dvr = p.dv + (((int64_t)b * p.S + pos) * p.Hkv + g) * D + lc;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      dkr[db * 32] += p.scale * dka[db][r];
      dvr[db * 32] += dva[db][r];
    }
  }
}

template <typename T, int D>
static hipError_t launch_bwd_t(const BwdParams& p, hipStream_t st) {
  constexpr int RPB = 256 / (D / 4);
  const int rows = p.seg_len * p.Hq;
  k_bwd_prep<T, D><<<dim3((rows + RPB - 1) / RPB, p.B), 256, 0, st>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int seg_end = min((p.seg + 1) * p.seg_len, p.max_kept_blocks * p.block);
  const int nkt = (seg_end + 127) / 128;
  k_bwd_main<T, D><<<dim3(nkt, p.Hkv, p.B), 256, 0, st>>>(p);
  return hipGetLastError();
}

// fp32 operands, head_dim 64 (the bf16 backward is attn64.hip)
hipError_t launch_bwd_segment_f32(const BwdParams& p, hipStream_t st) { return launch_bwd_t<float, 64>(p, st); }
}  // namespace jenga
