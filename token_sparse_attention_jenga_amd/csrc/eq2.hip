// Eq. 2 literal block scoring for gfx950 (bf16).
//
// Jenga (aipaper summary, §4.2.2 Eq. 2): the informativeness of a score block is the maximum,
// over its elements, of the attention scores aggregated across heads, where only positive
// scores enter the aggregation and the sum is divided by the number of heads; §4.2.3: a token
// block's score sums its score blocks.  Here score block (m, n) pairs query block m with key
// block n (m >= n, causal):
//   e_ij = (1/Hq) sum_h max(c q_i^h . k_j^g(h), 0),  B(m,n) = max_{i in m, j in n, j <= i} e_ij,
//   s_n  = sum_{m >= n} B(m,n).
//
//   k_eq2_tiles   one workgroup per causal score block: loops over the query heads, S^h = Q K^T
//                 per 32x32 sub-tile with MFMA, acc += max(S^h, 0); then the causal mask on the
//                 diagonal block and the block maximum, times c / Hq (c > 0 factors out of the
//                 positive part and the maximum).  Q and K tiles load in 64-column chunks of
//                 head_dim; the next chunk loads into a second LDS buffer while the current one
//                 is multiplied.  A head's positive part is added while the next head's
//                 products run.
//   k_eq2_reduce  s_n = sum over m >= n in a fixed order (fp64), rounded once to fp32.
#include "common.h"
#include "kernels.h"
#include "tiles64.h"

namespace jenga {

// Score blocks are visited in super-tiles of kSM query blocks x kSN key blocks, one
// workgroup per block: the kSM * kSN = 32 consecutive workgroups of an XCD's range run side by
// side and share kSM Q and kSN K blocks per head in that XCD's L2, instead of one Q block and
// 32 different K blocks.  (8 x 8 super-tiles, as many as the XCD's 32 compute units hold at two
// workgroups each, measured no faster.)  Super-tile (M, N) holds the blocks m in [kSM M, kSM M + kSM),
// n in [kSN N, kSN N + kSN); only super-tiles holding some causal block (m >= n) are
// launched, N-major, and slots with m < n or past the last block exit at once.
constexpr int kSM = 4, kSN = 8;

__host__ __device__ inline int eq2_super_rows(int nkb) { return (nkb + kSM - 1) / kSM; }
// first super-row M holding a causal block of super-column N: kSM M + kSM - 1 >= kSN N
__host__ __device__ inline int eq2_first_row(int N) {
  const int need = kSN * N - (kSM - 1);
  return need <= 0 ? 0 : (need + kSM - 1) / kSM;
}
__host__ __device__ inline int eq2_super_tiles(int nkb) {
  const int R = eq2_super_rows(nkb), Cn = (nkb + kSN - 1) / kSN;
  int n = 0;
  for (int N = 0; N < Cn; ++N) n += R - eq2_first_row(N);
  return n;
}

// (m, n) of workgroup slot t; false for a slot without a causal block
__device__ inline bool pair_of(int t, int nkb, int& m, int& n) {
  const int slot = t % (kSM * kSN);
  int st = t / (kSM * kSN), N = 0;
  const int R = eq2_super_rows(nkb);
  for (;;) {
    const int cnt = R - eq2_first_row(N);
    if (st < cnt) break;
    st -= cnt;
    ++N;
  }
  m = kSM * (eq2_first_row(N) + st) + slot / kSN;
  n = kSN * N + slot % kSN;
  return m < nkb && n <= m;
}

// max(x, 0) as one integer max on the bits: a float with the sign bit set is a negative int32
// (-0 included), any other a non-negative one, so this gives x for x > 0 and +0 otherwise.
// (fmaxf first quietens an operand that comes out of an MFMA, one more VALU instruction per
// element: 4.9 against 5.3 ms per 32K-token layer.)
__device__ inline float pos_part(float x) {
  return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
}

// One 64-column head_dim chunk of a wave's HB x HB sub-tiles: W += Q K^T over the chunk's k-steps
// (from zero on a head's first chunk), with the positive part of sub-tiles [R0, R1) of the
// previous head's scores R added to acc between the MFMAs, so that the VALU work of one head
// runs under the MFMA work of the next within the wave.  The operand reads run two k-steps
// ahead.
template <int HB, int R0, int R1, bool FIRST>
__device__ __attribute__((always_inline)) inline void eq2_chunk(const char* Q0, const char* K0,
                                                                const int* nat, f32x16* W,
                                                                const f32x16* R, f32x16* acc) {
  using C = T64<64>;
#pragma unroll
  for (int s = 0; s < C::NS; ++s) {
    bf16x8 a[HB], bk[HB];
#pragma unroll
    for (int i = 0; i < HB; ++i) a[i] = ldo(Q0 + i * C::NAT32, nat[s]);
#pragma unroll
    for (int i = 0; i < HB; ++i) bk[i] = ldo(K0 + i * C::NAT32, nat[s]);
#pragma unroll
    for (int i = 0; i < HB; ++i)
#pragma unroll
      for (int j = 0; j < HB; ++j)
        W[HB * i + j] = Mfma<bf16>::mma(a[i], bk[j], (FIRST && s == 0) ? zero16() : W[HB * i + j]);
  }
#pragma unroll
  for (int t = R0; t < R1; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] += pos_part(R[t][r]);
  // reads of k-steps 0 and 1; then per k-step s its MFMAs, each followed by its share of the
  // VALU work, and the reads of step s + 2
  constexpr int MF = C::NS * HB * HB, VPM = 2 * 16 * (R1 - R0) / MF;
  static_assert(VPM * MF == 2 * 16 * (R1 - R0), "VALU work spreads evenly over the MFMAs");
  __builtin_amdgcn_sched_group_barrier(0x100, 4 * HB, 0);
#pragma unroll
  for (int s = 0; s < C::NS; ++s) {
#pragma unroll
    for (int m = 0; m < HB * HB; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (VPM > 0) __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
    }
    if (s + 2 < C::NS) __builtin_amdgcn_sched_group_barrier(0x100, 2 * HB, 0);
  }
}

template <int D, int BLK>
__global__ __launch_bounds__(256, 2) void k_eq2_tiles(Eq2Params p) {
  // Tiles are staged in 64-column chunks of head_dim (the scores of a head are summed over its
  // chunks before the positive part is taken): a stage is then small enough for two
  // workgroups per compute unit, each covering the other's load latency.
  using C = T64<64>;
  constexpr int DC = D / 64;                              // head_dim chunks per head
  constexpr int NW = 4;
  constexpr int SB = BLK / 32;                            // 32-row sub-blocks per block
  constexpr int SPW = SB * SB / NW;                       // sub-tiles per wave
  static_assert(SPW >= 1 && SB * SB == SPW * NW, "block must be 64 or 128");
  constexpr int STAGE = 2 * SB * C::NAT32;                // Q tiles then K tiles of one chunk
  __shared__ __attribute__((aligned(1024))) char sA[STAGE];
  __shared__ __attribute__((aligned(1024))) char sB[STAGE];
  __shared__ float wmax[NW];

  const Tile3 tl = xcd_tile();
  const int b = tl.y;
  int m, n;
  if (!pair_of(tl.x, p.nkb, m, n)) return;
  const int G = p.Hq / p.Hkv;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, hl = l >> 5, lc = l & 31;

  const int64_t qstride = p.qs[1] * 2, kstride = p.ks[1] * 2;
  NatPlan<64, NW> qplan, kplan;
  qplan.init(qstride);
  kplan.init(kstride);
  ReadPlan<64> rp;
  rp.init();
  const rsrc_t rq = make_rsrc((const bf16*)p.q + b * p.qs[0]);
  const rsrc_t rk = make_rsrc((const bf16*)p.k + b * p.ks[0]);
  const int nu = p.Hq * DC;                               // (head, chunk) steps
  auto issue = [&](int u, char* buf) {
    const int h = u / DC, c = u - h * DC, g = h / G;
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
      qplan.issue(buf + sb * C::NAT32, rq,
                  (uint32_t)((h * p.qs[2] + (int64_t)(m * BLK + 32 * sb) * p.qs[1]) * 2 + 128 * c));
      kplan.issue(buf + (SB + sb) * C::NAT32, rk,
                  (uint32_t)((g * p.ks[2] + (int64_t)(n * BLK + 32 * sb) * p.ks[1]) * 2 + 128 * c));
    }
  };

  // sub-tile t = HB i + j of this wave: query sub-block qsb0 + i, key sub-block ksb0 + j.  The
  // waves take the four quadrants of the SB x SB sub-tiles, so a wave's HB query and HB key
  // operand reads of a k-step serve HB^2 MFMAs
  constexpr int HB = SB / 2;
  static_assert(HB * HB == SPW, "one quadrant of sub-tiles per wave");
  const int qsb0 = (w >> 1) * HB, ksb0 = (w & 1) * HB;

  // Heads in pairs: head 2i's products go to sx, head 2i+1's to sy; chunk c of a head adds the
  // positive part of sub-tiles [c SPW / DC, (c + 1) SPW / DC) of the previous head.  Before the
  // first head the array read holds zeros, which add nothing.
  f32x16 acc[SPW], sx[SPW], sy[SPW];
#pragma unroll
  for (int t = 0; t < SPW; ++t) acc[t] = sx[t] = sy[t] = zero16();

  issue(0, sA);
  wait_all_mem();
  __syncthreads();
  // chunk c of head h: stage u = h DC + c, in buffer u % 2; stage u + 1 loads meanwhile
#define EQ2_CHUNK(W, R, c, cur, nxt)                                                               \
  do {                                                                                           \
    const int u_ = h * DC + (c);                                                                 \
    if (u_ + 1 < nu) issue(u_ + 1, nxt);                                                         \
    eq2_chunk<HB, (c) * SPW / DC, ((c) + 1) * SPW / DC, (c) == 0>(                               \
        cur + qsb0 * C::NAT32, cur + (SB + ksb0) * C::NAT32, rp.nat, W, R, acc);                \
    wait_all_mem();                                                                              \
    stage_barrier();                                                                             \
  } while (0)
  static_assert(DC == 1 || DC == 2, "head_dim 64 or 128");
  // (one loop with the exit between the two heads of a pair: with a loop over pairs and the
  // last head of an odd count after it, the compiler spilled 68 registers)
  for (int h = 0;; ++h) {
    // stage h DC + c sits in buffer (h DC + c) % 2
    if constexpr (DC == 1) {
      EQ2_CHUNK(sx, sy, 0, sA, sB);
      if (++h >= p.Hq) break;
      EQ2_CHUNK(sy, sx, 0, sB, sA);
    } else {
      EQ2_CHUNK(sx, sy, 0, sA, sB);
      EQ2_CHUNK(sx, sy, 1, sB, sA);
      if (++h >= p.Hq) break;
      EQ2_CHUNK(sy, sx, 0, sA, sB);
      EQ2_CHUNK(sy, sx, 1, sB, sA);
    }
    if (h + 1 >= p.Hq) break;
  }
#undef EQ2_CHUNK
  // the positive part of the last head
  const bool last_in_x = p.Hq % 2 != 0;
#pragma unroll
  for (int t = 0; t < SPW; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] += pos_part(last_in_x ? sx[t][r] : sy[t][r]);
  auto qsb = [&](int t) { return qsb0 + t / HB; };
  auto ksb = [&](int t) { return ksb0 + t % HB; };

  // lane = key n*BLK + 32 ksb + lc; register r = query m*BLK + 32 qsb + 8(r/4) + 4hl + r%4.
  // Every e >= 0, so a masked element set to 0 cannot raise the maximum.
  float mx = 0.f;
#pragma unroll
  for (int t = 0; t < SPW; ++t) {
    const int qrow0 = 32 * qsb(t) + 4 * hl, kcol = 32 * ksb(t) + lc;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const bool masked = m == n && kcol > qrow0 + 8 * (r >> 2) + (r & 3);
      mx = fmaxf(mx, masked ? 0.f : acc[t][r]);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if (l == 0) wmax[w] = mx;
  __syncthreads();
  if (tid == 0) {
    float v = wmax[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) v = fmaxf(v, wmax[i]);
    p.tilemax[((int64_t)b * p.nkb + m) * p.nkb + n] = v * p.scale / (float)p.Hq;
  }
}

__global__ __launch_bounds__(256) void k_eq2_reduce(Eq2Params p) {
  const int b = blockIdx.y, n = blockIdx.x * 256 + threadIdx.x;
  if (n >= p.nkb) return;
  const float* col = p.tilemax + (int64_t)b * p.nkb * p.nkb + n;
  // the sum runs over m in ascending order; the reads of 16 terms are issued before they are
  // added, so the loop waits once per 16 terms instead of once per term
  constexpr int U = 16;
  double s = 0.0;
  int m = n;
  for (; m + U <= p.nkb; m += U) {
    float t[U];
#pragma unroll
    for (int i = 0; i < U; ++i) t[i] = col[(int64_t)(m + i) * p.nkb];
#pragma unroll
    for (int i = 0; i < U; ++i) s += (double)t[i];
  }
  for (; m < p.nkb; ++m) s += (double)col[(int64_t)m * p.nkb];
  p.scores[(int64_t)b * p.nkb + n] = (float)s;
}

template <int D, int BLK>
static hipError_t launch_eq2_t(const Eq2Params& p, hipStream_t st) {
  const int pairs = eq2_super_tiles(p.nkb) * kSM * kSN;         // workgroup slots
  {
    TimedLaunch tl("k_eq2_tiles", st);
    k_eq2_tiles<D, BLK><<<dim3(pairs, p.B), 256, 0, st>>>(p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  TimedLaunch tl("k_eq2_reduce", st);
  k_eq2_reduce<<<dim3((p.nkb + 255) / 256, p.B), 256, 0, st>>>(p);
  return hipGetLastError();
}

hipError_t launch_score_eq2(const Eq2Params& p, int D, int block, hipStream_t st) {
  if (D == 64) return block == 64 ? launch_eq2_t<64, 64>(p, st) : launch_eq2_t<64, 128>(p, st);
  return block == 64 ? launch_eq2_t<128, 64>(p, st) : launch_eq2_t<128, 128>(p, st);
}

}  // namespace jenga
