// Permutation-free token movement fused into the projections, and the MLP block's activation
// with its token informativeness, for gfx950 (bf16 MFMA).
//
// Jenga (papercache notes, §4.4; aipaper summary, §4.4.1): the kept tokens are loaded straight
// from the full hidden-state tensor by the projection that consumes them, and the projected
// output is added into the residual stream in place, so no gathered copy, padding or separate
// residual pass exists.  Aipaper summary §4.2.4: token elimination extends to the MLP block,
// a token's informativeness coming from the block's intermediate activation (the ReLU output,
// or SiLU(gate) * up).
//
//   k_proj<kGather>         y[b][r][:]          = x[b][pos(r)][:] . W^T   gathered rows in, compact rows out (bf16)
//   k_proj<kScatter>        resid[b][pos(r)][:] += y[b][r][:] . W^T      compact rows in, residual updated in place
//   k_proj<kGatherScatter>  resid[b][pos(r)][:] += a[b][pos(r)][:] . W^T  gathered rows in, residual updated in place
//   k_proj<kPlain>          out[r][:]           = a[r][:] . W^T          contiguous rows (fp32 out), r < rows
//   k_proj<kMlpGated>       act[b][r][c]        = silu(x . Wg^T) * (x . Wu^T)   (bf16 out)
//   k_proj<kMlpRelu>        act[b][r][c]        = max(x . W1^T, 0)              (bf16 out)
// pos(r) is the token position of kept rank r (kept-block list); W is [N][K] (out x in features).
// The MLP modes also write, per row and per group of 32 units, the sum of |activation| (fp32,
// before rounding); k_mlp_block turns those into token and token-block scores.
//
// Workgroup: a 256 (rows) x 128 (GEMM columns) tile, 8 waves of 64 x 64 (2 x 2 MFMA blocks).
// In the gated mode the 128 GEMM columns are 64 gate and the matching 64 up columns, placed so
// that each wave holds the gate and up values of the same 32 units.  The reduction runs in
// 64-wide chunks; a chunk's 8 A tiles and 4 W tiles (32 x 64 bf16 each) are copied by
// direct-to-LDS loads spread evenly over the waves (6 per wave), through a three-buffer ring
// so that chunk t+2 loads while chunk t is multiplied.
#include "common.h"
#include "kernels.h"
#include "tiles64.h"

namespace jenga {

// v[0..15]: one value per accumulator register (a row) in each lane of a 32-lane half-wave.
// Sums every register over the 32 lanes of the half by halving exchanges (16 shuffles instead
// of 80): lane lc ends with the full sum of register ((lc>>4)&1)*8 + ((lc>>3)&1)*4 +
// ((lc>>2)&1)*2 + ((lc>>1)&1); lanes lc and lc^1 hold the same sum.
__device__ inline float half_wave_row_sums(float (&v)[16], int lc) {
#pragma unroll
  for (int n = 16, off = 16; n >= 2; n >>= 1, off >>= 1) {
    const bool hi = (lc & off) != 0;
#pragma unroll
    for (int j = 0; j < n / 2; ++j) {
      const float keep = hi ? v[n / 2 + j] : v[j];
      const float send = hi ? v[j] : v[n / 2 + j];
      v[j] = keep + __shfl_xor(send, off, 64);
    }
  }
  return v[0] + __shfl_xor(v[0], 1, 64);
}

template <int MODE>
__global__ __launch_bounds__(512, 1) void k_proj(ProjParams p) {
  constexpr bool AGATHER = MODE == kGather || MODE == kGatherScatter;
  constexpr bool DENSE = MODE == kPlain || MODE == kMlpGated || MODE == kMlpRelu;
  constexpr bool GATED = MODE == kMlpGated, RELU = MODE == kMlpRelu;
  using C = T64<64>;                                      // one reduction chunk: 32 x 64 tiles
  constexpr int NW = 8, TM = 256, TN = 128;
  constexpr int AT = TM / 32, BT = TN / 32;               // 8 A tiles, 4 W tiles per chunk
  constexpr int STAGE = (AT + BT) * C::NAT32;             // 48 KB
  constexpr int PER = (AT + BT) * 4 / NW;                 // direct-to-LDS loads per wave per chunk
  static_assert(PER == 6, "12 tiles x 4 loads over 8 waves");
  __shared__ __attribute__((aligned(1024))) char sA[STAGE];
  __shared__ __attribute__((aligned(1024))) char sB[STAGE];
  __shared__ __attribute__((aligned(1024))) char sC[STAGE];
  __shared__ int ktab[kKeptTab];

  // row tiles per visiting group, as measured on the c5-sized projections: gathered rows favour
  // two (QKV 1846 -> 1500 us against row tiles fastest), contiguous rows four (O scatter-add
  // 746 -> 662, logits 1175 -> 1038 us)
  const Tile3 tl = xcd_tile_grouped<AGATHER ? 2 : 4>();
  const int mt = tl.x, nt = tl.y, b = tl.z;
  const int32_t* kept = DENSE ? nullptr : p.kept + (int64_t)b * p.nkb;
  const int Nk = DENSE ? p.rows : min(p.n_kept[b], p.max_kept_blocks) * p.block;
  const int r0 = mt * TM, n0 = nt * TN;
  if (r0 >= Nk) return;
  if (!DENSE) stage_kept(ktab, kept, (min(r0 + TM, Nk) - 1) / p.block + 1);
  __syncthreads();
  const KeptTab kt{(const LDS_AS int*)ktab, kept, p.block};
  const int tid = threadIdx.x, l = tid & 63, hl = l >> 5, lc = l & 31;
  const int w = tid >> 6;
  // the same wave index taken through readfirstlane, for what the direct-to-LDS loads need in
  // scalar registers (row offsets, LDS destination): computed from the plain index the
  // compiler cannot prove them uniform and wraps every load in a waterfall loop
  const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w & 3, wn = w >> 2;                       // the wave's 64-row / 64-column group

  // Load j = w + 8i of a chunk (i = 0..5) covers quarter (w % 4) of tile 2i + w/4: tiles 0..7
  // are the A row tiles, 8..11 the W row tiles.  Per lane: row (w%4)*8 + l/8 of the tile,
  // 16-byte chunk l%8 stored at chunk (l%8) ^ (row % 8).
  const int trow = (w & 3) * 8 + (l >> 3);
  const int tchunk = ((l & 7) ^ (trow & 7)) << 4;
  const int64_t abytes = p.as1 * 2, wbytes = (int64_t)p.K * 2;
  const uint32_t voff_a = (uint32_t)(trow * abytes + tchunk);
  const uint32_t voff_w = (uint32_t)(trow * wbytes + tchunk);
  const int tsel = wu >> 2;
  const rsrc_t ra = make_rsrc_u((const bf16*)p.a + b * p.as0);
  // Gated mode: W tile slot 2i + tsel holds rows c0 + 32i of the gate (tsel 0) or the up
  // projection (tsel 1), c0 = 64 nt, so wave column group wn reads gate and up of units
  // c0 + 32wn .. +31.  Otherwise slot t holds W rows n0 + 32t.
  const rsrc_t rw = make_rsrc_u(GATED && tsel ? p.w2 : p.w);
  auto wrow = [&](int i) -> int64_t { return GATED ? nt * 64 + 32 * i : n0 + 32 * (2 * i + tsel); };
  // first row of A tile t (rows past the row count load a harmless valid row instead, so
  // that every wave issues the same number of loads per chunk)
  // (the row count is a multiple of 32 in every mode, so a 32-row group is whole or past it)
  auto arow0 = [&](int t) -> int64_t {
    const int r = r0 + 32 * t < Nk ? r0 + 32 * t : 0;
    return AGATHER ? kt.pos_u(r) : r;
  };
  int64_t abase[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) abase[i] = arow0(2 * i + tsel) * abytes;

  auto issue = [&](int c, char* buf) {
    const uint32_t koff = (uint32_t)c * 128u;               // 64 bf16 per chunk
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dma16b(ra, voff_a, (uint32_t)abase[i] + koff, buf + (2 * i + tsel) * C::NAT32 + (wu & 3) * 1024);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      dma16b(rw, voff_w, (uint32_t)(wrow(i) * wbytes) + koff,
             buf + (AT + 2 * i + tsel) * C::NAT32 + (wu & 3) * 1024);
  };

  ReadPlan<64> rp;
  rp.init();
  f32x16 acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = zero16();

  // C[m][n]: A operand = rows m (lane = row), B operand = W rows n (lane = output column)
  auto compute = [&](const char* buf) {
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) af[mb] = ldo(buf + (2 * wm + mb) * C::NAT32, rp.nat[s]);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) bfr[nb] = ldo(buf + (AT + 2 * wn + nb) * C::NAT32, rp.nat[s]);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = Mfma<bf16>::mma(af[mb], bfr[nb], acc[mb][nb]);
    }
  };

  const int nch = p.K / 64;
  auto stage = [&](int t, const char* cur, char* nxt) {
    // every chunk issues one set of loads (past the end, a reload of the last chunk that
    // nobody reads), so exactly one set may still be in flight when chunk t is needed
    wait_vm<PER>();
    stage_barrier();
    issue(min(t + 2, nch - 1), nxt);
    compute(cur);
  };
  issue(0, sA);
  issue(min(1, nch - 1), sB);
  for (int t = 0; t < nch; t += 3) {
    stage(t, sA, sC);
    if (t + 1 >= nch) break;
    stage(t + 1, sB, sA);
    if (t + 2 >= nch) break;
    stage(t + 2, sC, sB);
  }
  wait_all_mem();                                          // drain the trailing reloads

  if constexpr (GATED || RELU) {
    // lane = unit column, register r = row rb + 8(r/4) + 4hl + r%4.
    // Gated: acc[mb][0] gate, acc[mb][1] up of units c0 + 32wn + lc.
    // ReLU:  acc[mb][nb] units n0 + 64wn + 32nb + lc.
    constexpr int NG = GATED ? 1 : 2;                      // 32-unit groups per wave
    const int ncg = p.N / 32;
    bf16* actb = (bf16*)p.out + b * p.os0;
    float* part = p.part + (int64_t)b * ncg * p.rows;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int rb = r0 + 64 * wm + 32 * mb;
      if (rb >= Nk) continue;                              // Nk is a multiple of 32
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const int unit = GATED ? nt * 64 + 32 * wn + lc : n0 + 64 * wn + 32 * g + lc;
        float av[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float a;
          if (GATED) {
            const float z = acc[mb][0][r];
            a = z / (1.f + __expf(-z)) * acc[mb][1][r];
          } else {
            a = fmaxf(acc[mb][g][r], 0.f);
          }
          const int row = rb + 8 * (r >> 2) + 4 * hl + (r & 3);
          actb[(int64_t)row * p.os1 + unit] = (bf16)a;
          av[r] = fabsf(a);
        }
        const float sum = half_wave_row_sums(av, lc);
        if ((lc & 1) == 0) {
          const int ri = ((lc >> 4) & 1) * 8 + ((lc >> 3) & 1) * 4 + ((lc >> 2) & 1) * 2 + ((lc >> 1) & 1);
          const int row = rb + 8 * (ri >> 2) + 4 * hl + (ri & 3);
          const int cg = (unit - lc) / 32;
          part[(int64_t)cg * p.rows + row] = sum;
        }
      }
    }
  } else {
    // lane = output column n0 + 64wn + 32nb + lc; register r = row r0 + 64wm + 32mb + 8(r/4) + 4hl + r%4
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int rb = r0 + 64 * wm + 32 * mb;
      if (rb >= Nk) continue;                              // Nk is a multiple of 32
      // the 32 ranks rb.. lie in one kept block (blocks are multiples of 64 rows): one lookup
      // places them all, where a lookup per row waited for every read issued before it
      const int pos0 = (MODE == kScatter || MODE == kGatherScatter) ? kt.pos_u(rb) : 0;
#pragma unroll
      for (int rg = 0; rg < 4; ++rg)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = rb + 8 * rg + 4 * hl + i;
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            const int col = n0 + 64 * wn + 32 * nb + lc;
            const float v = acc[mb][nb][4 * rg + i];
            if (MODE == kGather) {
              bf16* orow = (bf16*)p.out + b * p.os0 + (int64_t)r * p.os1;
              orow[col] = (bf16)v;
            } else if (MODE == kPlain) {
              float* orow = (float*)p.out + b * p.os0 + (int64_t)r * p.os1;
              orow[col] = v;
            } else {                                       // kScatter, kGatherScatter
              float* orow = (float*)p.out + b * p.os0 + (int64_t)(pos0 + (r - rb)) * p.os1;
              orow[col] += v;
            }
          }
        }
    }
  }
}

// Token and token-block informativeness of the MLP block from the per-32-unit partial sums:
// e_t = (sum over groups, fixed order, fp64) / F, rounded once to fp32; block score = the
// largest e_t of the block's tokens.  One workgroup per (token block, batch row).
__global__ __launch_bounds__(256) void k_mlp_block(MlpBlockParams p) {
  __shared__ float wmax[4];
  const int n = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const float* part = p.part + (int64_t)b * p.ncg * p.S;
  float mx = 0.f;                                          // every score is >= 0
  for (int j = tid; j < p.block; j += 256) {
    const int t = n * p.block + j;
    double s = 0.0;
    for (int c = 0; c < p.ncg; ++c) s += (double)part[(int64_t)c * p.S + t];
    const float e = (float)(s / (double)p.F);
    p.token_scores[(int64_t)b * p.S + t] = e;
    mx = fmaxf(mx, e);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if ((tid & 63) == 0) wmax[tid >> 6] = mx;
  __syncthreads();
  if (tid == 0)
    p.block_scores[(int64_t)b * p.nkb + n] = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
}

template <int MODE>
static hipError_t launch_proj_t(const ProjParams& p, const char* name, hipStream_t st) {
  TimedLaunch tl(name, st);
  const bool dense = MODE == kPlain || MODE == kMlpGated || MODE == kMlpRelu;
  const int rows = dense ? p.rows : p.ncap;
  const int cols = MODE == kMlpGated ? p.N / 64 : p.N / 128;
  k_proj<MODE><<<dim3((rows + 255) / 256, cols, p.B), 512, 0, st>>>(p);
  return hipGetLastError();
}

hipError_t launch_proj(const ProjParams& p, int mode, const char* name, hipStream_t st) {
  switch (mode) {
    case kGather: return launch_proj_t<kGather>(p, name, st);
    case kScatter: return launch_proj_t<kScatter>(p, name, st);
    case kGatherScatter: return launch_proj_t<kGatherScatter>(p, name, st);
    case kMlpGated: return launch_proj_t<kMlpGated>(p, name, st);
    case kMlpRelu: return launch_proj_t<kMlpRelu>(p, name, st);
    default: return launch_proj_t<kPlain>(p, name, st);
  }
}

hipError_t launch_mlp_block(const MlpBlockParams& p, hipStream_t st) {
  TimedLaunch tl("k_mlp_block", st);
  k_mlp_block<<<dim3(p.nkb, p.B), 256, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace jenga
