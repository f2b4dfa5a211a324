// Permutation-free token movement fused into the projections, for gfx950 (bf16 MFMA).
//
// Jenga (papercache notes, §4.4; aipaper summary, §4.4.1): the kept tokens are loaded straight
// from the full hidden-state tensor by the projection that consumes them, and the projected
// output is added into the residual stream in place, so no gathered copy, padding or separate
// residual pass exists.
//
//   k_proj<kGather>   y[b][r][:]          = x[b][pos(r)][:] . W^T   gathered rows in, compact rows out (bf16)
//   k_proj<kScatter>  resid[b][pos(r)][:] += y[b][r][:] . W^T      compact rows in, residual updated in place
//   k_proj<kPlain>    out[r][:]           = a[r][:] . W^T          contiguous rows (fp32 out), r < rows
// pos(r) is the token position of kept rank r (kept-block list); W is [N][K] (out x in features).
//
// Workgroup: a 256 (rows) x 128 (output columns) tile, 8 waves of 64 x 64 (2 x 2 MFMA blocks).
// The reduction runs in 64-wide chunks; a chunk's 8 A tiles and 4 W tiles (32 x 64 bf16 each)
// are copied by direct-to-LDS loads spread evenly over the waves (6 per wave), through a
// three-buffer ring so that chunk t+2 loads while chunk t is multiplied.
#include "common.h"
#include "kernels.h"
#include "tiles64.h"

namespace jenga {

template <int MODE>
__global__ __launch_bounds__(512, 1) void k_proj(ProjParams p) {
  constexpr bool GATHER = MODE == kGather, PLAIN = MODE == kPlain;
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

  const Tile3 tl = xcd_tile();
  const int mt = tl.x, nt = tl.y, b = tl.z;
  const int32_t* kept = PLAIN ? nullptr : p.kept + (int64_t)b * p.nkb;
  const int Nk = PLAIN ? p.rows : min(p.n_kept[b], p.max_kept_blocks) * p.block;
  const int r0 = mt * TM, n0 = nt * TN;
  if (r0 >= Nk) return;
  if (!PLAIN) stage_kept(ktab, kept, (min(r0 + TM, Nk) - 1) / p.block + 1);
  __syncthreads();
  const KeptTab kt{(const LDS_AS int*)ktab, kept, p.block};
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, hl = l >> 5, lc = l & 31;
  const int wm = w & 3, wn = w >> 2;                       // the wave's 64-row / 64-column group

  // Load j = w + 8i of a chunk (i = 0..5) covers quarter (w % 4) of tile 2i + w/4: tiles 0..7
  // are the A row tiles, 8..11 the W row tiles.  Per lane: row (w%4)*8 + l/8 of the tile,
  // 16-byte chunk l%8 stored at chunk (l%8) ^ (row % 8).
  const int trow = (w & 3) * 8 + (l >> 3);
  const int tchunk = ((l & 7) ^ (trow & 7)) << 4;
  const int64_t abytes = p.as1 * 2, wbytes = (int64_t)p.K * 2;
  const uint32_t voff_a = (uint32_t)(trow * abytes + tchunk);
  const uint32_t voff_w = (uint32_t)(trow * wbytes + tchunk);
  const int tsel = w >> 2;
  const rsrc_t ra = make_rsrc((const bf16*)p.a + b * p.as0);
  const rsrc_t rw = make_rsrc(p.w);
  // first row of A tile t (rows past the kept count load a harmless valid row instead, so
  // that every wave issues the same number of loads per chunk)
  // (the row count is a multiple of 32 in every mode, so a 32-row group is whole or past it)
  auto arow0 = [&](int t) -> int64_t {
    const int r = r0 + 32 * t < Nk ? r0 + 32 * t : 0;
    return GATHER ? kt.pos_u(r) : r;
  };
  int64_t abase[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) abase[i] = arow0(2 * i + tsel) * abytes;

  auto issue = [&](int c, char* buf) {
    const uint32_t koff = (uint32_t)c * 128u;               // 64 bf16 per chunk
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dma16b(ra, voff_a, (uint32_t)abase[i] + koff, buf + (2 * i + tsel) * C::NAT32 + (w & 3) * 1024);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      dma16b(rw, voff_w, (uint32_t)((int64_t)(n0 + 32 * (2 * i + tsel)) * wbytes) + koff,
             buf + (AT + 2 * i + tsel) * C::NAT32 + (w & 3) * 1024);
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

  // lane = output column n0 + 64wn + 32nb + lc; register r = row r0 + 64wm + 32mb + 8(r/4) + 4hl + r%4
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int rb = r0 + 64 * wm + 32 * mb;
    if (rb >= Nk) continue;                                // Nk is a multiple of 32
#pragma unroll
    for (int rg = 0; rg < 4; ++rg)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rb + 8 * rg + 4 * hl + i;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int col = n0 + 64 * wn + 32 * nb + lc;
          const float v = acc[mb][nb][4 * rg + i];
          if (GATHER) {
            bf16* orow = (bf16*)p.out + b * p.os0 + (int64_t)r * p.os1;
            orow[col] = (bf16)v;
          } else if (PLAIN) {
            float* orow = (float*)p.out + b * p.os0 + (int64_t)r * p.os1;
            orow[col] = v;
          } else {
            float* orow = (float*)p.out + b * p.os0 + (int64_t)kt.pos(r) * p.os1;
            orow[col] += v;
          }
        }
      }
  }
}

template <int MODE>
static hipError_t launch_proj_t(const ProjParams& p, const char* name, hipStream_t st) {
  TimedLaunch tl(name, st);
  const int rows = MODE == kPlain ? p.rows : p.ncap;
  k_proj<MODE><<<dim3((rows + 255) / 256, p.N / 128, p.B), 512, 0, st>>>(p);
  return hipGetLastError();
}

hipError_t launch_proj(const ProjParams& p, int mode, const char* name, hipStream_t st) {
  if (mode == kGather) return launch_proj_t<kGather>(p, name, st);
  if (mode == kScatter) return launch_proj_t<kScatter>(p, name, st);
  return launch_proj_t<kPlain>(p, name, st);
}

}  // namespace jenga
