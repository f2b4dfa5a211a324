// Tile plumbing for the bf16 kernels that give each wave 64 rows (two 32-row MFMA blocks).
//
// Two LDS tile forms, both filled with gfx950 direct-to-LDS loads (global_load_lds_dwordx4:
// lane i of a wave writes its 16 bytes at LDS base + 16*i, from any global address):
//   natural tile  [32 rows][D] bf16, 16-byte chunk c of row r stored at chunk c ^ natswz(r)
//                 (a bijection on r % CPR, CPR = chunks per row); read as MFMA operands whose
//                 reduction runs along head_dim, or transposed (TrPlan) as operands whose
//                 reduction runs down its rows.
//   TP tile       [D][32 positions] bf16: row r of the source tile sits at position pi(r),
//                 pi swapping bits 2 and 3 of r.  Chunk c of line d stored at c ^ tpswz(d).
// Both swizzles make every 16-lane (and every 8-lane) group of a 16-byte read hit distinct
// banks for the access patterns below.
//                 One 16-byte read at line d, chunk 2j + h gives the 8 source rows that lane
//                 half h needs for k-step j when the other operand comes straight from a
//                 32x32 accumulator (registers 8j..8j+7 hold rows 16j + pi(8h + i)).
// TP tiles are produced in global memory by k_pack_tp / the backward prologue, so the hot
// kernels only copy them.
#pragma once

#include "common.h"

namespace jenga {

__host__ __device__ constexpr int pi16(int p) { return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1); }

// Natural-tile swizzle: chunk c of row r is stored at chunk c ^ natswz(r).  A bijection on
// r % CPR, so 16 consecutive rows read at one logical chunk hit 16 distinct chunks.  With
// 16 chunks per row the two low row bits go to the two high chunk bits: a transposing read
// (four consecutive rows x four consecutive chunks per 32 lanes) then also covers all 16 chunk
// positions, i.e. all 64 banks.
template <int CPR>
__host__ __device__ constexpr int natswz(int r) {
  return CPR == 16 ? (((r & 3) << 2) | ((r >> 2) & 3)) : (r & (CPR - 1));
}

template <int D>
struct T64 {
  static constexpr int ROWB = D * 2;       // natural row bytes
  static constexpr int CPR = ROWB / 16;    // 16-byte chunks per natural row
  static constexpr int NAT32 = 32 * ROWB;  // natural 32-row tile bytes
  static constexpr int TP32 = D * 64;      // TP tile bytes
  static constexpr int NS = D / 16;        // MFMA k-steps over head_dim
  static constexpr int NDB = D / 32;       // 32-wide head_dim blocks
};

// Direct-to-LDS copies through raw buffer loads.  The resource holds a wave-uniform base (kept in
// SGPRs); a copy adds a per-lane offset (voff, a register computed once per kernel) and a
// wave-uniform one (soff, per step).  Keeping the per-lane part in a long-lived register matters:
// when a 64-bit address register of an outstanding direct-to-LDS load is reused, the compiler
// first waits for all outstanding vector-memory work, prefetched tiles included.  Every caller
// keeps voff + soff inside the tensor the base points into (below 4 GiB); the range field is
// not relied on.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ inline rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
}

// The same for a base that is the same in every lane of the wave, taken through readfirstlane
// so that the resource is built in scalar registers: where the compiler cannot prove the
// address uniform it otherwise keeps the resource in vector registers and wraps every load
// that uses it in a waterfall loop.
__device__ inline rsrc_t make_rsrc_u(const void* base) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return make_rsrc((const void*)(uintptr_t)(lo | (hi << 32)));
}

__device__ inline void dma16b(rsrc_t r, uint32_t voff, uint32_t soff, char* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS_AS void*)lds, 16, voff, soff, 0, 0);
}

// Wait for every outstanding memory operation of this wave (direct-to-LDS loads included).
__device__ inline void wait_all_mem() { __builtin_amdgcn_s_waitcnt(0); }

// Wait until at most N vector-memory operations of this wave are outstanding (they complete in
// issue order), leaving the newest N -- later pipeline stages -- in flight.
template <int N>
__device__ inline void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0xF70 | (N & 15) | ((N >> 4) << 14));
}

// Scheduling groups for a run of NSTEP k-steps, each READS LDS operand reads feeding MFMAS
// MFMAs, placed right after that run in the same basic block: the reads of step i+1 are issued
// before the MFMAs of step i, so each MFMA finds its operands already on the way instead of
// waiting out a whole LDS round trip (left alone, the compiler pairs each read with its use).
// Runs that can end up in one basic block take different SYNC ids.
// (A macro, not a function: the groups then stay attached to the caller's instructions.)
#define SCHED_READS_AHEAD(NSTEP, READS, MFMAS, SYNC)                                             \
  do {                                                                                          \
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * (READS), SYNC); /* reads of steps 0, 1 */  \
    _Pragma("unroll") for (int i_ = 0; i_ < (NSTEP) - 2; ++i_) {                                \
      __builtin_amdgcn_sched_group_barrier(0x008, MFMAS, SYNC);     /* MFMAs of step i */       \
      __builtin_amdgcn_sched_group_barrier(0x100, READS, SYNC);     /* reads of step i + 2 */   \
    }                                                                                           \
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * (MFMAS), SYNC); /* last two steps */        \
  } while (0)

// The staged loop over a three-buffer LDS ring: stage(t, cur, nxt) computes tile t from cur
// while tile t + 2 loads into nxt (tile t lives in buffer t % 3).  Six steps per iteration:
// where the loop's back edge joins, the compiler no longer knows which buffer a pending
// direct-to-LDS load targets and makes the first buffer read after the join wait for all of
// them; with six steps per iteration that exposed wait comes once per six steps, not three.
template <class Stage>
__device__ inline void ring3_loop(int n, char* A, char* B, char* C, Stage&& stage) {
  for (int t = 0; t < n; t += 6) {
    stage(t, A, C);
    if (t + 1 >= n) break;
    stage(t + 1, B, A);
    if (t + 2 >= n) break;
    stage(t + 2, C, B);
    if (t + 3 >= n) break;
    stage(t + 3, A, C);
    if (t + 4 >= n) break;
    stage(t + 4, B, A);
    if (t + 5 >= n) break;
    stage(t + 5, C, B);
  }
}

// Workgroup barrier for the staged loops.  __syncthreads() also fences memory, which makes
// the compiler wait for every outstanding vector-memory operation -- including the
// direct-to-LDS loads of tiles still being prefetched.  Here each wave first waits for its own
// loads of the tile about to be read (the caller's wait_vm / wait_all_mem) and for its LDS
// reads of the tile about to be overwritten; the asm memory clobbers keep the compiler from
// moving LDS accesses across the barrier.
__device__ inline void stage_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);                    // lgkmcnt(0) only
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Direct-to-LDS instructions one wave issues for a tile (uniform across waves iff exact).
template <int D, int NW>
struct DmaCount {
  static constexpr int NAT = 32 * T64<D>::CPR / 64;
  static constexpr int TP = D * 64 / 1024;
  static constexpr bool EXACT = NAT % NW == 0 && TP % NW == 0;
  static constexpr int NAT_W = NAT / NW, TP_W = TP / NW;
};

__device__ inline int tpswz(int d) { return ((d >> 1) & 3) ^ ((d >> 3) & 1); }

// Per-lane address offsets of one wave's direct-to-LDS instructions, computed once per kernel
// so that a step only adds its (wave-uniform) base address.  The offsets are unsigned 32-bit so
// that the loads take the scalar-base form (uniform base in SGPRs + per-lane offset register):
// with a fresh 64-bit address register per load, the compiler waits for every outstanding
// vector-memory operation before it may reuse that register.
template <int D, int NW>
struct NatPlan {
  static constexpr int NI = DmaCount<D, NW>::NAT;
  static constexpr int MAXW = (NI + NW - 1) / NW;
  uint32_t off[MAXW];
  __device__ void init(int64_t row_stride) {
    constexpr int CPR = T64<D>::CPR;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < MAXW; ++i) {
      const int idx = (w + i * NW) * 64 + l;
      const int row = idx / CPR, phys = idx % CPR;
      off[i] = (uint32_t)(row * row_stride) + ((phys ^ natswz<CPR>(row)) << 4);
    }
  }
  // rows at byte offset soff (row 0) from the resource's base
  __device__ void issue(char* lds_tile, rsrc_t r, uint32_t soff) const {
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < MAXW; ++i)
      // (when NW divides the load count every wave issues all of its loads; the bound check
      // then stays out of the code, so the loads are not placed in branches of their own)
      if (NI % NW == 0 || w + i * NW < NI) dma16b(r, off[i], soff, lds_tile + (w + i * NW) * 1024);
  }
};

template <int D, int NW>
struct TpPlan {
  static constexpr int NI = DmaCount<D, NW>::TP;
  static constexpr int MAXW = (NI + NW - 1) / NW;
  uint32_t off[MAXW];
  __device__ void init() {
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < MAXW; ++i) {
      const int idx = (w + i * NW) * 64 + l;
      const int d = idx >> 2, phys = idx & 3;
      off[i] = (uint32_t)(d * 64 + ((phys ^ tpswz(d)) << 4));
    }
  }
  // the TP tile at byte offset soff from the resource's base
  __device__ void issue(char* lds_tile, rsrc_t r, uint32_t soff) const {
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < MAXW; ++i)
      if (NI % NW == 0 || w + i * NW < NI) dma16b(r, off[i], soff, lds_tile + (w + i * NW) * 1024);
  }
};

// Per-lane LDS read offsets for the MFMA operands of a wave whose rows are its lane index:
// natural tile, k-step s:  row lc, chunk 2s + hl;   TP tile, 32-wide block db, k-step j:
// line db*32 + lc, chunk 2j + hl (the db part is a constant 2048*db).
template <int D>
struct ReadPlan {
  int nat[T64<D>::NS];
  int tp[2];
  __device__ void init() {
    const int l = threadIdx.x & 63, hl = l >> 5, lc = l & 31;
    constexpr int CPR = T64<D>::CPR;
#pragma unroll
    for (int s = 0; s < T64<D>::NS; ++s) nat[s] = lc * T64<D>::ROWB + (((2 * s + hl) ^ natswz<CPR>(lc)) << 4);
#pragma unroll
    for (int j = 0; j < 2; ++j) tp[j] = lc * 64 + (((2 * j + hl) ^ tpswz(lc)) << 4);
  }
};

__device__ inline bf16x8 ldo(const char* tile, int off) { return *(const bf16x8*)(tile + off); }

// Per-lane LDS offsets for an operand whose reduction runs down the rows of a natural tile (the
// transposed operand of a 32x32x16 product), read with two transposing 8-byte reads.  The
// operand pairs with a 32x32 accumulator's registers 8j..8j+7 as the other operand, whose
// reduction index i = 0..7 of lane half h is row 16j + pi16(8h + i): rows 16j + 4h + 0..3
// (first read, t = 0) and 16j + 8 + 4h + 0..3 (second read, t = 1).  Lane l's column is
// 32 db + l % 32.  Within a 16-lane group, lane s addresses row R + s/4 at column
// C + 4 (s % 4), and receives rows R..R+3 of column C + s.  k-step j adds 16 j rows, which
// leave the swizzle unchanged: a constant j * 16 * ROWB.
template <int D>
struct TrPlan {
  int off[2][T64<D>::NDB];
  __device__ void init() {
    constexpr int CPR = T64<D>::CPR, ROWB = T64<D>::ROWB;
    const int l = threadIdx.x & 63, hl = l >> 5, s = l & 15, grp = (l >> 4) & 1;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < T64<D>::NDB; ++db) {
        const int row = 8 * t + 4 * hl + (s >> 2);
        const int col = 32 * db + 16 * grp + 4 * (s & 3);
        off[t][db] = row * ROWB + (((col >> 3) ^ natswz<CPR>(row)) << 4) + (col & 7) * 2;
      }
  }
};

__device__ inline bf16x8 ldtr(const char* tile, int off0, int off1) {
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(tile + off0));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(tile + off1));
  const s16x8 c = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, c);
}

// Kept-block table staged in LDS once per workgroup, so the hot loops resolve a kept rank to
// its token position without a global-memory round trip.  Blocks beyond the table's capacity
// fall back to the global list.
constexpr int kKeptTab = 1024;

struct KeptTab {
  const LDS_AS int* s;     // LDS copy of kept[0 .. min(n, kKeptTab))
  const int32_t* g;        // the global list
  int block;
  // The table is typed as LDS so that the two reads stay an LDS read and a global read: merged
  // into one flat load, every lookup would also wait for all outstanding vector-memory work,
  // including tiles still being prefetched.
  __device__ int pos(int r) const {
    const int kb = r / block;
    const int v = kb < kKeptTab ? s[kb] : g[kb];
    return v * block + (r - kb * block);
  }
  // kept[kb] for a wave-uniform kb, as used by the staged loops.  Each branch ends in a scalar
  // register, and the global branch waits for its own load: were the two joined in one vector
  // register, the common path would wait for every outstanding vector-memory operation.
  __device__ int entry_u(int kb) const {
    if (kb < kKeptTab) return __builtin_amdgcn_readfirstlane(s[kb]);
    const int x = g[kb];
    __builtin_amdgcn_s_waitcnt(0);
    return __builtin_amdgcn_readfirstlane(x);
  }
  // pos() for a wave-uniform rank
  __device__ int pos_u(int r) const {
    const int kb = r / block;
    return entry_u(kb) * block + (r - kb * block);
  }
};

// pos_u over consecutive 32-rank steps, walked without a division per step: the kept block
// and the offset in it of the next step's first rank.  Staged loops issue steps in order and
// call advance() after each step they issue, except past their last one.
struct StepPos {
  int kb, off;
  __device__ void init(int rank, int block) {
    kb = rank / block;
    off = rank - kb * block;
  }
  __device__ int pos(const KeptTab& kt) const { return kt.entry_u(kb) * kt.block + off; }
  __device__ void advance(int block) {
    off += 32;
    if (off == block) {
      off = 0;
      ++kb;
    }
  }
};

// All threads of the workgroup: copy kept[0..nb) (clipped to the table) into LDS.  The caller
// synchronises before the first lookup.
__device__ inline void stage_kept(int* tab, const int32_t* kept, int nb) {
  const int n = min(nb, kKeptTab);
  for (int i = threadIdx.x; i < n; i += blockDim.x) tab[i] = kept[i];
}

__device__ inline bf16x8 frag_from_acc(const f32x16& a, int j) {
  return to_frag8(a[8 * j + 0], a[8 * j + 1], a[8 * j + 2], a[8 * j + 3], a[8 * j + 4],
                  a[8 * j + 5], a[8 * j + 6], a[8 * j + 7]);
}

}  // namespace jenga
