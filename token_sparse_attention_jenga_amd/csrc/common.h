// Shared device helpers for the gfx950 kernels: MFMA operand traits, LDS transpose reads,
// bf16 conversion, and the kept-rank -> token-position map.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))

namespace jenga {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------------------
// MFMA 32x32 traits.  For both operand types the accumulator layout is the same: lane l,
// register r holds C[8*(r/4) + 4*(l/32) + r%4][l%32].  Operands: lane l supplies
// A[l%32][KSTEP*s + KPL*(l/32) + i] and B[KSTEP*s + KPL*(l/32) + i][l%32], i < KPL.
// ---------------------------------------------------------------------------------------
template <typename T> struct Mfma;

template <> struct Mfma<bf16> {
  using frag = bf16x8;
  static constexpr int KPL = 8;
  static constexpr int KSTEP = 16;
  __device__ static inline f32x16 mma(const frag& a, const frag& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<float> {
  using frag = float;
  static constexpr int KPL = 1;
  static constexpr int KSTEP = 2;
  __device__ static inline f32x16 mma(const frag& a, const frag& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

__device__ inline f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

// float -> bf16 with round-to-nearest-even (gfx950 v_cvt_pk_bf16_f32).
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Eight fp32 values -> one bf16x8 MFMA operand.
__device__ inline bf16x8 to_frag8(float a0, float a1, float a2, float a3, float a4, float a5,
                                  float a6, float a7) {
  const f32x8 v = {a0, a1, a2, a3, a4, a5, a6, a7};
  return __builtin_convertvector(v, bf16x8);
}

// LDS transpose read of 16-bit data (gfx950).  Within every group of 16 lanes, lane j
// receives element j%4 of the 8-byte words addressed by lanes 4*i + j/4, i = 0..3.  If lane s
// of the group addresses row R + s/4, column C + 4*(s%4) of a row-major tile, lane j
// therefore receives tile[R + i][C + j] for i = 0..3: four consecutive rows of one column.
__device__ inline s16x4 lds_read_tr16(const LDS_AS char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)p);
}

// bf16 A/B operand whose reduction index runs down the rows of a row-major LDS tile:
// lane l receives tile[row0(t) + s/4 ... ][col] for two instructions t = 0, 1, where the
// caller supplies the first row of each 4-row run seen by this lane's half-wave.
// col0: first column of the 32-wide operand block (elements).
__device__ inline bf16x8 lds_frag_tr(const LDS_AS char* tile, int ld_bytes, int row_t0,
                                     int row_t1, int col0) {
  const int l = threadIdx.x & 63;
  const int s = l & 15;
  const int col = col0 + 16 * ((l >> 4) & 1) + 4 * (s & 3);
  const LDS_AS char* p0 = tile + (row_t0 + (s >> 2)) * ld_bytes + col * 2;
  const LDS_AS char* p1 = tile + (row_t1 + (s >> 2)) * ld_bytes + col * 2;
  s16x4 a = lds_read_tr16(p0);
  s16x4 b = lds_read_tr16(p1);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 c = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, c);
}

// Token position of kept rank r (ranks are in ascending position order).
__device__ inline int rank_to_pos(const int32_t* __restrict__ kept, int block, int r) {
  const int kb = r / block;
  return kept[kb] * block + (r - kb * block);
}

// 16-byte global load / store helpers.
__device__ inline u32x4 ld16(const void* p) { return *(const u32x4*)p; }

__device__ inline float wave_xor32(float x) { return __shfl_xor(x, 32, 64); }

// Combine lane l with lane l ^ 32 through the cross-half lane swap (a VALU operation, no LDS
// round trip): the swap of x with itself returns (x[l], x[l + 32]) in lanes l < 32 and
// (x[l - 32], x[l]) in lanes l >= 32, so both lanes of a pair see the same two values.
// Maximum of three floats in one v_max3_f32.  Written out because fmaxf makes the compiler
// first quiet each operand that might be a signalling NaN (one v_max_f32 x, x per operand that
// does not come from an earlier max), which here costs almost as much as the maximum itself;
// the operands are scores, never NaN.
__device__ inline float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Maximum of the 16 values of a 32x32 accumulator block held by one lane: a tree of v_max3.
__device__ inline float max16(const f32x16& v) {
  const float a = max3f(v[0], v[1], v[2]), b = max3f(v[3], v[4], v[5]), c = max3f(v[6], v[7], v[8]);
  const float d = max3f(v[9], v[10], v[11]), e = max3f(v[12], v[13], v[14]);
  const float f = max3f(a, b, c), g = max3f(d, e, v[15]);
  return max3f(f, g, g);
}

__device__ inline float half_pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max3f(__uint_as_float(r[0]), __uint_as_float(r[1]), __uint_as_float(r[1]));
}
__device__ inline float half_pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// XCD-aware workgroup numbering.  An MI355X has 8 XCDs, each with its own L2, and the
// dispatcher hands workgroups, in linear launch order, to XCD (index % 8) in turn.  xcd_tile()
// renumbers them so that XCD x runs one contiguous range of logical tiles (x fastest, then y,
// then z) in launch order; the tiles of one (batch, head) then share one L2 instead of
// streaming the same K/V or Q rows through all eight.  A bijection for any grid size.
struct Tile3 {
  int x, y, z;
};
__device__ inline Tile3 xcd_tile() {
  const int nx = gridDim.x, ny = gridDim.y;
  const int nwg = nx * ny * (int)gridDim.z;
  const int lin = (int)blockIdx.x + nx * ((int)blockIdx.y + ny * (int)blockIdx.z);
  const int q = nwg >> 3, r = nwg & 7, xcd = lin & 7, slot = lin >> 3;
  const int L = xcd * q + min(xcd, r) + slot;
  return {L % nx, (L / nx) % ny, L / (nx * ny)};
}

// The same ranges, visited weight-major in groups, for grids whose tiles get lighter along x
// (causal row tiles numbered heaviest first).  When XCD x's range holds whole rows (y, z) of
// tiles, its workgroups take tiles 0..G-1 of every row of the range, then tiles G..2G-1 of every
// row, and so on (G = kWeightMajorGroup; the last group may be shorter).  Row by row, the heavy
// tiles of the range's later rows went out after the light tiles of its first rows and the
// launch ended on them; tile by tile across the rows, the XCD swept several rows' K at once and
// fetched twice the bytes from beyond its L2.  Groups of 32 tiles keep most of the balance and
// the fetch of the row-by-row order.  Otherwise (ranges that split a row) the order of
// xcd_tile().
constexpr int kWeightMajorGroup = 32;

__device__ inline Tile3 xcd_tile_weight_major() {
  const int nx = gridDim.x, ny = gridDim.y;
  const int nwg = nx * ny * (int)gridDim.z;
  const int lin = (int)blockIdx.x + nx * ((int)blockIdx.y + ny * (int)blockIdx.z);
  const int q = nwg >> 3, r = nwg & 7, xcd = lin & 7, slot = lin >> 3;
  int L;
  if (r == 0 && q % nx == 0) {
    const int rows = q / nx;                             // whole rows per XCD range
    const int G = min(kWeightMajorGroup, nx);
    const int nfull = nx / G, full_slots = nfull * rows * G;
    int row, t;
    if (slot < full_slots) {                             // a group of G tiles of every row
      const int grp = slot / (rows * G), in = slot - grp * rows * G;
      row = in / G;
      t = grp * G + (in - row * G);
    } else {                                             // the last, shorter group
      const int P = nx - nfull * G, in = slot - full_slots;
      row = in / P;
      t = nfull * G + (in - row * P);
    }
    L = (xcd * rows + row) * nx + t;
  } else {
    L = xcd * q + min(xcd, r) + slot;
  }
  return {L % nx, (L / nx) % ny, L / (nx * ny)};
}

// The same XCD-contiguous ranges for a GEMM grid (x = row tiles, y = column tiles), with the
// tiles of a range visited in groups of GM row tiles: within a group the row tile runs fastest,
// so the workgroups an XCD runs side by side cover GM row panels and a few column panels, and
// each panel's reduction chunks serve several of them from the L2 (row tile fastest over all
// row tiles would have them share column panels only).
template <int GM>
__device__ inline Tile3 xcd_tile_grouped() {
  const int nx = gridDim.x, ny = gridDim.y;
  const int nwg = nx * ny * (int)gridDim.z;
  const int lin = (int)blockIdx.x + nx * ((int)blockIdx.y + ny * (int)blockIdx.z);
  const int q = nwg >> 3, r = nwg & 7, xcd = lin & 7, slot = lin >> 3;
  const int L = xcd * q + min(xcd, r) + slot;
  const int per = nx * ny, z = L / per, Lr = L - z * per;
  const int grp = Lr / (GM * ny), first = grp * GM, g = min(nx - first, GM);
  const int in = Lr - grp * GM * ny;
  return {first + in % g, in / g, z};
}

}  // namespace jenga
