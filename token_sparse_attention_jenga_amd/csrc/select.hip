// Token-block elimination on gfx950: top-k by keep ratio or a per-layer threshold, then
// wavefront ballot / prefix compaction of the kept block indices.
//
// Jenga (papercache notes, §4.2 layer-specific threshold; aipaper summary, §4.2.3 Algorithm
// 1 step 1: the layer threshold starts from the average token-block score).  One workgroup
// per batch row; the whole decision is exact and deterministic.
#include "common.h"
#include "kernels.h"

namespace jenga {

// Order key: larger key = better block.  NaN maps below every number; -0 and +0 tie.
__device__ inline uint32_t order_key(float x) {
  if (x != x) return 0u;
  if (x == 0.f) x = 0.f;
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kSelThreads = 1024;

__global__ __launch_bounds__(kSelThreads) void k_select(SelectParams p) {
  extern __shared__ uint32_t keys[];            // [nkb]
  __shared__ double thr_s;
  __shared__ int wave_tot[kSelThreads / 64];
  __shared__ int running_s;

  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nkb = p.nkb;
  const float* x = p.scores + (int64_t)b * nkb;
  const bool force = (p.flags & 1u) != 0;
  for (int n = tid; n < nkb; n += kSelThreads) keys[n] = order_key(x[n]);
  if (tid == 0) {
    running_s = 0;
    if (p.mode == 1) {
      double total = 0.0;
      for (int n = 0; n < nkb; ++n) total += (double)x[n];   // left to right, as specified
      thr_s = (double)p.param * (total / (double)nkb);
    } else {
      thr_s = (double)p.param;
    }
  }
  __syncthreads();
  const double thr = thr_s;
  // top-k among the candidates (all blocks, or blocks 1.. when block 0 is forced)
  const int kc = force ? p.kcount - 1 : p.kcount;
  const int first = force ? 1 : 0;

  for (int base = 0; base < nkb; base += kSelThreads) {
    const int n = base + tid;
    bool keep = false;
    if (n < nkb) {
      if (force && n == 0) {
        keep = true;
      } else if (p.mode == 0) {
        const uint32_t kn = keys[n];
        int rank = 0;
        for (int m = first; m < nkb && rank < kc; ++m) {
          const uint32_t km = keys[m];
          rank += (km > kn) || (km == kn && m < n);
        }
        keep = rank < kc;
      } else {
        keep = (double)x[n] >= thr;                       // NaN compares false
      }
    }
    const uint64_t mask = __ballot(keep);
    const int before = __popcll(mask & ((1ull << lane) - 1ull));
    if (lane == 0) wave_tot[wv] = __popcll(mask);
    __syncthreads();
    int off = running_s;
    for (int i = 0; i < wv; ++i) off += wave_tot[i];
    if (keep) p.kept_idx[(int64_t)b * nkb + off + before] = n;
    __syncthreads();
    if (tid == 0) {
      int t = running_s;
      for (int i = 0; i < kSelThreads / 64; ++i) t += wave_tot[i];
      running_s = t;
    }
    __syncthreads();
  }
  const int total = running_s;
  for (int n = total + tid; n < nkb; n += kSelThreads) p.kept_idx[(int64_t)b * nkb + n] = -1;
  if (tid == 0) p.n_kept[b] = total;
}

hipError_t launch_select(const SelectParams& p, hipStream_t st) {
  TimedLaunch tl("k_select", st);
  k_select<<<p.B, kSelThreads, (size_t)p.nkb * sizeof(uint32_t), st>>>(p);
  return hipGetLastError();
}

}  // namespace jenga
