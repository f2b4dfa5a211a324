// Cross-entropy of the language-model head, segment by segment, for gfx950.
//
// Jenga (aipaper summary, §4.4.2; papercache notes, §4.4 segment-based peak cutting): the loss
// computation's transient -- the full [tokens x vocab] logits -- is cut into segments that are
// processed one after another, so the peak follows the segment instead of the sequence.
//
//   k_ce_rows    one workgroup per logits row: the row stays in registers (one read), then
//                lse = max + log sum exp(x - max), row_loss = lse - x[target], and the gradient
//                (exp(x - lse) - [v == target]) * grad_scale written as bf16 for the next GEMM
//   k_loss_mean  mean of the row losses in a fixed order (fp64)
#include "common.h"
#include "kernels.h"

namespace jenga {

// One workgroup of 1024 threads per row; thread t holds the float4 groups t, t + 1024, ... of
// the row (vocab is a multiple of 128, so a group is wholly inside or past the row).  With 32
// values per thread a wave issues its 8 loads at once and several workgroups share a compute
// unit; a 256-thread workgroup holding 128 values per thread ran one wave per SIMD and waited
// out two memory round trips per row.  (Launch bounds: at least 8 waves per SIMD, i.e. two
// workgroups per compute unit, which keeps a thread within 64 registers.)
constexpr int kCeThreads = 1024;
constexpr int kCeGroups = 8;                              // float4 groups per thread: vocab <= 32768

__device__ inline float block_reduce(float v, float* red, bool is_max) {
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float o = __shfl_xor(v, off, 64);
    v = is_max ? fmaxf(v, o) : v + o;
  }
  if (l == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kCeThreads / 64; ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kCeThreads, 8) void k_ce_rows(CeParams p) {
  __shared__ float red[kCeThreads / 64];
  const int row = blockIdx.x, tid = threadIdx.x;
  const float* x = p.logits + (int64_t)row * p.V;
  bf16* g = (bf16*)p.dlogits + (int64_t)row * p.V;
  f32x4 v[kCeGroups];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < kCeGroups; ++i) {
    const int c = 4 * (i * kCeThreads + tid);
    v[i] = c < p.V ? *(const f32x4*)(x + c) : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    mx = fmaxf(mx, fmaxf(fmaxf(v[i][0], v[i][1]), fmaxf(v[i][2], v[i][3])));
  }
  mx = block_reduce(mx, red, true);
  float se = 0.f;
#pragma unroll
  for (int i = 0; i < kCeGroups; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) se += __expf(v[i][e] - mx);
  se = block_reduce(se, red, false);
  const float lse = mx + __logf(se);
  const int t = p.targets[row];
  if (tid == 0) p.row_loss[row] = lse - x[t];
#pragma unroll
  for (int i = 0; i < kCeGroups; ++i) {
    const int c = 4 * (i * kCeThreads + tid);
    if (c < p.V) {
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = (__expf(v[i][e] - lse) - (c + e == t ? 1.f : 0.f)) * p.grad_scale;
      u32x2 w;
      w[0] = pack_bf16x2(y[0], y[1]);
      w[1] = pack_bf16x2(y[2], y[3]);
      *(u32x2*)(g + c) = w;
    }
  }
}

__global__ __launch_bounds__(256) void k_loss_mean(const float* row_loss, int rows, float* loss) {
  __shared__ double part[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < rows; i += 256) s += (double)row_loss[i];
  part[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int i = 0; i < 256; ++i) t += part[i];
    *loss = (float)(t / rows);
  }
}

hipError_t launch_ce_rows(const CeParams& p, hipStream_t st) {
  TimedLaunch tl("k_ce_rows", st);
  k_ce_rows<<<p.rows, kCeThreads, 0, st>>>(p);
  return hipGetLastError();
}

hipError_t launch_loss_mean(const float* row_loss, int rows, float* loss, hipStream_t st) {
  k_loss_mean<<<1, 256, 0, st>>>(row_loss, rows, loss);
  return hipGetLastError();
}

}  // namespace jenga
