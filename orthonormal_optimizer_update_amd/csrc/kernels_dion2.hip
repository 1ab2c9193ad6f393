// Dion2 (agentlenshq "microsoft/dion", sections "How it works" and
// "Highlights"; hysenlabs "Microsoft Dion: orthonormal optimizers that assume
// DTensor parallelism", section "Dion3 is not a retuning of Dion2, and the
// README says so"): with B = M + G, the k rows of B with the largest l2 norm
// are orthonormalised together (Newton-Schulz) and applied; error feedback
// keeps mu times the applied rows and every other row whole.  The pages print
// no selection rule; largest row norm, ties by lower row index, is the
// reading.  Four launches around the Newton-Schulz of the block:
//   norms   sum of squares of every row of B (fp32, a fixed order)
//   rank    rank of every row in (norm descending, index ascending) order --
//           a strict total order, so ranks are a permutation of 0 .. m-1 and
//           sel[rank] = row for rank < k names every selected row once
//   gather  block[t] = B[sel[t]]
//   update  selected row i (rank t): M = mu B, X = X - c U[t]; other rows: M = B
#include "launch.h"

namespace ortho {

namespace {

// Sum over the 256 threads of a workgroup in a fixed order; every thread gets
// the total.
__device__ __forceinline__ float block_sum256(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

template <typename GT>
__global__ __launch_bounds__(256) void dion2_norms_kernel(Dion2Args a) {
  __shared__ float red[4];
  const int bi = blockIdx.z, i = blockIdx.y;
  const float* M = static_cast<const float*>(a.m.p[bi]) + (int64_t)i * a.m.ld;
  const GT* G = static_cast<const GT*>(a.g.p[bi]) + (int64_t)i * a.g.ld;
  const bool vec = a.m.vec && a.g.vec;
  float s = 0.f;
  for (int c = threadIdx.x * 4; c < a.cols; c += 1024) {
    const float4 mv = load4<float>(M, c, a.cols, vec);
    const float4 gv = load4<GT>(G, c, a.cols, vec);
    const float x0 = mv.x + gv.x, x1 = mv.y + gv.y, x2 = mv.z + gv.z, x3 = mv.w + gv.w;
    s += (x0 * x0 + x1 * x1) + (x2 * x2 + x3 * x3);
  }
  s = block_sum256(s, red);
  if (threadIdx.x == 0) a.norms[bi * a.vec_stride + i] = s;
}

// One thread per row; the norms pass through LDS in chunks of 4096.
__global__ __launch_bounds__(256) void dion2_rank_kernel(Dion2Args a) {
  __shared__ float keys[4096];
  const int bi = blockIdx.z;
  const int i = blockIdx.x * 256 + threadIdx.x;
  const float* norms = a.norms + bi * a.vec_stride;
  auto key = [](float v) { return v != v ? -1.0f : v; };   // NaN after everything
  const float ki = i < a.rows ? key(norms[i]) : 0.f;
  int rank = 0;
  for (int j0 = 0; j0 < a.rows; j0 += 4096) {
    const int nj = min(4096, a.rows - j0);
    __syncthreads();
    for (int t = threadIdx.x; t < nj; t += 256) keys[t] = key(norms[j0 + t]);
    __syncthreads();
    for (int t = 0; t < nj; ++t) {
      const float kj = keys[t];
      rank += (kj > ki) || (kj == ki && j0 + t < i);
    }
  }
  if (i < a.rows) {
    a.rank[bi * a.vec_stride + i] = rank;
    if (rank < a.k) a.sel[bi * a.vec_stride + rank] = i;
  }
}

// block row t = B[sel[t]], four columns per thread.
template <typename GT>
__global__ __launch_bounds__(256) void dion2_gather_kernel(Dion2Args a) {
  const int bi = blockIdx.z, t = blockIdx.y;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= a.cols) return;
  const int row = a.sel[bi * a.vec_stride + t];
  const float* M = static_cast<const float*>(a.m.p[bi]) + (int64_t)row * a.m.ld;
  const GT* G = static_cast<const GT*>(a.g.p[bi]) + (int64_t)row * a.g.ld;
  float* dst = static_cast<float*>(const_cast<void*>(a.blk.p[bi])) + (int64_t)t * a.blk.ld;
  const bool vec = a.m.vec && a.g.vec && a.blk.vec;
  const float4 mv = load4<float>(M, c, a.cols, vec);
  const float4 gv = load4<GT>(G, c, a.cols, vec);
  const float v[4] = {mv.x + gv.x, mv.y + gv.y, mv.z + gv.z, mv.w + gv.w};
  if (vec && c + 4 <= a.cols) {
    *reinterpret_cast<float4*>(dst + c) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (c + e < a.cols) dst[c + e] = v[e];
  }
}

// Error feedback and the update, one row per blockIdx.y, four columns per
// thread: rank t < k: M = mu (M + G), X = X - c U[t] (RNE into X's dtype);
// otherwise M = M + G and X is untouched.
template <typename XT>
__global__ __launch_bounds__(256) void dion2_update_kernel(Dion2Args a) {
  const int bi = blockIdx.z, i = blockIdx.y;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= a.cols) return;
  const int t = a.rank[bi * a.vec_stride + i];
  const bool applied = t < a.k;
  float* M = static_cast<float*>(const_cast<void*>(a.m.p[bi])) + (int64_t)i * a.m.ld;
  const XT* G = static_cast<const XT*>(a.g.p[bi]) + (int64_t)i * a.g.ld;
  const bool vec = a.m.vec && a.g.vec && a.x.vec && a.blk.vec;
  const float4 mv = load4<float>(M, c, a.cols, vec);
  const float4 gv = load4<XT>(G, c, a.cols, vec);
  const float f = applied ? a.mu : 1.0f;
  const float mn[4] = {f * (mv.x + gv.x), f * (mv.y + gv.y), f * (mv.z + gv.z), f * (mv.w + gv.w)};
  if (vec && c + 4 <= a.cols) {
    *reinterpret_cast<float4*>(M + c) = make_float4(mn[0], mn[1], mn[2], mn[3]);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (c + e < a.cols) M[c + e] = mn[e];
  }
  if (!applied) return;
  XT* X = static_cast<XT*>(const_cast<void*>(a.x.p[bi])) + (int64_t)i * a.x.ld;
  const float* U = static_cast<const float*>(a.blk.p[bi]) + (int64_t)t * a.blk.ld;
  const float4 xv = load4<XT>(X, c, a.cols, vec);
  const float4 uv = load4<float>(U, c, a.cols, vec);
  const float xn[4] = {xv.x - a.c * uv.x, xv.y - a.c * uv.y, xv.z - a.c * uv.z, xv.w - a.c * uv.w};
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (c + e < a.cols) store_from_f32<XT>(X, c + e, xn[e]);
}

inline int cdiv(int64_t a, int64_t b) { return static_cast<int>((a + b - 1) / b); }

}  // namespace

hipError_t launch_dion2_select(const Dion2Args& a, bool g_bf16, int members, hipStream_t s) {
  if (a.rows < 1 || a.rows > 65535 || a.k < 1 || a.k > a.rows) return hipErrorInvalidValue;
  if (g_bf16)
    hipLaunchKernelGGL(dion2_norms_kernel<uint16_t>, dim3(1, a.rows, members), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(dion2_norms_kernel<float>, dim3(1, a.rows, members), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dion2_rank_kernel, dim3(cdiv(a.rows, 256), 1, members), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid(cdiv(a.cols, 1024), a.k, members);
  if (g_bf16) hipLaunchKernelGGL(dion2_gather_kernel<uint16_t>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(dion2_gather_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dion2_update(const Dion2Args& a, bool x_bf16, int members, hipStream_t s) {
  dim3 grid(cdiv(a.cols, 1024), a.rows, members);
  if (x_bf16) hipLaunchKernelGGL(dion2_update_kernel<uint16_t>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(dion2_update_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ortho
