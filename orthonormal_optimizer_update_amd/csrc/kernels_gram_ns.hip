// Gram Newton-Schulz for a small Gram side (M <= 128 rows, wide orientation):
// the iteration X_{k+1} = (a I + b A_k + c A_k^2) X_k, A_k = X_k X_k^T, run on
// the M x M side.  With X_k = Q_k X_0 and A_0 = X_0 X_0^T,
//     A_k     = Q_k A_0 Q_k^T
//     Q_{k+1} = (a I + b A_k + c A_k^2) Q_k,   Q_0 = I,
// and the result is X_steps = Q_steps X_0 (one product with the wide matrix,
// made by the split-precision apply).  This is the same iteration rewritten on
// the Gram side (hysenlabs "Microsoft Dion: orthonormal optimizers that assume
// DTensor parallelism", section on installing with the optional kernels, which
// names a Gram Newton-Schulz option; agentlenshq "microsoft/dion", section
// "Highlights", per-head orthogonalisation).  Every Q_k is a polynomial in A_0,
// so every matrix here is symmetric (up to rounding) and nothing is inverted.
#include "launch.h"

namespace ortho {

namespace {

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ floatx16 mfma(const bf16x8& x, const bf16x8& y, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c, 0, 0, 0);
}

}  // namespace

// One workgroup (4 waves, 2 x 2 layout, WT x WT per wave) per member; MP = 64
// or 128 is M rounded up (padded rows and columns of A_0 are zero, and the
// identity term is added on the M real rows only, so every padded entry stays
// zero).  Q_k and one work matrix (T, A_k, then P_k) live in LDS as two bf16
// pieces each (x = hi + lo + O(2^-16 |x|); row pitch MP + 8 elements), so the
// products read their fragments directly; A_0 lives in the member's global
// scratch as three pieces and is read from L2 once per iteration.  The products
// T = Q_k A_0 (A_0 is exactly symmetric), A_k = T Q_k^T and S = A_k A_k^T read
// rows of their right operand; Q_{k+1} = P_k Q_k reads Q_k's columns (see
// prod_lc).  Precision, from emulating the
// iteration against fp64: hi*hi + hi*lo + lo*hi for T Q_k, A_k A_k and P_k Q_k,
// and the five products of Q_k's two pieces with A_0's three pieces (i + j <=
// 2) for Q_k A_0, whose small eigen-directions need them (rank-1 inputs).
template <int MP>
__global__ __launch_bounds__(256) void ns_gram_iter_kernel(NsGramIterArgs a) {
  constexpr int LD = MP + 8;
  constexpr int WT = MP / 2, NB = WT / 32;
  constexpr int PS = MP * LD;  // elements per LDS piece
  __shared__ __attribute__((aligned(16))) uint16_t sQ[2 * PS];
  __shared__ __attribute__((aligned(16))) uint16_t sW[2 * PS];
  const int bi = blockIdx.x;
  const int M = a.M;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // A_0's three pieces, MP x MP each with ld MP
  uint16_t* a0 = static_cast<uint16_t*>(const_cast<void*>(a.a0.p[bi]));
  const float sc = a.scale ? a.scale[bi * a.scale_stride] : 1.0f;

  // A_0 = sc^2 * (the sum of the k-split Gram slices in slice order, ld M),
  // zero-padded to MP x MP: three pieces to the global scratch, two to sW.
  {
    const float* part = a.part + bi * a.part_member_stride;
    constexpr int PER = MP * MP / 256;
    float v[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) v[q] = 0.f;
    for (int sl = 0; sl < a.splits; ++sl) {
      const float* src = part + sl * a.slice;
      float t[PER];
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const int e = tid + q * 256, i = e / MP, j = e % MP;
        t[q] = (i < M && j < M) ? src[i * M + j] : 0.f;
      }
#pragma unroll
      for (int q = 0; q < PER; ++q) v[q] += t[q];
    }
    const float sc2 = sc * sc;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = tid + q * 256, i = e / MP, j = e % MP;
      const float x = sc2 * v[q];
      const bf16 h = to_bf16(x);
      const float r1 = x - static_cast<float>(h);
      const bf16 md = to_bf16(r1);
      const bf16 l = to_bf16(r1 - static_cast<float>(md));
      a0[i * MP + j] = __builtin_bit_cast(uint16_t, h);
      a0[MP * MP + i * MP + j] = __builtin_bit_cast(uint16_t, md);
      a0[2 * MP * MP + i * MP + j] = __builtin_bit_cast(uint16_t, l);
      sW[i * LD + j] = __builtin_bit_cast(uint16_t, h);
      sW[PS + i * LD + j] = to_bf16_bits(r1);
    }
  }
  // the scratch copy is read back by other waves: complete the stores and
  // drop stale cache lines before they read it
  __threadfence();
  __syncthreads();

  const int fr = lane & 31, fk = (lane >> 5) * 8;
  floatx16 acc[NB][NB], keep[NB][NB];
  auto zero = [&]() {
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  };
  // acc = X Y^T over k < MP, both from LDS pieces: hi*hi + hi*lo + lo*hi.
  // The fragments of the next k step are read while this step's products run,
  // and each product kind goes over all accumulators before the next kind, so
  // consecutive products never wait on each other.
  auto prod_ll = [&](const uint16_t* X, const uint16_t* Y) {
    zero();
    bf16x8 xh[2][NB], xl[2][NB], yh[2][NB], yl[2][NB];
    auto load = [&](int buf, int k0) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int o = (wm * WT + i * 32 + fr) * LD + k0 + fk;
        xh[buf][i] = ld8(X + o);
        xl[buf][i] = ld8(X + PS + o);
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int o = (wn * WT + j * 32 + fr) * LD + k0 + fk;
        yh[buf][j] = ld8(Y + o);
        yl[buf][j] = ld8(Y + PS + o);
      }
    };
    load(0, 0);
#pragma unroll
    for (int k0 = 0; k0 < MP; k0 += 16) {
      const int cur = (k0 >> 4) & 1;
      if (k0 + 16 < MP) load(cur ^ 1, k0 + 16);
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = mfma(xh[cur][i], yh[cur][j], acc[i][j]);
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = mfma(xh[cur][i], yl[cur][j], acc[i][j]);
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = mfma(xl[cur][i], yh[cur][j], acc[i][j]);
    }
  };
  // acc = X Y with Y read down its columns (both from LDS pieces, hi*hi +
  // hi*lo + lo*hi).  Q_{k+1} = P_k Q_k needs the true product: Q_k is symmetric
  // only up to rounding, and P_k Q_k^T lets that asymmetry grow with the
  // iteration's gain on rank-deficient inputs (found by emulating the kernel's
  // arithmetic against fp64: 1e-1 instead of 1.5e-3 on a rank-1 input).
  auto prod_lc = [&](const uint16_t* X, const uint16_t* Y) {
    zero();
    bf16x8 xh[2][NB], xl[2][NB], yh[2][NB], yl[2][NB];
    auto load = [&](int buf, int k0) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int o = (wm * WT + i * 32 + fr) * LD + k0 + fk;
        xh[buf][i] = ld8(X + o);
        xl[buf][i] = ld8(X + PS + o);
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int col = wn * WT + j * 32 + fr;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int o = (k0 + fk + t) * LD + col;
          yh[buf][j][t] = __builtin_bit_cast(bf16, Y[o]);
          yl[buf][j][t] = __builtin_bit_cast(bf16, Y[PS + o]);
        }
      }
    };
    load(0, 0);
#pragma unroll
    for (int k0 = 0; k0 < MP; k0 += 16) {
      const int cur = (k0 >> 4) & 1;
      if (k0 + 16 < MP) load(cur ^ 1, k0 + 16);
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = mfma(xh[cur][i], yh[cur][j], acc[i][j]);
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = mfma(xh[cur][i], yl[cur][j], acc[i][j]);
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = mfma(xl[cur][i], yh[cur][j], acc[i][j]);
    }
  };
  // acc = X A_0 (A_0 symmetric): X's two LDS pieces against A_0's three
  // global pieces, the five products with piece indices summing to <= 2; the
  // fragments of the next k step are loaded while this one's run
  auto prod_lg = [&](const uint16_t* X) {
    zero();
    bf16x8 g[2][NB][3], xh[2][NB], xl[2][NB];
    auto load = [&](int buf, int k0) {
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int p = 0; p < 3; ++p)
          g[buf][j][p] = ld8(a0 + p * MP * MP + (wn * WT + j * 32 + fr) * MP + k0 + fk);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int o = (wm * WT + i * 32 + fr) * LD + k0 + fk;
        xh[buf][i] = ld8(X + o);
        xl[buf][i] = ld8(X + PS + o);
      }
    };
    load(0, 0);
#pragma unroll
    for (int k0 = 0; k0 < MP; k0 += 16) {
      const int cur = (k0 >> 4) & 1;
      if (k0 + 16 < MP) load(cur ^ 1, k0 + 16);
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = mfma(xh[cur][i], g[cur][j][0], acc[i][j]);
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = mfma(xh[cur][i], g[cur][j][1], acc[i][j]);
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = mfma(xl[cur][i], g[cur][j][0], acc[i][j]);
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = mfma(xh[cur][i], g[cur][j][2], acc[i][j]);
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = mfma(xl[cur][i], g[cur][j][1], acc[i][j]);
    }
  };
  // element (row, col) of accumulator (i, j), register g * 4 + t
  auto rc = [&](int i, int j, int g, int t, int& row, int& col) {
    row = wm * WT + i * 32 + g * 8 + (lane >> 5) * 4 + t;
    col = wn * WT + j * 32 + (lane & 31);
  };
  // the accumulators as two bf16 pieces into D
  auto store = [&](uint16_t* D) {
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            int row, col;
            rc(i, j, g, t, row, col);
            const float x = acc[i][j][g * 4 + t];
            const bf16 h = to_bf16(x);
            D[row * LD + col] = __builtin_bit_cast(uint16_t, h);
            D[PS + row * LD + col] = to_bf16_bits(x - static_cast<float>(h));
          }
  };
  // P = a I + b A + c S with S = A A in the accumulators and A in `keep`; the
  // identity only on the M real rows
  auto poly = [&]() {
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            int row, col;
            rc(i, j, g, t, row, col);
            const float eye = (row == col && row < M) ? a.a : 0.f;
            acc[i][j][g * 4 + t] = eye + a.b * keep[i][j][g * 4 + t] + a.c * acc[i][j][g * 4 + t];
          }
  };

  // k = 0: A_0 (fp32 value from its three pieces) kept; Q_1 = P_0
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          int row, col;
          rc(i, j, g, t, row, col);
          const int o = row * MP + col;
          keep[i][j][g * 4 + t] = bf16_bits_to_f32(a0[o]) + bf16_bits_to_f32(a0[MP * MP + o]) +
                                  bf16_bits_to_f32(a0[2 * MP * MP + o]);
        }
  prod_ll(sW, sW);
  poly();
  __syncthreads();
  store(sQ);
  __syncthreads();
  for (int k = 1; k < a.steps; ++k) {
    prod_lg(sQ);           // T = Q_k A_0
    store(sW);             // sW held P_{k-1}, last read before the previous barrier
    __syncthreads();
    prod_ll(sW, sQ);       // A_k = T Q_k^T
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) keep[i][j] = acc[i][j];
    __syncthreads();
    store(sW);
    __syncthreads();
    prod_ll(sW, sW);       // S = A_k A_k^T
    poly();                // P_k
    __syncthreads();
    store(sW);
    __syncthreads();
    prod_lc(sW, sQ);       // Q_{k+1} = P_k Q_k
    if (k + 1 < a.steps) {
      __syncthreads();
      store(sQ);
      __syncthreads();
    }
  }
  // sc * Q_steps (the M x M real block, fp32 from the accumulators) for the apply
  float* q = static_cast<float*>(const_cast<void*>(a.q.p[bi]));
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          int row, col;
          rc(i, j, g, t, row, col);
          if (row < M && col < M) q[(int64_t)row * a.q.ld + col] = sc * acc[i][j][g * 4 + t];
        }
}

hipError_t launch_ns_gram_iter(const NsGramIterArgs& a, int members, hipStream_t s) {
  if (a.M < 1 || a.M > 128 || a.steps < 1 || a.a0.ld != (a.M <= 64 ? 64 : 128))
    return hipErrorInvalidValue;
  if (a.M <= 64)
    hipLaunchKernelGGL(ns_gram_iter_kernel<64>, dim3(members), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(ns_gram_iter_kernel<128>, dim3(members), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ortho
