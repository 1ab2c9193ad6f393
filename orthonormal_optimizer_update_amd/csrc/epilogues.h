// Epilogue policies for gemm_kernel.  apply() receives rows row0..row0+3 of
// column col (acc values v0..v3); apply2() also receives a second accumulator.
#pragma once

#include "common.h"

namespace ortho {

// fp32 store of C (optionally also C^T), or of one split-K slice of C.
struct EpiStoreF32 {
  struct Args {
    MatArg c;              // destination, fp32
    int64_t split_stride;  // elements between split-K slices (0: no split)
    MatArg ct;             // transposed copy, fp32 (used when has_t)
    int has_t;
    MatArg cb;             // bf16 copy (used when has_b)
    int has_b;
  };
  float* c;
  float* ct;
  uint16_t* cb;
  int64_t ld, ldt, ldb;
  bool has_t, has_b;
  __device__ EpiStoreF32(const Args& a, int bi, int split)
      : c(static_cast<float*>(const_cast<void*>(a.c.p[bi])) + split * a.split_stride),
        ct(a.has_t ? static_cast<float*>(const_cast<void*>(a.ct.p[bi])) : nullptr),
        cb(a.has_b ? static_cast<uint16_t*>(const_cast<void*>(a.cb.p[bi])) : nullptr),
        ld(a.c.ld), ldt(a.ct.ld), ldb(a.cb.ld), has_t(a.has_t), has_b(a.has_b) {}
  __device__ __forceinline__ void apply(int row0, int col, int M, int N, float v0, float v1,
                                        float v2, float v3) {
    if (col >= N) return;
    const float v[4] = {v0, v1, v2, v3};
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (row0 + t < M) c[(int64_t)(row0 + t) * ld + col] = v[t];
    if (has_t) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (row0 + t < M) ct[(int64_t)col * ldt + row0 + t] = v[t];
    }
    if (has_b) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (row0 + t < M) cb[(int64_t)(row0 + t) * ldb + col] = to_bf16_bits(v[t]);
    }
  }
};

// Newton-Schulz Gram A = X X^T, stored as bf16.
struct EpiNSGram {
  struct Args {
    MatArg a;  // bf16 bits, M x N
  };
  uint16_t* a;
  int64_t ld;
  __device__ EpiNSGram(const Args& g, int bi, int)
      : a(static_cast<uint16_t*>(const_cast<void*>(g.a.p[bi]))), ld(g.a.ld) {}
  __device__ __forceinline__ void apply(int row0, int col, int M, int N, float v0, float v1,
                                        float v2, float v3) {
    if (col >= N) return;
    const float v[4] = {v0, v1, v2, v3};
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (row0 + t < M) a[(int64_t)(row0 + t) * ld + col] = to_bf16_bits(v[t]);
  }
};

// Newton-Schulz polynomial Bp = b A + c (A A), stored as bf16.
struct EpiNSPoly {
  struct Args {
    MatArg a;     // bf16 A (read)
    MatArg bp;    // bf16 Bp (written)
    MatArg bp32;  // fp32 Bp (written when has32)
    float b, c;
    int has32;
  };
  const uint16_t* a;
  uint16_t* bp;
  float* bp32;
  int64_t lda, ldb, ldb32;
  float b, c;
  __device__ EpiNSPoly(const Args& g, int bi, int)
      : a(static_cast<const uint16_t*>(g.a.p[bi])),
        bp(static_cast<uint16_t*>(const_cast<void*>(g.bp.p[bi]))),
        bp32(g.has32 ? static_cast<float*>(const_cast<void*>(g.bp32.p[bi])) : nullptr),
        lda(g.a.ld), ldb(g.bp.ld), ldb32(g.bp32.ld), b(g.b), c(g.c) {}
  __device__ __forceinline__ void apply(int row0, int col, int M, int N, float v0, float v1,
                                        float v2, float v3) {
    if (col >= N) return;
    const float v[4] = {v0, v1, v2, v3};
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (row0 + t < M) {
        const float av = bf16_bits_to_f32(a[(int64_t)(row0 + t) * lda + col]);
        const float y = b * av + c * v[t];
        bp[(int64_t)(row0 + t) * ldb + col] = to_bf16_bits(y);
        if (bp32) bp32[(int64_t)(row0 + t) * ldb32 + col] = y;
      }
  }
};

// Newton-Schulz apply X <- a X + Bp X.  The fp32 iterate is updated in place;
// bf16 copies in both orientations feed the next iteration's products.  On the
// last iteration the result goes to the caller's output instead, in its dtype,
// transposed back when the input was tall.
template <typename OUT_T>
struct EpiNSApply {
  struct Args {
    MatArg x32;   // fp32 iterate, M x N (read and written)
    MatArg xb;    // bf16 M x N (written unless last)
    MatArg xbt;   // bf16 N x M (written unless last)
    MatArg out;   // caller's output (written when last)
    float a;
    int last;
    int out_transposed;  // out is N x M
  };
  float* x32;
  uint16_t* xb;
  uint16_t* xbt;
  OUT_T* out;
  int64_t ldx, ldb, ldbt, ldo;
  float a;
  bool last, out_t;
  __device__ EpiNSApply(const Args& g, int bi, int)
      : x32(static_cast<float*>(const_cast<void*>(g.x32.p[bi]))),
        xb(static_cast<uint16_t*>(const_cast<void*>(g.xb.p[bi]))),
        xbt(static_cast<uint16_t*>(const_cast<void*>(g.xbt.p[bi]))),
        out(static_cast<OUT_T*>(const_cast<void*>(g.out.p[bi]))),
        ldx(g.x32.ld), ldb(g.xb.ld), ldbt(g.xbt.ld), ldo(g.out.ld), a(g.a), last(g.last),
        out_t(g.out_transposed) {}
  __device__ __forceinline__ void apply(int row0, int col, int M, int N, float v0, float v1,
                                        float v2, float v3) {
    if (col >= N) return;
    const float v[4] = {v0, v1, v2, v3};
    uint16_t hb[4] = {0, 0, 0, 0};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row = row0 + t;
      if (row >= M) continue;
      const int64_t ix = (int64_t)row * ldx + col;
      const float xn = a * x32[ix] + v[t];
      if (last) {
        if (out_t) store_from_f32<OUT_T>(out, (int64_t)col * ldo + row, xn);
        else store_from_f32<OUT_T>(out, (int64_t)row * ldo + col, xn);
      } else {
        x32[ix] = xn;
        hb[t] = to_bf16_bits(xn);
        xb[(int64_t)row * ldb + col] = hb[t];
      }
    }
    if (!last) {
      // The four rows are consecutive elements of one row of X^T: one 8-byte
      // store when they are all inside (row0 is a multiple of 4 and the
      // transposed buffer's leading dimension a multiple of 8).
      uint16_t* dst = xbt + (int64_t)col * ldbt + row0;
      if (row0 + 4 <= M) {
        *reinterpret_cast<uint2*>(dst) =
            make_uint2(hb[0] | (uint32_t(hb[1]) << 16), hb[2] | (uint32_t(hb[3]) << 16));
      } else {
        for (int t = 0; t < 4 && row0 + t < M; ++t) dst[t] = hb[t];
      }
    }
  }
};

// Dion sweep 3: with B = M + G recomputed from the inputs,
//   M <- B - c1 * (P R^T),   X <- X - c2 * (P Q'^T)
// where c1 = 1 - mu and c2 = lr * scale.  X is rounded to its storage dtype.
template <typename XT>
struct EpiDion {
  struct Args {
    MatArg m;  // fp32 momentum (read and written)
    MatArg g;  // gradient, XT
    MatArg x;  // weight, XT (read and written)
    float c1, c2;
  };
  float* m;
  const XT* g;
  XT* x;
  int64_t ldm, ldg, ldx;
  float c1, c2;
  __device__ EpiDion(const Args& e, int bi, int)
      : m(static_cast<float*>(const_cast<void*>(e.m.p[bi]))),
        g(static_cast<const XT*>(e.g.p[bi])),
        x(static_cast<XT*>(const_cast<void*>(e.x.p[bi]))),
        ldm(e.m.ld), ldg(e.g.ld), ldx(e.x.ld), c1(e.c1), c2(e.c2) {}
  __device__ __forceinline__ void apply2(int row0, int col, int M, int N, float u0, float u1,
                                         float u2, float u3, float w0, float w1, float w2,
                                         float w3) {
    if (col >= N) return;
    const float u[4] = {u0, u1, u2, u3};
    const float w[4] = {w0, w1, w2, w3};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row = row0 + t;
      if (row >= M) continue;
      const int64_t im = (int64_t)row * ldm + col;
      const int64_t ig = (int64_t)row * ldg + col;
      const int64_t ix = (int64_t)row * ldx + col;
      const float bval = m[im] + load_as_f32<XT>(g, ig);
      m[im] = bval - c1 * u[t];
      store_from_f32<XT>(x, ix, load_as_f32<XT>(x, ix) - c2 * w[t]);
    }
  }
};

}  // namespace ortho
