// Epilogue policies for the GEMM kernels.  apply() receives rows row0..row0+3
// of column col (acc values v0..v3); apply2() also receives a second
// accumulator.  A policy with kPreload = true also provides init() (init2()),
// which sets the accumulators before the main loop: terms of the result that
// come from memory are loaded there, where no store precedes them and the loads
// can all be in flight at once, so the epilogue itself only stores.
#pragma once

#include <type_traits>

#include "common.h"

namespace ortho {

// Tile-aligned interface used by the 256 x 256 kernel (every tile is full):
//   kFastPre      0: accumulators start at zero; 1: at fast_pre_scale() times a
//                 bf16 M x N matrix; 2: the same for an fp32 matrix
//                 (fast_pre_src(), fast_pre_ld()).  The kernel stages that
//                 matrix through LDS with coalesced copies.
//   kSegs         1, or 3: the product is a*b0 + a*b0s + a2*b0 over bf16x2
//                 pieces (hi*hi + hi*lo + lo*hi).
//   kFastPre2     0, or 1: a second (bf16) matrix added the same way
//                 (fast_pre2_src(), fast_pre2_ld(), fast_pre2_scale()).
//   fast_store4   receives four consecutive columns of one row of the result.
//   kFastT / fast_store_t4  receive four consecutive rows of one column
//                 (transposed outputs), straight from the accumulators; a
//                 kFastT policy also names, through fast_t_rows(ld), a
//                 16-byte-aligned bf16 destination that the kernel fills with
//                 whole row pieces of the transposed tile instead (null: use
//                 fast_store_t4, or nothing when fast_t_any() is false).
//   kFastSym      the result is symmetric: with GemmParams::sym the kernel
//                 computes the tiles on and above the diagonal only and hands
//                 each off-diagonal tile to fast_store_t4 as well (its mirror).

// Four consecutive values at p[idx..idx+3]; one vector store when vec.
template <class T>
__device__ __forceinline__ void store4_from_f32(T* p, int64_t idx, floatx4 v, bool vec);
template <>
__device__ __forceinline__ void store4_from_f32<float>(float* p, int64_t idx, floatx4 v, bool vec) {
  if (vec) {
    *reinterpret_cast<floatx4*>(p + idx) = v;
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) p[idx + t] = v[t];
  }
}
template <>
__device__ __forceinline__ void store4_from_f32<uint16_t>(uint16_t* p, int64_t idx, floatx4 v,
                                                          bool vec) {
  if (vec) {
    *reinterpret_cast<uint2*>(p + idx) = pack_bf16x4(v);
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) p[idx + t] = to_bf16_bits(v[t]);
  }
}

// fp32 store of C (optionally also C^T), or of one split-K slice of C.
struct EpiStoreF32 {
  static constexpr bool kPreload = false;
  struct Args {
    MatArg c;              // destination, fp32
    int64_t split_stride;  // elements between split-K slices (0: no split)
    MatArg ct;             // transposed copy, fp32 (used when has_t)
    int has_t;
    MatArg cb;             // bf16 copy (used when has_b)
    int has_b;
    // bf16 hi and lo pieces of the transpose, k-blocked: element (row k,
    // column j) at (k / 16) * N * 16 + j * 16 + k % 16 (used when has_p; the
    // workgroup's rows come in groups of 4 inside one block of 16)
    MatArg phi, plo;
    int has_p;
    // bf16 copy in MFMA fragment order (used when has_f; N a multiple of 16):
    // element (i, k) at (((i / 32) * N / 16 + k / 16) * 64 + i % 32 +
    // 32 * (k / 8 % 2)) * 8 + k % 8
    MatArg pf;
    int has_f;
  };
  float* c;
  float* ct;
  uint16_t* cb;
  uint16_t* phi;
  uint16_t* plo;
  uint16_t* pf;
  int64_t ld, ldt, ldb;
  bool has_t, has_b, has_p, has_f;
  __device__ EpiStoreF32(const Args& a, int bi, int split)
      : c(static_cast<float*>(const_cast<void*>(a.c.p[bi])) + split * a.split_stride),
        ct(a.has_t ? static_cast<float*>(const_cast<void*>(a.ct.p[bi])) : nullptr),
        cb(a.has_b ? static_cast<uint16_t*>(const_cast<void*>(a.cb.p[bi])) : nullptr),
        phi(a.has_p ? static_cast<uint16_t*>(const_cast<void*>(a.phi.p[bi])) : nullptr),
        plo(a.has_p ? static_cast<uint16_t*>(const_cast<void*>(a.plo.p[bi])) : nullptr),
        pf(a.has_f ? static_cast<uint16_t*>(const_cast<void*>(a.pf.p[bi])) : nullptr),
        ld(a.c.ld), ldt(a.ct.ld), ldb(a.cb.ld), has_t(a.has_t), has_b(a.has_b),
        has_p(a.has_p), has_f(a.has_f) {}
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
    if (has_f) {
      const int64_t ks = N >> 4;
      const int64_t base = ((int64_t)(col >> 4) * 64 + 32 * ((col >> 3) & 1)) * 8 + (col & 7);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int i = row0 + t;
        if (i < M) pf[(((int64_t)(i >> 5) * ks) * 64 + (i & 31)) * 8 + base] = to_bf16_bits(v[t]);
      }
    }
    if (has_p) {
      uint16_t h[4], l[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        bf16 bh, bl;
        split_bf16(row0 + t < M ? v[t] : 0.f, bh, bl);
        h[t] = __builtin_bit_cast(uint16_t, bh);
        l[t] = __builtin_bit_cast(uint16_t, bl);
      }
      const int64_t o = (int64_t)(row0 >> 4) * N * 16 + (int64_t)col * 16 + (row0 & 15);
      if (row0 + 3 < M) {
        *reinterpret_cast<uint2*>(phi + o) =
            make_uint2(h[0] | (uint32_t(h[1]) << 16), h[2] | (uint32_t(h[3]) << 16));
        *reinterpret_cast<uint2*>(plo + o) =
            make_uint2(l[0] | (uint32_t(l[1]) << 16), l[2] | (uint32_t(l[3]) << 16));
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (row0 + t < M) {
            phi[o + t] = h[t];
            plo[o + t] = l[t];
          }
      }
    }
  }
};

// Newton-Schulz Gram A = X X^T, stored as bf16.
struct EpiNSGram {
  static constexpr bool kPreload = false;
  struct Args {
    MatArg a;  // bf16 bits, M x N
  };
  uint16_t* a;
  int64_t ld;
  __device__ EpiNSGram(const Args& g, int bi, int)
      : a(static_cast<uint16_t*>(const_cast<void*>(g.a.p[bi]))), ld(g.a.ld) {}
  static constexpr int kFastPre = 0;
  static constexpr int kSegs = 1;
  static constexpr int kFastPre2 = 0;
  static constexpr bool kFastT = false;
  static constexpr bool kFastSym = true;
  __device__ const void* fast_pre_src() const { return nullptr; }
  __device__ int64_t fast_pre_ld() const { return 0; }
  __device__ float fast_pre_scale() const { return 0.f; }
  __device__ __forceinline__ void fast_store4(int row, int col, floatx4 v) {
    *reinterpret_cast<uint2*>(a + (int64_t)row * ld + col) = pack_bf16x4(v);
  }
  // mirror: A[col][row0 .. row0 + 3] = A[row0 .. row0 + 3][col]
  __device__ __forceinline__ void fast_store_t4(int col, int row0, floatx4 v) {
    *reinterpret_cast<uint2*>(a + (int64_t)col * ld + row0) = pack_bf16x4(v);
  }
  __device__ const void* fast_pre2_src() const { return nullptr; }
  __device__ int64_t fast_pre2_ld() const { return 0; }
  __device__ float fast_pre2_scale() const { return 0.f; }
  __device__ __forceinline__ void apply(int row0, int col, int M, int N, float v0, float v1,
                                        float v2, float v3) {
    if (col >= N) return;
    const float v[4] = {v0, v1, v2, v3};
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (row0 + t < M) a[(int64_t)(row0 + t) * ld + col] = to_bf16_bits(v[t]);
  }
};

// Newton-Schulz polynomial Bp = b A + c (A A), stored as bf16 (and fp32 when
// has32).  The accumulator starts at (b/c) A, so the result is c * acc (c != 0;
// the launcher handles c == 0 without a product).
struct EpiNSPoly {
  static constexpr bool kPreload = true;
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
  float boc, c;
  __device__ EpiNSPoly(const Args& g, int bi, int)
      : a(static_cast<const uint16_t*>(g.a.p[bi])),
        bp(static_cast<uint16_t*>(const_cast<void*>(g.bp.p[bi]))),
        bp32(g.has32 ? static_cast<float*>(const_cast<void*>(g.bp32.p[bi])) : nullptr),
        lda(g.a.ld), ldb(g.bp.ld), ldb32(g.bp32.ld), boc(g.b / g.c), c(g.c) {}
  static constexpr int kFastPre = 1;
  static constexpr int kSegs = 1;
  static constexpr int kFastPre2 = 0;
  static constexpr bool kFastT = false;
  static constexpr bool kFastSym = true;
  __device__ const void* fast_pre_src() const { return a; }
  __device__ int64_t fast_pre_ld() const { return lda; }
  __device__ float fast_pre_scale() const { return boc; }
  __device__ __forceinline__ void fast_store4(int row, int col, floatx4 v) {
    const floatx4 y = c * v;
    *reinterpret_cast<uint2*>(bp + (int64_t)row * ldb + col) = pack_bf16x4(y);
    if (bp32) *reinterpret_cast<floatx4*>(bp32 + (int64_t)row * ldb32 + col) = y;
  }
  // mirror: Bp[col][row0 .. row0 + 3] = Bp[row0 .. row0 + 3][col]
  __device__ __forceinline__ void fast_store_t4(int col, int row0, floatx4 v) {
    const floatx4 y = c * v;
    *reinterpret_cast<uint2*>(bp + (int64_t)col * ldb + row0) = pack_bf16x4(y);
    if (bp32) *reinterpret_cast<floatx4*>(bp32 + (int64_t)col * ldb32 + row0) = y;
  }
  __device__ const void* fast_pre2_src() const { return nullptr; }
  __device__ int64_t fast_pre2_ld() const { return 0; }
  __device__ float fast_pre2_scale() const { return 0.f; }
  // Preloads run before the main loop: clamped addresses and a select (no
  // branch per element), so all of a thread's loads are in flight together.
  __device__ __forceinline__ void init(int row0, int col, int M, int N, float* v) const {
    const int cc = min(col, N - 1);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float x = bf16_bits_to_f32(a[(int64_t)min(row0 + t, M - 1) * lda + cc]);
      v[t] = (col < N && row0 + t < M) ? boc * x : 0.f;
    }
  }
  __device__ __forceinline__ void apply(int row0, int col, int M, int N, float v0, float v1,
                                        float v2, float v3) {
    if (col >= N) return;
    const float v[4] = {v0, v1, v2, v3};
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (row0 + t < M) {
        const float y = c * v[t];
        bp[(int64_t)(row0 + t) * ldb + col] = to_bf16_bits(y);
        if (bp32) bp32[(int64_t)(row0 + t) * ldb32 + col] = y;
      }
  }
};

// Newton-Schulz apply X <- a X + Bp X.  The accumulator starts at a X (the
// fp32 iterate), so the result is the accumulator: it overwrites the fp32
// iterate and its bf16 copies in both orientations, or, on the last
// iteration, goes to the caller's output in its dtype (transposed back when
// the input was tall).
template <typename OUT_T>
struct EpiNSApply {
  static constexpr bool kPreload = true;
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
  bool last, out_t, out_vec;
  __device__ EpiNSApply(const Args& g, int bi, int)
      : x32(static_cast<float*>(const_cast<void*>(g.x32.p[bi]))),
        xb(static_cast<uint16_t*>(const_cast<void*>(g.xb.p[bi]))),
        xbt(static_cast<uint16_t*>(const_cast<void*>(g.xbt.p[bi]))),
        out(static_cast<OUT_T*>(const_cast<void*>(g.out.p[bi]))),
        ldx(g.x32.ld), ldb(g.xb.ld), ldbt(g.xbt.ld), ldo(g.out.ld), a(g.a), last(g.last),
        out_t(g.out_transposed), out_vec(g.out.vec) {}
  static constexpr int kFastPre = 2;
  static constexpr int kSegs = 1;
  static constexpr int kFastPre2 = 0;
  static constexpr bool kFastT = true;
  static constexpr bool kFastSym = false;
  __device__ const void* fast_pre_src() const { return x32; }
  __device__ int64_t fast_pre_ld() const { return ldx; }
  __device__ float fast_pre_scale() const { return a; }
  __device__ __forceinline__ void fast_store4(int row, int col, floatx4 v) {
    if (last) {
      if (!out_t) store4_from_f32<OUT_T>(out, (int64_t)row * ldo + col, v, out_vec);
      return;
    }
    *reinterpret_cast<floatx4*>(x32 + (int64_t)row * ldx + col) = v;
    *reinterpret_cast<uint2*>(xb + (int64_t)row * ldb + col) = pack_bf16x4(v);
  }
  __device__ const void* fast_pre2_src() const { return nullptr; }
  __device__ int64_t fast_pre2_ld() const { return 0; }
  __device__ float fast_pre2_scale() const { return 0.f; }
  // The transposed bf16 destination when whole 16-byte pieces of its rows
  // may be stored (X^T, or the caller's transposed bf16 output on the last
  // iteration), else null; fast_t_any: whether there is a transposed output.
  __device__ uint16_t* fast_t_rows(int64_t& ld) const {
    uint16_t* d = nullptr;
    if (!last) {
      d = xbt;
      ld = ldbt;
    } else if (out_t && std::is_same<OUT_T, uint16_t>::value) {
      d = reinterpret_cast<uint16_t*>(out);
      ld = ldo;
    }
    if (d == nullptr || reinterpret_cast<uintptr_t>(d) % 16 != 0 || ld % 8 != 0) return nullptr;
    return d;
  }
  __device__ bool fast_t_any() const { return last ? out_t : xbt != nullptr; }
  // rows row0..row0+3 of column col: consecutive elements of one row of X^T
  __device__ __forceinline__ void fast_store_t4(int col, int row0, floatx4 v) {
    if (last) {
      if (out_t) store4_from_f32<OUT_T>(out, (int64_t)col * ldo + row0, v, out_vec);
      return;
    }
    if (xbt == nullptr) return;  // no product reads a transposed copy
    *reinterpret_cast<uint2*>(xbt + (int64_t)col * ldbt + row0) = pack_bf16x4(v);
  }
  __device__ __forceinline__ void init(int row0, int col, int M, int N, float* v) const {
    const int cc = min(col, N - 1);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float x = x32[(int64_t)min(row0 + t, M - 1) * ldx + cc];
      v[t] = (col < N && row0 + t < M) ? a * x : 0.f;
    }
  }
  __device__ __forceinline__ void apply(int row0, int col, int M, int N, float v0, float v1,
                                        float v2, float v3) {
    if (col >= N) return;
    const float v[4] = {v0, v1, v2, v3};
    if (last) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int row = row0 + t;
        if (row >= M) continue;
        if (out_t) store_from_f32<OUT_T>(out, (int64_t)col * ldo + row, v[t]);
        else store_from_f32<OUT_T>(out, (int64_t)row * ldo + col, v[t]);
      }
      return;
    }
    uint16_t hb[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      hb[t] = to_bf16_bits(v[t]);
      const int row = row0 + t;
      if (row < M) {
        x32[(int64_t)row * ldx + col] = v[t];
        xb[(int64_t)row * ldb + col] = hb[t];
      }
    }
    // The four rows are consecutive elements of one row of X^T: one 8-byte
    // store when they are all inside (row0 is a multiple of 4 and the
    // transposed buffer's leading dimension a multiple of 8).  No transposed
    // copy is kept when no product reads it (xbt NULL).
    if (xbt == nullptr) return;
    uint16_t* dst = xbt + (int64_t)col * ldbt + row0;
    if (row0 + 4 <= M) {
      *reinterpret_cast<uint2*>(dst) =
          make_uint2(hb[0] | (uint32_t(hb[1]) << 16), hb[2] | (uint32_t(hb[3]) << 16));
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (row0 + t < M) dst[t] = hb[t];
    }
  }
};

// Newton-Schulz with fp32-accurate products (fp32 inputs): the polynomial
// Bp = b A + c (A A) from the fp32 Gram, stored as fp32.
struct EpiNSPoly32 {
  static constexpr bool kPreload = false;
  struct Args {
    MatArg a32;   // fp32 A (read)
    MatArg bp32;  // fp32 Bp (written)
    float b, c;
  };
  const float* a;
  float* bp;
  int64_t lda, ldb;
  float b, c;
  __device__ EpiNSPoly32(const Args& g, int bi, int)
      : a(static_cast<const float*>(g.a32.p[bi])),
        bp(static_cast<float*>(const_cast<void*>(g.bp32.p[bi]))),
        lda(g.a32.ld), ldb(g.bp32.ld), b(g.b), c(g.c) {}
  __device__ __forceinline__ void apply(int row0, int col, int M, int N, float v0, float v1,
                                        float v2, float v3) {
    if (col >= N) return;
    const float v[4] = {v0, v1, v2, v3};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row = row0 + t;
      if (row < M) bp[(int64_t)row * ldb + col] = b * a[(int64_t)row * lda + col] + c * v[t];
    }
  }
};

// Newton-Schulz apply with fp32-accurate products: X' = a X + Bp X, read from
// one fp32 iterate and written to the other (the product of every row tile
// reads all rows of X, so the update cannot be made in place), or, on the last
// iteration, to the caller's output in its dtype (transposed back when the
// input was tall).
template <typename OUT_T>
struct EpiNSApply32 {
  static constexpr bool kPreload = false;
  struct Args {
    MatArg x;      // fp32 iterate (read)
    MatArg xn;     // fp32 next iterate (written unless last)
    MatArg out;    // caller's output (written when last)
    float a;
    int last;
    int out_transposed;  // out is N x M
  };
  const float* x;
  float* xn;
  OUT_T* out;
  int64_t ldx, ldn, ldo;
  float a;
  bool last, out_t;
  __device__ EpiNSApply32(const Args& g, int bi, int)
      : x(static_cast<const float*>(g.x.p[bi])),
        xn(g.last ? nullptr : static_cast<float*>(const_cast<void*>(g.xn.p[bi]))),
        out(g.last ? static_cast<OUT_T*>(const_cast<void*>(g.out.p[bi])) : nullptr),
        ldx(g.x.ld), ldn(g.xn.ld), ldo(g.out.ld), a(g.a), last(g.last), out_t(g.out_transposed) {}
  __device__ __forceinline__ void apply(int row0, int col, int M, int N, float v0, float v1,
                                        float v2, float v3) {
    if (col >= N) return;
    const float v[4] = {v0, v1, v2, v3};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row = row0 + t;
      if (row >= M) continue;
      const float y = a * x[(int64_t)row * ldx + col] + v[t];
      if (!last) xn[(int64_t)row * ldn + col] = y;
      else if (out_t) store_from_f32<OUT_T>(out, (int64_t)col * ldo + row, y);
      else store_from_f32<OUT_T>(out, (int64_t)row * ldo + col, y);
    }
  }
};

// A result written straight to the caller's output in its dtype, transposed
// when out_transposed (Gram Newton-Schulz apply).
template <typename OUT_T>
struct EpiStoreOut {
  static constexpr bool kPreload = false;
  struct Args {
    MatArg out;
    int out_transposed;
  };
  OUT_T* out;
  int64_t ldo;
  bool out_t;
  __device__ EpiStoreOut(const Args& g, int bi, int)
      : out(static_cast<OUT_T*>(const_cast<void*>(g.out.p[bi]))), ldo(g.out.ld),
        out_t(g.out_transposed) {}
  __device__ __forceinline__ void apply(int row0, int col, int M, int N, float v0, float v1,
                                        float v2, float v3) {
    if (col >= N) return;
    const float v[4] = {v0, v1, v2, v3};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row = row0 + t;
      if (row >= M) continue;
      if (out_t) store_from_f32<OUT_T>(out, (int64_t)col * ldo + row, v[t]);
      else store_from_f32<OUT_T>(out, (int64_t)row * ldo + col, v[t]);
    }
  }
};

// Dion sweep 3 (fp32 weights): with B = M + G recomputed from the inputs,
//   M <- B - c1 * (P R^T),   X <- X - c2 * (P Q'^T)
// where c1 = 1 - mu and c2 = lr * scale.
template <typename XT>
struct EpiDion {
  static constexpr bool kPreload = false;
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

// Dion sweep 3 (bf16 weights) with the factors pre-scaled (R by c1, Q' by
// c2): the accumulators start at -(M + G) and -X, so after the products
// M' = -acc1 and X' = -acc2 (rounded to bf16); the epilogue only stores.
struct EpiDionPre {
  static constexpr bool kPreload = true;
  struct Args {
    MatArg m;  // fp32 momentum (read and written)
    MatArg g;  // bf16 gradient
    MatArg x;  // bf16 weight (read and written)
    float c1, c2;
  };
  float* m;
  const uint16_t* g;
  uint16_t* x;
  int64_t ldm, ldg, ldx;
  __device__ EpiDionPre(const Args& e, int bi, int)
      : m(static_cast<float*>(const_cast<void*>(e.m.p[bi]))),
        g(static_cast<const uint16_t*>(e.g.p[bi])),
        x(static_cast<uint16_t*>(const_cast<void*>(e.x.p[bi]))),
        ldm(e.m.ld), ldg(e.g.ld), ldx(e.x.ld) {}
  __device__ __forceinline__ void init2(int row0, int col, int M, int N, float* u, float* w) const {
    const int cc = min(col, N - 1);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row = row0 + t;
      const bool ok = col < N && row < M;
      const int64_t rr = min(row, M - 1);
      const float mv = m[rr * ldm + cc], gv = bf16_bits_to_f32(g[rr * ldg + cc]);
      const float xv = bf16_bits_to_f32(x[rr * ldx + cc]);
      u[t] = ok ? -(mv + gv) : 0.f;
      w[t] = ok ? -xv : 0.f;
    }
  }
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
      m[(int64_t)row * ldm + col] = -u[t];
      x[(int64_t)row * ldx + col] = to_bf16_bits(-w[t]);
    }
  }
};

// Dion update on the 256 x 256 kernel, bf16 weights, as two launches whose
// products P (c1 R)^T and P (c2 Q')^T arrive pre-scaled (bf16 operands):
//   momentum: accumulators start at -(M + G); M' = -acc = B - c1 P R^T;
//   weight:   accumulators start at -X;       X' = -acc = X - c2 P Q'^T,
//             rounded to bf16.
struct EpiDionFastM {
  static constexpr bool kPreload = false;
  struct Args {
    MatArg m;  // fp32 momentum (read and written)
    MatArg g;  // bf16 gradient
  };
  float* m;
  const uint16_t* g;
  int64_t ldm, ldg;
  __device__ EpiDionFastM(const Args& e, int bi, int)
      : m(static_cast<float*>(const_cast<void*>(e.m.p[bi]))),
        g(static_cast<const uint16_t*>(e.g.p[bi])), ldm(e.m.ld), ldg(e.g.ld) {}
  static constexpr int kFastPre = 2;
  static constexpr int kSegs = 1;
  static constexpr int kFastPre2 = 1;
  static constexpr bool kFastT = false;
  static constexpr bool kFastSym = false;
  __device__ const void* fast_pre_src() const { return m; }
  __device__ int64_t fast_pre_ld() const { return ldm; }
  __device__ float fast_pre_scale() const { return -1.f; }
  __device__ const void* fast_pre2_src() const { return g; }
  __device__ int64_t fast_pre2_ld() const { return ldg; }
  __device__ float fast_pre2_scale() const { return -1.f; }
  __device__ __forceinline__ void fast_store4(int row, int col, floatx4 v) {
    *reinterpret_cast<floatx4*>(m + (int64_t)row * ldm + col) = -v;
  }
  __device__ __forceinline__ void fast_store_t4(int, int, floatx4) {}
};

struct EpiDionFastX {
  static constexpr bool kPreload = false;
  struct Args {
    MatArg x;  // bf16 weight (read and written)
  };
  uint16_t* x;
  int64_t ldx;
  __device__ EpiDionFastX(const Args& e, int bi, int)
      : x(static_cast<uint16_t*>(const_cast<void*>(e.x.p[bi]))), ldx(e.x.ld) {}
  static constexpr int kFastPre = 1;
  static constexpr int kSegs = 1;
  static constexpr int kFastPre2 = 0;
  static constexpr bool kFastT = false;
  static constexpr bool kFastSym = false;
  __device__ const void* fast_pre_src() const { return x; }
  __device__ int64_t fast_pre_ld() const { return ldx; }
  __device__ float fast_pre_scale() const { return -1.f; }
  __device__ const void* fast_pre2_src() const { return nullptr; }
  __device__ int64_t fast_pre2_ld() const { return 0; }
  __device__ float fast_pre2_scale() const { return 0.f; }
  __device__ __forceinline__ void fast_store4(int row, int col, floatx4 v) {
    *reinterpret_cast<uint2*>(x + (int64_t)row * ldx + col) = pack_bf16x4(-v);
  }
  __device__ __forceinline__ void fast_store_t4(int, int, floatx4) {}
};

// fp32 store of C, or of split-K slice `split` of C, from the 256 x 256 kernel
// over bf16 pieces (kS segments: 3 for bf16x2 pieces, 6 for bf16x3 pieces).
template <int kS>
struct EpiFastSplitSegs {
  static constexpr bool kPreload = false;
  struct Args {
    MatArg c;              // destination, fp32 (ld a multiple of 4, 16-byte aligned)
    int64_t split_stride;  // elements between split-K slices
  };
  float* c;
  int64_t ld;
  __device__ EpiFastSplitSegs(const Args& a, int bi, int split)
      : c(static_cast<float*>(const_cast<void*>(a.c.p[bi])) + split * a.split_stride),
        ld(a.c.ld) {}
  static constexpr int kFastPre = 0;
  static constexpr int kSegs = kS;
  static constexpr int kFastPre2 = 0;
  static constexpr bool kFastT = false;
  static constexpr bool kFastSym = false;
  __device__ const void* fast_pre_src() const { return nullptr; }
  __device__ int64_t fast_pre_ld() const { return 0; }
  __device__ float fast_pre_scale() const { return 0.f; }
  __device__ const void* fast_pre2_src() const { return nullptr; }
  __device__ int64_t fast_pre2_ld() const { return 0; }
  __device__ float fast_pre2_scale() const { return 0.f; }
  __device__ __forceinline__ void fast_store4(int row, int col, floatx4 v) {
    *reinterpret_cast<floatx4*>(c + (int64_t)row * ld + col) = v;
  }
  __device__ __forceinline__ void fast_store_t4(int, int, floatx4) {}
};
using EpiFastSplitF32 = EpiFastSplitSegs<3>;   // bf16x3
using EpiFastSplit6F32 = EpiFastSplitSegs<6>;  // bf16x6

}  // namespace ortho


