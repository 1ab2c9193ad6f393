// Generic LDS-staged MFMA GEMM for gfx950:  C[i, j] = sum_k A[i, k] * Bop[j, k]
// ("NT" form: both operands are consumed with the reduction index k contiguous
// in LDS).  Loaders bring a tile of each operand from HBM into registers, turn
// it into one to three bf16 pieces (x = hi + lo + ...) and store it to LDS in the
// k-contiguous layout the MFMA fragments want; transposing loaders do the
// transpose in registers, so every global access stays row-coalesced.
//
// Products: PRODS = 1 uses hi*hi; PRODS = 2 (two pieces of the left operand,
// one of the right: a right operand that is exact in bf16) adds lo*hi;
// PRODS = 3 (two pieces, x = hi + lo) adds
// lo*hi and hi*lo, about 2^-16 relative accuracy; PRODS = 6 (three pieces
// x = p0 + p1 + p2) keeps every product p_i*q_j with i + j <= 2, about fp32
// accuracy.  NBOP = 2 runs two right operands against the same left tile with
// two accumulator sets.
//
// Matrix core: v_mfma_f32_32x32x16_bf16.  Each lane supplies eight consecutive
// k values of one row (lanes 0-31: k 0-7, lanes 32-63: k 8-15) for both A and
// Bop, so the pairing of k slots is identical for the two operands.  The fp32
// result of lane l, element e is row 8*(e/4) + 4*(l/32) + e%4, column l%32.
#pragma once

#include "common.h"

namespace ortho {

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int NA_, int NB_, int PRODS_,
          int NBOP_>
struct GemmCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NT = WAVES_M * WAVES_N * 64;
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  static constexpr int MI = WTM / 32, NI = WTN / 32;
  static constexpr int NA = NA_, NB = NB_, PRODS = PRODS_, NBOP = NBOP_;
  static constexpr int LDS_LD = BK + 8;  // bf16 elements per LDS row; +16 B breaks bank aliasing
  static constexpr int A_ELEMS = BM * LDS_LD;
  static constexpr int B_ELEMS = BN * LDS_LD;
  static constexpr int STAGE = NA * A_ELEMS + NBOP * NB * B_ELEMS;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(BK % 16 == 0, "BK must be a multiple of 16");
  static_assert(PRODS == 1 || (PRODS == 2 && NA == 2 && NB == 1) ||
                    (PRODS == 3 && NA == 2 && NB == 2) || (PRODS == 6 && NA == 3 && NB == 3),
                "bad product set");
};

// ---------------------------------------------------------------------------
// Loaders.  A loader instance owns one ROWS x BK tile of one operand.
// load(row0, k0, kend) issues the global loads for rows [row0, row0+ROWS) and
// k in [k0, k0+BK) (zero outside the matrix and for k >= kend); store() writes
// the NP bf16 pieces to LDS (piece p at s + p*pstride, row stride LDS_LD).
// ---------------------------------------------------------------------------

template <int NP>
__device__ __forceinline__ void put4(bf16* s, int pstride, float a, float b, float c, float d) {
  if constexpr (NP == 1) {
    bf16x4 h = {to_bf16(a), to_bf16(b), to_bf16(c), to_bf16(d)};
    *reinterpret_cast<bf16x4*>(s) = h;
  } else if constexpr (NP == 3) {
    const float x[4] = {a, b, c, d};
    bf16x4 p0, p1, p2;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bf16 h = to_bf16(x[t]);
      const float r1 = x[t] - static_cast<float>(h);   // exact
      const bf16 mid = to_bf16(r1);
      p0[t] = h;
      p1[t] = mid;
      p2[t] = to_bf16(r1 - static_cast<float>(mid));   // exact argument
    }
    *reinterpret_cast<bf16x4*>(s) = p0;
    *reinterpret_cast<bf16x4*>(s + pstride) = p1;
    *reinterpret_cast<bf16x4*>(s + 2 * pstride) = p2;
  } else {
    bf16 h0, h1, h2, h3, l0, l1, l2, l3;
    split_bf16(a, h0, l0);
    split_bf16(b, h1, l1);
    split_bf16(c, h2, l2);
    split_bf16(d, h3, l3);
    bf16x4 h = {h0, h1, h2, h3};
    bf16x4 l = {l0, l1, l2, l3};
    *reinterpret_cast<bf16x4*>(s) = h;
    *reinterpret_cast<bf16x4*>(s + pstride) = l;
  }
}

// Four consecutive elements as loaded, before any conversion (Raw4: fp32 as
// a float4, bf16 as the raw 8 bytes).  Loaders of one source keep this form
// until store(), with rows outside the matrix masked by a zero limit rather than a
// branch (measured: the triangular and correction applies of the
// orthonormalisation 29 -> 24 us and 28 -> 22 us at 4096 x 256).  Loaders that
// add two sources (M + G) add at load time: deferring that add to store()
// measured slower (Dion sweeps at 4096 x 4096, r = 256: 81 -> 101 us and
// 78 -> 89 us).

template <typename T>
__device__ __forceinline__ typename Raw4<T>::type load_raw4(const T* row, int c, int limit, bool vec);
template <>
__device__ __forceinline__ float4 load_raw4<float>(const float* row, int c, int limit, bool vec) {
  return load4<float>(row, c, limit, vec);
}
template <>
__device__ __forceinline__ uint2 load_raw4<uint16_t>(const uint16_t* row, int c, int limit, bool vec) {
  if (vec && c + 4 <= limit) return *reinterpret_cast<const uint2*>(row + c);
  uint16_t t[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) t[j] = (c + j < limit) ? row[c + j] : 0;
  return make_uint2(t[0] | (uint32_t(t[1]) << 16), t[2] | (uint32_t(t[3]) << 16));
}


// Row-major source, k contiguous: element (i, k) = S[i*ld + k].  The source
// is SRC_T (float or bf16 bits); with ADD = true the element is
// S[i*ld+k] + S2[i*ld2+k] (momentum plus gradient).
template <int ROWS, int BK, int NT, int NP, typename SRC_T, bool ADD, typename SRC2_T>
struct LdRow {
  static constexpr int CPR = BK / 4;
  static constexpr int NCH = ROWS * CPR / NT;
  static_assert(ROWS * CPR % NT == 0, "tile does not divide among threads");
  const SRC_T* p;
  const SRC2_T* p2;
  int64_t ld, ld2;
  int rows;
  bool vec;
  typename Raw4<SRC_T>::type v[ADD ? 1 : NCH];
  float4 vs[ADD ? NCH : 1];   // M + G

  __device__ LdRow(const MatArg& a, const MatArg& a2, int bi)
      : p(static_cast<const SRC_T*>(a.p[bi])),
        p2(ADD ? static_cast<const SRC2_T*>(a2.p[bi]) : nullptr),
        ld(a.ld), ld2(a2.ld), rows(a.rows), vec(a.vec && (!ADD || a2.vec)) {}

  // Without ADD, rows past the end load nothing: every column index is then
  // past the zero limit.  A tile wholly inside the source (a uniform test)
  // takes plain vector loads: with the per-lane choice between the vector and
  // the element-wise path, both ran under exec masks and each vector load
  // waited for every load before it.
  __device__ __forceinline__ void load(int row0, int k0, int kend) {
    if (vec && row0 + ROWS <= rows && k0 + BK <= kend) {
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int idx = threadIdx.x + c * NT;
        const int r = idx / CPR, kc = (idx % CPR) * 4;
        const SRC_T* src = p + (int64_t)(row0 + r) * ld + k0 + kc;
        if constexpr (ADD) {
          const float4 mv = raw_to_f4(*reinterpret_cast<const typename Raw4<SRC_T>::type*>(src));
          const float4 g = raw_to_f4(*reinterpret_cast<const typename Raw4<SRC2_T>::type*>(
              p2 + (int64_t)(row0 + r) * ld2 + k0 + kc));
          vs[c] = make_float4(mv.x + g.x, mv.y + g.y, mv.z + g.z, mv.w + g.w);
        } else {
          v[c] = *reinterpret_cast<const typename Raw4<SRC_T>::type*>(src);
        }
      }
      return;
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int idx = threadIdx.x + c * NT;
      const int r = idx / CPR, kc = (idx % CPR) * 4;
      const int gr = row0 + r;
      const bool in = gr < rows;
      const int grc = in ? gr : 0;
      if constexpr (ADD) {
        if (in) {
          vs[c] = load4<SRC_T>(p + gr * ld, k0 + kc, kend, vec);
          const float4 g = load4<SRC2_T>(p2 + gr * ld2, k0 + kc, kend, vec);
          vs[c].x += g.x; vs[c].y += g.y; vs[c].z += g.z; vs[c].w += g.w;
        } else {
          vs[c] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      } else {
        v[c] = load_raw4<SRC_T>(p + grc * ld, k0 + kc, in ? kend : 0, vec);
      }
    }
  }

  template <int LDS_LD>
  __device__ __forceinline__ void store(bf16* s, int pstride) const {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int idx = threadIdx.x + c * NT;
      const int r = idx / CPR, kc = (idx % CPR) * 4;
      float4 x;
      if constexpr (ADD) x = vs[c];
      else x = raw_to_f4(v[c]);
      put4<NP>(s + r * LDS_LD + kc, pstride, x.x, x.y, x.z, x.w);
    }
  }
};

// Row-major bf16 source used as-is (one piece), 8 elements per access.
template <int ROWS, int BK, int NT>
struct LdRowBf16 {
  static constexpr int CPR = BK / 8;
  static constexpr int NCH = ROWS * CPR / NT;
  static_assert(ROWS * CPR % NT == 0, "tile does not divide among threads");
  const uint16_t* p;
  int64_t ld;
  int rows;
  bool vec;
  uint4 v[NCH];

  __device__ LdRowBf16(const MatArg& a, const MatArg&, int bi)
      : p(static_cast<const uint16_t*>(a.p[bi])), ld(a.ld), rows(a.rows), vec(a.vec) {}

  __device__ __forceinline__ void load(int row0, int k0, int kend) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int idx = threadIdx.x + c * NT;
      const int r = idx / CPR, kc = (idx % CPR) * 8;
      const int gr = row0 + r, gk = k0 + kc;
      if (gr < rows && vec && gk + 8 <= kend) {
        v[c] = *reinterpret_cast<const uint4*>(p + gr * ld + gk);
      } else {
        uint16_t t[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) t[j] = (gr < rows && gk + j < kend) ? p[gr * ld + gk + j] : 0;
        v[c] = make_uint4(t[0] | (uint32_t(t[1]) << 16), t[2] | (uint32_t(t[3]) << 16),
                          t[4] | (uint32_t(t[5]) << 16), t[6] | (uint32_t(t[7]) << 16));
      }
    }
  }

  template <int LDS_LD>
  __device__ __forceinline__ void store(bf16* s, int) const {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int idx = threadIdx.x + c * NT;
      const int r = idx / CPR, kc = (idx % CPR) * 8;
      *reinterpret_cast<uint4*>(s + r * LDS_LD + kc) = v[c];
    }
  }
};

// Transposing loader: element (j, k) of the operand is S[k*ld + j] (the source
// is stored with j contiguous).  Each thread reads a 4(k) x 4(j) block with
// row-coalesced loads and writes it transposed to LDS.  `rows` is the j extent.
template <int ROWS, int BK, int NT, int NP, typename SRC_T, bool ADD, typename SRC2_T>
struct LdCol {
  static constexpr int JC = ROWS / 4, KC = BK / 4;
  static constexpr int NCH = JC * KC / NT;
  static_assert(JC * KC % NT == 0, "tile does not divide among threads");
  const SRC_T* p;
  const SRC2_T* p2;
  int64_t ld, ld2;
  int rows;
  bool vec;
  typename Raw4<SRC_T>::type v[ADD ? 1 : NCH][4];
  float4 vs[ADD ? NCH : 1][4];   // M + G

  __device__ LdCol(const MatArg& a, const MatArg& a2, int bi)
      : p(static_cast<const SRC_T*>(a.p[bi])),
        p2(ADD ? static_cast<const SRC2_T*>(a2.p[bi]) : nullptr),
        ld(a.ld), ld2(a2.ld), rows(a.rows), vec(a.vec && (!ADD || a2.vec)) {}

  // Without ADD, source rows past kend load nothing: every column index is
  // then past the zero limit.  A tile wholly inside the source takes plain
  // vector loads (as in LdRow).
  __device__ __forceinline__ void load(int row0, int k0, int kend) {
    if (vec && row0 + ROWS <= rows && k0 + BK <= kend) {
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int idx = threadIdx.x + c * NT;
        const int jc = (idx % JC) * 4, kc = (idx / JC) * 4;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int64_t gk = k0 + kc + t;
          const SRC_T* src = p + gk * ld + row0 + jc;
          if constexpr (ADD) {
            const float4 mv = raw_to_f4(*reinterpret_cast<const typename Raw4<SRC_T>::type*>(src));
            const float4 g = raw_to_f4(
                *reinterpret_cast<const typename Raw4<SRC2_T>::type*>(p2 + gk * ld2 + row0 + jc));
            vs[c][t] = make_float4(mv.x + g.x, mv.y + g.y, mv.z + g.z, mv.w + g.w);
          } else {
            v[c][t] = *reinterpret_cast<const typename Raw4<SRC_T>::type*>(src);
          }
        }
      }
      return;
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int idx = threadIdx.x + c * NT;
      const int jc = (idx % JC) * 4, kc = (idx / JC) * 4;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int gk = k0 + kc + t;
        const bool in = gk < kend;
        const int gkc = in ? gk : 0;
        if constexpr (ADD) {
          if (in) {
            vs[c][t] = load4<SRC_T>(p + gk * ld, row0 + jc, rows, vec);
            const float4 g = load4<SRC2_T>(p2 + gk * ld2, row0 + jc, rows, vec);
            vs[c][t].x += g.x; vs[c][t].y += g.y; vs[c][t].z += g.z; vs[c][t].w += g.w;
          } else {
            vs[c][t] = make_float4(0.f, 0.f, 0.f, 0.f);
          }
        } else {
          v[c][t] = load_raw4<SRC_T>(p + gkc * ld, row0 + jc, in ? rows : 0, vec);
        }
      }
    }
  }

  template <int LDS_LD>
  __device__ __forceinline__ void store(bf16* s, int pstride) const {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int idx = threadIdx.x + c * NT;
      const int jc = (idx % JC) * 4, kc = (idx / JC) * 4;
      float4 x[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if constexpr (ADD) x[t] = vs[c][t];
        else x[t] = raw_to_f4(v[c][t]);
      }
      put4<NP>(s + (jc + 0) * LDS_LD + kc, pstride, x[0].x, x[1].x, x[2].x, x[3].x);
      put4<NP>(s + (jc + 1) * LDS_LD + kc, pstride, x[0].y, x[1].y, x[2].y, x[3].y);
      put4<NP>(s + (jc + 2) * LDS_LD + kc, pstride, x[0].z, x[1].z, x[2].z, x[3].z);
      put4<NP>(s + (jc + 3) * LDS_LD + kc, pstride, x[0].w, x[1].w, x[2].w, x[3].w);
    }
  }
};

// ---------------------------------------------------------------------------
// Kernel parameters and body
// ---------------------------------------------------------------------------

template <typename EpiArgs>
struct GemmParams {
  MatArg a, a2;      // left operand (a2: second source when the loader adds two)
  MatArg b0, b0s;    // right operand 0 (b0s: second source)
  MatArg b1, b1s;    // right operand 1 (NBOP = 2 only)
  EpiArgs e;
  int M, N, K;       // C is M x N, reduction length K
  int tiles_n;       // column tiles
  int splits;        // split-K factor (blockIdx.y = member * splits + split)
  int kchunk;        // k range per split, a multiple of BK
  int tri;           // right operand is zero for k > j (triangular factor)
  int sym;           // 256x256 kernel: C symmetric, upper tiles only (mirrored on store)
  MatArg a3, b0t;    // 256x256 kernel, six k segments: third pieces of A and B
};

template <class Cfg, class LA, class LB, class Epi>
__global__ __launch_bounds__(Cfg::NT) void gemm_kernel(GemmParams<typename Epi::Args> p) {
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * Cfg::STAGE];
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, LDS_LD = Cfg::LDS_LD;
  constexpr int MI = Cfg::MI, NI = Cfg::NI, NBOP = Cfg::NBOP;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;

  // Consecutive workgroup ids go round-robin over the 8 XCDs; give each XCD a
  // contiguous run of tiles so that neighbouring tiles share its L2.
  int bid = blockIdx.x;
  const int nwg = gridDim.x;
  if ((nwg & 7) == 0) bid = (bid & 7) * (nwg >> 3) + (bid >> 3);
  const int tm = bid / p.tiles_n, tn = bid % p.tiles_n;
  const int bi = blockIdx.y / p.splits, split = blockIdx.y % p.splits;
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbeg = split * p.kchunk;
  int kend = min(p.K, kbeg + p.kchunk);
  if (p.tri) kend = min(kend, n0 + BN);
  const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

  floatx16 acc[NBOP][MI][NI];
#pragma unroll
  for (int q = 0; q < NBOP; ++q)
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[q][i][j][e] = 0.f;

  Epi epi(p.e, bi, split);
  if constexpr (Epi::kPreload) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int row0 = m0 + wm * Cfg::WTM + i * 32 + g * 8 + (lane >> 5) * 4;
          const int col = n0 + wn * Cfg::WTN + j * 32 + (lane & 31);
          float u[4], w[4];
          if constexpr (NBOP == 1) {
            epi.init(row0, col, p.M, p.N, u);
          } else {
            epi.init2(row0, col, p.M, p.N, u, w);
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[NBOP - 1][i][j][g * 4 + t] = w[t];
          }
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[0][i][j][g * 4 + t] = u[t];
        }
  }

  LA la(p.a, p.a2, bi);
  LB lb0(p.b0, p.b0s, bi);
  LB lb1(NBOP == 2 ? p.b1 : p.b0, NBOP == 2 ? p.b1s : p.b0s, bi);

  auto stage_a = [&](int s) { return smem + s * Cfg::STAGE; };
  auto stage_b = [&](int s, int q) {
    return smem + s * Cfg::STAGE + Cfg::NA * Cfg::A_ELEMS + q * Cfg::NB * Cfg::B_ELEMS;
  };

  if (nk > 0) {
    la.load(m0, kbeg, kend);
    lb0.load(n0, kbeg, kend);
    if constexpr (NBOP == 2) lb1.load(n0, kbeg, kend);
    la.template store<LDS_LD>(stage_a(0), Cfg::A_ELEMS);
    lb0.template store<LDS_LD>(stage_b(0, 0), Cfg::B_ELEMS);
    if constexpr (NBOP == 2) lb1.template store<LDS_LD>(stage_b(0, 1), Cfg::B_ELEMS);
  }

  const int frag_row = lane & 31;
  const int frag_k = (lane >> 5) * 8;

  // products of one LDS stage into the accumulators
  // Products of one LDS stage into the accumulators.  The fragments of the
  // next 16-deep k step are read before this step's products are issued
  // (two fragment sets, indices fixed by the full unroll), so the LDS reads'
  // latency sits under the matrix-core work instead of in front of it.
  auto compute = [&](int cur) {
    const bf16* sa = stage_a(cur);
    constexpr int KS = BK / 16;
    bf16x8 af[2][Cfg::NA][MI];
    bf16x8 bfr[2][NBOP][Cfg::NB][NI];
#pragma unroll
    for (int t = -1; t < KS; ++t) {
      if (t + 1 < KS) {
        const int nb = (t + 1) & 1, kk = (t + 1) * 16;
#pragma unroll
        for (int pa = 0; pa < Cfg::NA; ++pa)
#pragma unroll
          for (int i = 0; i < MI; ++i)
            af[nb][pa][i] = *reinterpret_cast<const bf16x8*>(
                sa + pa * Cfg::A_ELEMS + (wm * Cfg::WTM + i * 32 + frag_row) * LDS_LD + kk + frag_k);
#pragma unroll
        for (int q = 0; q < NBOP; ++q) {
          const bf16* sb = stage_b(cur, q);
#pragma unroll
          for (int pb = 0; pb < Cfg::NB; ++pb)
#pragma unroll
            for (int j = 0; j < NI; ++j)
              bfr[nb][q][pb][j] = *reinterpret_cast<const bf16x8*>(
                  sb + pb * Cfg::B_ELEMS + (wn * Cfg::WTN + j * 32 + frag_row) * LDS_LD + kk + frag_k);
        }
      }
      if (t < 0) continue;
      const int b = t & 1;
#pragma unroll
      for (int q = 0; q < NBOP; ++q)
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NI; ++j) {
            if constexpr (Cfg::PRODS == 6) {
              acc[q][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[b][2][i], bfr[b][q][0][j], acc[q][i][j], 0, 0, 0);
              acc[q][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[b][1][i], bfr[b][q][1][j], acc[q][i][j], 0, 0, 0);
              acc[q][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[b][0][i], bfr[b][q][2][j], acc[q][i][j], 0, 0, 0);
            }
            if constexpr (Cfg::PRODS >= 3) {
              acc[q][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[b][1][i], bfr[b][q][0][j], acc[q][i][j], 0, 0, 0);
              acc[q][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[b][0][i], bfr[b][q][1][j], acc[q][i][j], 0, 0, 0);
            }
            if constexpr (Cfg::PRODS == 2)
              acc[q][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[b][1][i], bfr[b][q][0][j], acc[q][i][j], 0, 0, 0);
            acc[q][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[b][0][i], bfr[b][q][0][j], acc[q][i][j], 0, 0, 0);
          }
    }
  };

  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int kn = kbeg + (kt + 1) * BK;
      la.load(m0, kn, kend);
      lb0.load(n0, kn, kend);
      if constexpr (NBOP == 2) lb1.load(n0, kn, kend);
    }
    compute(cur);
    if (more) {
      const int nxt = cur ^ 1;
      la.template store<LDS_LD>(stage_a(nxt), Cfg::A_ELEMS);
      lb0.template store<LDS_LD>(stage_b(nxt, 0), Cfg::B_ELEMS);
      if constexpr (NBOP == 2) lb1.template store<LDS_LD>(stage_b(nxt, 1), Cfg::B_ELEMS);
    }
  }

  // Epilogue: hand each lane's four consecutive rows of one column to the
  // policy, which applies bounds and writes.
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int row0 = m0 + wm * Cfg::WTM + i * 32 + g * 8 + (lane >> 5) * 4;
        const int col = n0 + wn * Cfg::WTN + j * 32 + (lane & 31);
        if constexpr (NBOP == 1) {
          epi.apply(row0, col, p.M, p.N, acc[0][i][j][g * 4 + 0], acc[0][i][j][g * 4 + 1],
                    acc[0][i][j][g * 4 + 2], acc[0][i][j][g * 4 + 3]);
        } else {
          epi.apply2(row0, col, p.M, p.N, acc[0][i][j][g * 4 + 0], acc[0][i][j][g * 4 + 1],
                     acc[0][i][j][g * 4 + 2], acc[0][i][j][g * 4 + 3], acc[1][i][j][g * 4 + 0],
                     acc[1][i][j][g * 4 + 1], acc[1][i][j][g * 4 + 2], acc[1][i][j][g * 4 + 3]);
        }
      }
}

}  // namespace ortho
