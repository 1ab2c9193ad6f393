// Instantiations of the MFMA GEMM core for every contraction of the Dion and
// Newton-Schulz paths, and their host launchers.
#include "epilogues.h"
#include "gemm_core.h"
#include "gemm_fast.h"
#include "gemm_sym.h"
#include "launch.h"
#include "plan.h"

namespace ortho {

namespace {

inline int cdiv(int64_t a, int64_t b) { return static_cast<int>((a + b - 1) / b); }

template <class Cfg, class LA, class LB, class Epi>
hipError_t run(GemmParams<typename Epi::Args>& p, int members, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0 || members <= 0) return hipSuccess;
  const int tm = cdiv(p.M, Cfg::BM), tn = cdiv(p.N, Cfg::BN);
  p.tiles_n = tn;
  if (p.splits < 1) p.splits = 1;
  if (p.kchunk <= 0) p.kchunk = cdiv(p.K, Cfg::BK) * Cfg::BK;
  dim3 grid(tm * tn, members * p.splits);
  hipLaunchKernelGGL((gemm_kernel<Cfg, LA, LB, Epi>), grid, dim3(Cfg::NT), 0, s, p);
  return hipGetLastError();
}

MatArg with_rows(MatArg a, int rows) {
  a.rows = rows;
  return a;
}

// Tall-skinny Dion contractions: 128 x 128 tiles, 4 waves, two bf16 pieces per
// operand and three products (hi*hi + lo*hi + hi*lo).
using CfgSplit = GemmCfg<128, 128, 32, 2, 2, 2, 2, 3, 1>;
// The same with three pieces and six products (fp32-level products).
using CfgSplit6 = GemmCfg<128, 128, 32, 2, 2, 3, 3, 6, 1>;
// Dion sweep 3 with bf16 weights: one product from pre-converted bf16 factors,
// two right operands, 256 x 128 tiles with 8 waves.
using CfgUpdBf = GemmCfg<256, 128, 32, 4, 2, 1, 1, 1, 2>;
// Dion sweep 3 with fp32 weights: split products, two right operands.
using CfgUpdF32 = GemmCfg<128, 128, 32, 2, 2, 2, 2, 3, 2>;
// Newton-Schulz: 256 x 256 tiles with 8 waves for large matrices, 128 x 128
// with 4 waves when the Gram side is small.
using CfgNsBig = GemmCfg<256, 256, 32, 2, 4, 1, 1, 1, 1>;
using CfgNsSmall = GemmCfg<128, 128, 32, 2, 2, 1, 1, 1, 1>;

template <int ROWS, int NT, int NP>
using RowF32 = LdRow<ROWS, 32, NT, NP, float, false, float>;
template <int ROWS, int NT, int NP, typename GT>
using RowMG = LdRow<ROWS, 32, NT, NP, float, true, GT>;
template <int ROWS, int NT, int NP>
using ColF32 = LdCol<ROWS, 32, NT, NP, float, false, float>;
template <int ROWS, int NT, int NP, typename GT>
using ColMG = LdCol<ROWS, 32, NT, NP, float, true, GT>;

// Few output tiles (few_tiles): 64 x 64 tiles, k 64 deep (the column
// loader's minimum for 64 rows), NP bf16 pieces per operand.
template <int NP>
using CfgSmall = GemmCfg<64, 64, 64, 2, 2, NP, NP, NP == 3 ? 6 : 3, 1>;

template <typename GT, class Cfg, int NP>
hipError_t dion_left_t(const DionLeftArgs& a, int members, hipStream_t s) {
  GemmParams<EpiStoreF32::Args> p{};
  p.a = with_rows(a.m, a.M);
  p.a2 = with_rows(a.g, a.M);
  p.b0 = with_rows(a.q, a.r);  // element (j, k) = Q[k][j]
  p.e.c = a.out;
  p.e.split_stride = a.splits > 1 ? a.split_stride : 0;
  p.e.has_t = 0;
  p.M = a.M; p.N = a.r; p.K = a.N;
  p.splits = a.splits; p.kchunk = a.kchunk; p.tri = 0;
  if (a.small && a.kchunk % 64 == 0)
    return run<CfgSmall<NP>, LdRow<64, 64, 256, NP, float, true, GT>,
               LdCol<64, 64, 256, NP, float, false, float>, EpiStoreF32>(p, members, s);
  return run<Cfg, RowMG<128, 256, NP, GT>, ColF32<128, 256, NP>, EpiStoreF32>(p, members, s);
}

template <typename GT, class Cfg, int NP>
hipError_t dion_right_t(const DionRightArgs& a, int members, hipStream_t s) {
  GemmParams<EpiStoreF32::Args> p{};
  p.a = with_rows(a.m, a.N);   // element (j, i) = M[i][j] + G[i][j]
  p.a2 = with_rows(a.g, a.N);
  p.b0 = with_rows(a.p, a.r);  // element (k, i) = P[i][k]
  p.e.c = a.out;
  p.e.split_stride = a.splits > 1 ? a.split_stride : 0;
  p.e.has_t = 0;
  p.M = a.N; p.N = a.r; p.K = a.M;
  p.splits = a.splits; p.kchunk = a.kchunk; p.tri = 0;
  if (a.small && a.kchunk % 64 == 0)
    return run<CfgSmall<NP>, LdCol<64, 64, 256, NP, float, true, GT>,
               LdCol<64, 64, 256, NP, float, false, float>, EpiStoreF32>(p, members, s);
  return run<Cfg, ColMG<128, 256, NP, GT>, ColF32<128, 256, NP>, EpiStoreF32>(p, members, s);
}

hipError_t dion_update_f32(const DionUpdateArgs& a, int members, hipStream_t s) {
  GemmParams<typename EpiDion<float>::Args> p{};
  p.a = with_rows(a.p, a.M);
  p.b0 = with_rows(a.r, a.N);
  p.b1 = with_rows(a.q, a.N);
  p.e.m = a.m; p.e.g = a.g; p.e.x = a.x;
  p.e.c1 = a.c1; p.e.c2 = a.c2;
  p.M = a.M; p.N = a.N; p.K = a.rank;
  p.splits = 1; p.kchunk = 0; p.tri = 0;
  if (few_tiles(a.M, a.N, members))
    return run<GemmCfg<64, 64, 32, 2, 2, 2, 2, 3, 2>, RowF32<64, 256, 2>, RowF32<64, 256, 2>,
               EpiDion<float>>(p, members, s);
  return run<CfgUpdF32, RowF32<128, 256, 2>, RowF32<128, 256, 2>, EpiDion<float>>(p, members, s);
}

bool fast_ok(int M, int N, int K, const MatArg& a, const MatArg& b);
template <class Epi>
hipError_t run_fast(GemmParams<typename Epi::Args>& p, int members, hipStream_t s);

// Every member's rows start on 16-byte boundaries (direct-to-LDS copies).
static bool rows16(const MatArg& t, int members, size_t esz) {
  if ((static_cast<size_t>(t.ld) * esz) % 16 != 0) return false;
  for (int i = 0; i < members; ++i)
    if (reinterpret_cast<uintptr_t>(t.p[i]) % 16 != 0) return false;
  return true;
}

hipError_t dion_update_bf16(const DionUpdateArgs& a, int members, hipStream_t s) {
  // r = 512 with P in fragment order: the streaming kernel
  if (a.rank == 512 && a.has_pf && dion_update_stream_ok(a, members))
    return launch_dion_update_stream(a, members, s);
  // From r = 768 on (and at r = 512 without the fragment-order P) the products
  // weigh enough that the 256 x 256 pair is the fastest (12-layer GPT groups at
  // r = 512: 15.7 ms per step against 16.5 with the streaming kernel reading P
  // row by row; 15.1 against 15.4 once it read the fragment-order copy); at
  // r = 256 the step is bound by its 14 mn bytes and the streaming kernel
  // (memory terms loaded under the products, 16-byte accesses) is; the
  // two-accumulator 256 x 128 kernel takes every other case.
  if (a.rank >= 512 && fast_ok(a.M, a.N, a.rank, a.pb, a.rb) && a.qb.vec && a.qb.ld % 8 == 0 &&
      rows16(a.m, members, 4) && rows16(a.g, members, 2) && rows16(a.x, members, 2)) {
    // two launches of the 256 x 256 kernel: momentum, then weight
    GemmParams<EpiDionFastM::Args> pm{};
    pm.a = with_rows(a.pb, a.M);
    pm.b0 = with_rows(a.rb, a.N);
    pm.e.m = a.m; pm.e.g = a.g;
    pm.M = a.M; pm.N = a.N; pm.K = a.rank;
    hipError_t e = run_fast<EpiDionFastM>(pm, members, s);
    if (e != hipSuccess) return e;
    GemmParams<EpiDionFastX::Args> px{};
    px.a = with_rows(a.pb, a.M);
    px.b0 = with_rows(a.qb, a.N);
    px.e.x = a.x;
    px.M = a.M; px.N = a.N; px.K = a.rank;
    return run_fast<EpiDionFastX>(px, members, s);
  }
  if (dion_update_stream_ok(a, members)) return launch_dion_update_stream(a, members, s);
  GemmParams<EpiDionPre::Args> p{};
  p.a = with_rows(a.pb, a.M);
  p.b0 = with_rows(a.rb, a.N);
  p.b1 = with_rows(a.qb, a.N);
  p.e.m = a.m; p.e.g = a.g; p.e.x = a.x;
  p.e.c1 = 1.0f; p.e.c2 = 1.0f;   // factors arrive pre-scaled
  p.M = a.M; p.N = a.N; p.K = a.rank;
  p.splits = 1; p.kchunk = 0; p.tri = 0;
  return run<CfgUpdBf, LdRowBf16<256, 32, 512>, LdRowBf16<128, 32, 512>, EpiDionPre>(p, members, s);
}

template <class Cfg>
using NsRow = LdRowBf16<Cfg::BM, Cfg::BK, Cfg::NT>;

// The 256 x 256 x 64 direct-to-LDS kernel applies when the product tiles
// exactly, every operand row is 16-byte aligned and a 256-row block of an
// operand spans less than 2 GiB (per-lane 32-bit load offsets).
bool fast_ok(int M, int N, int K, const MatArg& a, const MatArg& b) {
  return M % 256 == 0 && N % 256 == 0 && K % 64 == 0 && a.vec && b.vec && a.ld % 8 == 0 &&
         b.ld % 8 == 0 && a.ld <= (int64_t{1} << 22) && b.ld <= (int64_t{1} << 22);
}

template <class Epi>
hipError_t run_fast(GemmParams<typename Epi::Args>& p, int members, hipStream_t s) {
  // every piece shares the first piece's row stride
  if (Epi::kSegs > 1 && (p.a2.ld != p.a.ld || p.b0s.ld != p.b0.ld)) return hipErrorInvalidValue;
  if (Epi::kSegs == 6 && (p.a3.ld != p.a.ld || p.b0t.ld != p.b0.ld)) return hipErrorInvalidValue;
  if (p.a.ld > (int64_t{1} << 22) || p.b0.ld > (int64_t{1} << 22)) return hipErrorInvalidValue;
  p.tiles_n = p.N / 256;
  if (p.splits < 1 || p.kchunk < 1) {  // one slice over every k tile
    p.splits = 1;
    p.kchunk = (p.K / 64) * Epi::kSegs;
  }
  // symmetric results (Gram, polynomial): tiles on and above the diagonal
  if (p.sym && (!Epi::kFastSym || p.M != p.N)) return hipErrorInvalidValue;
  const int tiles = p.sym ? p.tiles_n * (p.tiles_n + 1) / 2 : (p.M / 256) * p.tiles_n;
  dim3 grid(tiles, members * p.splits);
  hipLaunchKernelGGL((gemm_bf16_256<Epi>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

// Symmetric products (Gram, polynomial) on the 256 x 256 grid's T^2
// equal-work workgroups (gemm_sym.h): M = N, the conditions of fast_ok.
template <class Epi>
hipError_t run_sym(GemmParams<typename Epi::Args>& p, int members, hipStream_t s) {
  if (p.M != p.N || p.M % 256 != 0 || p.K % 64 != 0 || p.K < 64) return hipErrorInvalidValue;
  p.tiles_n = p.M / 256;
  p.splits = 1;
  dim3 grid(p.tiles_n * p.tiles_n, members);
  hipLaunchKernelGGL((gemm_bf16_sym<Epi>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

// Newton-Schulz products whose 256 x 256 grid (upper tiles for the symmetric
// ones) would give fewer than 128 workgroups over a launch's members run on
// the 128 x 128 kernel instead: four times the workgroups (full tiles, so the
// symmetric products compute both halves).
// 64 deep in k: 16 products per wave cover each tile's loads, and at 73 KB of
// LDS and 150 registers two workgroups share a CU.
using CfgNsMid = GemmCfg<128, 128, 64, 2, 2, 1, 1, 1, 1>;

inline bool ns_few_fast_tiles(int M, int N, int members, bool sym) {
  const int64_t tm = (M + 255) / 256, tn = (N + 255) / 256;
  const int64_t tiles = sym ? tm * (tm + 1) / 2 : tm * tn;
  return tiles * members < 128;
}

template <class Cfg>
hipError_t ns_gram_t(const NsGramArgs& a, int members, hipStream_t s) {
  GemmParams<EpiNSGram::Args> p{};
  p.a = with_rows(a.x, a.M);
  p.b0 = with_rows(a.x, a.M);
  p.e.a = a.a;
  p.M = a.M; p.N = a.M; p.K = a.K;
  p.splits = 1; p.kchunk = 0; p.tri = 0;
  if (ns_few_fast_tiles(a.M, a.M, members, true))
    return run<CfgNsMid, NsRow<CfgNsMid>, NsRow<CfgNsMid>, EpiNSGram>(p, members, s);
  if (fast_ok(p.M, p.N, p.K, p.a, p.b0) && p.K >= 64) return run_sym<EpiNSGram>(p, members, s);  // X X^T
  return run<Cfg, NsRow<Cfg>, NsRow<Cfg>, EpiNSGram>(p, members, s);
}

template <class Cfg>
hipError_t ns_poly_t(const NsPolyArgs& a, int members, hipStream_t s) {
  GemmParams<EpiNSPoly::Args> p{};
  p.a = with_rows(a.a, a.M);
  p.b0 = with_rows(a.a, a.M);   // A is symmetric: A A = A A^T
  p.e.a = a.a; p.e.bp = a.bp; p.e.bp32 = a.bp32; p.e.b = a.b; p.e.c = a.c;
  p.e.has32 = a.M <= kNsSplitRows;
  p.M = a.M; p.N = a.M; p.K = a.M;
  p.splits = 1; p.kchunk = 0; p.tri = 0;
  if (ns_few_fast_tiles(a.M, a.M, members, true))
    return run<CfgNsMid, NsRow<CfgNsMid>, NsRow<CfgNsMid>, EpiNSPoly>(p, members, s);
  // b A + c A A is symmetric with A
  if (fast_ok(p.M, p.N, p.K, p.a, p.b0) && p.K >= 64) return run_sym<EpiNSPoly>(p, members, s);
  return run<Cfg, NsRow<Cfg>, NsRow<Cfg>, EpiNSPoly>(p, members, s);
}

template <class Cfg, typename OUT_T>
hipError_t ns_apply_t(const NsApplyArgs& a, int members, hipStream_t s) {
  GemmParams<typename EpiNSApply<OUT_T>::Args> p{};
  p.a = with_rows(a.bp, a.M);
  p.b0 = with_rows(a.xbt, a.N);   // element (j, k) = X^T[j][k] = X[k][j]
  p.e.x32 = a.x32; p.e.xb = a.xb_next; p.e.xbt = a.xbt_next; p.e.out = a.out;
  p.e.a = a.a; p.e.last = a.last; p.e.out_transposed = a.out_transposed;
  p.M = a.M; p.N = a.N; p.K = a.M;
  p.splits = 1; p.kchunk = 0; p.tri = 0;
  if (ns_few_fast_tiles(a.M, a.N, members, false))
    return run<CfgNsMid, NsRow<CfgNsMid>, NsRow<CfgNsMid>, EpiNSApply<OUT_T>>(p, members, s);
  if (fast_ok(p.M, p.N, p.K, p.a, p.b0)) return run_fast<EpiNSApply<OUT_T>>(p, members, s);
  return run<Cfg, NsRow<Cfg>, NsRow<Cfg>, EpiNSApply<OUT_T>>(p, members, s);
}

// Small Gram side: split bf16 products from the fp32 Bp and the fp32 iterate
// (read transposed: element (j, k) = X[k][j]).
template <typename OUT_T>
hipError_t ns_apply_split_t(const NsApplyArgs& a, int members, hipStream_t s) {
  GemmParams<typename EpiNSApply<OUT_T>::Args> p{};
  p.a = with_rows(a.bp32, a.M);
  p.b0 = with_rows(a.x32, a.N);
  p.e.x32 = a.x32; p.e.xb = a.xb_next; p.e.xbt = a.xbt_next; p.e.out = a.out;
  p.e.a = a.a; p.e.last = a.last; p.e.out_transposed = a.out_transposed;
  p.M = a.M; p.N = a.N; p.K = a.M;
  p.splits = 1; p.kchunk = 0; p.tri = 0;
  return run<CfgSplit, RowF32<128, 256, 2>, ColF32<128, 256, 2>, EpiNSApply<OUT_T>>(p, members, s);
}

}  // namespace

// bf16 weights: bf16x3 sweeps.  fp32 weights: bf16x6 sweeps.
hipError_t launch_dion_left(const DionLeftArgs& a, bool bf16, int members, hipStream_t s) {
  return bf16 ? dion_left_t<uint16_t, CfgSplit, 2>(a, members, s)
              : dion_left_t<float, CfgSplit6, 3>(a, members, s);
}

hipError_t launch_dion_right(const DionRightArgs& a, bool bf16, int members, hipStream_t s) {
  return bf16 ? dion_right_t<uint16_t, CfgSplit, 2>(a, members, s)
              : dion_right_t<float, CfgSplit6, 3>(a, members, s);
}

// The orthonormalisation products of a small rank (r < 512) have few 128 x 128
// tiles (m = 4096, r = 256: 64 output tiles, 4 for P1^T P1); 64 x 64 tiles,
// four waves of 32 x 32, give the chip four times the workgroups.
using CfgSplit6S = GemmCfg<64, 64, 32, 2, 2, 3, 3, 6, 1>;
using CfgSplitS = GemmCfg<64, 64, 32, 2, 2, 2, 2, 3, 1>;
using CfgSplitS64 = GemmCfg<64, 64, 64, 2, 2, 2, 2, 3, 1>;   // k 64 deep: the column loader's minimum

hipError_t launch_apply_t(const ApplyArgs& a, bool six_products, int members, hipStream_t s) {
  GemmParams<EpiStoreF32::Args> p{};
  p.a = with_rows(a.pt, a.M);
  p.b0 = with_rows(a.tt, a.r);   // element (j, k) = T^T[j][k], zero for k > j
  p.e.c = a.out;
  p.e.split_stride = 0;
  p.e.has_t = 0;
  p.e.cb = a.out_bf16;
  p.e.has_b = a.has_bf16;
  p.e.phi = a.piece_hi; p.e.plo = a.piece_lo;
  p.e.has_p = a.has_pieces;
  p.e.pf = a.frag;
  p.e.has_f = a.has_frag;
  if (a.has_pieces && a.M % 4 != 0) return hipErrorInvalidValue;
  if (a.has_frag && a.r % 16 != 0) return hipErrorInvalidValue;
  p.M = a.M; p.N = a.r; p.K = a.r;
  p.splits = 1; p.kchunk = 0; p.tri = 1;
  if (static_cast<int64_t>(cdiv(a.M, 128)) * cdiv(a.r, 128) * members < 256) {
    if (six_products)
      return run<CfgSplit6S, RowF32<64, 256, 3>, RowF32<64, 256, 3>, EpiStoreF32>(p, members, s);
    return run<CfgSplitS, RowF32<64, 256, 2>, RowF32<64, 256, 2>, EpiStoreF32>(p, members, s);
  }
  if (six_products)
    return run<CfgSplit6, RowF32<128, 256, 3>, RowF32<128, 256, 3>, EpiStoreF32>(p, members, s);
  return run<CfgSplit, RowF32<128, 256, 2>, RowF32<128, 256, 2>, EpiStoreF32>(p, members, s);
}

hipError_t launch_gram_tn(const GramTnArgs& a, int members, hipStream_t s) {
  GemmParams<EpiStoreF32::Args> p{};
  p.a = with_rows(a.p, a.r);     // element (j, i) = P[i][j]
  p.b0 = with_rows(a.p, a.r);
  p.e.c = a.out;
  p.e.split_stride = a.splits > 1 ? a.split_stride : 0;
  p.e.has_t = 0;
  p.M = a.r; p.N = a.r; p.K = a.m;
  p.splits = a.splits; p.kchunk = a.kchunk; p.tri = 0;
  if (gram_tn_small_tiles(a.r) && a.kchunk % 64 == 0)
    return run<CfgSplitS64, LdCol<64, 64, 256, 2, float, false, float>,
               LdCol<64, 64, 256, 2, float, false, float>, EpiStoreF32>(p, members, s);
  return run<CfgSplit, ColF32<128, 256, 2>, ColF32<128, 256, 2>, EpiStoreF32>(p, members, s);
}

hipError_t launch_dion_update(const DionUpdateArgs& a, bool bf16, int members, hipStream_t s) {
  return bf16 ? dion_update_bf16(a, members, s) : dion_update_f32(a, members, s);
}

hipError_t launch_ns_gram(const NsGramArgs& a, int members, hipStream_t s) {
  return a.M > 128 ? ns_gram_t<CfgNsBig>(a, members, s) : ns_gram_t<CfgNsSmall>(a, members, s);
}

hipError_t launch_ns_gram_split(const NsGramArgs& a, const MatArg& part, int64_t split_stride,
                                int splits, int kchunk, int members, hipStream_t s) {
  if (splits < 2 || kchunk % 32 != 0) return hipErrorInvalidValue;
  GemmParams<EpiStoreF32::Args> p{};
  p.a = with_rows(a.x, a.M);
  p.b0 = with_rows(a.x, a.M);
  p.e.c = part;
  p.e.split_stride = split_stride;
  p.e.has_t = 0;
  p.M = a.M; p.N = a.M; p.K = a.K;
  p.splits = splits; p.kchunk = kchunk; p.tri = 0;
  return run<CfgNsSmall, NsRow<CfgNsSmall>, NsRow<CfgNsSmall>, EpiStoreF32>(p, members, s);
}

hipError_t launch_ns_gram32_split(const NsGramArgs& a, const MatArg& part, int64_t split_stride,
                                  int splits, int kchunk, int members, hipStream_t s) {
  if (a.M > 128 || splits < 1 || kchunk % 32 != 0) return hipErrorInvalidValue;
  GemmParams<EpiStoreF32::Args> p{};
  p.a = with_rows(a.x, a.M);
  p.b0 = with_rows(a.x, a.M);   // element (j, k) = X[j][k]
  p.e.c = part;
  p.e.split_stride = split_stride;
  p.e.has_t = 0;
  p.M = a.M; p.N = a.M; p.K = a.K;
  p.splits = splits; p.kchunk = kchunk; p.tri = 0;
  return run<CfgSplit, RowF32<128, 256, 2>, RowF32<128, 256, 2>, EpiStoreF32>(p, members, s);
}

hipError_t launch_ns_gram_g(const NsGramArgs& a, bool g_bf16, const MatArg& part,
                            int64_t split_stride, int splits, int kchunk, int members,
                            hipStream_t s) {
  if (!g_bf16) return launch_ns_gram32_split(a, part, split_stride, splits, kchunk, members, s);
  if (a.M > 128 || splits < 1 || kchunk % 32 != 0) return hipErrorInvalidValue;
  GemmParams<EpiStoreF32::Args> p{};
  p.a = with_rows(a.x, a.M);
  p.b0 = with_rows(a.x, a.M);   // element (j, k) = G[j][k]
  p.e.c = part;
  p.e.split_stride = split_stride;
  p.e.has_t = 0;
  p.M = a.M; p.N = a.M; p.K = a.K;
  p.splits = splits; p.kchunk = kchunk; p.tri = 0;
  return run<CfgNsSmall, NsRow<CfgNsSmall>, NsRow<CfgNsSmall>, EpiStoreF32>(p, members, s);
}

// Two pieces of the fp32 left operand against an exact bf16 right operand.
using CfgSplit2 = GemmCfg<128, 128, 32, 2, 2, 2, 1, 2, 1>;

template <class Cfg, class LB, typename OUT_T>
hipError_t ns_gram_apply_t(const NsGramApplyArgs& a, int members, hipStream_t s) {
  GemmParams<typename EpiStoreOut<OUT_T>::Args> p{};
  p.a = with_rows(a.q, a.M);
  p.b0 = with_rows(a.x, a.N);   // element (j, k) = x[k][j]
  p.e.out = a.out;
  p.e.out_transposed = a.out_transposed;
  p.M = a.M; p.N = a.N; p.K = a.M;
  p.splits = 1; p.kchunk = 0; p.tri = 0;
  return run<Cfg, RowF32<128, 256, Cfg::NA>, LB, EpiStoreOut<OUT_T>>(p, members, s);
}

hipError_t launch_ns_gram_apply(const NsGramApplyArgs& a, bool x_bf16, bool out_bf16, int members,
                                hipStream_t s) {
  if (a.M > 128) return hipErrorInvalidValue;
  using ColBf = LdCol<128, 32, 256, 1, uint16_t, false, uint16_t>;
  if (x_bf16)
    return out_bf16 ? ns_gram_apply_t<CfgSplit2, ColBf, uint16_t>(a, members, s)
                    : ns_gram_apply_t<CfgSplit2, ColBf, float>(a, members, s);
  return out_bf16 ? ns_gram_apply_t<CfgSplit, ColF32<128, 256, 2>, uint16_t>(a, members, s)
                  : ns_gram_apply_t<CfgSplit, ColF32<128, 256, 2>, float>(a, members, s);
}

hipError_t launch_ns_poly(const NsPolyArgs& a, int members, hipStream_t s) {
  if (a.c == 0.0f) return launch_ns_linear(a, members, s);
  return a.M > 128 ? ns_poly_t<CfgNsBig>(a, members, s) : ns_poly_t<CfgNsSmall>(a, members, s);
}

hipError_t launch_ns_apply(const NsApplyArgs& a, bool out_bf16, int members, hipStream_t s) {
  if (a.M <= kNsSplitRows)
    return out_bf16 ? ns_apply_split_t<uint16_t>(a, members, s) : ns_apply_split_t<float>(a, members, s);
  // larger sides read X^T as bf16, and every iteration but the last writes it
  if (a.xbt.p[0] == nullptr || (!a.last && a.xbt_next.p[0] == nullptr)) return hipErrorInvalidValue;
  return out_bf16 ? ns_apply_t<CfgNsBig, uint16_t>(a, members, s)
                  : ns_apply_t<CfgNsBig, float>(a, members, s);
}

// Newton-Schulz with fp32-accurate products: bf16x6 splits of the fp32
// operands, formed in the loaders of the 128 x 128 kernel.
hipError_t launch_ns32_gram(const Ns32Args& a, int members, hipStream_t s) {
  GemmParams<EpiStoreF32::Args> p{};
  p.a = with_rows(a.x, a.M);
  p.b0 = with_rows(a.x, a.M);    // element (j, k) = X[j][k]
  p.e.c = a.a32;
  p.e.split_stride = 0;
  p.M = a.M; p.N = a.M; p.K = a.N;
  p.splits = 1; p.kchunk = 0; p.tri = 0;
  return run<CfgSplit6, RowF32<128, 256, 3>, RowF32<128, 256, 3>, EpiStoreF32>(p, members, s);
}

hipError_t launch_ns32_poly(const Ns32Args& a, int members, hipStream_t s) {
  GemmParams<EpiNSPoly32::Args> p{};
  p.a = with_rows(a.a32, a.M);
  p.b0 = with_rows(a.a32, a.M);  // A is symmetric: A A = A A^T
  p.e.a32 = a.a32; p.e.bp32 = a.bp32; p.e.b = a.b; p.e.c = a.c;
  p.M = a.M; p.N = a.M; p.K = a.M;
  p.splits = 1; p.kchunk = 0; p.tri = 0;
  return run<CfgSplit6, RowF32<128, 256, 3>, RowF32<128, 256, 3>, EpiNSPoly32>(p, members, s);
}

template <typename OUT_T>
hipError_t ns32_apply_t(const Ns32Args& a, int members, hipStream_t s) {
  GemmParams<typename EpiNSApply32<OUT_T>::Args> p{};
  p.a = with_rows(a.bp32, a.M);
  p.b0 = with_rows(a.x, a.N);    // element (j, k) = X[k][j]
  p.e.x = a.x; p.e.xn = a.xn; p.e.out = a.out;
  p.e.a = a.a; p.e.last = a.last; p.e.out_transposed = a.out_transposed;
  p.M = a.M; p.N = a.N; p.K = a.M;
  p.splits = 1; p.kchunk = 0; p.tri = 0;
  return run<CfgSplit6, RowF32<128, 256, 3>, ColF32<128, 256, 3>, EpiNSApply32<OUT_T>>(p, members, s);
}

hipError_t launch_ns32_apply(const Ns32Args& a, bool out_bf16, int members, hipStream_t s) {
  return out_bf16 ? ns32_apply_t<uint16_t>(a, members, s) : ns32_apply_t<float>(a, members, s);
}

hipError_t launch_fast_split6(const Split6Args& a, int members, hipStream_t s) {
  GemmParams<EpiFastSplit6F32::Args> p{};
  p.a = with_rows(a.a[0], a.M);
  p.a2 = with_rows(a.a[1], a.M);
  p.a3 = with_rows(a.a[2], a.M);
  p.b0 = with_rows(a.b[0], a.N);
  p.b0s = with_rows(a.b[1], a.N);
  p.b0t = with_rows(a.b[2], a.N);
  p.e.c = a.out;
  p.e.split_stride = a.split_stride;
  p.M = a.M; p.N = a.N; p.K = a.K;
  p.splits = a.splits; p.kchunk = a.kchunk;
  return run_fast<EpiFastSplit6F32>(p, members, s);
}

hipError_t launch_fast_split3(const Split3Args& a, int members, hipStream_t s) {
  GemmParams<EpiFastSplitF32::Args> p{};
  p.a = with_rows(a.ahi, a.M);
  p.a2 = with_rows(a.alo, a.M);
  p.b0 = with_rows(a.bhi, a.N);
  p.b0s = with_rows(a.blo, a.N);
  p.e.c = a.out;
  p.e.split_stride = a.split_stride;
  p.M = a.M; p.N = a.N; p.K = a.K;
  p.splits = a.splits; p.kchunk = a.kchunk;
  return run_fast<EpiFastSplitF32>(p, members, s);
}

}  // namespace ortho
