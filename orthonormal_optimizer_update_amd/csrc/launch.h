// Host-side launchers of the gfx950 kernels (internal to libortho.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace ortho {

struct RedArgs {
  const float* part;          // member 0 partials; slices of rows x cols (ld = cols)
  int64_t part_member_stride;
  int64_t slice;              // elements per slice
  int splits, rows, cols;
  MatArg out;                 // fp32 destination
  MatArg out_bf16;            // optional bf16 copy of the result (has_bf16; vector path only)
  int has_bf16;
  float* colsq;               // optional per-64-row-block column sums of squares
  int64_t colsq_member_stride;
  int no_store;               // splits == 1 and part is out's memory: column sums only
};

struct ColnormArgs {
  MatArg r;                   // fp32 source
  MatArg q;                   // fp32 destination
  float* colsq;               // per-row-block column sums of squares; row 0 receives 1/norm
  int64_t colsq_member_stride;
  int nrb, rows, cols;
  int32_t* status;
  // optional bf16 operands of the last sweep: rb = c1 * R, qb = c2 * Q'
  MatArg rb, qb;
  float c1, c2;
  int has_bf16;
};

struct SumsqArgs {
  MatArg g;
  float* partial;
  int64_t partial_stride;
  int64_t chunk;       // rows per block
};

struct NsInitArgs {
  MatArg g;            // caller's input (storage dtype)
  MatArg x32, xb, xbt; // iterate (M x N fp32), bf16 M x N, bf16 N x M
  const float* scale;
  int64_t scale_stride;
  int M, N;            // wide orientation, M <= N
  int transposed;      // X = G^T
};

struct Gram64Args {
  MatArg p;            // fp32 m x r
  double* part;        // slices of r x r
  int64_t part_member_stride;
  int64_t slice;
  int m, r, kchunk;
  int big;             // 128 x 128 tiles (r % 128 == 0; the plan's split is for them)
};

struct CholArgs {
  const double* part;  // Gram slices (lower tiles valid)
  int64_t part_member_stride;
  int64_t slice;
  int splits;
  double* s;           // r x r: scaled Gram, then L (lower)
  double* x;           // r x r: L^{-1} (lower)
  double* d;           // r: column scaling 1/sqrt(W_ii)
  int64_t mat_stride, vec_stride;
  int r;
  int32_t* status;
};

// bf16x2 pieces (x = hi + lo + O(2^-16 |x|)) for the 256 x 256 product kernel.
// B = M + G of an m x n fp32 M and bf16 G, written row-major (hi, lo: m x n)
// and transposed (hit, lot: n x m).  rows, cols multiples of 64; M rows 16-byte
// aligned, G and outputs 8-byte aligned.
struct SplitSumArgs {
  MatArg m, g;
  MatArg hi, lo, hit, lot;
  int rows, cols;
};
hipError_t launch_split_sum(const SplitSumArgs& a, int members, hipStream_t s);
// Transposed pieces of an fp32 rows x cols matrix: hit, lot are cols x rows
// (leading dimension hit.ld), or, with blocked, k-blocked: element (j, k) at
// (k / 16) * cols * 16 + j * 16 + k % 16.
struct SplitTArgs {
  MatArg src;
  MatArg hit, lot;
  int rows, cols;
  int blocked;
};
hipError_t launch_split_t(const SplitTArgs& a, int members, hipStream_t s);

// C (+ split-K slices) = A B^T over bf16x2 pieces, hi*hi + hi*lo + lo*hi, on
// the 256 x 256 kernel: A pieces M x K, B pieces N x K (k contiguous), C fp32
// M x N.  M, N multiples of 256, K a multiple of 64; kchunk k tiles per split.
struct Split3Args {
  MatArg ahi, alo, bhi, blo;
  MatArg out;
  int64_t split_stride;
  int M, N, K;
  int splits, kchunk;
};
hipError_t launch_fast_split3(const Split3Args& a, int members, hipStream_t s);
// The same over bf16x3 pieces (x = p0 + p1 + p2), six products p0 q0, p0 q1,
// p1 q0, p0 q2, p1 q1, p2 q0 (fp32-accurate products of fp32 data).
struct Split6Args {
  MatArg a[3], b[3];
  MatArg out;
  int64_t split_stride;
  int M, N, K;
  int splits, kchunk;
};
hipError_t launch_fast_split6(const Split6Args& a, int members, hipStream_t s);
// np (2 or 3) row-major bf16 pieces of an fp32 rows x cols matrix:
// x = p0 + p1 (+ p2), each piece rounded to nearest even from what the
// earlier pieces leave.  grid over 64 x 64 tiles.
struct SplitRowsArgs {
  MatArg src;
  MatArg piece[3];
  int rows, cols, np;
};
hipError_t launch_split_rows(const SplitRowsArgs& a, int members, hipStream_t s);
// Sum of split-K slices (as RedArgs, rows x cols with ld = cols; rows and cols
// multiples of 64, 16-byte aligned rows), written as any of: fp32 (has_out),
// bf16 (has_bf16), np (2 or 3) row-major bf16 pieces, and the transposed
// bf16x2 pieces (has_t; cols x rows).
struct RedPiecesArgs {
  const float* part;
  int64_t part_member_stride;
  int64_t slice;
  int splits, rows, cols;
  MatArg out;
  int has_out;
  MatArg out_bf16;
  int has_bf16;
  MatArg piece[3];
  int np;
  MatArg tpiece[2];
  int has_t;
  // transposed pieces k-blocked, as the streaming sweeps read them: element
  // (j, i) (column j, row i of the result) at (i / 16) * cols * 16 + j * 16 + i % 16
  int t_blocked;
  // bf16 copy in MFMA fragment order (see EpiStoreF32), cols % 16 == 0
  MatArg frag;
  int has_frag;
};
hipError_t launch_reduce_pieces(const RedPiecesArgs& a, int members, hipStream_t s);

hipError_t launch_reduce_splits(const RedArgs& a, int members, hipStream_t s);
hipError_t launch_colnorm(const ColnormArgs& a, int members, hipStream_t s);
// The split-K reduce of R followed by the column normalisation (a.out is cn.r):
// one launch (reduce_colnorm_kernel) when R is short (rows <= kFusedColnormRows,
// at most 16 slice loads per thread) and the reduce's vector path applies, else
// the launches above.
constexpr int kFusedColnormRows = 512;
hipError_t launch_reduce_colnorm(const RedArgs& a, const ColnormArgs& cn, int members, hipStream_t s);
// Whether small_ortho_kernel can sum P~'s split-K slices itself (see
// SmallOrthoArgs::splits): 16-byte alignment of the slices and their rows.
bool small_ortho_reduce_ok(const RedArgs& a);
hipError_t launch_sumsq(const SumsqArgs& a, int nblocks, int members, bool bf16, hipStream_t s);
hipError_t launch_ns_scale(const float* partial, int64_t partial_stride, int nparts, float* scale,
                           int64_t scale_stride, float eps, int members, hipStream_t s);
hipError_t launch_ns_init(const NsInitArgs& a, int members, bool bf16, hipStream_t s);
hipError_t launch_ns_store(const NsInitArgs& a, const MatArg& out, int members, bool bf16,
                           hipStream_t s);
hipError_t launch_gram64(const Gram64Args& a, int splits, int members, hipStream_t s);
// P = P~ T1 with fp64 products (apply64_kernel): t holds T1^T, r x r fp64,
// lower triangular (ld r), as make_t writes it into ttd.
struct Apply64Args {
  MatArg pt;                  // fp32 m x r
  const double* t;            // member 0's T1^T
  int64_t t_member_stride;
  MatArg out;                 // fp32 m x r (must not alias pt)
  MatArg out_bf16;            // optional bf16 copy (has_bf16)
  int has_bf16;
  int m, r;
  // optional further copies of P (m and r multiples of 64), in the layouts of
  // reduce_pieces_kernel: bf16 in MFMA fragment order (has_frag) and the
  // transposed hi / lo pieces (has_t; k-blocked when t_blocked)
  MatArg frag;
  int has_frag;
  MatArg tpiece[2];
  int has_t, t_blocked;
};
hipError_t launch_apply64(const Apply64Args& a, int members, hipStream_t s);

// The whole orthonormalisation (fp64 Gram, scaled Cholesky and inverse,
// P = P~ T1 in fp64) in one workgroup per member, for r <= 64 and a short P~
// (small_ortho_kernel).  ca supplies r, the status word and the s / x
// scratch that the diagonal factorisation writes; out must not alias pt.
struct SmallOrthoArgs {
  MatArg pt;                  // fp32 m x r (read when splits == 0)
  MatArg out;                 // fp32 m x r
  MatArg out_bf16;            // optional bf16 copy (has_bf16)
  int has_bf16;
  int m;
  CholArgs ca;
  // splits > 0: P~ is instead the sum, in slice order, of `splits` split-K
  // slices at part (ld r, slice stride `slice`, member stride
  // part_member_stride), as reduce_splits_vec_kernel would store it
  const float* part;
  int64_t part_member_stride, slice;
  int splits;
};
hipError_t launch_small_ortho(const SmallOrthoArgs& a, int members, hipStream_t s);

// T1^T into tt (fp32) and / or ttd (fp64, when not null).
hipError_t launch_cholesky_inverse(const CholArgs& a, float* tt, int64_t tt_stride, int members,
                                   hipStream_t s, double* ttd = nullptr, int64_t ttd_stride = 0);

// --- GEMM-family sweeps (kernels_gemm.hip) ---------------------------------

// Dion sweep 1: C = (M + G) Q, C is m x r.  G/X dtype: bf16 (true) or fp32.
// Writes split-K slices to `out` (slice stride `split_stride`, ld = r) or, with
// splits == 1, directly.
struct DionLeftArgs {
  MatArg m, g, q;
  MatArg out;
  int64_t split_stride;
  int M, N, r;           // B is M x N
  int splits, kchunk;
  int small;             // 64 x 64 tiles, k 64 deep (kchunk a multiple of 64)
};
hipError_t launch_dion_left(const DionLeftArgs& a, bool bf16, int members, hipStream_t s);

// Dion sweep 2: C = (M + G)^T P, C is n x r (split-K over m).
struct DionRightArgs {
  MatArg m, g, p;
  MatArg out;
  int64_t split_stride;
  int M, N, r;
  int splits, kchunk;
  int small;             // 64 x 64 tiles, k 64 deep (kchunk a multiple of 64)
};
hipError_t launch_dion_right(const DionRightArgs& a, bool bf16, int members, hipStream_t s);

// Dion sweeps for bf16 weights at r = 64, 128, 256 or 512 (kernels_sweep.hip):
// trans = false: out = (M + G) F^T, out rows = rows of M (sweep 1, F = Q^T);
// trans = true:  out = (M + G)^T F^T, out rows = columns of M (sweep 2, F = P^T).
// F is given as two bf16 pieces (hi, lo), r x K k-blocked as split_t writes
// them with blocked set.  Each split-K slice of kchunk k goes to
// out + split * split_stride (ld r).
struct SweepArgs {
  MatArg m, g;             // fp32 M and bf16 G, M_rows x (K or rows)
  MatArg f[2];             // factor pieces, r x K
  float* out;              // member 0's partial slices
  int64_t out_member_stride, split_stride;
  int rows, K, r, kchunk, M_rows;
};
bool dion_sweep_ok(const SweepArgs& a, int members);
hipError_t launch_dion_sweep(const SweepArgs& a, bool trans, int members, hipStream_t s);

// Dion2 (kernels_dion2.hip): select the k rows of B = M + G with the largest
// norm and gather them into blk (launch_dion2_select), then, after
// Newton-Schulz of blk in place, apply it with error feedback
// (launch_dion2_update).  rows <= 65535.
struct Dion2Args {
  MatArg x, g, m;          // caller's X, G (X's dtype) and fp32 M
  MatArg blk;              // fp32 k x cols block, ld a multiple of 4
  float* norms;            // member 0's row sums of squares (rows)
  int* rank;               // member 0's row ranks (rows)
  int* sel;                // member 0's selected rows, in rank order (k)
  int64_t vec_stride;      // elements between members' norms, rank and sel
  int rows, cols, k;
  float mu, c;             // c = lr * scale
};
hipError_t launch_dion2_select(const Dion2Args& a, bool g_bf16, int members, hipStream_t s);
hipError_t launch_dion2_update(const Dion2Args& a, bool x_bf16, int members, hipStream_t s);

// Orthonormalisation apply: P1 = Pt * T with T upper triangular, given as T^T
// (r x r fp32, row-major).
struct ApplyArgs {
  MatArg pt, tt;
  MatArg out;
  MatArg out_bf16;   // optional bf16 copy of the result (has_bf16)
  int has_bf16;
  // optional k-blocked transposed bf16 pieces of the result (has_pieces):
  // element (i, j) at (i / 16) * r * 16 + j * 16 + i % 16; M a multiple of 4
  MatArg piece_hi, piece_lo;
  int has_pieces;
  // optional bf16 copy in MFMA fragment order (see EpiStoreF32), r % 16 == 0
  MatArg frag;
  int has_frag;
  int M, r;
};
hipError_t launch_apply_t(const ApplyArgs& a, bool six_products, int members, hipStream_t s);

// Gram of an m x r fp32 matrix, C = P^T P (r x r), bf16x3 products, split-K
// slices (ld = r, slice stride split_stride) when splits > 1.
struct GramTnArgs {
  MatArg p;
  MatArg out;
  int64_t split_stride;
  int m, r, splits, kchunk;
};
// 64 x 64 tiles (k in steps of 64) where gram_tn_small_tiles(r) and kchunk is
// a multiple of 64, else 128 x 128.
hipError_t launch_gram_tn(const GramTnArgs& a, int members, hipStream_t s);

// T2^T = I - Phi(E) with E = W2 - I (W2 summed from `splits` r x r slices) and
// Phi(E) the lower triangle of E with its diagonal halved: the first-order
// inverse Cholesky factor of a nearly orthonormal basis.
hipError_t launch_correction(const float* part, int64_t part_member_stride, int64_t slice, int splits,
                             int r, float* tt, int64_t tt_stride, int members, hipStream_t s);

// Dion sweep 3: M <- (M+G) - c1 P R^T,  X <- X - c2 P Q'^T.  With bf16
// weights the factors come pre-scaled as bf16 (pb, rb = c1 R, qb = c2 Q');
// with fp32 weights as fp32 (p, r, q) scaled in the epilogue.
struct DionUpdateArgs {
  MatArg p, r, q;        // P m x r, R n x r, Q' n x r (fp32)
  MatArg pb, rb, qb;     // bf16 copies (bf16 weights)
  MatArg pf;             // bf16 P in MFMA fragment order (has_pf; streaming update only)
  int has_pf;
  MatArg m, g, x;
  float c1, c2;
  int M, N, rank;
};
hipError_t launch_dion_update(const DionUpdateArgs& a, bool bf16, int members, hipStream_t s);
// bf16 weights, r = 256 or 512, M % 128 == 0, N % 32 == 0, 16-byte rows of M and
// the bf16 factors, 8-byte rows of G and X: the HBM-streaming update kernel.
bool dion_update_stream_ok(const DionUpdateArgs& a, int members);
hipError_t launch_dion_update_stream(const DionUpdateArgs& a, int members, hipStream_t s);

// Muon step: M = mu M + G (fp32 momentum), then X = X - c U after Newton-Schulz
// of M into the fp32 U.  Grid: 1024 columns x one row per workgroup.
struct MuonArgs {
  MatArg m, g, x, u;
  float mu, c;
  int rows, cols;
  const float* rowf;       // per-row factors of U (NULL: none), rowf_stride floats per member
  int64_t rowf_stride;
};
// Neuron-wise normalisation factors of U (fp32, rows x cols per member):
// rowf[i] = t / |U_i| with t = |U|_F / sqrt(rows), 0 for a zero row.  Two
// launches: one workgroup per row sums its squares, then one workgroup per
// member sums the rows in a fixed order and turns the sums into factors.
struct RowNormArgs {
  MatArg u;
  float* rowf;
  int64_t rowf_stride;
  int rows, cols;
};
hipError_t launch_row_factors(const RowNormArgs& a, int members, hipStream_t s);
hipError_t launch_muon_momentum(const MuonArgs& a, bool g_bf16, int members, hipStream_t s);
hipError_t launch_muon_update(const MuonArgs& a, bool x_bf16, int members, hipStream_t s);

// Newton-Schulz products (bf16 operands, fp32 accumulation).
struct NsGramArgs { MatArg x; MatArg a; int M, K; };                 // A = X X^T
struct NsPolyArgs { MatArg a; MatArg bp; MatArg bp32; float b, c; int M; };  // Bp = bA + cAA
// X = aX + Bp X.  When M <= kNsSplitRows the product uses split bf16 operands
// read from bp32 and the fp32 iterate (one row tile, so updating the iterate in
// place cannot race with another tile's reads).
constexpr int kNsSplitRows = 128;
struct NsApplyArgs {
  MatArg bp, xbt, x32, xb_next, xbt_next, out, bp32;
  float a;
  int M, N, last, out_transposed;
};
hipError_t launch_ns_gram(const NsGramArgs& a, int members, hipStream_t s);
// X X^T for a Gram side of at most 128 rows, split over k into fp32 partials
// (member pointers in `part`, slice `split_stride` elements apart, ld = M).
hipError_t launch_ns_gram_split(const NsGramArgs& a, const MatArg& part, int64_t split_stride,
                                int splits, int kchunk, int members, hipStream_t s);
hipError_t launch_ns_poly(const NsPolyArgs& a, int members, hipStream_t s);
// Gram side of 64 or 128 rows after the split Gram: per member, A = sum of the
// k-split partials (slice order) rounded to bf16, then Bp = c ((b/c) A + A A) into
// bp (bf16) and bp32 (fp32), in one launch with one workgroup per member.
struct NsSmallPolyArgs {
  const float* part;
  int64_t part_member_stride, slice;
  int splits, M;
  MatArg bp, bp32;
  float b, c;
};
hipError_t launch_ns_small_poly(const NsSmallPolyArgs& a, int members, hipStream_t s);
hipError_t launch_ns_linear(const NsPolyArgs& a, int members, hipStream_t s);  // c == 0
// Newton-Schulz with fp32-accurate products (fp32 inputs): bf16x6 splits of
// the fp32 operands.  A32 = X X^T; Bp32 = b A32 + c A32 A32; then
// Xn = a X + Bp32 X, or the caller's output on the last iteration.
struct Ns32Args {
  MatArg x, xn;        // fp32 iterates M x N (read / written)
  MatArg a32, bp32;    // fp32 M x M
  MatArg out;          // caller's output (storage dtype; N x M when out_transposed)
  float a, b, c;
  int M, N, last, out_transposed;
};
hipError_t launch_ns32_gram(const Ns32Args& a, int members, hipStream_t s);
hipError_t launch_ns32_poly(const Ns32Args& a, int members, hipStream_t s);
hipError_t launch_ns32_apply(const Ns32Args& a, bool out_bf16, int members, hipStream_t s);

// Gram Newton-Schulz on a Gram side of M <= 128 rows: A_0 = X_0 X_0^T from the
// fp32 iterate with bf16x3 products, split over k into fp32 slices (ld M)...
hipError_t launch_ns_gram32_split(const NsGramArgs& a, const MatArg& part, int64_t split_stride,
                                  int splits, int kchunk, int members, hipStream_t s);
// ...then, one workgroup per member, the iteration on the M x M side with
// bf16x6 products: Q_{k+1} = (a I + b A_k + c A_k^2) Q_k, A_k = Q_k A_0 Q_k^T,
// Q_0 = I, for `steps` >= 1 iterations; Q_steps goes to q (fp32 M x M).  The
// apply X = Q_steps X_0 is launch_ns_apply with a = 0 and bp32 = q.
struct NsGramIterArgs {
  const float* part;           // member 0's k-split Gram slices (ld M)
  int64_t part_member_stride, slice;
  int splits;
  const float* scale;          // per-member factor sc (NULL: 1): A_0 = sc^2 * sum, q = sc * Q
  int64_t scale_stride;
  MatArg a0;                   // scratch per member: three bf16 MP x MP pieces (ld MP, MP = 64 or 128)
  MatArg q;                    // fp32 result, M x M
  float a, b, c;
  int M, steps;
};
hipError_t launch_ns_gram_iter(const NsGramIterArgs& a, int members, hipStream_t s);
// The Gram of the caller's wide G itself (M <= 128 rows): exact bf16 products
// for bf16 G, bf16x3 for fp32 G; k-split fp32 slices (ld M) as above.
hipError_t launch_ns_gram_g(const NsGramArgs& a, bool g_bf16, const MatArg& part,
                            int64_t split_stride, int splits, int kchunk, int members,
                            hipStream_t s);
// The apply of Gram Newton-Schulz: out = Q x (M x N), Q fp32 M x M (two bf16
// pieces), x M x N (bf16: exact; fp32: two pieces); out in its dtype,
// transposed (N x M) when out_transposed.
struct NsGramApplyArgs {
  MatArg q, x, out;
  int M, N, out_transposed;
};
hipError_t launch_ns_gram_apply(const NsGramApplyArgs& a, bool x_bf16, bool out_bf16, int members,
                                hipStream_t s);
hipError_t launch_ns_apply(const NsApplyArgs& a, bool out_bf16, int members, hipStream_t s);

}  // namespace ortho
