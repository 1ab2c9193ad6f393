// Workspace planning and argument validation for libortho.so.  Plain C++ with
// no HIP calls, so it can be built and tested on a host without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/ortho.h"

namespace ortho {

constexpr int kMaxMembersPerLaunch = 32;  // must match kMaxBatch in common.h
constexpr size_t kWsAlign = 256;
// Largest rank whose orthonormalisation takes one fp64 pass (apply64).
constexpr int kOrtho64MaxRank = 2048;
// Longest P~ whose whole orthonormalisation runs in one workgroup (r <= 64).
constexpr int kSmallOrthoMaxRows = 256;

// P1^T P1 of the correction pass runs on 64 x 64 tiles below this rank (a
// 256 x 256 result is only 4 tiles of 128); the plan sizes its split for them.
inline bool gram_tn_small_tiles(int r) { return r < 512; }

// A contraction with fewer than 64 output tiles of 128 x 128 over a launch's
// members leaves most of the chip idle: the Dion sweeps then run on 64 x 64
// tiles (k 64 deep), and every split-K reduction may cut k down to 64.
// The fp64 Gram of P~ on 128 x 128 tiles (eight waves each) from r = 1024 on
// (at r = 512 the 64 x 64 tiles were faster, batched or not: 12-layer GPT
// groups 468 against 434 us per call).
inline bool gram_big_tiles(int r, int members) {
  (void)members;
  return r % 128 == 0 && r >= 1024;
}

inline bool few_tiles(int64_t rows, int64_t cols, int members) {
  return ((rows + 127) / 128) * ((cols + 127) / 128) * members < 64;
}

// Byte offsets of one member's regions inside the Dion workspace, and the
// split-K factors chosen for the three reductions over a long dimension.
struct DionPlan {
  int64_t m, n;
  int r;
  int64_t rp;                // leading dimension of m x r / n x r fp32 buffers (r rounded to 4)
  int chunk;                 // members per launch
  int split_left, kchunk_left;    // B Q: split over n
  int split_right, kchunk_right;  // B^T P: split over m
  int split_gram, kchunk_gram;    // fp64 P^T P: split over m
  int split_gram2, kchunk_gram2;  // bf16x3 P1^T P1 (correction pass): split over m
  int gram_big;                   // fp64 Gram on 128 x 128 tiles (gram_big_tiles)
  int small_left, small_right;    // sweeps on 64 x 64 tiles (few_tiles), kchunk a multiple of 64
  int nrb;                   // 64-row blocks of R (column-norm partials)
  size_t off_pt, off_p1, off_part, off_s, off_x, off_d, off_tt, off_r, off_colsq;
  int64_t rpb;               // leading dimension of the bf16 factor copies (r rounded to 8)
  size_t off_pb, off_rb, off_qb;  // bf16 P, (1-mu) R, lr*scale*Q' for the last sweep
  // bf16 P in MFMA fragment order for the streaming update (frag_p): 32-row
  // blocks, then 16-deep k steps, then 64 lanes of 8 (element (i, k) at
  // (((i / 32) * r / 16 + k / 16) * 64 + i % 32 + 32 * (k / 8 % 2)) * 8 + k % 8)
  bool frag_p;
  size_t off_pf;
  // Sweeps on the 256 x 256 kernel (m, n, r multiples of 256, r >= 768, bf16 weights):
  // bf16x2 pieces of B = M + G (m x n) and B^T, of Q^T (r x n) and of P^T (r x m),
  // and split-K factors in k tiles of the three-segment reductions.
  bool fast_sweeps;
  int split_fl, kchunk_fl, split_fr, kchunk_fr;
  // Streaming sweeps (r = 64, 128, 256 or 512, m and n multiples of 64, bf16
  // weights): split-K factors of sweep 1 (over n) and sweep 2 (over m), with
  // the transposed bf16 pieces of Q and P in off_qhit.. off_plot.
  bool stream_sweeps;
  int split_sl, kchunk_sl, split_sr, kchunk_sr;
  size_t off_bhi, off_blo, off_bhit, off_blot, off_qhit, off_qlot, off_phit, off_plot;
  // P = P~ T1 in one pass of fp64 products (apply64), T1^T in fp64 in the
  // scaled-Gram region and P in off_p1, for r <= kOrtho64MaxRank; above it the
  // two passes over bf16 pieces (first-order correction) below.
  bool ortho64;
  // r <= 64 and m <= kSmallOrthoMaxRows: Gram, Cholesky and the fp64 apply in
  // one workgroup per member (small_ortho_kernel).
  bool small_ortho;
  // Orthonormalisation products on the 256 x 256 kernel (with fast_sweeps, or
  // with the streaming sweeps at r = 512 and m a multiple of 256; and 3 r <= n):
  // bf16 pieces in the B-piece buffers, free between the sweeps, or (streaming)
  // in off_bhi (three m x r sets) and off_blo (three r x r sets).
  int fast_ortho;
  int split_ap6, kchunk_ap6;  // P1 = P~ T1, six segments of r
  int split_ap3, kchunk_ap3;  // P = P1 T2, three segments of r
  int split_e, kchunk_e;      // E = P1^T P1, three segments of m
  size_t member_bytes;       // stride between members
  size_t total_bytes;
};

struct NsPlan {
  int64_t M, N;              // wide orientation, M <= N
  int transposed;
  int64_t ld_x, ld_xt;       // leading dims of the M x N and N x M / M x M buffers (rounded to 8)
  int chunk;
  int nparts;
  int64_t part_chunk;        // rows per sum-of-squares block
  size_t off_x32, off_xb0, off_xb1, off_xbt0, off_xbt1, off_a, off_bp, off_bp32, off_partial,
      off_scale;
  // Gram side of 64 or 128 rows: X X^T is one tile per member, so it is split
  // over k (gram_splits slices of gram_kchunk columns, fp32 partials at
  // off_gpart) and reduced in a fixed order into A.
  int gram_splits, gram_kchunk;
  size_t off_gpart;
  // Gram Newton-Schulz (bf16 products, M <= 128 and N >= 4 M): k-split fp32
  // slices of X_0 X_0^T (ld M) and A_0's three bf16 MP x MP pieces (MP = M
  // rounded up to 64 or 128) per member.
  int gram_ns;
  int gns_splits, gns_kchunk, gns_mp;
  size_t off_gns_part, off_gns_a0;
  size_t member_bytes;
  size_t total_bytes;
};

// Muon step: the Newton-Schulz workspace followed, per member of a launch
// chunk, by the fp32 orthogonalised momentum U (m x ld_u, ld_u = n rounded to 4).
struct MuonPlan {
  NsPlan ns;
  int64_t ld_u;
  size_t off_u;              // after the Newton-Schulz part
  size_t u_bytes;            // per member
  size_t off_rowf;           // NorMuon: row factors of U, rows floats per member
  size_t rowf_bytes;         // per member (0 for Muon)
  size_t total_bytes;
};

// Dion2 step on one m x n matrix with k selected rows: the Newton-Schulz
// workspace of the k x n block first, then the block (fp32, ld_blk) and the
// row norms, ranks and selection.
struct Dion2Plan {
  NsPlan ns;
  int64_t ld_blk;
  size_t off_blk, off_norms, off_rank, off_sel;
  size_t total_bytes;
};

bool plan_dion(int64_t m, int64_t n, int32_t r, int32_t batch, DionPlan* out);
bool plan_dion2(int64_t m, int64_t n, int32_t k, Dion2Plan* out);
ortho_status validate_dion2(const ortho_mat& X, const ortho_mat& G, const ortho_mat& M, int32_t k,
                            int32_t steps, const float* abc, float mu, float lr, float scale,
                            const void* ws, size_t ws_bytes);
bool plan_muon(int64_t m, int64_t n, int32_t batch, MuonPlan* out, bool row_norm = false);
bool plan_ns(int64_t m, int64_t n, int32_t batch, NsPlan* out);

ortho_status validate_dion(int32_t batch, const ortho_mat* X, const ortho_mat* G, const ortho_mat* M,
                           const ortho_mat* Q, int32_t r, float mu, float lr, float scale,
                           const ortho_mat* P_out, const ortho_mat* R_out, const void* ws,
                           size_t ws_bytes);

ortho_status validate_ns(int32_t batch, const ortho_mat* G, const ortho_mat* Out, int32_t steps,
                         const float* abc, const void* ws, size_t ws_bytes);

ortho_status validate_muon(int32_t batch, const ortho_mat* X, const ortho_mat* G, const ortho_mat* M,
                           int32_t steps, const float* abc, float mu, float lr, float scale,
                           const void* ws, size_t ws_bytes, bool row_norm = false);

}  // namespace ortho
