// C-ABI entry points of libortho.so: argument checks, workspace carving and the
// stream-ordered kernel sequence of each operation.  No allocation, no host
// synchronisation.
#include <string.h>

#include "../../include/ortho.h"
#include "launch.h"
#include "plan.h"
#include "run.h"

using namespace ortho;

namespace {

constexpr float kMuonA = 3.4445f, kMuonB = -4.7750f, kMuonC = 2.0315f;
constexpr float kNsEps = 1e-7f;

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

// Pointer table over caller matrices [b0, b0 + nb).  `vec_bytes` is the width
// of the vector accesses the consuming kernel makes.
MatArg user_table(const ortho_mat* mats, int b0, int nb, size_t vec_bytes) {
  MatArg t;
  memset(&t, 0, sizeof(t));
  const size_t esz = mats[b0].dtype == ORTHO_BF16 ? 2 : 4;
  t.ld = mats[b0].ld;
  t.rows = static_cast<int>(mats[b0].rows);
  t.cols = static_cast<int>(mats[b0].cols);
  bool vec = (static_cast<size_t>(t.ld) * esz) % vec_bytes == 0;
  for (int i = 0; i < nb; ++i) {
    t.p[i] = mats[b0 + i].data;
    vec = vec && aligned(t.p[i], vec_bytes);
  }
  t.vec = vec;
  return t;
}

// Pointer table over one workspace region of members [0, nb).
MatArg ws_table(char* base, size_t member_bytes, size_t off, int nb, int64_t ld, int rows,
                int cols, size_t esz, size_t vec_bytes) {
  MatArg t;
  memset(&t, 0, sizeof(t));
  t.ld = ld;
  t.rows = rows;
  t.cols = cols;
  for (int i = 0; i < nb; ++i) t.p[i] = base + i * member_bytes + off;
  t.vec = (static_cast<size_t>(ld) * esz) % vec_bytes == 0;
  return t;
}

#define ORTHO_TRY(expr)                               \
  do {                                                \
    if ((expr) != hipSuccess) return ORTHO_E_HIP;     \
  } while (0)

ortho_status run_dion(int32_t batch, const ortho_mat* X, const ortho_mat* G, const ortho_mat* M,
                      const ortho_mat* Q, int32_t r, float mu, float lr, float scale,
                      const ortho_mat* P_out, const ortho_mat* R_out, int32_t* status, void* ws,
                      void* stream) {
  const int64_t m = X[0].rows, n = X[0].cols;
  DionPlan pl;
  if (!plan_dion(m, n, r, batch, &pl)) return ORTHO_E_SHAPE;
  const bool bf = X[0].dtype == ORTHO_BF16;
  const hipStream_t s = as_stream(stream);
  char* base = static_cast<char*>(ws);
  const size_t mb = pl.member_bytes;
  const int mi = static_cast<int>(m), ni = static_cast<int>(n);
  const int64_t rp = pl.rp;
  const size_t gvec = bf ? 8 : 16;

  for (int b0 = 0; b0 < batch; b0 += pl.chunk) {
    const int nb = batch - b0 < pl.chunk ? batch - b0 : pl.chunk;
    const MatArg tX = user_table(X, b0, nb, gvec);
    const MatArg tG = user_table(G, b0, nb, gvec);
    const MatArg tM = user_table(M, b0, nb, 16);
    const MatArg tQ = user_table(Q, b0, nb, 16);
    const MatArg tPt = ws_table(base, mb, pl.off_pt, nb, rp, mi, r, 4, 16);
    const MatArg tP1 = ws_table(base, mb, pl.off_p1, nb, rp, mi, r, 4, 16);
    const MatArg tPart = ws_table(base, mb, pl.off_part, nb, r, 0, r, 4, 16);
    const MatArg tR = ws_table(base, mb, pl.off_r, nb, rp, ni, r, 4, 16);
    const MatArg tTt = ws_table(base, mb, pl.off_tt, nb, r, r, r, 4, 16);
    const MatArg tPb = ws_table(base, mb, pl.off_pb, nb, pl.rpb, mi, r, 2, 16);
    const MatArg tRb = ws_table(base, mb, pl.off_rb, nb, pl.rpb, ni, r, 2, 16);
    const MatArg tQb = ws_table(base, mb, pl.off_qb, nb, pl.rpb, ni, r, 2, 16);
    float* part_f = reinterpret_cast<float*>(base + pl.off_part);
    double* part_d = reinterpret_cast<double*>(base + pl.off_part);
    // bf16 pieces of the orthonormalisation products on the 256 x 256 kernel:
    // A pieces (m x r) in the row-major B-piece buffer and B pieces (r x r) in
    // the second one, both free once sweep 1 is done (3 r <= n), or in regions
    // of their own with the streaming sweeps; m, r multiples of 256, so every
    // piece starts 256-byte aligned.
    MatArg ap[3], bp[3];
    for (int k = 0; k < 3; ++k) {
      ap[k] = ws_table(base, mb, pl.off_bhi + k * static_cast<size_t>(mi) * r * 2, nb, r, mi, r, 2, 16);
      bp[k] = ws_table(base, mb, pl.off_blo + k * static_cast<size_t>(r) * r * 2, nb, r, r, r, 2, 16);
    }
    bool pt_pieces = false;  // P_tilde's bf16x3 pieces already in ap

    // Sweeps on the 256 x 256 kernel over bf16x2 pieces (bf16 weights, sizes
    // multiples of 256, 16-byte rows of M and Q; G rows 8-byte aligned).
    const bool fast_sw = bf && pl.fast_sweeps && tM.vec && tQ.vec && tG.vec;
    if (fast_sw) {
      const MatArg tBhi = ws_table(base, mb, pl.off_bhi, nb, n, mi, ni, 2, 16);
      const MatArg tBlo = ws_table(base, mb, pl.off_blo, nb, n, mi, ni, 2, 16);
      const MatArg tBhiT = ws_table(base, mb, pl.off_bhit, nb, m, ni, mi, 2, 16);
      const MatArg tBloT = ws_table(base, mb, pl.off_blot, nb, m, ni, mi, 2, 16);
      const MatArg tQhiT = ws_table(base, mb, pl.off_qhit, nb, n, r, ni, 2, 16);
      const MatArg tQloT = ws_table(base, mb, pl.off_qlot, nb, n, r, ni, 2, 16);
      SplitSumArgs sa{};
      sa.m = tM; sa.g = tG; sa.hi = tBhi; sa.lo = tBlo; sa.hit = tBhiT; sa.lot = tBloT;
      sa.rows = mi; sa.cols = ni;
      ORTHO_TRY(launch_split_sum(sa, nb, s));
      SplitTArgs qa{};
      qa.src = tQ; qa.hit = tQhiT; qa.lot = tQloT; qa.rows = ni; qa.cols = r;
      ORTHO_TRY(launch_split_t(qa, nb, s));
      // Sweep 1 over n: P_tilde = (Bhi, Blo) (Qhi, Qlo)^T
      Split3Args l3{};
      l3.ahi = tBhi; l3.alo = tBlo; l3.bhi = tQhiT; l3.blo = tQloT;
      l3.out = pl.split_fl > 1 ? tPart : tPt;
      l3.split_stride = m * r;
      l3.M = mi; l3.N = r; l3.K = ni;
      l3.splits = pl.split_fl; l3.kchunk = pl.kchunk_fl;
      ORTHO_TRY(launch_fast_split3(l3, nb, s));
      if (pl.split_fl > 1 && pl.fast_ortho) {
        // the reduce also writes the bf16x3 pieces of P_tilde for P1 = P~ T1
        RedPiecesArgs ra{};
        ra.part = part_f; ra.part_member_stride = static_cast<int64_t>(mb / 4);
        ra.slice = m * r; ra.splits = pl.split_fl; ra.rows = mi; ra.cols = r;
        ra.out = tPt; ra.has_out = 1;
        for (int k = 0; k < 3; ++k) ra.piece[k] = ap[k];
        ra.np = 3;
        ORTHO_TRY(launch_reduce_pieces(ra, nb, s));
        pt_pieces = true;
      } else if (pl.split_fl > 1) {
        RedArgs ra{};
        ra.part = part_f; ra.part_member_stride = static_cast<int64_t>(mb / 4);
        ra.slice = m * r; ra.splits = pl.split_fl; ra.rows = mi; ra.cols = r;
        ra.out = tPt; ra.colsq = nullptr; ra.colsq_member_stride = 0;
        ORTHO_TRY(launch_reduce_splits(ra, nb, s));
      }
    }

    // The split-K reduce of P~ into tPt, or, when the one-workgroup
    // orthonormalisation follows, left to that kernel (it sums the slices as
    // it loads P~, in the same order).
    RedArgs pt_red{};
    bool pt_red_pending = false;
    auto reduce_pt = [&](const RedArgs& ra) -> hipError_t {
      if (pl.small_ortho && small_ortho_reduce_ok(ra)) {
        pt_red = ra;
        pt_red_pending = true;
        return hipSuccess;
      }
      return launch_reduce_splits(ra, nb, s);
    };

    // Streaming sweeps (bf16 weights, r = 64, 128, 256 or 512): the pieces of
    // Q^T, then one pass over M and G into split-K slices.
    SweepArgs sw{};
    bool stream_sw = false;
    if (bf && !fast_sw && pl.stream_sweeps) {
      sw.m = tM; sw.g = user_table(G, b0, nb, 16);
      sw.f[0] = ws_table(base, mb, pl.off_qhit, nb, n, r, ni, 2, 16);
      sw.f[1] = ws_table(base, mb, pl.off_qlot, nb, n, r, ni, 2, 16);
      // one k slice: the sweep writes P~ itself (ld r), no reduce follows
      sw.out = pl.split_sl == 1 ? reinterpret_cast<float*>(base + pl.off_pt) : part_f;
      sw.out_member_stride = static_cast<int64_t>(mb / 4);
      sw.split_stride = m * r;
      sw.rows = mi; sw.K = ni; sw.r = r; sw.kchunk = pl.kchunk_sl; sw.M_rows = mi;
      stream_sw = dion_sweep_ok(sw, nb);
    }
    // orthonormalisation products on the 256 x 256 kernel over bf16 pieces
    const bool fast_or = bf && pl.fast_ortho && (fast_sw || stream_sw);
    if (stream_sw) {
      SplitTArgs qa{};
      qa.src = tQ; qa.hit = sw.f[0]; qa.lot = sw.f[1]; qa.rows = ni; qa.cols = r; qa.blocked = 1;
      ORTHO_TRY(launch_split_t(qa, nb, s));
      ORTHO_TRY(launch_dion_sweep(sw, false, nb, s));
      if (pl.split_sl == 1 && !fast_or) {
        // P~ is already in tPt
      } else if (fast_or) {
        // the reduce also writes the bf16x3 pieces of P_tilde for P1 = P~ T1
        RedPiecesArgs ra{};
        ra.part = part_f; ra.part_member_stride = static_cast<int64_t>(mb / 4);
        ra.slice = m * r; ra.splits = pl.split_sl; ra.rows = mi; ra.cols = r;
        ra.out = tPt; ra.has_out = 1;
        for (int k = 0; k < 3; ++k) ra.piece[k] = ap[k];
        ra.np = 3;
        ORTHO_TRY(launch_reduce_pieces(ra, nb, s));
        pt_pieces = true;
      } else {
        RedArgs ra{};
        ra.part = part_f; ra.part_member_stride = static_cast<int64_t>(mb / 4);
        ra.slice = m * r; ra.splits = pl.split_sl; ra.rows = mi; ra.cols = r;
        ra.out = tPt; ra.colsq = nullptr; ra.colsq_member_stride = 0;
        ORTHO_TRY(reduce_pt(ra));
      }
    }

    // Sweep 1: P_tilde = (M + G) Q.
    DionLeftArgs la{};
    la.m = tM; la.g = tG; la.q = tQ;
    la.out = pl.split_left > 1 ? tPart : tPt;
    la.split_stride = m * r;
    la.M = mi; la.N = ni; la.r = r;
    la.splits = pl.split_left; la.kchunk = pl.kchunk_left; la.small = pl.small_left;
    if (!fast_sw && !stream_sw) ORTHO_TRY(launch_dion_left(la, bf, nb, s));
    if (!fast_sw && !stream_sw && pl.split_left > 1) {
      RedArgs ra{};
      ra.part = part_f; ra.part_member_stride = static_cast<int64_t>(mb / 4);
      ra.slice = m * r; ra.splits = pl.split_left; ra.rows = mi; ra.cols = r;
      ra.out = tPt; ra.colsq = nullptr; ra.colsq_member_stride = 0;
      ORTHO_TRY(reduce_pt(ra));
    }

    // Orthonormalisation of P_tilde (Q-factor of its thin QR, diag(R) > 0):
    // fp64 Gram, column-scaled fp64 Cholesky and triangular inverse, then
    // P = P_tilde T1 (T1 = D L^-T, upper triangular).
    CholArgs ca{};
    ca.part = part_d; ca.part_member_stride = static_cast<int64_t>(mb / 8);
    ca.slice = static_cast<int64_t>(r) * r; ca.splits = pl.split_gram;
    ca.s = reinterpret_cast<double*>(base + pl.off_s);
    ca.x = reinterpret_cast<double*>(base + pl.off_x);
    ca.d = reinterpret_cast<double*>(base + pl.off_d);
    ca.mat_stride = static_cast<int64_t>(mb / 8); ca.vec_stride = static_cast<int64_t>(mb / 8);
    ca.r = r; ca.status = status;
    float* tt = reinterpret_cast<float*>(base + pl.off_tt);
    // P ends up in tP (off_p): tPt, or tP1 when the fp64 pass writes it
    MatArg tP = tPt;
    size_t off_p = pl.off_pt;
    if (!pl.small_ortho) {
      Gram64Args ga{};
      ga.p = tPt; ga.part = part_d; ga.part_member_stride = static_cast<int64_t>(mb / 8);
      ga.slice = static_cast<int64_t>(r) * r; ga.m = mi; ga.r = r; ga.kchunk = pl.kchunk_gram;
      ga.big = pl.gram_big;
      ORTHO_TRY(launch_gram64(ga, pl.split_gram, nb, s));
    }
    if (pl.small_ortho || pl.ortho64) {
      if (pl.small_ortho) {
        // r <= 64 and a short P~: the whole chain in one workgroup per member
        SmallOrthoArgs so{};
        so.pt = tPt; so.out = tP1; so.out_bf16 = tPb; so.has_bf16 = bf; so.m = mi; so.ca = ca;
        if (pt_red_pending) {   // sweep 1's split-K slices, summed by the kernel
          so.part = pt_red.part; so.part_member_stride = pt_red.part_member_stride;
          so.slice = pt_red.slice; so.splits = pt_red.splits;
          pt_red_pending = false;
        }
        ORTHO_TRY(launch_small_ortho(so, nb, s));
      } else {
        // T1^T in fp64 into the scaled-Gram region (free once the chain is
        // done), then P = P~ T1 in one pass of fp64 products into tP1, with
        // the bf16 copy the update reads
        double* ttd = reinterpret_cast<double*>(base + pl.off_s);
        ORTHO_TRY(launch_cholesky_inverse(ca, nullptr, 0, nb, s, ttd, static_cast<int64_t>(mb / 8)));
        Apply64Args a64{};
        a64.pt = tPt; a64.t = ttd; a64.t_member_stride = static_cast<int64_t>(mb / 8);
        a64.out = tP1; a64.out_bf16 = tPb; a64.has_bf16 = bf; a64.m = mi; a64.r = r;
        // the fragment-order copy and sweep 2's transposed pieces from the same
        // tiles (every path that reads them has m and r multiples of 64)
        if (bf && pl.frag_p) {
          a64.frag = ws_table(base, mb, pl.off_pf, nb, r, mi, r, 2, 16);
          a64.has_frag = 1;
        }
        if (stream_sw || fast_sw) {
          a64.tpiece[0] = ws_table(base, mb, pl.off_phit, nb, m, r, mi, 2, 16);
          a64.tpiece[1] = ws_table(base, mb, pl.off_plot, nb, m, r, mi, 2, 16);
          a64.has_t = 1;
          a64.t_blocked = stream_sw;
        }
        ORTHO_TRY(launch_apply64(a64, nb, s));
      }
      tP = tP1;
      off_p = pl.off_p1;
      // after the one-workgroup path: the fragment-order copy (streaming
      // update) and the transposed pieces (sweep 2: k-blocked for the
      // streaming kernel, ld m for the 256 x 256 one); every path that reads
      // them has m and r multiples of 64
      const bool need_frag = pl.small_ortho && bf && pl.frag_p;
      const bool need_t = pl.small_ortho && (stream_sw || fast_sw);
      if (need_frag || need_t) {
        RedPiecesArgs rd{};
        rd.part = reinterpret_cast<const float*>(base + pl.off_p1);
        rd.part_member_stride = static_cast<int64_t>(mb / 4);
        rd.slice = m * r; rd.splits = 1; rd.rows = mi; rd.cols = r;
        if (need_t) {
          rd.tpiece[0] = ws_table(base, mb, pl.off_phit, nb, m, r, mi, 2, 16);
          rd.tpiece[1] = ws_table(base, mb, pl.off_plot, nb, m, r, mi, 2, 16);
          rd.has_t = 1;
          rd.t_blocked = stream_sw;
        }
        if (need_frag) {
          rd.frag = ws_table(base, mb, pl.off_pf, nb, r, mi, r, 2, 16);
          rd.has_frag = 1;
        }
        ORTHO_TRY(launch_reduce_pieces(rd, nb, s));
      }
    } else {
    ORTHO_TRY(launch_cholesky_inverse(ca, tt, static_cast<int64_t>(mb / 4), nb, s));
    if (fast_or) {
      // The same three products on the 256 x 256 kernel over bf16 pieces
      // (split-K, fixed-order reduces that also write the next product's
      // pieces).
      const MatArg tPhiT = ws_table(base, mb, pl.off_phit, nb, m, r, mi, 2, 16);
      const MatArg tPloT = ws_table(base, mb, pl.off_plot, nb, m, r, mi, 2, 16);
      const int64_t mr = static_cast<int64_t>(mi) * r;
      // P1 = P~ T1, six products of bf16x3 pieces
      if (!pt_pieces) {
        SplitRowsArgs sp{};
        sp.src = tPt; sp.piece[0] = ap[0]; sp.piece[1] = ap[1]; sp.piece[2] = ap[2];
        sp.rows = mi; sp.cols = r; sp.np = 3;
        ORTHO_TRY(launch_split_rows(sp, nb, s));
      }
      SplitRowsArgs st{};
      st.src = tTt; st.piece[0] = bp[0]; st.piece[1] = bp[1]; st.piece[2] = bp[2];
      st.rows = r; st.cols = r; st.np = 3;
      ORTHO_TRY(launch_split_rows(st, nb, s));
      Split6Args a6{};
      for (int k = 0; k < 3; ++k) { a6.a[k] = ap[k]; a6.b[k] = bp[k]; }
      a6.out = tPart; a6.split_stride = mr;
      a6.M = mi; a6.N = r; a6.K = r; a6.splits = pl.split_ap6; a6.kchunk = pl.kchunk_ap6;
      ORTHO_TRY(launch_fast_split6(a6, nb, s));
      // P1 itself is not kept: the reduce writes its bf16x2 pieces, row-major
      // for P = P1 T2 and transposed for E = P1^T P1 (pass 2, see below).
      RedPiecesArgs rp1{};
      rp1.part = part_f; rp1.part_member_stride = static_cast<int64_t>(mb / 4);
      rp1.slice = mr; rp1.splits = pl.split_ap6; rp1.rows = mi; rp1.cols = r;
      rp1.piece[0] = ap[0]; rp1.piece[1] = ap[1]; rp1.np = 2;
      rp1.tpiece[0] = tPhiT; rp1.tpiece[1] = tPloT; rp1.has_t = 1;
      ORTHO_TRY(launch_reduce_pieces(rp1, nb, s));
      Split3Args e3{};
      e3.ahi = tPhiT; e3.alo = tPloT; e3.bhi = tPhiT; e3.blo = tPloT;
      e3.out = tPart; e3.split_stride = static_cast<int64_t>(r) * r;
      e3.M = r; e3.N = r; e3.K = mi; e3.splits = pl.split_e; e3.kchunk = pl.kchunk_e;
      ORTHO_TRY(launch_fast_split3(e3, nb, s));
      ORTHO_TRY(launch_correction(part_f, static_cast<int64_t>(mb / 4), static_cast<int64_t>(r) * r,
                                  pl.split_e, r, tt, static_cast<int64_t>(mb / 4), nb, s));
      // P = P1 T2, bf16x3; the bf16 copy and the transposed pieces of P feed
      // sweeps 2 and 3
      st.np = 2;
      ORTHO_TRY(launch_split_rows(st, nb, s));
      Split3Args a3{};
      a3.ahi = ap[0]; a3.alo = ap[1]; a3.bhi = bp[0]; a3.blo = bp[1];
      a3.out = tPart; a3.split_stride = mr;
      a3.M = mi; a3.N = r; a3.K = r; a3.splits = pl.split_ap3; a3.kchunk = pl.kchunk_ap3;
      ORTHO_TRY(launch_fast_split3(a3, nb, s));
      RedPiecesArgs rp2{};
      rp2.part = part_f; rp2.part_member_stride = static_cast<int64_t>(mb / 4);
      rp2.slice = mr; rp2.splits = pl.split_ap3; rp2.rows = mi; rp2.cols = r;
      rp2.out = tPt; rp2.has_out = 1; rp2.out_bf16 = tPb; rp2.has_bf16 = 1;
      rp2.tpiece[0] = tPhiT; rp2.tpiece[1] = tPloT; rp2.has_t = 1;
      rp2.t_blocked = stream_sw;   // the streaming sweep 2 reads them k-blocked
      if (pl.frag_p) {
        rp2.frag = ws_table(base, mb, pl.off_pf, nb, r, mi, r, 2, 16);
        rp2.has_frag = 1;
      }
      ORTHO_TRY(launch_reduce_pieces(rp2, nb, s));
    } else {
    ApplyArgs aa{};
    aa.pt = tPt; aa.tt = tTt; aa.out = tP1; aa.M = mi; aa.r = r;
    aa.out_bf16 = tPb; aa.has_bf16 = 0;
    ORTHO_TRY(launch_apply_t(aa, true, nb, s));
    // Pass 2: P1 is orthonormal to about 2^-24 * cond; E = P1^T P1 - I (bf16x3)
    // and the first-order factor T2 = I - Phi(E)^T give P = P1 T2.
    GramTnArgs g2{};
    g2.p = tP1; g2.out = tPart; g2.split_stride = static_cast<int64_t>(r) * r;
    g2.m = mi; g2.r = r; g2.splits = pl.split_gram2; g2.kchunk = pl.kchunk_gram2;
    ORTHO_TRY(launch_gram_tn(g2, nb, s));
    ORTHO_TRY(launch_correction(part_f, static_cast<int64_t>(mb / 4), static_cast<int64_t>(r) * r,
                                pl.split_gram2, r, tt, static_cast<int64_t>(mb / 4), nb, s));
    aa.pt = tP1; aa.out = tPt; aa.has_bf16 = bf;   // bf16 P feeds the last sweep
    if (bf && pl.frag_p) {
      // and its fragment-order copy the streaming update
      aa.frag = ws_table(base, mb, pl.off_pf, nb, r, mi, r, 2, 16);
      aa.has_frag = 1;
    }
    if (stream_sw) {
      // the k-blocked transposed pieces of P that the streaming sweep 2 reads
      aa.piece_hi = ws_table(base, mb, pl.off_phit, nb, m, r, mi, 2, 16);
      aa.piece_lo = ws_table(base, mb, pl.off_plot, nb, m, r, mi, 2, 16);
      aa.has_pieces = 1;
    }
    ORTHO_TRY(launch_apply_t(aa, false, nb, s));
    }
    }

    // Sweep 2: R = (M + G)^T P, then Q' = column-normalised R.
    int split_r = pl.split_right;
    if (fast_sw) {
      // over m: R = (Bhi^T, Blo^T) (Phi^T, Plo^T)^T
      const MatArg tBhiT = ws_table(base, mb, pl.off_bhit, nb, m, ni, mi, 2, 16);
      const MatArg tBloT = ws_table(base, mb, pl.off_blot, nb, m, ni, mi, 2, 16);
      const MatArg tPhiT = ws_table(base, mb, pl.off_phit, nb, m, r, mi, 2, 16);
      const MatArg tPloT = ws_table(base, mb, pl.off_plot, nb, m, r, mi, 2, 16);
      if (!pl.fast_ortho && !pl.ortho64) {  // else the last orthonormalisation reduce wrote them
        SplitTArgs pa{};
        pa.src = tPt; pa.hit = tPhiT; pa.lot = tPloT; pa.rows = mi; pa.cols = r;
        ORTHO_TRY(launch_split_t(pa, nb, s));
      }
      Split3Args r3{};
      r3.ahi = tBhiT; r3.alo = tBloT; r3.bhi = tPhiT; r3.blo = tPloT;
      r3.out = tPart; r3.split_stride = n * r;
      r3.M = ni; r3.N = r; r3.K = mi;
      r3.splits = pl.split_fr; r3.kchunk = pl.kchunk_fr;
      ORTHO_TRY(launch_fast_split3(r3, nb, s));
      split_r = pl.split_fr;
    } else if (stream_sw) {
      // over m: the pieces of P^T, then one pass over M and G
      SweepArgs sr = sw;
      sr.f[0] = ws_table(base, mb, pl.off_phit, nb, m, r, mi, 2, 16);
      sr.f[1] = ws_table(base, mb, pl.off_plot, nb, m, r, mi, 2, 16);
      sr.split_stride = n * r;
      sr.rows = ni; sr.K = mi; sr.kchunk = pl.kchunk_sr;
      // one k slice: the sweep writes R itself (ld r), the reduce only sums squares
      sr.out = pl.split_sr == 1 ? reinterpret_cast<float*>(base + pl.off_r) : part_f;
      // (the pieces were written by the last orthonormalisation product)
      ORTHO_TRY(launch_dion_sweep(sr, true, nb, s));
      split_r = pl.split_sr;
    } else {
      DionRightArgs rb{};
      rb.m = tM; rb.g = tG; rb.p = tP; rb.out = tPart;
      rb.split_stride = n * r;
      rb.M = mi; rb.N = ni; rb.r = r;
      rb.splits = pl.split_right; rb.kchunk = pl.kchunk_right; rb.small = pl.small_right;
      ORTHO_TRY(launch_dion_right(rb, bf, nb, s));
    }
    RedArgs rr{};
    rr.part = part_f; rr.part_member_stride = static_cast<int64_t>(mb / 4);
    rr.slice = n * r; rr.splits = split_r; rr.rows = ni; rr.cols = r;
    rr.out = tR;
    if (stream_sw && split_r == 1) {
      rr.part = reinterpret_cast<const float*>(base + pl.off_r);
      rr.no_store = 1;
    }
    rr.colsq = reinterpret_cast<float*>(base + pl.off_colsq);
    rr.colsq_member_stride = static_cast<int64_t>(mb / 4);
    ColnormArgs cn{};
    cn.r = tR; cn.q = tQ; cn.colsq = rr.colsq; cn.colsq_member_stride = rr.colsq_member_stride;
    cn.nrb = pl.nrb; cn.rows = ni; cn.cols = r; cn.status = status;
    cn.rb = tRb; cn.qb = tQb; cn.c1 = 1.0f - mu; cn.c2 = lr * scale; cn.has_bf16 = bf;
    ORTHO_TRY(launch_reduce_colnorm(rr, cn, nb, s));

    if (P_out)
      ORTHO_TRY(hipMemcpy2DAsync(P_out->data, P_out->ld * 4, base + off_p, rp * 4, r * 4, m,
                                 hipMemcpyDeviceToDevice, s));
    if (R_out)
      ORTHO_TRY(hipMemcpy2DAsync(R_out->data, R_out->ld * 4, base + pl.off_r, rp * 4, r * 4, n,
                                 hipMemcpyDeviceToDevice, s));

    // Sweep 3: error feedback into M and the weight update into X.
    DionUpdateArgs ua{};
    ua.p = tP; ua.r = tR; ua.q = tQ; ua.m = tM; ua.g = tG; ua.x = tX;
    ua.pb = tPb; ua.rb = tRb; ua.qb = tQb;
    // the fragment-order P, written by the last orthonormalisation product or
    // its reduce
    ua.has_pf = bf && pl.frag_p;
    if (ua.has_pf) ua.pf = ws_table(base, mb, pl.off_pf, nb, r, mi, r, 2, 16);
    ua.c1 = 1.0f - mu; ua.c2 = lr * scale;
    ua.M = mi; ua.N = ni; ua.rank = r;
    ORTHO_TRY(launch_dion_update(ua, bf, nb, s));
  }
  return ORTHO_OK;
}

// fp32-accurate Newton-Schulz (`precise`): the three products of every
// iteration on bf16x6 splits of fp32 operands.  The iterate ping-pongs between
// the fp32 slot and the region of the two bf16 copies (which holds M x ld_x
// fp32); the fp32 Gram takes the two transposed-copy regions and the fp32 Bp
// the A and Bp regions, so the workspace size does not depend on the dtype.
ortho_status run_ns_precise(const NsPlan& pl, int nb, const MatArg& tG, const MatArg& tOut,
                            bool out_bf, int32_t steps, float a, float b, float c, char* base,
                            hipStream_t s) {
  const size_t mb = pl.member_bytes;
  const int M = static_cast<int>(pl.M), N = static_cast<int>(pl.N);
  const MatArg xs[2] = {ws_table(base, mb, pl.off_x32, nb, pl.ld_x, M, N, 4, 16),
                        ws_table(base, mb, pl.off_xb0, nb, pl.ld_x, M, N, 4, 16)};
  float* partial = reinterpret_cast<float*>(base + pl.off_partial);
  float* scl = reinterpret_cast<float*>(base + pl.off_scale);
  SumsqArgs sa{};
  sa.g = tG; sa.partial = partial; sa.partial_stride = static_cast<int64_t>(mb / 4);
  sa.chunk = pl.part_chunk;
  ORTHO_TRY(launch_sumsq(sa, pl.nparts, nb, out_bf, s));
  ORTHO_TRY(launch_ns_scale(partial, static_cast<int64_t>(mb / 4), pl.nparts, scl,
                            static_cast<int64_t>(mb / 4), kNsEps, nb, s));
  MatArg none;
  memset(&none, 0, sizeof(none));
  NsInitArgs ia{};
  ia.g = tG; ia.x32 = xs[0]; ia.xb = none; ia.xbt = none;
  ia.scale = scl; ia.scale_stride = static_cast<int64_t>(mb / 4);
  ia.M = M; ia.N = N; ia.transposed = pl.transposed;
  ORTHO_TRY(launch_ns_init(ia, nb, out_bf, s));
  if (steps == 0) ORTHO_TRY(launch_ns_store(ia, tOut, nb, out_bf, s));
  Ns32Args na{};
  na.a32 = ws_table(base, mb, pl.off_xbt0, nb, pl.ld_xt, M, M, 4, 16);
  na.bp32 = ws_table(base, mb, pl.off_a, nb, pl.ld_xt, M, M, 4, 16);
  na.out = tOut;
  na.a = a; na.b = b; na.c = c;
  na.M = M; na.N = N; na.out_transposed = pl.transposed;
  for (int it = 0; it < steps; ++it) {
    na.x = xs[it & 1];
    na.xn = xs[(it & 1) ^ 1];
    na.last = it == steps - 1;
    ORTHO_TRY(launch_ns32_gram(na, nb, s));
    ORTHO_TRY(launch_ns32_poly(na, nb, s));
    ORTHO_TRY(launch_ns32_apply(na, out_bf, nb, s));
  }
  return ORTHO_OK;
}

// Gram Newton-Schulz (bf16-product path, Gram side M <= 128 with N >= 4 M).
// Wide G (no transposition): X_0 = sc G is never formed; A_0 = sc^2 G G^T
// (exact bf16 products for bf16 G, bf16x3 for fp32 G, k-split), the iteration
// on the M x M side gives sc Q_steps, and the apply writes (sc Q_steps) G to
// the caller's output.  Tall G: X_0 = sc G^T goes through the fp32 iterate
// first, and the output is written transposed back.
ortho_status run_ns_gram(const NsPlan& pl, int nb, const ortho_mat* G, int b0, const MatArg& tG,
                         const MatArg& tOut, bool g_bf, int32_t steps, float a, float b, float c,
                         char* base, hipStream_t s) {
  const size_t mb = pl.member_bytes;
  const int M = static_cast<int>(pl.M), N = static_cast<int>(pl.N);
  const MatArg x32 = ws_table(base, mb, pl.off_x32, nb, pl.ld_x, M, N, 4, 16);
  const MatArg tbp32 = ws_table(base, mb, pl.off_bp32, nb, pl.ld_xt, M, M, 4, 16);
  float* partial = reinterpret_cast<float*>(base + pl.off_partial);
  float* scl = reinterpret_cast<float*>(base + pl.off_scale);
  SumsqArgs sa{};
  sa.g = tG; sa.partial = partial; sa.partial_stride = static_cast<int64_t>(mb / 4);
  sa.chunk = pl.part_chunk;
  ORTHO_TRY(launch_sumsq(sa, pl.nparts, nb, g_bf, s));
  ORTHO_TRY(launch_ns_scale(partial, static_cast<int64_t>(mb / 4), pl.nparts, scl,
                            static_cast<int64_t>(mb / 4), kNsEps, nb, s));
  const bool direct = !pl.transposed;
  if (!direct) {
    MatArg none;
    memset(&none, 0, sizeof(none));
    NsInitArgs ia{};
    ia.g = tG; ia.x32 = x32; ia.xb = none; ia.xbt = none;
    ia.scale = scl; ia.scale_stride = static_cast<int64_t>(mb / 4);
    ia.M = M; ia.N = N; ia.transposed = 1;
    ORTHO_TRY(launch_ns_init(ia, nb, g_bf, s));
  }
  const MatArg gpart = ws_table(base, mb, pl.off_gns_part, nb, M, M, M, 4, 4);
  const int64_t slice = static_cast<int64_t>(M) * M;
  NsGramArgs g1{};
  g1.M = M; g1.K = N;
  if (direct) {
    // 16-byte row loads of bf16 G need 16-byte aligned rows
    g1.x = user_table(G, b0, nb, 16);
    ORTHO_TRY(launch_ns_gram_g(g1, g_bf, gpart, slice, pl.gns_splits, pl.gns_kchunk, nb, s));
  } else {
    g1.x = x32;
    ORTHO_TRY(launch_ns_gram_g(g1, false, gpart, slice, pl.gns_splits, pl.gns_kchunk, nb, s));
  }
  NsGramIterArgs gi{};
  gi.part = reinterpret_cast<const float*>(base + pl.off_gns_part);
  gi.part_member_stride = static_cast<int64_t>(mb / 4);
  gi.slice = slice; gi.splits = pl.gns_splits;
  gi.scale = direct ? scl : nullptr;
  gi.scale_stride = static_cast<int64_t>(mb / 4);
  gi.a0 = ws_table(base, mb, pl.off_gns_a0, nb, pl.gns_mp, pl.gns_mp, pl.gns_mp, 2, 16);
  gi.q = tbp32;
  gi.a = a; gi.b = b; gi.c = c;
  gi.M = M; gi.steps = steps;
  ORTHO_TRY(launch_ns_gram_iter(gi, nb, s));
  NsGramApplyArgs ap{};
  ap.q = tbp32; ap.x = direct ? tG : x32; ap.out = tOut;
  ap.M = M; ap.N = N; ap.out_transposed = !direct;
  ORTHO_TRY(launch_ns_gram_apply(ap, direct && g_bf, g_bf, nb, s));
  return ORTHO_OK;
}

// Newton-Schulz over a group.  The products use bf16 operands with fp32
// accumulation, or fp32-accurate split products when `precise` (fp32 inputs).
ortho_status run_ns(int32_t batch, const ortho_mat* G, const ortho_mat* Out, int32_t steps,
                    const float* abc, void* ws, void* stream, bool precise) {
  NsPlan pl;
  if (!plan_ns(G[0].rows, G[0].cols, batch, &pl)) return ORTHO_E_SHAPE;
  const bool bf = G[0].dtype == ORTHO_BF16;
  const float a = abc ? abc[0] : kMuonA, b = abc ? abc[1] : kMuonB, c = abc ? abc[2] : kMuonC;
  const hipStream_t s = as_stream(stream);
  char* base = static_cast<char*>(ws);
  const size_t mb = pl.member_bytes;
  const int M = static_cast<int>(pl.M), N = static_cast<int>(pl.N);
  const size_t gvec = bf ? 8 : 16;

  for (int b0 = 0; b0 < batch; b0 += pl.chunk) {
    const int nb = batch - b0 < pl.chunk ? batch - b0 : pl.chunk;
    const MatArg tG = user_table(G, b0, nb, gvec);
    const MatArg tOut = user_table(Out, b0, nb, gvec);
    if (precise) {
      const ortho_status st = run_ns_precise(pl, nb, tG, tOut, bf, steps, a, b, c, base, s);
      if (st != ORTHO_OK) return st;
      continue;
    }
    if (pl.gram_ns && steps > 0) {
      const ortho_status st = run_ns_gram(pl, nb, G, b0, tG, tOut, bf, steps, a, b, c, base, s);
      if (st != ORTHO_OK) return st;
      continue;
    }
    const MatArg x32 = ws_table(base, mb, pl.off_x32, nb, pl.ld_x, M, N, 4, 16);
    const MatArg xb[2] = {ws_table(base, mb, pl.off_xb0, nb, pl.ld_x, M, N, 2, 16),
                          ws_table(base, mb, pl.off_xb1, nb, pl.ld_x, M, N, 2, 16)};
    const MatArg xbt[2] = {ws_table(base, mb, pl.off_xbt0, nb, pl.ld_xt, N, M, 2, 16),
                           ws_table(base, mb, pl.off_xbt1, nb, pl.ld_xt, N, M, 2, 16)};
    const MatArg ta = ws_table(base, mb, pl.off_a, nb, pl.ld_xt, M, M, 2, 16);
    const MatArg tbp = ws_table(base, mb, pl.off_bp, nb, pl.ld_xt, M, M, 2, 16);
    const MatArg tbp32 = ws_table(base, mb, pl.off_bp32, nb, pl.ld_xt, M, M, 4, 16);
    float* partial = reinterpret_cast<float*>(base + pl.off_partial);
    float* scl = reinterpret_cast<float*>(base + pl.off_scale);

    SumsqArgs sa{};
    sa.g = tG; sa.partial = partial; sa.partial_stride = static_cast<int64_t>(mb / 4);
    sa.chunk = pl.part_chunk;
    ORTHO_TRY(launch_sumsq(sa, pl.nparts, nb, bf, s));
    ORTHO_TRY(launch_ns_scale(partial, static_cast<int64_t>(mb / 4), pl.nparts, scl,
                              static_cast<int64_t>(mb / 4), kNsEps, nb, s));
    // With a side of at most kNsSplitRows rows the apply takes both operands
    // from the fp32 iterate, so no transposed bf16 copy is written.
    const bool keep_t = M > kNsSplitRows;
    MatArg no_t;
    memset(&no_t, 0, sizeof(no_t));
    NsInitArgs ia{};
    ia.g = tG; ia.x32 = x32; ia.xb = xb[0]; ia.xbt = keep_t ? xbt[0] : no_t;
    ia.scale = scl; ia.scale_stride = static_cast<int64_t>(mb / 4);
    ia.M = M; ia.N = N; ia.transposed = pl.transposed;
    ORTHO_TRY(launch_ns_init(ia, nb, bf, s));
    if (steps == 0) ORTHO_TRY(launch_ns_store(ia, tOut, nb, bf, s));
    for (int it = 0; it < steps; ++it) {
      const int cur = it & 1;
      NsGramArgs g1{};
      g1.x = xb[cur]; g1.a = ta; g1.M = M; g1.K = N;
      // the fused reduce-and-polynomial kernel holds a side of at most 128 rows
      const bool small_poly = pl.gram_splits > 1 && c != 0.0f && M <= 128;
      if (pl.gram_splits > 1) {
        const MatArg gpart = ws_table(base, mb, pl.off_gpart, nb, M, M, M, 4, 16);
        const int64_t slice = static_cast<int64_t>(M) * M;
        ORTHO_TRY(launch_ns_gram_split(g1, gpart, slice, pl.gram_splits, pl.gram_kchunk, nb, s));
        if (small_poly) {
          // the reduce and the polynomial in one launch, one workgroup per member
          NsSmallPolyArgs sp{};
          sp.part = reinterpret_cast<const float*>(base + pl.off_gpart);
          sp.part_member_stride = static_cast<int64_t>(mb / 4);
          sp.slice = slice; sp.splits = pl.gram_splits; sp.M = M;
          sp.bp = tbp; sp.bp32 = tbp32; sp.b = b; sp.c = c;
          ORTHO_TRY(launch_ns_small_poly(sp, nb, s));
        } else {
          RedPiecesArgs rg{};
          rg.part = reinterpret_cast<const float*>(base + pl.off_gpart);
          rg.part_member_stride = static_cast<int64_t>(mb / 4);
          rg.slice = slice; rg.splits = pl.gram_splits; rg.rows = M; rg.cols = M;
          rg.out_bf16 = ta; rg.has_bf16 = 1;
          ORTHO_TRY(launch_reduce_pieces(rg, nb, s));
        }
      } else {
        ORTHO_TRY(launch_ns_gram(g1, nb, s));
      }
      if (!small_poly) {
        NsPolyArgs g2{};
        g2.a = ta; g2.bp = tbp; g2.bp32 = tbp32; g2.b = b; g2.c = c; g2.M = M;
        ORTHO_TRY(launch_ns_poly(g2, nb, s));
      }
      NsApplyArgs g3{};
      g3.bp = tbp; g3.xbt = keep_t ? xbt[cur] : no_t; g3.x32 = x32; g3.xb_next = xb[cur ^ 1];
      g3.xbt_next = keep_t ? xbt[cur ^ 1] : no_t; g3.out = tOut; g3.bp32 = tbp32; g3.a = a;
      g3.M = M; g3.N = N; g3.last = it == steps - 1; g3.out_transposed = pl.transposed;
      ORTHO_TRY(launch_ns_apply(g3, bf, nb, s));
    }
  }
  return ORTHO_OK;
}

// Muon step on each member: M = mu M + G; U = Newton-Schulz of M (fp32, in
// the workspace after the Newton-Schulz part); X = X - lr * scale * U.  Launch
// chunks as in run_ns, so U needs one slot per member of a chunk.
ortho_status run_muon(int32_t batch, const ortho_mat* X, const ortho_mat* G, const ortho_mat* M,
                      int32_t steps, const float* abc, float mu, float lr, float scale, void* ws,
                      void* stream, bool row_norm = false) {
  MuonPlan pl;
  const int64_t m = X[0].rows, n = X[0].cols;
  if (!plan_muon(m, n, batch, &pl, row_norm)) return ORTHO_E_SHAPE;
  const bool bf = X[0].dtype == ORTHO_BF16;
  const hipStream_t s = as_stream(stream);
  char* base = static_cast<char*>(ws);
  const size_t gvec = bf ? 8 : 16;
  const int chunk = pl.ns.chunk;
  for (int b0 = 0; b0 < batch; b0 += chunk) {
    const int nb = batch - b0 < chunk ? batch - b0 : chunk;
    MuonArgs a{};
    a.m = user_table(M, b0, nb, 16);
    a.g = user_table(G, b0, nb, gvec);
    a.x = user_table(X, b0, nb, gvec);
    a.u = ws_table(base, pl.u_bytes, pl.off_u, nb, pl.ld_u, static_cast<int>(m), static_cast<int>(n),
                   4, 16);
    a.mu = mu; a.c = lr * scale;
    a.rows = static_cast<int>(m); a.cols = static_cast<int>(n);
    ORTHO_TRY(launch_muon_momentum(a, bf, nb, s));
    ortho_mat us[kMaxBatch];
    for (int i = 0; i < nb; ++i)
      us[i] = ortho_mat{base + pl.off_u + i * pl.u_bytes, m, n, pl.ld_u, ORTHO_F32};
    // the fp32 momentum is orthogonalised with fp32-accurate products when
    // the weights are fp32, with bf16 products when they are bf16
    const ortho_status st = run_ns(nb, M + b0, us, steps, abc, ws, stream, !bf);
    if (st != ORTHO_OK) return st;
    if (row_norm) {
      // NorMuon: every row of U scaled to the common norm |U|_F / sqrt(m)
      RowNormArgs rn{};
      rn.u = a.u;
      rn.rowf = reinterpret_cast<float*>(base + pl.off_rowf);
      rn.rowf_stride = static_cast<int64_t>(pl.rowf_bytes / 4);
      rn.rows = a.rows; rn.cols = a.cols;
      ORTHO_TRY(launch_row_factors(rn, nb, s));
      a.rowf = rn.rowf;
      a.rowf_stride = rn.rowf_stride;
    }
    ORTHO_TRY(launch_muon_update(a, bf, nb, s));
  }
  return ORTHO_OK;
}

ortho_status run_dion2(const ortho_mat& X, const ortho_mat& G, const ortho_mat& M, int32_t k,
                       int32_t steps, const float* abc, float mu, float lr, float scale,
                       int32_t* selected, void* ws, void* stream) {
  Dion2Plan pl;
  if (!plan_dion2(X.rows, X.cols, k, &pl)) return ORTHO_E_SHAPE;
  const bool bf = X.dtype == ORTHO_BF16;
  const hipStream_t s = as_stream(stream);
  char* base = static_cast<char*>(ws);
  const size_t gvec = bf ? 8 : 16;
  const int m = static_cast<int>(X.rows), n = static_cast<int>(X.cols);
  Dion2Args a{};
  a.x = user_table(&X, 0, 1, gvec);
  a.g = user_table(&G, 0, 1, gvec);
  a.m = user_table(&M, 0, 1, 16);
  a.blk = ws_table(base, 0, pl.off_blk, 1, pl.ld_blk, k, n, 4, 16);
  a.norms = reinterpret_cast<float*>(base + pl.off_norms);
  a.rank = reinterpret_cast<int*>(base + pl.off_rank);
  a.sel = reinterpret_cast<int*>(base + pl.off_sel);
  a.vec_stride = 0;
  a.rows = m; a.cols = n; a.k = k;
  a.mu = mu; a.c = lr * scale;
  ORTHO_TRY(launch_dion2_select(a, bf, 1, s));
  // Newton-Schulz of the block in place: fp32-accurate products for fp32
  // weights, bf16 products for bf16 weights
  const ortho_mat blk{base + pl.off_blk, k, n, pl.ld_blk, ORTHO_F32};
  const ortho_status st = run_ns(1, &blk, &blk, steps, abc, ws, stream, !bf);
  if (st != ORTHO_OK) return st;
  ORTHO_TRY(launch_dion2_update(a, bf, 1, s));
  if (selected)
    ORTHO_TRY(hipMemcpyAsync(selected, a.sel, static_cast<size_t>(k) * 4, hipMemcpyDeviceToDevice, s));
  return ORTHO_OK;
}

}  // namespace

namespace ortho {
ortho_status dion_run(int32_t batch, const ortho_mat* X, const ortho_mat* G, const ortho_mat* M,
                      const ortho_mat* Q, int32_t r, float mu, float lr, float scale, void* ws,
                      void* stream) {
  return run_dion(batch, X, G, M, Q, r, mu, lr, scale, nullptr, nullptr, nullptr, ws, stream);
}
}  // namespace ortho

extern "C" {

size_t ortho_muon_workspace_size(int64_t m, int64_t n, int32_t batch) {
  MuonPlan p;
  return plan_muon(m, n, batch, &p) ? p.total_bytes : 0;
}

ortho_status muon_step(ortho_mat X, ortho_mat G, ortho_mat M, int32_t steps, const float* abc,
                       float mu, float lr, float scale, void* ws, size_t ws_bytes, void* stream) {
  const ortho_status st = validate_muon(1, &X, &G, &M, steps, abc, mu, lr, scale, ws, ws_bytes);
  if (st != ORTHO_OK) return st;
  return run_muon(1, &X, &G, &M, steps, abc, mu, lr, scale, ws, stream);
}

ortho_status muon_step_batched(int32_t batch, const ortho_mat* X, const ortho_mat* G,
                               const ortho_mat* M, int32_t steps, const float* abc, float mu,
                               float lr, float scale, void* ws, size_t ws_bytes, void* stream) {
  const ortho_status st = validate_muon(batch, X, G, M, steps, abc, mu, lr, scale, ws, ws_bytes);
  if (st != ORTHO_OK) return st;
  return run_muon(batch, X, G, M, steps, abc, mu, lr, scale, ws, stream);
}

size_t ortho_normuon_workspace_size(int64_t m, int64_t n, int32_t batch) {
  MuonPlan p;
  return plan_muon(m, n, batch, &p, true) ? p.total_bytes : 0;
}

ortho_status normuon_step(ortho_mat X, ortho_mat G, ortho_mat M, int32_t steps, const float* abc,
                          float mu, float lr, float scale, void* ws, size_t ws_bytes,
                          void* stream) {
  const ortho_status st =
      validate_muon(1, &X, &G, &M, steps, abc, mu, lr, scale, ws, ws_bytes, true);
  if (st != ORTHO_OK) return st;
  return run_muon(1, &X, &G, &M, steps, abc, mu, lr, scale, ws, stream, true);
}

ortho_status normuon_step_batched(int32_t batch, const ortho_mat* X, const ortho_mat* G,
                                  const ortho_mat* M, int32_t steps, const float* abc, float mu,
                                  float lr, float scale, void* ws, size_t ws_bytes, void* stream) {
  const ortho_status st =
      validate_muon(batch, X, G, M, steps, abc, mu, lr, scale, ws, ws_bytes, true);
  if (st != ORTHO_OK) return st;
  return run_muon(batch, X, G, M, steps, abc, mu, lr, scale, ws, stream, true);
}

size_t ortho_dion_workspace_size(int64_t m, int64_t n, int32_t r, int32_t batch) {
  DionPlan p;
  return plan_dion(m, n, r, batch, &p) ? p.total_bytes : 0;
}

size_t ortho_ns_workspace_size(int64_t m, int64_t n, int32_t batch) {
  NsPlan p;
  return plan_ns(m, n, batch, &p) ? p.total_bytes : 0;
}

ortho_status dion_step_ex(ortho_mat X, ortho_mat G, ortho_mat M, ortho_mat Q, int32_t r, float mu,
                          float lr, float scale, const ortho_mat* P_out, const ortho_mat* R_out,
                          int32_t* dev_status, void* ws, size_t ws_bytes, void* stream) {
  const ortho_status st =
      validate_dion(1, &X, &G, &M, &Q, r, mu, lr, scale, P_out, R_out, ws, ws_bytes);
  if (st != ORTHO_OK) return st;
  return run_dion(1, &X, &G, &M, &Q, r, mu, lr, scale, P_out, R_out, dev_status, ws, stream);
}

ortho_status dion_step(ortho_mat X, ortho_mat G, ortho_mat M, ortho_mat Q, int32_t r, float mu,
                       float lr, void* ws, size_t ws_bytes, void* stream) {
  return dion_step_ex(X, G, M, Q, r, mu, lr, 1.0f, nullptr, nullptr, nullptr, ws, ws_bytes, stream);
}

ortho_status dion_step_batched(int32_t batch, const ortho_mat* X, const ortho_mat* G,
                               const ortho_mat* M, const ortho_mat* Q, int32_t r, float mu, float lr,
                               float scale, int32_t* dev_status, void* ws, size_t ws_bytes,
                               void* stream) {
  const ortho_status st =
      validate_dion(batch, X, G, M, Q, r, mu, lr, scale, nullptr, nullptr, ws, ws_bytes);
  if (st != ORTHO_OK) return st;
  return run_dion(batch, X, G, M, Q, r, mu, lr, scale, nullptr, nullptr, dev_status, ws, stream);
}

ortho_status newton_schulz(ortho_mat G, ortho_mat Out, int32_t steps, const float* abc, void* ws,
                           size_t ws_bytes, void* stream) {
  const ortho_status st = validate_ns(1, &G, &Out, steps, abc, ws, ws_bytes);
  if (st != ORTHO_OK) return st;
  return run_ns(1, &G, &Out, steps, abc, ws, stream, G.dtype == ORTHO_F32);
}

ortho_status newton_schulz_batched(int32_t batch, const ortho_mat* G, const ortho_mat* Out,
                                   int32_t steps, const float* abc, void* ws, size_t ws_bytes,
                                   void* stream) {
  const ortho_status st = validate_ns(batch, G, Out, steps, abc, ws, ws_bytes);
  if (st != ORTHO_OK) return st;
  return run_ns(batch, G, Out, steps, abc, ws, stream, G[0].dtype == ORTHO_F32);
}

size_t ortho_dion2_workspace_size(int64_t m, int64_t n, int32_t k) {
  Dion2Plan p;
  return plan_dion2(m, n, k, &p) ? p.total_bytes : 0;
}

ortho_status dion2_step(ortho_mat X, ortho_mat G, ortho_mat M, int32_t k, int32_t steps,
                        const float* abc, float mu, float lr, float scale, int32_t* selected,
                        void* ws, size_t ws_bytes, void* stream) {
  const ortho_status st = validate_dion2(X, G, M, k, steps, abc, mu, lr, scale, ws, ws_bytes);
  if (st != ORTHO_OK) return st;
  return run_dion2(X, G, M, k, steps, abc, mu, lr, scale, selected, ws, stream);
}

const char* ortho_status_str(int32_t status) {
  switch (status) {
    case ORTHO_OK: return "ok";
    case ORTHO_E_NULL: return "a required pointer is NULL";
    case ORTHO_E_SHAPE: return "matrix shapes disagree or a dimension is out of range";
    case ORTHO_E_DTYPE: return "unsupported or mismatched dtype";
    case ORTHO_E_RANK: return "rank r outside [1, min(m, n)] or different from Q.cols";
    case ORTHO_E_LAYOUT: return "leading dimension smaller than cols, or differs within a group";
    case ORTHO_E_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case ORTHO_E_PARAM: return "invalid scalar parameter (mu, lr, scale, abc, steps or batch)";
    case ORTHO_E_HIP: return "a HIP launch failed";
    case ORTHO_E_SCRATCH:
      return "the problem needs more scratch memory than the no-allocation entry point holds";
    default: return "unknown status";
  }
}

int32_t ortho_abi_version(void) { return ORTHO_ABI_VERSION; }

}  // extern "C"
