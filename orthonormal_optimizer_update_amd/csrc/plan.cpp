// Workspace planning and argument validation (host only, no HIP calls).
#include "plan.h"

#include <math.h>

namespace ortho {

namespace {

constexpr int64_t kMaxDim = (int64_t{1} << 30);   // rows/cols index with int32
constexpr int kTargetWorkgroups = 512;            // ~2 workgroups per CU
constexpr int kMinSplitK = 256;                   // rows per split-K slice, at least

size_t align_up(size_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Split a reduction of length K so that tiles * members * splits reaches the
// target, with each slice a multiple of 32 and at least kMinSplitK long.
void choose_split(int64_t K, int64_t tiles, int members, int* splits, int* kchunk,
                  int64_t min_k = kMinSplitK, int64_t multiple = 32) {
  int64_t want = cdiv(kTargetWorkgroups, tiles * members);
  int64_t cap = K / min_k;
  if (cap < 1) cap = 1;
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  int64_t kc = cdiv(cdiv(K, want), multiple) * multiple;
  *kchunk = static_cast<int>(kc);
  *splits = static_cast<int>(cdiv(K, kc));
}

// Slices of 64 (a multiple of 64 when the kernel's k step is 64) for
// contractions with few output tiles.
constexpr int64_t kMinSplitKSmall = 64;

// Split nkt k tiles so that tiles * members * splits reaches one workgroup per
// CU of the 256 x 256 kernel, with at least 8 k tiles per split.
void choose_split_tiles(int64_t nkt, int64_t tiles, int members, int* splits, int* kchunk) {
  int64_t want = cdiv(256, tiles * members);
  int64_t cap = nkt / 8;
  if (cap < 1) cap = 1;
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  const int64_t kc = cdiv(nkt, want);
  *kchunk = static_cast<int>(kc);
  *splits = static_cast<int>(cdiv(nkt, kc));
}

bool finite(float v) { return isfinite(v) != 0; }

ortho_status check_mat(const ortho_mat& a) {
  if (a.data == nullptr) return ORTHO_E_NULL;
  if (a.rows < 1 || a.cols < 1 || a.rows > kMaxDim || a.cols > kMaxDim) return ORTHO_E_SHAPE;
  if (a.ld < a.cols || a.ld > (int64_t{1} << 40)) return ORTHO_E_LAYOUT;
  if (a.dtype != ORTHO_F32 && a.dtype != ORTHO_BF16) return ORTHO_E_DTYPE;
  return ORTHO_OK;
}

bool same_geometry(const ortho_mat& a, const ortho_mat& b) {
  return a.rows == b.rows && a.cols == b.cols && a.dtype == b.dtype;
}

}  // namespace

bool plan_dion(int64_t m, int64_t n, int32_t r, int32_t batch, DionPlan* p) {
  if (m < 1 || n < 1 || r < 1 || batch < 1 || m > kMaxDim || n > kMaxDim) return false;
  if (r > m || r > n || r > 16384) return false;
  DionPlan d{};
  d.m = m;
  d.n = n;
  d.r = r;
  d.chunk = batch < kMaxMembersPerLaunch ? batch : kMaxMembersPerLaunch;
  d.small_left = few_tiles(m, r, d.chunk);
  d.small_right = few_tiles(n, r, d.chunk);
  if (d.small_left)
    choose_split(n, cdiv(m, 64) * cdiv(r, 64), d.chunk, &d.split_left, &d.kchunk_left,
                 kMinSplitKSmall, 64);
  else
    choose_split(n, cdiv(m, 128) * cdiv(r, 128), d.chunk, &d.split_left, &d.kchunk_left);
  if (d.small_right)
    choose_split(m, cdiv(n, 64) * cdiv(r, 64), d.chunk, &d.split_right, &d.kchunk_right,
                 kMinSplitKSmall, 64);
  else
    choose_split(m, cdiv(n, 128) * cdiv(r, 128), d.chunk, &d.split_right, &d.kchunk_right);
  const int64_t tg = cdiv(r, 64);
  const bool small_gram = tg * (tg + 1) / 2 * d.chunk < 64;
  choose_split(m, tg * (tg + 1) / 2, d.chunk, &d.split_gram, &d.kchunk_gram,
               small_gram ? kMinSplitKSmall : kMinSplitK);
  d.gram_big = gram_big_tiles(r, d.chunk);
  if (d.gram_big) {
    // 128 x 128 fp64 Gram tiles: at most one workgroup per CU (a second round
    // on a few CUs would double the time), at least eight 32-row k tiles each
    const int64_t tb = r / 128, tiles = tb * (tb + 1) / 2 * d.chunk;
    int64_t want = 256 / tiles, cap = m / 256;
    if (cap < 1) cap = 1;
    if (want > cap) want = cap;
    if (want < 1) want = 1;
    const int64_t kc = cdiv(cdiv(m, want), 32) * 32;
    d.kchunk_gram = static_cast<int>(kc);
    d.split_gram = static_cast<int>(cdiv(m, kc));
  }
  if (gram_tn_small_tiles(r)) {
    const int64_t t64 = cdiv(r, 64) * cdiv(r, 64);
    choose_split(m, t64, d.chunk, &d.split_gram2, &d.kchunk_gram2,
                 t64 * d.chunk < 64 ? kMinSplitKSmall : kMinSplitK, 64);
  } else {
    choose_split(m, cdiv(r, 128) * cdiv(r, 128), d.chunk, &d.split_gram2, &d.kchunk_gram2);
  }
  d.nrb = static_cast<int>(cdiv(n, 64));
  d.rp = cdiv(r, 4) * 4;
  const size_t mr = static_cast<size_t>(m) * r, nr = static_cast<size_t>(n) * r;
  const size_t mrp = static_cast<size_t>(m) * d.rp, nrp = static_cast<size_t>(n) * d.rp;
  const size_t rr = static_cast<size_t>(r) * r;
  size_t part = static_cast<size_t>(d.split_left) * mr * 4;
  const size_t pr = static_cast<size_t>(d.split_right) * nr * 4;
  const size_t pg = static_cast<size_t>(d.split_gram) * rr * 8;
  const size_t pg2 = static_cast<size_t>(d.split_gram2) * rr * 4;
  if (pr > part) part = pr;
  if (pg > part) part = pg;
  if (pg2 > part) part = pg2;
  // Up to r = 512 the sweeps stream M and G (below); from r = 1024 on they
  // are product-bound and a pass that stores the pieces of B pays for itself.
  d.stream_sweeps = (r == 64 || r == 128 || r == 256 || r == 512) && m % 64 == 0 && n % 64 == 0;
  d.fast_sweeps = !d.stream_sweeps && m % 256 == 0 && n % 256 == 0 && r % 256 == 0 && r >= 512;
  if (d.fast_sweeps) {
    choose_split_tiles(3 * n / 64, (m / 256) * (r / 256), d.chunk, &d.split_fl, &d.kchunk_fl);
    choose_split_tiles(3 * m / 64, (n / 256) * (r / 256), d.chunk, &d.split_fr, &d.kchunk_fr);
    const size_t pfl = static_cast<size_t>(d.split_fl) * mr * 4;
    const size_t pfr = static_cast<size_t>(d.split_fr) * nr * 4;
    if (pfl > part) part = pfl;
    if (pfr > part) part = pfr;
  }
  // The orthonormalisation products on the 256 x 256 kernel: with the piece
  // sweeps, their pieces live in the B-piece buffers (three m x r and r x r
  // sets fit when 3 r <= n); with the streaming sweeps at r = 512, in regions
  // of their own.
  d.ortho64 = r <= kOrtho64MaxRank;
  d.small_ortho = r <= 64 && m <= kSmallOrthoMaxRows;
  d.fast_ortho = !d.ortho64 && (d.fast_sweeps || (d.stream_sweeps && r == 512 && m % 256 == 0)) &&
                 3 * r <= n;
  if (d.fast_ortho) {
    choose_split_tiles(6 * r / 64, (m / 256) * (r / 256), d.chunk, &d.split_ap6, &d.kchunk_ap6);
    choose_split_tiles(3 * r / 64, (m / 256) * (r / 256), d.chunk, &d.split_ap3, &d.kchunk_ap3);
    choose_split_tiles(3 * m / 64, (r / 256) * (r / 256), d.chunk, &d.split_e, &d.kchunk_e);
    const size_t pa = static_cast<size_t>(d.split_ap6 > d.split_ap3 ? d.split_ap6 : d.split_ap3) * mr * 4;
    const size_t pe = static_cast<size_t>(d.split_e) * rr * 4;
    if (pa > part) part = pa;
    if (pe > part) part = pe;
  }
  if (d.stream_sweeps) {
    // one 128-row workgroup per CU over the chunk's members, at least 128 k
    // (eight 16-deep stages) per slice
    auto pick = [&](int64_t rows, int64_t K, int* splits, int* kchunk) {
      int64_t want = cdiv(256, cdiv(rows, 128) * d.chunk), cap = K / 128;
      if (want > cap) want = cap;
      if (want < 1) want = 1;
      const int64_t kc = cdiv(cdiv(K, want), 16) * 16;
      *kchunk = static_cast<int>(kc);
      *splits = static_cast<int>(cdiv(K, kc));
    };
    pick(m, n, &d.split_sl, &d.kchunk_sl);
    pick(n, m, &d.split_sr, &d.kchunk_sr);
    const size_t psl = static_cast<size_t>(d.split_sl) * mr * 4;
    const size_t psr = static_cast<size_t>(d.split_sr) * nr * 4;
    if (psl > part) part = psl;
    if (psr > part) part = psr;
  }
  size_t o = 0;
  d.off_pt = o;    o = align_up(o + mrp * 4);
  d.off_p1 = o;    o = align_up(o + mrp * 4);
  d.off_part = o;  o = align_up(o + part);
  d.off_s = o;     o = align_up(o + rr * 8);
  d.off_x = o;     o = align_up(o + rr * 8);
  d.off_d = o;     o = align_up(o + static_cast<size_t>(r) * 8);
  d.off_tt = o;    o = align_up(o + rr * 4);
  d.off_r = o;     o = align_up(o + nrp * 4);
  d.off_colsq = o; o = align_up(o + static_cast<size_t>(d.nrb) * r * 4);
  d.rpb = cdiv(r, 8) * 8;
  d.off_pb = o;    o = align_up(o + static_cast<size_t>(m) * d.rpb * 2);
  d.off_rb = o;    o = align_up(o + static_cast<size_t>(n) * d.rpb * 2);
  d.off_qb = o;    o = align_up(o + static_cast<size_t>(n) * d.rpb * 2);
  d.frag_p = (r == 256 || r == 512) && m % 128 == 0;
  d.off_pf = o;    o = align_up(o + (d.frag_p ? mr * 2 : 0));
  if (d.fast_sweeps) {
    const size_t mn2 = static_cast<size_t>(m) * n * 2;
    d.off_bhi = o;   o = align_up(o + mn2);
    d.off_blo = o;   o = align_up(o + mn2);
    d.off_bhit = o;  o = align_up(o + mn2);
    d.off_blot = o;  o = align_up(o + mn2);
  } else if (d.fast_ortho) {
    // the three m x r and r x r piece sets of the orthonormalisation products
    d.off_bhi = o;   o = align_up(o + 3 * mr * 2);
    d.off_blo = o;   o = align_up(o + 3 * rr * 2);
  }
  if (d.fast_sweeps || d.stream_sweeps) {
    d.off_qhit = o;  o = align_up(o + nr * 2);
    d.off_qlot = o;  o = align_up(o + nr * 2);
    d.off_phit = o;  o = align_up(o + mr * 2);
    d.off_plot = o;  o = align_up(o + mr * 2);
  }
  d.member_bytes = o;
  d.total_bytes = o * static_cast<size_t>(d.chunk);
  *p = d;
  return true;
}

bool plan_ns(int64_t m, int64_t n, int32_t batch, NsPlan* p) {
  if (m < 1 || n < 1 || batch < 1 || m > kMaxDim || n > kMaxDim) return false;
  NsPlan s{};
  s.transposed = m > n;
  s.M = s.transposed ? n : m;
  s.N = s.transposed ? m : n;
  s.chunk = batch < kMaxMembersPerLaunch ? batch : kMaxMembersPerLaunch;
  // sum-of-squares blocks: whole rows, about 16K elements each, at most 2048
  int64_t parts = cdiv(m * n, 16384);
  if (parts > 2048) parts = 2048;
  if (parts > m) parts = m;
  if (parts < 1) parts = 1;
  s.part_chunk = cdiv(m, parts);
  s.nparts = static_cast<int>(cdiv(m, s.part_chunk));
  s.ld_x = cdiv(s.N, 8) * 8;
  s.ld_xt = cdiv(s.M, 8) * 8;
  const size_t mn = static_cast<size_t>(s.M) * s.ld_x, nm = static_cast<size_t>(s.N) * s.ld_xt;
  const size_t mm = static_cast<size_t>(s.M) * s.ld_xt;
  size_t o = 0;
  s.off_x32 = o;     o = align_up(o + mn * 4);
  s.off_xb0 = o;     o = align_up(o + mn * 2);
  s.off_xb1 = o;     o = align_up(o + mn * 2);
  s.off_xbt0 = o;    o = align_up(o + nm * 2);
  s.off_xbt1 = o;    o = align_up(o + nm * 2);
  s.off_a = o;       o = align_up(o + mm * 2);
  s.off_bp = o;      o = align_up(o + mm * 2);
  // fp32 copy of Bp, used by the split-precision apply when M <= 128
  s.off_bp32 = o;    o = align_up(o + (s.M <= 128 ? mm * 4 : 0));
  s.gram_splits = 1;
  s.gram_kchunk = 0;
  // A Gram side of 64 or 128 rows is one 128 x 128 tile per member; a larger
  // side whose symmetric 256 x 256 grid gives under 128 workgroups runs on
  // 128 x 128 tiles (see the Newton-Schulz launchers).  Both split k (the
  // fixed-order reduce takes sides that are multiples of 64).
  const int64_t t256 = cdiv(s.M, 256), t128 = cdiv(s.M, 128);
  const bool few = s.M > 128 && s.M % 64 == 0 && t256 * (t256 + 1) / 2 * s.chunk < 128;
  if ((s.M <= 128 && s.M % 64 == 0) || few) {
    // one workgroup per CU over the chunk's members, at least 8 k steps of 32 each
    int64_t want = cdiv(256, s.chunk * (s.M <= 128 ? 1 : t128 * t128)), cap = s.N / 256;
    if (want > cap) want = cap;
    if (want > 1) {
      s.gram_kchunk = static_cast<int>(cdiv(cdiv(s.N, want), 32) * 32);
      s.gram_splits = static_cast<int>(cdiv(s.N, s.gram_kchunk));
    }
  }
  s.off_gpart = o;   o = align_up(o + (s.gram_splits > 1 ? static_cast<size_t>(s.gram_splits) * mm * 4 : 0));
  // Gram Newton-Schulz when the Gram side is small against the long side
  s.gram_ns = s.M <= 128 && s.N >= 4 * s.M;
  s.gns_splits = 1;
  s.gns_kchunk = static_cast<int>(cdiv(s.N, 32) * 32);
  s.gns_mp = s.M <= 64 ? 64 : 128;
  if (s.gram_ns) {
    // one workgroup per CU over the chunk's members, at least 8 k steps of 32
    int64_t want = cdiv(256, s.chunk), cap = s.N / 256;
    if (want > cap) want = cap;
    if (want > 1) {
      s.gns_kchunk = static_cast<int>(cdiv(cdiv(s.N, want), 32) * 32);
      s.gns_splits = static_cast<int>(cdiv(s.N, s.gns_kchunk));
    }
  }
  const size_t gmm = static_cast<size_t>(s.M) * s.M;
  s.off_gns_part = o;
  o = align_up(o + (s.gram_ns ? static_cast<size_t>(s.gns_splits) * gmm * 4 : 0));
  s.off_gns_a0 = o;
  o = align_up(o + (s.gram_ns ? static_cast<size_t>(s.gns_mp) * s.gns_mp * 6 : 0));
  s.off_partial = o; o = align_up(o + static_cast<size_t>(s.nparts) * 4);
  s.off_scale = o;   o = align_up(o + 4);
  s.member_bytes = o;
  s.total_bytes = o * static_cast<size_t>(s.chunk);
  *p = s;
  return true;
}

bool plan_muon(int64_t m, int64_t n, int32_t batch, MuonPlan* p, bool row_norm) {
  MuonPlan d{};
  if (!plan_ns(m, n, batch, &d.ns)) return false;
  d.ld_u = cdiv(n, 4) * 4;
  // The step runs Newton-Schulz once per launch chunk, each call laid out for
  // its own member count; U goes after the larger of the full and the last
  // chunk's layouts.
  size_t ns_bytes = d.ns.total_bytes;
  const int32_t last = batch % d.ns.chunk;
  if (last != 0) {
    NsPlan tail;
    if (!plan_ns(m, n, last, &tail)) return false;
    if (tail.total_bytes > ns_bytes) ns_bytes = tail.total_bytes;
  }
  d.off_u = align_up(ns_bytes);
  d.u_bytes = align_up(static_cast<size_t>(m) * d.ld_u * 4);
  d.off_rowf = align_up(d.off_u + d.u_bytes * static_cast<size_t>(d.ns.chunk));
  d.rowf_bytes = row_norm ? align_up(static_cast<size_t>(m) * 4) : 0;
  d.total_bytes = row_norm ? d.off_rowf + d.rowf_bytes * static_cast<size_t>(d.ns.chunk)
                           : d.off_u + d.u_bytes * static_cast<size_t>(d.ns.chunk);
  *p = d;
  return true;
}

bool plan_dion2(int64_t m, int64_t n, int32_t k, Dion2Plan* p) {
  if (m < 1 || n < 1 || k < 1 || k > m || m > 65535 || n > kMaxDim) return false;
  Dion2Plan d{};
  if (!plan_ns(k, n, 1, &d.ns)) return false;
  d.ld_blk = cdiv(n, 4) * 4;
  size_t o = align_up(d.ns.total_bytes);
  d.off_blk = o;    o = align_up(o + static_cast<size_t>(k) * d.ld_blk * 4);
  d.off_norms = o;  o = align_up(o + static_cast<size_t>(m) * 4);
  d.off_rank = o;   o = align_up(o + static_cast<size_t>(m) * 4);
  d.off_sel = o;    o = align_up(o + static_cast<size_t>(k) * 4);
  d.total_bytes = o;
  *p = d;
  return true;
}

ortho_status validate_dion2(const ortho_mat& X, const ortho_mat& G, const ortho_mat& M, int32_t k,
                            int32_t steps, const float* abc, float mu, float lr, float scale,
                            const void* ws, size_t ws_bytes) {
  if (steps < 0) return ORTHO_E_PARAM;
  if (!(mu >= 0.f && mu <= 1.f) || !finite(lr) || !finite(scale)) return ORTHO_E_PARAM;
  if (abc && (!finite(abc[0]) || !finite(abc[1]) || !finite(abc[2]))) return ORTHO_E_PARAM;
  ortho_status st;
  if ((st = check_mat(X)) != ORTHO_OK) return st;
  if ((st = check_mat(G)) != ORTHO_OK) return st;
  if ((st = check_mat(M)) != ORTHO_OK) return st;
  if (G.dtype != X.dtype || M.dtype != ORTHO_F32) return ORTHO_E_DTYPE;
  if (G.rows != X.rows || G.cols != X.cols || M.rows != X.rows || M.cols != X.cols)
    return ORTHO_E_SHAPE;
  if (X.rows > 65535) return ORTHO_E_SHAPE;
  if (k < 1 || k > X.rows) return ORTHO_E_RANK;
  Dion2Plan plan;
  if (!plan_dion2(X.rows, X.cols, k, &plan)) return ORTHO_E_SHAPE;
  if (ws == nullptr || ws_bytes < plan.total_bytes) return ORTHO_E_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % kWsAlign != 0) return ORTHO_E_WORKSPACE;
  return ORTHO_OK;
}

ortho_status validate_dion(int32_t batch, const ortho_mat* X, const ortho_mat* G, const ortho_mat* M,
                           const ortho_mat* Q, int32_t r, float mu, float lr, float scale,
                           const ortho_mat* P_out, const ortho_mat* R_out, const void* ws,
                           size_t ws_bytes) {
  if (batch < 1) return ORTHO_E_PARAM;
  if (!X || !G || !M || !Q) return ORTHO_E_NULL;
  if (!(mu >= 0.f && mu <= 1.f) || !finite(lr) || !finite(scale)) return ORTHO_E_PARAM;
  for (int32_t b = 0; b < batch; ++b) {
    ortho_status st;
    if ((st = check_mat(X[b])) != ORTHO_OK) return st;
    if ((st = check_mat(G[b])) != ORTHO_OK) return st;
    if ((st = check_mat(M[b])) != ORTHO_OK) return st;
    if ((st = check_mat(Q[b])) != ORTHO_OK) return st;
    if (G[b].dtype != X[b].dtype || M[b].dtype != ORTHO_F32 || Q[b].dtype != ORTHO_F32)
      return ORTHO_E_DTYPE;
    if (G[b].rows != X[b].rows || G[b].cols != X[b].cols || M[b].rows != X[b].rows ||
        M[b].cols != X[b].cols || Q[b].rows != X[b].cols)
      return ORTHO_E_SHAPE;
    // every member's right factor has exactly r columns (the kernels read and
    // write r columns of each)
    if (Q[b].cols != r) return ORTHO_E_RANK;
    if (b > 0) {
      if (!same_geometry(X[b], X[0])) return ORTHO_E_SHAPE;
      if (X[b].ld != X[0].ld || G[b].ld != G[0].ld || M[b].ld != M[0].ld || Q[b].ld != Q[0].ld)
        return ORTHO_E_LAYOUT;
    }
  }
  const int64_t m = X[0].rows, n = X[0].cols;
  if (r < 1 || r > m || r > n || r > 16384 || Q[0].cols != r) return ORTHO_E_RANK;
  if (P_out) {
    ortho_status st = check_mat(*P_out);
    if (st != ORTHO_OK) return st;
    if (P_out->dtype != ORTHO_F32) return ORTHO_E_DTYPE;
    if (P_out->rows != m || P_out->cols != r) return ORTHO_E_SHAPE;
  }
  if (R_out) {
    ortho_status st = check_mat(*R_out);
    if (st != ORTHO_OK) return st;
    if (R_out->dtype != ORTHO_F32) return ORTHO_E_DTYPE;
    if (R_out->rows != n || R_out->cols != r) return ORTHO_E_SHAPE;
  }
  DionPlan plan;
  if (!plan_dion(m, n, r, batch, &plan)) return ORTHO_E_SHAPE;
  if (ws == nullptr || ws_bytes < plan.total_bytes) return ORTHO_E_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % kWsAlign != 0) return ORTHO_E_WORKSPACE;
  return ORTHO_OK;
}

ortho_status validate_ns(int32_t batch, const ortho_mat* G, const ortho_mat* Out, int32_t steps,
                         const float* abc, const void* ws, size_t ws_bytes) {
  if (batch < 1 || steps < 0) return ORTHO_E_PARAM;
  if (!G || !Out) return ORTHO_E_NULL;
  if (abc && (!finite(abc[0]) || !finite(abc[1]) || !finite(abc[2]))) return ORTHO_E_PARAM;
  for (int32_t b = 0; b < batch; ++b) {
    ortho_status st;
    if ((st = check_mat(G[b])) != ORTHO_OK) return st;
    if ((st = check_mat(Out[b])) != ORTHO_OK) return st;
    if (!same_geometry(G[b], Out[b])) return Out[b].dtype != G[b].dtype ? ORTHO_E_DTYPE : ORTHO_E_SHAPE;
    if (b > 0) {
      if (!same_geometry(G[b], G[0])) return ORTHO_E_SHAPE;
      if (G[b].ld != G[0].ld || Out[b].ld != Out[0].ld) return ORTHO_E_LAYOUT;
    }
  }
  NsPlan plan;
  if (!plan_ns(G[0].rows, G[0].cols, batch, &plan)) return ORTHO_E_SHAPE;
  if (ws == nullptr || ws_bytes < plan.total_bytes) return ORTHO_E_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % kWsAlign != 0) return ORTHO_E_WORKSPACE;
  return ORTHO_OK;
}

ortho_status validate_muon(int32_t batch, const ortho_mat* X, const ortho_mat* G, const ortho_mat* M,
                           int32_t steps, const float* abc, float mu, float lr, float scale,
                           const void* ws, size_t ws_bytes, bool row_norm) {
  if (batch < 1 || steps < 0) return ORTHO_E_PARAM;
  if (!X || !G || !M) return ORTHO_E_NULL;
  if (!(mu >= 0.f && mu <= 1.f) || !finite(lr) || !finite(scale)) return ORTHO_E_PARAM;
  if (abc && (!finite(abc[0]) || !finite(abc[1]) || !finite(abc[2]))) return ORTHO_E_PARAM;
  for (int32_t b = 0; b < batch; ++b) {
    ortho_status st;
    if ((st = check_mat(X[b])) != ORTHO_OK) return st;
    if ((st = check_mat(G[b])) != ORTHO_OK) return st;
    if ((st = check_mat(M[b])) != ORTHO_OK) return st;
    if (G[b].dtype != X[b].dtype || M[b].dtype != ORTHO_F32) return ORTHO_E_DTYPE;
    if (G[b].rows != X[b].rows || G[b].cols != X[b].cols || M[b].rows != X[b].rows ||
        M[b].cols != X[b].cols)
      return ORTHO_E_SHAPE;
    if (b > 0) {
      if (!same_geometry(X[b], X[0])) return ORTHO_E_SHAPE;
      if (X[b].ld != X[0].ld || G[b].ld != G[0].ld || M[b].ld != M[0].ld) return ORTHO_E_LAYOUT;
    }
  }
  MuonPlan plan;
  if (!plan_muon(X[0].rows, X[0].cols, batch, &plan, row_norm)) return ORTHO_E_SHAPE;
  if (ws == nullptr || ws_bytes < plan.total_bytes) return ORTHO_E_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % kWsAlign != 0) return ORTHO_E_WORKSPACE;
  return ORTHO_OK;
}

}  // namespace ortho
