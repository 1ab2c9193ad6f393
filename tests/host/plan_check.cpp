// Host-only check of libortho's workspace planning and argument validation
// (plan.cpp), built with g++ under AddressSanitizer and UndefinedBehavior-
// Sanitizer by tests/test_plan_sanitized.py.  It needs no GPU and no HIP.
//
// Plans: over a grid of shapes (edge sizes, ragged sizes, the workloads'
// sizes, the largest dimensions accepted), every region must sit inside the
// member stride, aligned, in the order the plan lays them out, and large
// enough for what the kernels write there; every split-K factor must cover its
// reduction exactly, with no empty slice.  Validation: a table of argument
// errors, each expected to give one status code.
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <initializer_list>
#include <vector>

#include "plan.h"

using namespace ortho;

static int failures = 0;
static long checks = 0;

#define EXPECT(cond, ...)                                 \
  do {                                                    \
    ++checks;                                             \
    if (!(cond)) {                                        \
      ++failures;                                         \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                       \
      fprintf(stderr, "\n");                              \
    }                                                     \
  } while (0)

static size_t cdiv(size_t a, size_t b) { return (a + b - 1) / b; }

// split-K factors: `splits` slices of `kchunk` cover K exactly, none empty
static void check_split(const char* what, int64_t K, int splits, int kchunk, int multiple,
                        int64_t m, int64_t n, int r) {
  EXPECT(splits >= 1 && kchunk >= 1, "%s: splits %d kchunk %d (m %lld n %lld r %d)", what, splits,
         kchunk, (long long)m, (long long)n, r);
  if (splits < 1 || kchunk < 1) return;
  EXPECT((int64_t)(splits - 1) * kchunk < K && (int64_t)splits * kchunk >= K,
         "%s: %d x %d does not cover K = %lld exactly (m %lld n %lld r %d)", what, splits, kchunk,
         (long long)K, (long long)m, (long long)n, r);
  if (splits > 1)
    EXPECT(kchunk % multiple == 0, "%s: kchunk %d not a multiple of %d (m %lld n %lld r %d)", what,
           kchunk, multiple, (long long)m, (long long)n, r);
}

// Regions in layout order: each aligned, after the previous one's end, and
// of at least `need` bytes (the next region's offset, or the member stride,
// bounds it).
struct Region {
  const char* name;
  size_t off, need;
};

static void check_regions(const char* what, const std::vector<Region>& rs, size_t end, int64_t m,
                          int64_t n, int r) {
  for (size_t i = 0; i < rs.size(); ++i) {
    const size_t next = i + 1 < rs.size() ? rs[i + 1].off : end;
    EXPECT(rs[i].off % kWsAlign == 0, "%s.%s offset %zu not aligned (m %lld n %lld r %d)", what,
           rs[i].name, rs[i].off, (long long)m, (long long)n, r);
    EXPECT(next >= rs[i].off && next - rs[i].off >= rs[i].need,
           "%s.%s: %zu bytes from %zu to %zu, needs %zu (m %lld n %lld r %d)", what, rs[i].name,
           next - rs[i].off, rs[i].off, next, rs[i].need, (long long)m, (long long)n, r);
  }
  EXPECT(end % kWsAlign == 0, "%s: stride %zu not aligned", what, end);
}

static void check_dion(int64_t m, int64_t n, int r, int batch) {
  DionPlan p;
  const bool ok = plan_dion(m, n, r, batch, &p);
  const bool valid = m >= 1 && n >= 1 && r >= 1 && batch >= 1 && r <= std::min(m, n) &&
                     r <= 16384 && m <= (int64_t{1} << 30) && n <= (int64_t{1} << 30);
  EXPECT(ok == valid, "plan_dion(%lld, %lld, %d, %d) returned %d", (long long)m, (long long)n, r,
         batch, ok);
  if (!ok) return;
  const size_t mr = (size_t)m * r, nr = (size_t)n * r, rr = (size_t)r * r;
  EXPECT(p.chunk == std::min(batch, 32), "chunk %d for batch %d", p.chunk, batch);
  EXPECT(p.total_bytes == p.member_bytes * (size_t)p.chunk, "total %zu != %zu x %d", p.total_bytes,
         p.member_bytes, p.chunk);
  EXPECT(p.rp >= r && p.rp % 4 == 0 && p.rpb >= r && p.rpb % 8 == 0, "rp %lld rpb %lld for r %d",
         (long long)p.rp, (long long)p.rpb, r);
  EXPECT(p.small_left == few_tiles(m, r, p.chunk) && p.small_right == few_tiles(n, r, p.chunk),
         "small sweeps flags (m %lld n %lld r %d)", (long long)m, (long long)n, r);
  // the 64 x 64 sweep kernels step k by 64
  check_split("left", n, p.split_left, p.kchunk_left, p.small_left ? 64 : 32, m, n, r);
  check_split("right", m, p.split_right, p.kchunk_right, p.small_right ? 64 : 32, m, n, r);
  if (p.small_left) EXPECT(p.kchunk_left % 64 == 0, "small left kchunk %d", p.kchunk_left);
  if (p.small_right) EXPECT(p.kchunk_right % 64 == 0, "small right kchunk %d", p.kchunk_right);
  check_split("gram", m, p.split_gram, p.kchunk_gram, 32, m, n, r);
  EXPECT(p.gram_big == gram_big_tiles(r, p.chunk), "fp64 Gram tile choice (r %d chunk %d)", r, p.chunk);
  check_split("gram2", m, p.split_gram2, p.kchunk_gram2, gram_tn_small_tiles(r) ? 64 : 32, m, n, r);
  // every split-K partial set that goes through the shared partial buffer
  size_t part = std::max({(size_t)p.split_left * mr * 4, (size_t)p.split_right * nr * 4,
                          (size_t)p.split_gram * rr * 8, (size_t)p.split_gram2 * rr * 4});
  const bool stream = (r == 64 || r == 128 || r == 256 || r == 512) && m % 64 == 0 && n % 64 == 0;
  EXPECT(p.stream_sweeps == stream, "stream sweeps flag on %lld x %lld r %d", (long long)m,
         (long long)n, r);
  EXPECT(p.fast_sweeps == (!stream && m % 256 == 0 && n % 256 == 0 && r % 256 == 0 && r >= 512),
         "fast sweeps flag on %lld x %lld r %d", (long long)m, (long long)n, r);
  EXPECT(p.ortho64 == (r <= kOrtho64MaxRank), "fp64 orthonormalisation flag for r %d", r);
  EXPECT(p.small_ortho == (r <= 64 && m <= kSmallOrthoMaxRows), "one-workgroup orthonormalisation flag (m %lld r %d)",
         (long long)m, r);
  EXPECT(!!p.fast_ortho == (!p.ortho64 && (p.fast_sweeps || (stream && r == 512 && m % 256 == 0)) &&
                            3 * r <= n),
         "fast orthonormalisation flag on %lld x %lld r %d", (long long)m, (long long)n, r);
  if (p.fast_sweeps) {
    check_split("fast left", 3 * n / 64, p.split_fl, p.kchunk_fl, 1, m, n, r);
    check_split("fast right", 3 * m / 64, p.split_fr, p.kchunk_fr, 1, m, n, r);
    part = std::max({part, (size_t)p.split_fl * mr * 4, (size_t)p.split_fr * nr * 4});
  }
  if (p.fast_ortho) {
    check_split("ap6", 6 * r / 64, p.split_ap6, p.kchunk_ap6, 1, m, n, r);
    check_split("ap3", 3 * r / 64, p.split_ap3, p.kchunk_ap3, 1, m, n, r);
    check_split("e", 3 * m / 64, p.split_e, p.kchunk_e, 1, m, n, r);
    part = std::max({part, (size_t)std::max(p.split_ap6, p.split_ap3) * mr * 4,
                     (size_t)p.split_e * rr * 4});
  }
  if (p.stream_sweeps) {
    check_split("stream left", n, p.split_sl, p.kchunk_sl, 16, m, n, r);
    check_split("stream right", m, p.split_sr, p.kchunk_sr, 16, m, n, r);
    part = std::max({part, (size_t)p.split_sl * mr * 4, (size_t)p.split_sr * nr * 4});
  }
  std::vector<Region> rs = {
      {"pt", p.off_pt, (size_t)m * p.rp * 4},  {"p1", p.off_p1, (size_t)m * p.rp * 4},
      {"part", p.off_part, part},              {"s", p.off_s, rr * 8},
      {"x", p.off_x, rr * 8},                  {"d", p.off_d, (size_t)r * 8},
      {"tt", p.off_tt, rr * 4},                {"r", p.off_r, (size_t)n * p.rp * 4},
      {"colsq", p.off_colsq, (size_t)cdiv(n, 64) * r * 4},
      {"pb", p.off_pb, (size_t)m * p.rpb * 2}, {"rb", p.off_rb, (size_t)n * p.rpb * 2},
      {"qb", p.off_qb, (size_t)n * p.rpb * 2},
      {"pf", p.off_pf, p.frag_p ? mr * 2 : 0}};
  EXPECT(p.frag_p == ((r == 256 || r == 512) && m % 128 == 0), "fragment-order P flag");
  if (p.fast_sweeps) {
    for (auto pr : {std::make_pair("bhi", p.off_bhi), std::make_pair("blo", p.off_blo),
                    std::make_pair("bhit", p.off_bhit), std::make_pair("blot", p.off_blot)})
      rs.push_back({pr.first, pr.second, (size_t)m * n * 2});
  } else if (p.fast_ortho) {
    rs.push_back({"ortho a pieces", p.off_bhi, 3 * mr * 2});
    rs.push_back({"ortho b pieces", p.off_blo, 3 * rr * 2});
  }
  if (p.fast_sweeps || p.stream_sweeps) {
    rs.push_back({"qhit", p.off_qhit, nr * 2});
    rs.push_back({"qlot", p.off_qlot, nr * 2});
    rs.push_back({"phit", p.off_phit, mr * 2});
    rs.push_back({"plot", p.off_plot, mr * 2});
  }
  check_regions("dion", rs, p.member_bytes, m, n, r);
}

static void check_ns(int64_t m, int64_t n, int batch) {
  NsPlan s;
  const bool ok = plan_ns(m, n, batch, &s);
  const bool valid = m >= 1 && n >= 1 && batch >= 1 && m <= (int64_t{1} << 30) && n <= (int64_t{1} << 30);
  EXPECT(ok == valid, "plan_ns(%lld, %lld, %d) returned %d", (long long)m, (long long)n, batch, ok);
  if (!ok) return;
  EXPECT(s.M == std::min(m, n) && s.N == std::max(m, n) && s.transposed == (m > n),
         "ns orientation for %lld x %lld", (long long)m, (long long)n);
  EXPECT(s.total_bytes == s.member_bytes * (size_t)s.chunk, "ns total");
  EXPECT(s.nparts >= 1 && (int64_t)s.nparts * s.part_chunk >= m && (int64_t)(s.nparts - 1) * s.part_chunk < m,
         "ns sum-of-squares blocks %d x %lld for m %lld", s.nparts, (long long)s.part_chunk, (long long)m);
  if (s.gram_splits > 1) check_split("ns gram", s.N, s.gram_splits, s.gram_kchunk, 32, m, n, 0);
  if (s.gram_ns) {
    EXPECT(s.M <= 128 && s.N >= 4 * s.M, "gram ns on %lld x %lld", (long long)m, (long long)n);
    check_split("ns gram-ns", s.N, s.gns_splits, s.gns_kchunk, 32, m, n, 0);
    EXPECT(s.gns_mp >= s.M && (s.gns_mp == 64 || s.gns_mp == 128), "gns_mp %d for M %lld", s.gns_mp,
           (long long)s.M);
  }
  const size_t mn = (size_t)s.M * s.ld_x, nm = (size_t)s.N * s.ld_xt, mm = (size_t)s.M * s.ld_xt;
  const size_t gmm = (size_t)s.M * s.M;
  std::vector<Region> rs = {
      {"x32", s.off_x32, mn * 4},
      {"xb0", s.off_xb0, mn * 2},
      {"xb1", s.off_xb1, mn * 2},
      {"xbt0", s.off_xbt0, nm * 2},
      {"xbt1", s.off_xbt1, nm * 2},
      {"a", s.off_a, mm * 2},
      {"bp", s.off_bp, mm * 2},
      {"bp32", s.off_bp32, s.M <= 128 ? mm * 4 : 0},
      {"gpart", s.off_gpart, s.gram_splits > 1 ? (size_t)s.gram_splits * mm * 4 : 0},
      {"gns_part", s.off_gns_part, s.gram_ns ? (size_t)s.gns_splits * gmm * 4 : 0},
      {"gns_a0", s.off_gns_a0, s.gram_ns ? (size_t)s.gns_mp * s.gns_mp * 6 : 0},
      {"partial", s.off_partial, (size_t)s.nparts * 4},
      {"scale", s.off_scale, 4}};
  check_regions("ns", rs, s.member_bytes, m, n, 0);
}

static void check_dion2(int64_t m, int64_t n, int k) {
  Dion2Plan d;
  const bool ok = plan_dion2(m, n, k, &d);
  const bool valid = m >= 1 && n >= 1 && k >= 1 && k <= m && m <= 65535 && n <= (int64_t{1} << 30);
  EXPECT(ok == valid, "plan_dion2(%lld, %lld, %d) returned %d", (long long)m, (long long)n, k, ok);
  if (!ok) return;
  std::vector<Region> rs = {{"ns", 0, d.ns.total_bytes},
                            {"blk", d.off_blk, (size_t)k * d.ld_blk * 4},
                            {"norms", d.off_norms, (size_t)m * 4},
                            {"rank", d.off_rank, (size_t)m * 4},
                            {"sel", d.off_sel, (size_t)k * 4}};
  check_regions("dion2", rs, d.total_bytes, m, n, k);
}

static void check_muon(int64_t m, int64_t n, int batch, bool row_norm) {
  MuonPlan p;
  if (!plan_muon(m, n, batch, &p, row_norm)) {
    EXPECT(false, "plan_muon(%lld, %lld, %d) failed", (long long)m, (long long)n, batch);
    return;
  }
  EXPECT(p.off_u >= p.ns.total_bytes && p.off_u % kWsAlign == 0, "muon U offset");
  EXPECT(p.u_bytes >= (size_t)m * n * 4, "muon U size");
  const size_t end_u = p.off_u + p.u_bytes * (size_t)p.ns.chunk;
  if (row_norm)
    EXPECT(p.off_rowf >= end_u && p.total_bytes >= p.off_rowf + (size_t)m * 4 * p.ns.chunk, "normuon row factors");
  else
    EXPECT(p.total_bytes >= end_u, "muon total");
  // a trailing chunk of fewer members still fits before U
  const int last = batch % p.ns.chunk;
  if (last) {
    NsPlan t;
    EXPECT(plan_ns(m, n, last, &t) && t.total_bytes <= p.off_u, "muon tail chunk");
  }
}

static ortho_mat mat(int64_t rows, int64_t cols, int dtype, int64_t ld = -1, void* data = (void*)0x1000) {
  ortho_mat a;
  a.data = data;
  a.rows = rows;
  a.cols = cols;
  a.ld = ld < 0 ? cols : ld;
  a.dtype = dtype;
  return a;
}

static void check_validation() {
  static char ws_store[1 << 16];
  void* ws = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(ws_store) + 255) & ~uintptr_t{255});
  const size_t big = size_t{1} << 60;   // a claimed size: validation never touches the memory
  const int64_t m = 96, n = 160;
  const int r = 24;
  struct Case {
    const char* name;
    ortho_mat X, G, M, Q;
    int r;
    float mu, lr, scale;
    void* ws;
    size_t ws_bytes;
    ortho_status want;
  };
  const ortho_mat X = mat(m, n, ORTHO_BF16), G = mat(m, n, ORTHO_BF16), M = mat(m, n, ORTHO_F32),
                  Q = mat(n, r, ORTHO_F32);
  DionPlan plan;
  plan_dion(m, n, r, 1, &plan);
  const float nan = __builtin_nanf("");
  const float inf = __builtin_inff();
  std::vector<Case> cases = {
      {"ok", X, G, M, Q, r, 0.9f, 0.1f, 1.f, ws, big, ORTHO_OK},
      {"exact workspace", X, G, M, Q, r, 0.9f, 0.1f, 1.f, ws, plan.total_bytes, ORTHO_OK},
      {"workspace one short", X, G, M, Q, r, 0.9f, 0.1f, 1.f, ws, plan.total_bytes - 1, ORTHO_E_WORKSPACE},
      {"null workspace", X, G, M, Q, r, 0.9f, 0.1f, 1.f, nullptr, big, ORTHO_E_WORKSPACE},
      {"misaligned workspace", X, G, M, Q, r, 0.9f, 0.1f, 1.f, (char*)ws + 16, big, ORTHO_E_WORKSPACE},
      {"null X", mat(m, n, ORTHO_BF16, -1, nullptr), G, M, Q, r, 0.9f, 0.1f, 1.f, ws, big, ORTHO_E_NULL},
      {"zero rows", mat(0, n, ORTHO_BF16), G, M, Q, r, 0.9f, 0.1f, 1.f, ws, big, ORTHO_E_SHAPE},
      {"negative cols", mat(m, -5, ORTHO_BF16), G, M, Q, r, 0.9f, 0.1f, 1.f, ws, big, ORTHO_E_SHAPE},
      {"huge rows", mat(int64_t{1} << 31, n, ORTHO_BF16), G, M, Q, r, 0.9f, 0.1f, 1.f, ws, big, ORTHO_E_SHAPE},
      {"ld < cols", mat(m, n, ORTHO_BF16, n - 1), G, M, Q, r, 0.9f, 0.1f, 1.f, ws, big, ORTHO_E_LAYOUT},
      {"ld too large", mat(m, n, ORTHO_BF16, int64_t{1} << 41), G, M, Q, r, 0.9f, 0.1f, 1.f, ws, big, ORTHO_E_LAYOUT},
      {"bad dtype", mat(m, n, 7), G, M, Q, r, 0.9f, 0.1f, 1.f, ws, big, ORTHO_E_DTYPE},
      {"G dtype differs", X, mat(m, n, ORTHO_F32), M, Q, r, 0.9f, 0.1f, 1.f, ws, big, ORTHO_E_DTYPE},
      {"bf16 momentum", X, G, mat(m, n, ORTHO_BF16), Q, r, 0.9f, 0.1f, 1.f, ws, big, ORTHO_E_DTYPE},
      {"G shape", X, mat(m + 1, n, ORTHO_BF16), M, Q, r, 0.9f, 0.1f, 1.f, ws, big, ORTHO_E_SHAPE},
      {"Q rows", X, G, M, mat(n + 1, r, ORTHO_F32), r, 0.9f, 0.1f, 1.f, ws, big, ORTHO_E_SHAPE},
      {"Q cols != r", X, G, M, mat(n, r + 1, ORTHO_F32), r, 0.9f, 0.1f, 1.f, ws, big, ORTHO_E_RANK},
      {"r = 0", X, G, M, mat(n, r, ORTHO_F32), 0, 0.9f, 0.1f, 1.f, ws, big, ORTHO_E_RANK},
      {"r > m", X, G, M, mat(n, 97, ORTHO_F32), 97, 0.9f, 0.1f, 1.f, ws, big, ORTHO_E_RANK},
      {"mu < 0", X, G, M, Q, r, -0.1f, 0.1f, 1.f, ws, big, ORTHO_E_PARAM},
      {"mu > 1", X, G, M, Q, r, 1.5f, 0.1f, 1.f, ws, big, ORTHO_E_PARAM},
      {"mu nan", X, G, M, Q, r, nan, 0.1f, 1.f, ws, big, ORTHO_E_PARAM},
      {"lr inf", X, G, M, Q, r, 0.9f, inf, 1.f, ws, big, ORTHO_E_PARAM},
      {"scale nan", X, G, M, Q, r, 0.9f, 0.1f, nan, ws, big, ORTHO_E_PARAM},
  };
  for (const Case& c : cases) {
    const ortho_status st = validate_dion(1, &c.X, &c.G, &c.M, &c.Q, c.r, c.mu, c.lr, c.scale, nullptr,
                                          nullptr, c.ws, c.ws_bytes);
    EXPECT(st == c.want, "validate_dion '%s': got %d, want %d", c.name, (int)st, (int)c.want);
  }
  // batches: one member that differs in leading dimension or shape
  {
    std::vector<ortho_mat> Xs(3, X), Gs(3, G), Ms(3, M), Qs(3, Q);
    DionPlan pb;
    plan_dion(m, n, r, 3, &pb);
    EXPECT(validate_dion(3, Xs.data(), Gs.data(), Ms.data(), Qs.data(), r, 0.9f, 0.1f, 1.f, nullptr,
                         nullptr, ws, pb.total_bytes) == ORTHO_OK, "batch of 3");
    EXPECT(validate_dion(3, Xs.data(), Gs.data(), Ms.data(), Qs.data(), r, 0.9f, 0.1f, 1.f, nullptr,
                         nullptr, ws, pb.total_bytes - 1) == ORTHO_E_WORKSPACE, "batch of 3, workspace short");
    Ms[2] = mat(m, n, ORTHO_F32, n + 4);
    EXPECT(validate_dion(3, Xs.data(), Gs.data(), Ms.data(), Qs.data(), r, 0.9f, 0.1f, 1.f, nullptr,
                         nullptr, ws, big) == ORTHO_E_LAYOUT, "batch member ld");
    Ms[2] = M;
    Qs[1] = mat(n, r - 1, ORTHO_F32);
    EXPECT(validate_dion(3, Xs.data(), Gs.data(), Ms.data(), Qs.data(), r, 0.9f, 0.1f, 1.f, nullptr,
                         nullptr, ws, big) == ORTHO_E_RANK, "batch member rank");
    EXPECT(validate_dion(0, Xs.data(), Gs.data(), Ms.data(), Qs.data(), r, 0.9f, 0.1f, 1.f, nullptr,
                         nullptr, ws, big) == ORTHO_E_PARAM, "batch of 0");
  }
  // Newton-Schulz, Muon, Dion2
  {
    const ortho_mat g = mat(m, n, ORTHO_BF16), o = mat(m, n, ORTHO_BF16);
    const float abc[3] = {3.4445f, -4.775f, 2.0315f}, bad[3] = {1.f, nan, 1.f};
    EXPECT(validate_ns(1, &g, &o, 5, abc, ws, big) == ORTHO_OK, "ns ok");
    EXPECT(validate_ns(1, &g, &o, -1, abc, ws, big) == ORTHO_E_PARAM, "ns steps < 0");
    EXPECT(validate_ns(1, &g, &o, 5, bad, ws, big) == ORTHO_E_PARAM, "ns coefficient nan");
    const ortho_mat ot = mat(n, m, ORTHO_BF16);
    EXPECT(validate_ns(1, &g, &ot, 5, abc, ws, big) == ORTHO_E_SHAPE, "ns output transposed");
    EXPECT(validate_ns(1, &g, &o, 5, abc, ws, 16) == ORTHO_E_WORKSPACE, "ns workspace short");
    const ortho_mat x = mat(m, n, ORTHO_BF16), mm = mat(m, n, ORTHO_F32);
    EXPECT(validate_muon(1, &x, &g, &mm, 5, abc, 0.95f, 0.02f, 1.f, ws, big) == ORTHO_OK, "muon ok");
    EXPECT(validate_muon(1, &x, &g, &mm, 5, abc, 0.95f, 0.02f, 1.f, ws, big, true) == ORTHO_OK, "normuon ok");
    EXPECT(validate_muon(1, &x, &g, &x, 5, abc, 0.95f, 0.02f, 1.f, ws, big) == ORTHO_E_DTYPE, "muon bf16 momentum");
    EXPECT(validate_dion2(x, g, mm, 24, 5, abc, 0.95f, 0.02f, 1.f, ws, big) == ORTHO_OK, "dion2 ok");
    EXPECT(validate_dion2(x, g, mm, 0, 5, abc, 0.95f, 0.02f, 1.f, ws, big) == ORTHO_E_RANK, "dion2 k = 0");
    EXPECT(validate_dion2(x, g, mm, (int)m + 1, 5, abc, 0.95f, 0.02f, 1.f, ws, big) == ORTHO_E_RANK, "dion2 k > m");
    const ortho_mat xt = mat(70000, 8, ORTHO_BF16), gt = mat(70000, 8, ORTHO_BF16), mt = mat(70000, 8, ORTHO_F32);
    EXPECT(validate_dion2(xt, gt, mt, 4, 5, abc, 0.95f, 0.02f, 1.f, ws, big) == ORTHO_E_SHAPE, "dion2 m > 65535");
  }
}

int main() {
  const std::vector<int64_t> dims = {1, 2, 63, 64, 65, 127, 128, 129, 200, 255, 256, 257, 320, 448, 512,
                                     1000, 1024, 2048, 4096, 8192, 12288, 16384, 53248};
  const std::vector<int> ranks = {1, 7, 24, 37, 63, 64, 65, 128, 255, 256, 257, 384, 511, 512, 1024,
                                  2048, 4096};
  for (int64_t m : dims)
    for (int64_t n : dims) {
      for (int r : ranks)
        if (r <= std::min(m, n)) check_dion(m, n, r, 1);
      check_ns(m, n, 1);
    }
  for (int batch : {2, 5, 12, 32, 33, 40, 64})
    for (auto mnr : {std::vector<int64_t>{2048, 2048, 512}, std::vector<int64_t>{2048, 8192, 512},
                     std::vector<int64_t>{8192, 2048, 512}, std::vector<int64_t>{256, 256, 64},
                     std::vector<int64_t>{300, 200, 37}}) {
      check_dion(mnr[0], mnr[1], (int)mnr[2], batch);
      check_ns(mnr[0], mnr[1], batch);
      check_muon(mnr[0], mnr[1], batch, false);
      check_muon(mnr[0], mnr[1], batch, true);
    }
  for (int heads : {1, 8, 32, 35, 40}) {
    check_ns(128, 4096, heads);
    check_ns(64, 4096, heads);
    check_muon(128, 4096, heads, true);
  }
  // rejected shapes
  check_dion(0, 10, 1, 1);
  check_dion(10, 10, 11, 1);
  check_dion(10, 10, 0, 1);
  check_dion(10, 10, 1, 0);
  check_dion((int64_t{1} << 30) + 1, 64, 8, 1);
  check_dion(65536, 65536, 16385, 1);
  check_ns(0, 5, 1);
  check_ns(5, 5, 0);
  // the largest dimensions accepted (sizes only; nothing is allocated)
  check_dion(int64_t{1} << 30, 64, 64, 1);
  check_dion(64, int64_t{1} << 30, 64, 1);
  check_ns(int64_t{1} << 30, 128, 1);
  check_ns(128, int64_t{1} << 30, 1);
  for (int64_t m : {1, 2, 100, 4096, 65535, 65536})
    for (int64_t n : {1, 64, 333, 4096})
      for (int k : {1, 24, 256, 1024, 4096, 65535})
        check_dion2(m, n, k);
  check_validation();
  printf("plan_check: %ld checks, %d failures\n", checks, failures);
  return failures == 0 ? 0 : 1;
}
