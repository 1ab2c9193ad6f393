// Dion's two power-iteration sweeps over B = M + G for bf16 weights and a
// rank r of 64, 128, 256 or 512 (MSR talk "Dion: The distributed orthonormal update
// revolution is here", passage on amortised power iteration):
//   left  (sweep 1):  P~ = B Q      (m x r, reduction over the n columns of B)
//   right (sweep 2):  R  = B^T P    (n x r, reduction over the m rows of B)
// Each is one streaming pass over M (fp32) and G (bf16) that is bound by HBM:
// at 4096 x 4096 and r = 256, 96 MB against 26 GFLOP of bf16x3 products.
//
// Design (gfx950): a workgroup of eight waves owns 128 output rows and all r
// columns, over one split-K slice of the reduction; wave (rb, ch) computes
// rows rb * 32 .. + 31 and half ch of the columns, so each SIMD runs two waves
// and one's LDS reads and conversions overlap the other's products.  The raw
// tiles of M and G and the bf16 pieces of the right factor (Q^T or P^T, hi and lo, k contiguous, prepared by
// split_t) go from HBM/L2 into LDS with global_load_lds_dwordx4 copies, four
// 16-deep k stages in flight.  Each wave builds its A fragments straight from
// the raw tiles -- B = M + G in fp32, split into bf16 hi and lo in registers --
// so B is never stored, and runs hi*hi + hi*lo + lo*hi on
// v_mfma_f32_32x32x16_bf16 (the same bf16x3 products as the generic path).
// The fp32 result of every slice goes to the split-K partial buffer, summed
// in a fixed order by the reduce kernel that follows.
//
// At r = 512 a wave holds eight 32 x 32 accumulators, and a 44 KB stage
// leaves room for three stages in LDS.  To keep two waves per SIMD within the
// register file, the factor fragments of a stage are held once (not double
// buffered): the hi*lo products run first, the next stage's lo fragments and
// A fragment are read under the hi*hi and lo*hi products, and its hi
// fragments after them.
//
// Requirements (checked by the launcher): r in {64, 128, 256, 512}; m and n
// multiples of 64; M and G rows 16-byte aligned; the factor pieces k-blocked
// (split_t with blocked set); kchunk a multiple of 16.
#include <type_traits>

#include "gemm_fast.h"
#include "launch.h"

namespace ortho {

namespace {

constexpr int kRows = 128;          // output rows per workgroup (4 row blocks of 32)
constexpr int kBK = 16;             // k per stage
constexpr int kMBytes = kRows * kBK * 4;   // raw fp32 M tile per stage
constexpr int kGBytes = kRows * kBK * 2;   // raw bf16 G tile per stage

constexpr int kWaves = 8;           // two per SIMD: 4 row blocks x 2 column halves

template <int R>
struct SweepLayout {
  static constexpr int kPieceBytes = R * kBK * 2;      // one bf16 piece of the factor
  static constexpr int kStageBytes = kMBytes + kGBytes + 2 * kPieceBytes;
  // four stages in flight (five, with the waits covering them, measured slower
  // at r = 256: 43 / 42 us against 42 / 42); three at r = 512 (132 KB)
  static constexpr int kStages = R == 512 ? 3 : 4;
  static constexpr int kMInstr = kMBytes / 1024;       // 1 KB per copy instruction
  static constexpr int kGInstr = kGBytes / 1024;
  static constexpr int kPInstr = 2 * kPieceBytes / 1024;
  static constexpr int kInstr = kMInstr + kGInstr + kPInstr;
  // wave w issues copies w, w + 8, ...: kLo or kLo + 1 of them per stage
  static constexpr int kLo = kInstr / kWaves;
  static constexpr int kHiWaves = kInstr % kWaves;     // waves 0 .. kHiWaves - 1 issue kLo + 1
  static constexpr int kMaxPerWave = kLo + (kHiWaves ? 1 : 0);
};

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// s_waitcnt lgkmcnt(0) as the compiler's own wait instruction (vmcnt and
// expcnt at their maxima), which its wait insertion takes into account
__device__ __forceinline__ void lds_reads_done() { __builtin_amdgcn_s_waitcnt(0xc07f); }

}  // namespace

// TRANS = false: sweep 1 (A rows are rows of B, k runs along a row of B);
// TRANS = true:  sweep 2 (A rows are columns of B, k runs down a column).
template <int R, bool TRANS>
__global__ __launch_bounds__(512, 1) void dion_sweep_kernel(SweepArgs a) {
  using L = SweepLayout<R>;
  using namespace fast;
  constexpr int kStages = L::kStages;
  __shared__ __attribute__((aligned(1024))) char smem[kStages * L::kStageBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int bi = blockIdx.z;
  // Workgroups are dealt to the 8 XCDs round robin in launch order.  When the
  // (row tile, split) grid divides evenly, XCD x takes the x-th eighth of the
  // grid in split-major order, so each XCD's L2 fetches only the factor rows
  // of its own k slices instead of all of them.
  int tile = blockIdx.x, split = blockIdx.y;
  {
    const int tiles = gridDim.x, total = tiles * gridDim.y;
    if (total % 8 == 0) {
      const int b = blockIdx.x + tiles * blockIdx.y;
      const int l = (b % 8) * (total / 8) + b / 8;
      split = l / tiles;
      tile = l - split * tiles;
    }
  }
  const int row0 = tile * kRows;                // first output row of the workgroup
  const int kbeg = split * a.kchunk;
  const int kend = min(a.K, kbeg + a.kchunk);
  const int nst = (kend - kbeg) / kBK;          // >= 1 (checked by the launcher)

  const float* M = static_cast<const float*>(a.m.p[bi]);
  const uint16_t* G = static_cast<const uint16_t*>(a.g.p[bi]);
  const uint16_t* F0 = static_cast<const uint16_t*>(a.f[0].p[bi]);
  const uint16_t* F1 = static_cast<const uint16_t*>(a.f[1].p[bi]);
  const int64_t ldm = a.m.ld, ldg = a.g.ld;
  const int out_rows = a.rows;                   // m (sweep 1) or n (sweep 2)

  // Per-lane byte offsets of this wave's copy instructions, relative to the
  // stage's k0 column (sweep 1) or row (sweep 2) of the source; the stage base
  // address is added per stage in scalar registers.  Copy instruction c of
  // the workgroup: M tiles first, then G, then the two factor pieces; wave w
  // issues instructions w, w + 8, ...
  const int ncopy = L::kLo + (wave < L::kHiWaves ? 1 : 0);
  unsigned off[L::kMaxPerWave];
  int kind[L::kMaxPerWave];   // 0: M, 1: G, 2: piece 0, 3: piece 1
#pragma unroll
  for (int u = 0; u < L::kMaxPerWave; ++u) {
    const int c = min(wave + kWaves * u, L::kInstr - 1);
    if (c < L::kMInstr) {
      kind[u] = 0;
      if (!TRANS) {
        // 16 rows of 64 B; lane: row c*16 + lane/4, stored chunk lane%4,
        // fetched chunk = stored ^ ((row >> 2) & 3)
        const int rl = c * 16 + (lane >> 2), pos = lane & 3;
        const int gr = min(row0 + rl, out_rows - 1);
        off[u] = static_cast<unsigned>((gr * ldm) * 4 + (pos ^ ((rl >> 2) & 3)) * 16);
      } else {
        // 2 k-rows of 128 floats (512 B); lane: k-row c*2 + lane/32, chunk lane%32
        const int kr = c * 2 + (lane >> 5), col = row0 + (lane & 31) * 4;
        off[u] = static_cast<unsigned>((kr * ldm + min(col, out_rows - 4)) * 4);
      }
    } else if (c < L::kMInstr + L::kGInstr) {
      kind[u] = 1;
      const int cg = c - L::kMInstr;
      if (!TRANS) {
        // 32 rows of 32 B; stored chunk lane%2, fetched = stored ^ ((row >> 3) & 1)
        const int rl = cg * 32 + (lane >> 1), pos = lane & 1;
        const int gr = min(row0 + rl, out_rows - 1);
        off[u] = static_cast<unsigned>((gr * ldg) * 2 + (pos ^ ((rl >> 3) & 1)) * 16);
      } else {
        // 4 k-rows of 128 bf16 (256 B); lane: k-row cg*4 + lane/16, chunk lane%16
        const int kr = cg * 4 + (lane >> 4), col = row0 + (lane & 15) * 8;
        off[u] = static_cast<unsigned>((kr * ldg + min(col, out_rows - 8)) * 2);
      }
    } else {
      const int cp = c - L::kMInstr - L::kGInstr;
      const int per = L::kPieceBytes / 1024;
      kind[u] = 2 + cp / per;
      // factor piece, k-blocked: the stage's 16 k of all R rows are one
      // contiguous run of R * 32 B; 32 rows (1 KB) per instruction, the same
      // swizzle as G
      const int j = (cp % per) * 32 + (lane >> 1), pos = lane & 1;
      off[u] = static_cast<unsigned>(j * 32 + (pos ^ ((j >> 3) & 1)) * 16);
    }
  }
  const unsigned lds0 = lds_addr(smem);
  auto issue = [&](int st) {
    const int k0 = kbeg + st * kBK;
    const int buf = st % kStages;
    // scalar stage bases
    const char* bm = TRANS ? reinterpret_cast<const char*>(M + (int64_t)k0 * ldm)
                           : reinterpret_cast<const char*>(M + k0);
    const char* bg = TRANS ? reinterpret_cast<const char*>(G + (int64_t)k0 * ldg)
                           : reinterpret_cast<const char*>(G + k0);
    const char* b0 = reinterpret_cast<const char*>(F0 + (int64_t)(k0 >> 4) * R * 16);
    const char* b1 = reinterpret_cast<const char*>(F1 + (int64_t)(k0 >> 4) * R * 16);
#pragma unroll
    for (int u = 0; u < L::kMaxPerWave; ++u) {
      if (u >= ncopy) break;
      const int c = wave + kWaves * u;
      const char* base = kind[u] == 0 ? bm : (kind[u] == 1 ? bg : (kind[u] == 2 ? b0 : b1));
      dma16(off[u], uniform_ptr(base), lds0 + buf * L::kStageBytes + c * 1024);
    }
  };
  // wait until at most `later` stages of this wave's copies are outstanding:
  // the steady state (kStages - 3 later stages in flight) has its own
  // immediate count, any other case waits for all copies (vector memory
  // loads complete in order, so a smaller count is always safe)
  auto wait_stages = [&](int later) {
    constexpr int kSteady = kStages > 3 ? kStages - 3 : 0;
    static_assert(kSteady * L::kMaxPerWave < 64, "vmcnt range");
    if (later >= kSteady) {
      if (ncopy == L::kLo) wait_vm<kSteady * L::kLo>();
      else wait_vm<kSteady * L::kMaxPerWave>();
    } else {
      wait_vm<0>();
    }
  };

  // wave (rb, ch): output rows rb * 32 .. + 31, columns ch * R / 2 .. + R / 2 - 1
  const int rb = wave & 3, ch = wave >> 2;
  constexpr int NB = R / 64;
  floatx16 acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;

  // Fragments of one stage: the A fragment (B = M + G split into hi and lo)
  // and the NB column blocks of both factor pieces.
  const int fr = lane & 31, half = lane >> 5;
  const int rl = rb * 32 + fr;
  // R <= 256: both stages' factor fragments in registers (fb[buf]); R = 512:
  // one stage's (fb[0]), refilled piece by piece
  constexpr int kFbBufs = R == 512 ? 1 : 2;
  bf16x8 fa[2][2], fb[kFbBufs][NB][2];
  // the factor fragments of piece `pc` of stage st into fb[buf]
  auto read_factor = [&](int st, int buf, int pc) {
    const char* sp = smem + (st % kStages) * L::kStageBytes + kMBytes + kGBytes;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int fj = ch * (R / 2) + j * 32 + fr;
      const int o = fj * 32 + ((half ^ ((fj >> 3) & 1)) * 16);
      fb[buf][j][pc] = *reinterpret_cast<const bf16x8*>(sp + pc * L::kPieceBytes + o);
    }
  };
  // The A fragment of a stage (output row rl, k = half*8 .. + 7 of the
  // stage) in two phases: the raw M and G values from LDS, then B = M + G in
  // fp32 split into bf16 hi and lo, in four parts of two k each, so the
  // conversions can sit between the products of the previous stage instead
  // of waiting on the LDS reads ahead of them.
  float rm[8];
  uint32_t rg[8];   // G's bf16 bits: two k per word (sweep 1), one per word (sweep 2)
  auto load_a = [&](int st) {
    const char* sb = smem + (st % kStages) * L::kStageBytes;
    const float* sm = reinterpret_cast<const float*>(sb);
    const uint16_t* sg = reinterpret_cast<const uint16_t*>(sb + kMBytes);
    if (!TRANS) {
      const floatx4 m0 = *reinterpret_cast<const floatx4*>(sm + rl * 16 + (((2 * half) ^ ((rl >> 2) & 3)) * 4));
      const floatx4 m1 = *reinterpret_cast<const floatx4*>(sm + rl * 16 + (((2 * half + 1) ^ ((rl >> 2) & 3)) * 4));
      const uint4 g = *reinterpret_cast<const uint4*>(sg + rl * 16 + ((half ^ ((rl >> 3) & 1)) * 8));
#pragma unroll
      for (int t = 0; t < 4; ++t) { rm[t] = m0[t]; rm[4 + t] = m1[t]; }
      rg[0] = g.x; rg[1] = g.y; rg[2] = g.z; rg[3] = g.w;   // two k per word
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int kr = half * 8 + t;
        rm[t] = sm[kr * 128 + rl];
        rg[t] = sg[kr * 128 + rl];
      }
    }
  };
  // part p (k = 2p, 2p + 1) of the split of the loaded values into fa[buf]
  auto convert_a = [&](int p, int buf) {
#pragma unroll
    for (int t = 2 * p; t < 2 * p + 2; ++t) {
      const uint32_t gb = TRANS ? (rg[t] << 16)
                                : ((t & 1) ? (rg[t >> 1] & 0xffff0000u) : (rg[t >> 1] << 16));
      const float x = rm[t] + __uint_as_float(gb);
      const bf16 h = to_bf16(x);
      fa[buf][0][t] = h;
      fa[buf][1][t] = to_bf16(x - static_cast<float>(h));
    }
    // pin the part here: without this the compiler sinks the arithmetic to
    // its first use, past the next barrier, where nothing hides it
    asm volatile("" : "+v"(fa[buf][0]), "+v"(fa[buf][1]));
  };
  auto read_a = [&](int st, int buf) {
    load_a(st);
#pragma unroll
    for (int p = 0; p < 4; ++p) convert_a(p, buf);
  };
  // wait until this wave's copies of stage `st` are done (at most the stages
  // issued after it still outstanding), then the barrier makes every wave's
  // copies visible
  auto ready = [&](int st, int issued_last) {
    asm volatile("" ::: "memory");
    wait_stages(issued_last - st);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // prologue: stages 0 .. kStages - 2 in flight, stage 0's fragments read
#pragma unroll
  for (int st = 0; st < kStages - 1; ++st)
    if (st < nst) issue(st);
  int issued_last = min(kStages - 2, nst - 1);
  ready(0, issued_last);
  read_a(0, 0);
  read_factor(0, 0, 0);
  read_factor(0, 0, 1);

  // MFMA q of a step's t products after which part p of the next stage's A
  // conversion runs: the last parts as late as possible, two products apart,
  // none before the middle, so the raw reads have landed
  auto conv_slot = [](int p, int t) {
    const int q = t - 1 - 2 * (3 - p);
    return q > t / 2 ? q : t / 2;
  };
  // one stage whose fragments are in buffer CUR (a compile-time index, so the
  // fragments stay in registers); the next stage's raw A values and factor
  // fragments are read ahead of the products and its A fragment is built
  // into buffer CUR ^ 1 between them.  Past the last stage the reads hit a
  // stale buffer and the values go unused.
  auto step = [&](auto cur_c, int st) {
    constexpr int CUR = decltype(cur_c)::value;
    constexpr int T = 3 * NB;
    if (st + 1 < nst) {
      // stage st + 1 in LDS; after this barrier every wave has read stage st's
      // fragments (previous step), so the buffer of stage st - 1 is free
      ready(st + 1, issued_last);
      if (st + kStages - 1 < nst) {
        issue(st + kStages - 1);
        issued_last = st + kStages - 1;
      }
    }
    // the previous step's reads are long done; saying so here keeps the
    // compiler from counting them behind this step's 24 reads (past the
    // 15 the LDS counter holds) and waiting on those before the products
    lds_reads_done();
    load_a(st + 1);
    read_factor(st + 1, CUR ^ 1, 0);
    read_factor(st + 1, CUR ^ 1, 1);
    __builtin_amdgcn_sched_barrier(0);
    // each product kind over all accumulators before the next kind
#pragma unroll
    for (int q = 0; q < T; ++q) {
      const int kind = q / NB, j = q % NB;
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[CUR][kind == 2 ? 1 : 0],
                                                       fb[CUR][j][kind == 1 ? 1 : 0], acc[j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int p = 0; p < 4; ++p)
        if (conv_slot(p, T) == q) convert_a(p, CUR ^ 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // r = 512: fa[CUR] and fb[0] hold stage st on entry
  auto step512 = [&](auto cur_c, int st) {
    constexpr int CUR = decltype(cur_c)::value;
    const bool more = st + 1 < nst;
#pragma unroll
    for (int j = 0; j < NB; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[CUR][0], fb[0][j][1], acc[j], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (more) {
      ready(st + 1, issued_last);
      if (st + kStages - 1 < nst) {
        issue(st + kStages - 1);
        issued_last = st + kStages - 1;
      }
      lds_reads_done();
      read_factor(st + 1, 0, 1);
    }
    load_a(st + 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 2 * NB; ++q) {
      const int j = q % NB;
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[CUR][q < NB ? 0 : 1], fb[0][j][0], acc[j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int p = 0; p < 4; ++p)
        if (conv_slot(p, 2 * NB) == q) convert_a(p, CUR ^ 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (more) read_factor(st + 1, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int st = 0; st < nst; st += 2) {
    if constexpr (R == 512) {
      step512(std::integral_constant<int, 0>{}, st);
      if (st + 1 < nst) step512(std::integral_constant<int, 1>{}, st + 1);
    } else {
      step(std::integral_constant<int, 0>{}, st);
      if (st + 1 < nst) step(std::integral_constant<int, 1>{}, st + 1);
    }
  }

  // slice `split` of the partial result, rows row0 + rb*32 .. + 31
  float* out = a.out + bi * a.out_member_stride + split * a.split_stride;
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int row = row0 + rb * 32 + g * 8 + half * 4 + t;
        if (row < out_rows) out[(int64_t)row * R + ch * (R / 2) + j * 32 + fr] = acc[j][g * 4 + t];
      }
}

bool dion_sweep_ok(const SweepArgs& a, int members) {
  if (a.r != 64 && a.r != 128 && a.r != 256 && a.r != 512) return false;
  if (a.rows % 64 != 0 || a.K % 64 != 0 || a.kchunk % kBK != 0 || a.kchunk < kBK) return false;
  if (a.m.ld % 4 != 0 || a.g.ld % 8 != 0) return false;
  // 32-bit per-lane offsets: every source the copies address spans < 4 GiB
  if ((int64_t)a.M_rows * a.m.ld * 4 >= (int64_t{1} << 32)) return false;
  for (int i = 0; i < members; ++i)
    if (reinterpret_cast<uintptr_t>(a.m.p[i]) % 16 || reinterpret_cast<uintptr_t>(a.g.p[i]) % 16 ||
        reinterpret_cast<uintptr_t>(a.f[0].p[i]) % 16 || reinterpret_cast<uintptr_t>(a.f[1].p[i]) % 16)
      return false;
  return true;
}

hipError_t launch_dion_sweep(const SweepArgs& a, bool trans, int members, hipStream_t s) {
  if (!dion_sweep_ok(a, members)) return hipErrorInvalidValue;
  dim3 grid((a.rows + kRows - 1) / kRows, (a.K + a.kchunk - 1) / a.kchunk, members);
#define ORTHO_SWEEP(RR)                                                                      \
  do {                                                                                       \
    if (trans) hipLaunchKernelGGL((dion_sweep_kernel<RR, true>), grid, dim3(512), 0, s, a);  \
    else hipLaunchKernelGGL((dion_sweep_kernel<RR, false>), grid, dim3(512), 0, s, a);      \
  } while (0)
  if (a.r == 64) ORTHO_SWEEP(64);
  else if (a.r == 128) ORTHO_SWEEP(128);
  else if (a.r == 256) ORTHO_SWEEP(256);
  else ORTHO_SWEEP(512);
#undef ORTHO_SWEEP
  return hipGetLastError();
}

}  // namespace ortho
