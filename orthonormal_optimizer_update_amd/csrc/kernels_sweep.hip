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

// wait until at most `later` stages of PER copies each are outstanding
template <int PER>
__device__ __forceinline__ void wait_later(int later) {
  switch (later) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<PER>(); break;
    case 2: wait_vm<2 * PER>(); break;
    case 3: wait_vm<3 * PER>(); break;
    case 4: wait_vm<4 * PER>(); break;
    case 5: wait_vm<5 * PER>(); break;
    default: wait_vm<6 * PER>(); break;
  }
}

__device__ __forceinline__ float2 bf16x2_to_f32(uint32_t u) {
  return make_float2(__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u));
}

// 8 fp32 values as two bf16 pieces (x = hi + lo + O(2^-16 |x|)).
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const bf16 h = to_bf16(x[t]);
    hi[t] = h;
    lo[t] = to_bf16(x[t] - static_cast<float>(h));
  }
}

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
  // wait until at most `later` stages of this wave's copies are outstanding
  auto wait_stages = [&](int later) {
    static_assert(kStages <= 8 && 6 * L::kMaxPerWave < 64, "wait cases cover up to six later stages");
    if (ncopy == L::kLo) wait_later<L::kLo>(later);
    else wait_later<L::kMaxPerWave>(later);
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
  // the A fragment of stage st into fa[buf]: B = M + G split into hi and lo
  auto read_a = [&](int st, int buf) {
    const char* sb = smem + (st % kStages) * L::kStageBytes;
    const float* sm = reinterpret_cast<const float*>(sb);
    const uint16_t* sg = reinterpret_cast<const uint16_t*>(sb + kMBytes);
    // output row rl, k = half*8 .. + 7 of the stage
    float x[8];
    if (!TRANS) {
      const floatx4 m0 = *reinterpret_cast<const floatx4*>(sm + rl * 16 + (((2 * half) ^ ((rl >> 2) & 3)) * 4));
      const floatx4 m1 = *reinterpret_cast<const floatx4*>(sm + rl * 16 + (((2 * half + 1) ^ ((rl >> 2) & 3)) * 4));
      const uint4 g = *reinterpret_cast<const uint4*>(sg + rl * 16 + ((half ^ ((rl >> 3) & 1)) * 8));
      const float2 g0 = bf16x2_to_f32(g.x), g1 = bf16x2_to_f32(g.y), g2 = bf16x2_to_f32(g.z),
                   g3 = bf16x2_to_f32(g.w);
      x[0] = m0[0] + g0.x; x[1] = m0[1] + g0.y; x[2] = m0[2] + g1.x; x[3] = m0[3] + g1.y;
      x[4] = m1[0] + g2.x; x[5] = m1[1] + g2.y; x[6] = m1[2] + g3.x; x[7] = m1[3] + g3.y;
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int kr = half * 8 + t;
        x[t] = sm[kr * 128 + rl] + bf16_bits_to_f32(sg[kr * 128 + rl]);
      }
    }
    split8(x, fa[buf][0], fa[buf][1]);
  };
  auto read_frags = [&](int st, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    read_a(st, buf);
    read_factor(st, buf, 0);
    read_factor(st, buf, 1);
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
  if constexpr (R == 512) {
    read_a(0, 0);
    read_factor(0, 0, 0);
    read_factor(0, 0, 1);
  } else {
    read_frags(0, std::integral_constant<int, 0>{});
  }

  // one stage whose fragments are in buffer CUR (a compile-time index, so the
  // fragments stay in registers); the next stage's go to buffer CUR ^ 1
  auto step = [&](auto cur_c, int st) {
    constexpr int CUR = decltype(cur_c)::value;
    if (st + 1 < nst) {
      // stage st + 1 in LDS; after this barrier every wave has read stage st's
      // fragments (previous step), so the buffer of stage st - 1 is free
      ready(st + 1, issued_last);
      if (st + kStages - 1 < nst) {
        issue(st + kStages - 1);
        issued_last = st + kStages - 1;
      }
      read_frags(st + 1, std::integral_constant<int, CUR ^ 1>{});
    }
    // each product kind over all accumulators before the next kind
#pragma unroll
    for (int j = 0; j < NB; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[CUR][0], fb[CUR][j][0], acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < NB; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[CUR][0], fb[CUR][j][1], acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < NB; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[CUR][1], fb[CUR][j][0], acc[j], 0, 0, 0);
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
      read_a(st + 1, CUR ^ 1);
      read_factor(st + 1, 0, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NB; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[CUR][0], fb[0][j][0], acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < NB; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[CUR][1], fb[0][j][0], acc[j], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
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
