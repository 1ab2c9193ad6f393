// Large bf16 "NT" GEMM for the Newton-Schulz products on gfx950:
//   C[i, j] = sum_k A[i, k] * B[j, k],  A: M x K, B: N x K, both row-major bf16
// (k contiguous), fp32 accumulation, result handed to an epilogue policy with
// the same interface as gemm_kernel's.
//
// 256 x 256 x 64 block tile, 4 waves in a 2 x 2 grid, 128 x 128 per wave
// (4 x 4 v_mfma_f32_32x32x16_bf16 accumulators).  Operand tiles go straight
// from HBM/L2 into LDS with global_load_lds_dwordx4 (each lane's 16 bytes land
// at LDS base + 16 * lane), two stages, one barrier per 64-wide k step.  The
// LDS row of a tile is 8 chunks of 16 bytes; chunk c of row r is stored at
// position c ^ ((r >> 1) & 7), which each lane realises by choosing which
// global chunk it fetches, so that the fragment reads of 16 consecutive rows
// hit 64 distinct banks.
//
// Requirements (checked by the launcher): M, N multiples of 256, K a multiple
// of 64, 16-byte aligned rows; every split-K slice holds at least one k tile.
#pragma once

#include "gemm_core.h"

namespace ortho {

namespace fast {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int TILE_BYTES = BM * BK * 2;  // 32 KB per operand per stage

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) const void* glb_ptr_t;

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// Issue the loads of one 256 x 64 operand tile into LDS (8 instructions per
// wave; instruction q of wave w fills rows (8w + q) * 8 .. + 7).
__device__ __forceinline__ void load_tile(const uint16_t* src, int64_t ld, int row0, int k0,
                                          char* lds_tile, int wave, int lane) {
  const int sub = lane >> 3;            // row within the 8-row group
  const int pos = lane & 7;             // stored chunk position
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int row = (wave * 8 + q) * 8 + sub;
    const int chunk = swz(row, pos);    // logical chunk this lane fetches
    const uint16_t* g = src + (int64_t)(row0 + row) * ld + k0 + chunk * 8;
    // address-space casts (generic -> global / local) need C-style casts
    __builtin_amdgcn_global_load_lds((glb_ptr_t)(g), (lds_ptr_t)(lds_tile + (wave * 8 + q) * 1024),
                                     16, 0, 0);
  }
}

__device__ __forceinline__ bf16x8 read_frag(const char* lds_tile, int row, int chunk) {
  return *reinterpret_cast<const bf16x8*>(lds_tile + (row * 8 + swz(row, chunk)) * 16);
}

}  // namespace fast

// Accumulators (+)= scale * S for a matrix S of the output's shape (bf16 or
// fp32, leading dimension ld): S's tile is copied row-major into LDS (1 KB per
// wave instruction, 128 KB per pass), then each wave reads its own elements in
// accumulator order.  bf16: one pass of all 256 rows.  fp32: two passes; pass
// p holds, for both row halves h of the tile, rows h * 128 + p * 64 .. + 63
// (LDS row h * 64 + r), i.e. accumulator rows i = 2p, 2p + 1 of every wave.
// Ends with a barrier, so the caller may reuse the LDS.
template <bool kBf, bool kAcc>
__device__ __forceinline__ void fast_preload(floatx16 (&acc)[4][4], const void* srcv, int64_t ldp,
                                             float sc, int m0, int n0, char* smem, int wave,
                                             int lane) {
  using namespace fast;
  constexpr int kEsz = kBf ? 2 : 4;
  constexpr int kRowsPerPass = kBf ? 256 : 128;
  constexpr int kRowsPerInstr = kBf ? 2 : 1;
  constexpr int kInstrPerWave = kRowsPerPass / kRowsPerInstr / 4;
  const int wm = wave >> 1, wn = wave & 1;
  const char* src = static_cast<const char*>(srcv);
  const int lrow = kBf ? (lane >> 5) : 0;
  const int lcol = kBf ? (lane & 31) * 8 : lane * 4;
#pragma unroll
  for (int pass = 0; pass < 256 / kRowsPerPass; ++pass) {
#pragma unroll 8
    for (int q = 0; q < kInstrPerWave; ++q) {
      const int ins = wave * kInstrPerWave + q;
      const int rl = ins * kRowsPerInstr + lrow;  // LDS row
      const int row = m0 + (kBf ? rl : (rl >> 6) * 128 + pass * 64 + (rl & 63));
      const char* g = src + ((int64_t)row * ldp + n0 + lcol) * kEsz;
      __builtin_amdgcn_global_load_lds((glb_ptr_t)(g), (lds_ptr_t)(smem + ins * 1024), 16, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!kBf && (i >> 1) != pass) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int rw = i * 32 + g * 8 + (lane >> 5) * 4 + t;  // row within the wave's 128
            const int rl = kBf ? wm * 128 + rw : wm * 64 + (rw & 63);
            const int cl = wn * 128 + j * 32 + (lane & 31);
            float v;
            if constexpr (kBf)
              v = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(smem)[rl * 256 + cl]);
            else
              v = reinterpret_cast<const float*>(smem)[rl * 256 + cl];
            if constexpr (kAcc)
              acc[i][j][g * 4 + t] += sc * v;
            else
              acc[i][j][g * 4 + t] = sc * v;
          }
        // one accumulator tile at a time keeps the values' live ranges short
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
  }
}

template <class Epi>
__global__ __launch_bounds__(256, 1) void gemm_bf16_256(GemmParams<typename Epi::Args> p) {
  using namespace fast;
  __shared__ __attribute__((aligned(1024))) char smem_fast[2 * 2 * TILE_BYTES];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // Tile order: each XCD (workgroup id mod 8) gets a contiguous run of
  // logical tiles, walked in groups of 4 tile rows so that a run shares A row
  // blocks and B column blocks in that XCD's L2.
  const int nwg = gridDim.x;
  int t = blockIdx.x;
  if ((nwg & 7) == 0) t = (t & 7) * (nwg >> 3) + (t >> 3);
  const int tiles_n = p.tiles_n, tiles_m = nwg / tiles_n;
  const int group = 4 * tiles_n;
  const int first_m = (t / group) * 4;
  const int gsize = min(tiles_m - first_m, 4);
  const int tm = first_m + (t % group) % gsize;
  const int tn = (t % group) / gsize;
  // blockIdx.y = member * splits + split (split-K over the k tiles)
  const int bi = blockIdx.y / p.splits, split = blockIdx.y % p.splits;
  const int m0 = tm * BM, n0 = tn * BN;

  // With Epi::kSegs == 3 the reduction runs over three segments of length K,
  // (a, b0), (a, b0s), (a2, b0): hi*hi + hi*lo + lo*hi of bf16x2 pieces.
  const uint16_t* A = static_cast<const uint16_t*>(p.a.p[bi]);
  const uint16_t* B = static_cast<const uint16_t*>(p.b0.p[bi]);
  const uint16_t* A2 = Epi::kSegs == 3 ? static_cast<const uint16_t*>(p.a2.p[bi]) : A;
  const uint16_t* B2 = Epi::kSegs == 3 ? static_cast<const uint16_t*>(p.b0s.p[bi]) : B;
  const int64_t lda = p.a.ld, ldb = p.b0.ld;
  const int nks = p.K / BK;                       // k tiles per segment
  const int kt_begin = split * p.kchunk;          // this split's k tiles
  const int kt_end = min(kt_begin + p.kchunk, nks * Epi::kSegs);
  auto seg_a = [&](int kt) { return Epi::kSegs == 3 && kt >= 2 * nks ? A2 : A; };
  auto seg_b = [&](int kt) { return Epi::kSegs == 3 && kt >= nks && kt < 2 * nks ? B2 : B; };
  auto seg_k = [&](int kt) {  // k offset within the segment (no division)
    if constexpr (Epi::kSegs == 3) kt -= kt >= 2 * nks ? 2 * nks : (kt >= nks ? nks : 0);
    return kt * BK;
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  Epi epi(p.e, bi, split);
  if constexpr (Epi::kFastPre != 0)
    fast_preload<Epi::kFastPre == 1, false>(acc, epi.fast_pre_src(), epi.fast_pre_ld(),
                                            epi.fast_pre_scale(), m0, n0, smem_fast, wave, lane);
  if constexpr (Epi::kFastPre2 != 0)
    fast_preload<true, true>(acc, epi.fast_pre2_src(), epi.fast_pre2_ld(), epi.fast_pre2_scale(),
                             m0, n0, smem_fast, wave, lane);

  auto sa = [&](int st) { return smem_fast + st * 2 * TILE_BYTES; };
  auto sb = [&](int st) { return smem_fast + st * 2 * TILE_BYTES + TILE_BYTES; };

  load_tile(seg_a(kt_begin), lda, m0, seg_k(kt_begin), sa(0), wave, lane);
  load_tile(seg_b(kt_begin), ldb, n0, seg_k(kt_begin), sb(0), wave, lane);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const int frow = lane & 31, fchunk = lane >> 5;
  // Fragments are double-buffered in registers: the reads for k step kk + 1
  // are issued before the 16 products of step kk, so LDS latency overlaps the
  // matrix cores (also across the k-tile barrier).
  bf16x8 fa[2][4], fb[2][4];
  auto read_frags = [&](bf16x8 (&a)[4], bf16x8 (&b)[4], const char* ta, const char* tb, int kk) {
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = read_frag(ta, wm * 128 + i * 32 + frow, kk * 2 + fchunk);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = read_frag(tb, wn * 128 + j * 32 + frow, kk * 2 + fchunk);
  };
  // One 64-wide k tile: loads of the next tile into the other stage, four
  // 16-wide steps of products on this one, barrier, first fragments of the
  // next tile.
  auto k_tile = [&](int kt) {
    const int cur = (kt - kt_begin) & 1;
    const bool more = kt + 1 < kt_end;
    if (more) {
      load_tile(seg_a(kt + 1), lda, m0, seg_k(kt + 1), sa(cur ^ 1), wave, lane);
      load_tile(seg_b(kt + 1), ldb, n0, seg_k(kt + 1), sb(cur ^ 1), wave, lane);
    }
    const char* ta = sa(cur);
    const char* tb = sb(cur);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk < 3) read_frags(fa[(kk + 1) & 1], fb[(kk + 1) & 1], ta, tb, kk + 1);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk & 1][i], fb[kk & 1][j], acc[i][j], 0, 0, 0);
    }
    // Instruction order for the scheduler: tile loads first, then for each k
    // step the next step's 8 fragment reads interleaved with its 16 products.
    __builtin_amdgcn_sched_group_barrier(0x020, 16, 0);  // VMEM reads (tile loads)
#pragma unroll
    for (int kk = 0; kk < 3; ++kk) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one DS read
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // two MFMAs
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (more) read_frags(fa[0], fb[0], sa(cur ^ 1), sb(cur ^ 1), 0);
  };
  read_frags(fa[0], fb[0], sa(0), sb(0), 0);
  // The first tile is peeled (K >= 64 is checked by the launcher): the
  // accumulators' initial values then feed products directly instead of also
  // reaching the epilogue through a zero-trip path.
  k_tile(kt_begin);
  for (int kt = kt_begin + 1; kt < kt_end; ++kt) k_tile(kt);

  // Transposed outputs straight from the accumulators (four consecutive rows
  // of one column per lane).
  if constexpr (Epi::kFastT) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int row0 = m0 + wm * 128 + i * 32 + g * 8 + (lane >> 5) * 4;
          const int col = n0 + wn * 128 + j * 32 + (lane & 31);
          const floatx4 v = {acc[i][j][g * 4 + 0], acc[i][j][g * 4 + 1], acc[i][j][g * 4 + 2],
                             acc[i][j][g * 4 + 3]};
          epi.fast_store_t4(col, row0, v);
        }
  }
  // Row-major outputs through LDS in two passes; pass p stages accumulator
  // rows i = 2p, 2p + 1 of every wave (tile rows h * 128 + p * 64 .. + 63 of
  // both row halves h, at LDS row h * 64 + r), then each wave hands one
  // 256-wide row at a time to the policy, four columns per lane.  The main
  // loop's last barrier has released the LDS.
  float* stage = reinterpret_cast<float*>(smem_fast);
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int i = 2 * pass; i < 2 * pass + 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int t = 0; t < 4; ++t)
            stage[(wm * 64 + (i & 1) * 32 + g * 8 + (lane >> 5) * 4 + t) * 256 + wn * 128 + j * 32 +
                  (lane & 31)] = acc[i][j][g * 4 + t];
    __syncthreads();
#pragma unroll 4
    for (int q = 0; q < 32; ++q) {
      const int rl = q * 4 + wave;
      const floatx4 v = *reinterpret_cast<const floatx4*>(stage + rl * 256 + lane * 4);
      epi.fast_store4(m0 + (rl >> 6) * 128 + pass * 64 + (rl & 63), n0 + lane * 4, v);
    }
    __syncthreads();
  }
}

}  // namespace ortho
