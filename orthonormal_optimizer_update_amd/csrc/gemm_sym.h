// Symmetric bf16 products C = A B^T with C symmetric (the Newton-Schulz Gram
// X X^T and polynomial b A + c A A, A symmetric), on gfx950, spread so that
// one 256-row tile grid of side T fills T^2 workgroups of about equal work:
//
// - each tile (tm, tn) above the diagonal is computed as two 256 x 128 column
//   halves, each by its own workgroup (four waves of 128 x 64: 4 x 2
//   v_mfma_f32_32x32x16_bf16 accumulators), and stored with its mirror;
// - each diagonal tile computes only its 36 upper 32 x 32 blocks: wave w owns
//   block rows w and 7 - w (8 - w and w + 1 blocks: nine per wave), and the
//   blocks above the diagonal are stored with their mirror.
// T (T - 1) half tiles and T diagonal tiles make T^2 workgroups: 256 at
// 4096 x 4096, one per CU, where the 256 x 256 kernel ran the T (T + 1) / 2
// upper tiles on 136 CUs.  A half tile carries half a tile's products, a
// diagonal tile 9/16 of them.
//
// Operand tiles (256 x 64 of A, 128 x 64 of B; a diagonal tile's B is its A)
// go straight from global memory into LDS with global_load_lds_dwordx4 in the
// same swizzled layout as the 256 x 256 kernel, three stages deep.  The issue
// order inside a k tile is fixed with scheduling fences: every slot of a
// 16-deep k step holds one product and at most one fragment read for the next
// step (left to itself the compiler sinks each read to just before its first
// product and waits on it there), and a tile's copies are spread over four k
// steps rather than issued in one burst.  After the loop, the policy's memory term (kFastPre == 1: a
// bf16 source S, symmetric like the result) is added as S[col][row .. row + 3]
// (one 8-byte read per lane), mirrors are stored straight from the
// accumulators (four consecutive rows of one column are contiguous in the
// mirror), and the direct blocks pass through a per-wave LDS transposition so
// that each store instruction covers eight whole 32-column row segments.
//
// Requirements (checked by the launcher): M = N, a multiple of 256; K a
// positive multiple of 64; 16-byte aligned rows; the operand-row conditions of the
// 256 x 256 kernel (fast_ok); one split.
#pragma once

#include <type_traits>

#include "gemm_fast.h"

namespace ortho {

namespace symk {

constexpr int BK = 64;
constexpr int A_BYTES = 256 * BK * 2;    // 32 KB
constexpr int B_BYTES = 128 * BK * 2;    // 16 KB
constexpr int STAGE = A_BYTES + B_BYTES;
constexpr int NSTAGE = 3;
constexpr int kTp = 36;                  // floats per row of a wave's 32 x 32 staging block

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// The policy's memory term (kFastPre == 1) for NB accumulator blocks at rows
// r0[b], columns c0[b]: S[row0 + t][col] read as S[col][row0 + t] (S
// symmetric), every load of the wave issued before any is added.
template <class Epi, int NB>
__device__ __forceinline__ void blocks_pre(const Epi& epi, floatx16 (&acc)[NB], const int (&r0)[NB],
                                           const int (&c0)[NB], int lane) {
  if constexpr (Epi::kFastPre == 1) {
    const uint16_t* src = static_cast<const uint16_t*>(epi.fast_pre_src());
    const int64_t ld = epi.fast_pre_ld();
    const float sc = epi.fast_pre_scale();
    uint2 u[NB][4];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int row0 = r0[b] + g * 8 + (lane >> 5) * 4, col = c0[b] + (lane & 31);
        u[b][g] = *reinterpret_cast<const uint2*>(src + (int64_t)col * ld + row0);
      }
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        acc[b][g * 4 + 0] += sc * __uint_as_float(u[b][g].x << 16);
        acc[b][g * 4 + 1] += sc * __uint_as_float(u[b][g].x & 0xffff0000u);
        acc[b][g * 4 + 2] += sc * __uint_as_float(u[b][g].y << 16);
        acc[b][g * 4 + 3] += sc * __uint_as_float(u[b][g].y & 0xffff0000u);
      }
  }
}

// The mirror and the direct store of one 32 x 32 accumulator block at rows
// r0, columns c0 (r0 < c0 unless the block is on the diagonal).  st: this
// wave's staging block in LDS.
template <class Epi>
__device__ __forceinline__ void block_out(Epi& epi, const floatx16& acc, int r0, int c0, bool mirror,
                                          float* st, int lane) {
  if (mirror) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int row0 = r0 + g * 8 + (lane >> 5) * 4, col = c0 + (lane & 31);
      const floatx4 v = {acc[g * 4 + 0], acc[g * 4 + 1], acc[g * 4 + 2], acc[g * 4 + 3]};
      epi.fast_store_t4(col, row0, v);
    }
  }
  // direct: transpose through LDS (the wave's own 32 x kTp floats; LDS
  // instructions of a wave run in order, so no barrier is needed)
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int t = 0; t < 4; ++t)
      st[(g * 8 + (lane >> 5) * 4 + t) * kTp + (lane & 31)] = acc[g * 4 + t];
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int rl = (lane >> 3) + 8 * q, cl = (lane & 7) * 4;
    const floatx4 v = *reinterpret_cast<const floatx4*>(st + rl * kTp + cl);
    epi.fast_store4(r0 + rl, c0 + cl, v);
  }
}

struct SymTile {
  int tm, tn, half;
};

// Unit u of the ordered walk over the upper triangle of a t x t tile grid:
// tile rows in order, each row's diagonal tile (one unit) first, then the two
// 256 x 128 halves of each tile to its right.
__host__ __device__ inline SymTile sym_walk(int t, int u) {
  int tm = 0;
  while (u >= 1 + 2 * (t - 1 - tm)) {
    u -= 1 + 2 * (t - 1 - tm);
    ++tm;
  }
  if (u == 0) return SymTile{tm, tm, 0};
  return SymTile{tm, tm + 1 + (u - 1) / 2, (u - 1) & 1};
}

// Workgroup b of the nwg = T^2 units of a T x T tile grid (T diagonal tiles,
// T (T - 1) halves).  Workgroups are dealt to the 8 XCDs round robin (XCD
// b mod 8, in the order b / 8), and both operands of these products are row
// blocks of one matrix, so an XCD's L2 fetches the union of the row blocks
// its tiles touch.  With T = 4 s, the grid splits into 4 x 4 blocks of s x s
// tiles: XCDs 0..5 each take one of the six blocks above the diagonal (2 s^2
// units, 2 s distinct row blocks) and XCDs 6 and 7 two of the four diagonal
// blocks each (s^2 units and s row blocks apiece): 16 s row blocks fetched
// in all, against about twice that for runs of the row-ordered walk.  Any
// other T takes, per XCD, a contiguous run of the walk.
__host__ __device__ inline SymTile sym_tile(int t, int nwg, int b) {
  if (nwg == t * t && t % 4 == 0) {
    const int s = t / 4, x = b & 7, l = b >> 3;
    if (x < 6) {
      // off-diagonal block (bi, bj) of the 4 x 4 block grid, tiles in row order
      const int bi = x < 3 ? 0 : (x < 5 ? 1 : 2);
      const int bj = x < 3 ? x + 1 : (x < 5 ? x - 1 : 3);
      const int i = l / (2 * s), rem = l - i * 2 * s;
      return SymTile{bi * s + i, bj * s + rem / 2, rem & 1};
    }
    // diagonal blocks 2 (x - 6) and 2 (x - 6) + 1, s^2 units each
    const int d = 2 * (x - 6) + (l >= s * s ? 1 : 0);
    const SymTile w = sym_walk(s, l % (s * s));
    return SymTile{d * s + w.tm, d * s + w.tn, w.half};
  }
  const int u = (nwg & 7) == 0 ? (b & 7) * (nwg >> 3) + (b >> 3) : b;
  return sym_walk(t, u);
}

}  // namespace symk

template <class Epi>
__global__ __launch_bounds__(256, 1) void gemm_bf16_sym(GemmParams<typename Epi::Args> p) {
  using namespace fast;
  static_assert(Epi::kSegs == 1 && Epi::kFastSym && Epi::kFastPre2 == 0, "symmetric single-segment policies");
  __shared__ __attribute__((aligned(1024))) char smem[symk::NSTAGE * symk::STAGE];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // Workgroup -> tile (symk::sym_tile): the tiles of one XCD share operand
  // row blocks in its L2.
  const symk::SymTile tile = symk::sym_tile(p.tiles_n, gridDim.x, blockIdx.x);
  const int tm = tile.tm, tn = tile.tn, half = tile.half;
  const bool diag = tm == tn;
  const int bi = blockIdx.y;
  const int m0 = tm * 256;
  const int n0 = tn * 256 + half * 128;

  const uint16_t* A = static_cast<const uint16_t*>(p.a.p[bi]);
  const uint16_t* B = static_cast<const uint16_t*>(p.b0.p[bi]);
  const int64_t lda = p.a.ld, ldb = p.b0.ld;
  const int nk = p.K / symk::BK;
  Epi epi(p.e, bi, 0);
  const unsigned lds0 = lds_addr(smem);

  // copy instruction q of wave w: A rows (8 w + q) * 8 .. + 7 (q < 8), B rows
  // (4 w + q) * 8 .. + 7 (q < 4); lane = 8 * (row within the group) + stored
  // chunk position, the fetched chunk swizzled as in the 256 x 256 kernel
  const int sub = lane >> 3, pos = lane & 7;
  unsigned offa[8], offb[4];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int row = (wave * 8 + q) * 8 + sub;
    offa[q] = static_cast<unsigned>((row * lda + swz(row, pos) * 8) * 2);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = (wave * 4 + q) * 8 + sub;
    offb[q] = static_cast<unsigned>((row * ldb + swz(row, pos) * 8) * 2);
  }
  auto base_a = [&](int kt) {
    return uniform_ptr(reinterpret_cast<const char*>(A + (int64_t)m0 * lda + kt * symk::BK));
  };
  auto base_b = [&](int kt) {
    return uniform_ptr(reinterpret_cast<const char*>(B + (int64_t)n0 * ldb + kt * symk::BK));
  };
  auto dma_a = [&](int q, const char* ba, int st) {
    dma16(offa[q], ba, lds0 + st * symk::STAGE + (wave * 8 + q) * 1024);
  };
  auto dma_b = [&](int q, const char* bb, int st) {
    dma16(offb[q], bb, lds0 + st * symk::STAGE + symk::A_BYTES + (wave * 4 + q) * 1024);
  };
  // copy c of a tile: c < 8 the A rows of dma_a(c), else the B rows of dma_b(c - 8)
  auto dma_c = [&](int c, const char* ba, const char* bb, int st) {
    if (c < 8) dma_a(c, ba, st);
    else dma_b(c - 8, bb, st);
  };
  // Stage of tile k: k mod 3.  Tile k + 3's copies are spread over the four
  // k steps that follow the barrier at which every wave is done with tile k
  // (E of them in tile k's last step, the rest in the first three steps of
  // tile k + 1), so that the copy instructions of the four waves never queue
  // up at once.  Before the loop: tiles 0 and 1 whole and tile 2's first E
  // copies, then wait for tile 0.  At every later wait each wave has exactly
  // one tile's copies (8 or 12) in flight.  A tile index past the last
  // reloads the last tile into a stage nobody reads.
  const int ncp = diag ? 8 : 12;          // copies per tile and wave
  const int ecp = diag ? 2 : 4;           // of them in the last k step
  {
#pragma unroll
    for (int k = 0; k < symk::NSTAGE; ++k) {
      const int kl = min(k, nk - 1);
      const char* ba = base_a(kl);
      const char* bb = base_b(kl);
      const int nc = k + 1 < symk::NSTAGE ? ncp : ecp;
#pragma unroll
      for (int c = 0; c < 12; ++c)
        if (c < nc) dma_c(c, ba, bb, k);
    }
    asm volatile("" ::: "memory");
    if (diag) symk::wait_vm<10>();
    else symk::wait_vm<16>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
  // end of a tile's first three k steps: this wave's fragment reads and tile
  // kt + 1's copies done (tile kt + 2's in flight), then every wave's
  auto tile_barrier = [&]() {
    asm volatile("" ::: "memory");
    if (diag) asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(12) lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  const int frow = lane & 31, fchunk = lane >> 5;
  float* stage_out = reinterpret_cast<float*>(smem) + wave * 32 * symk::kTp;

  if (!diag) {
    // ---- half tile: wave (wm, wn) rows wm * 128 .. + 127, columns wn * 64 .. + 63.
    // Issue order fixed by scheduling fences: each of the 8 slots of a
    // 16-deep k step holds one product and (slots 0 .. 5) one fragment read
    // for the next step, in the order the next step consumes them (a0 b0 b1
    // a1 a2 a3); slots 0, 3, 6 of the first three steps carry copies 4 .. 11
    // of tile kt + 2, slots 0 .. 3 of the fourth step copies 0 .. 3 of tile
    // kt + 3, and the fourth step reads the first step of tile kt + 1.
    const int wm = wave >> 1, wn = wave & 1;
    floatx16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    bf16x8 fa[2][4], fb[2][2];
    auto rd = [&](int buf, int q, const char* ta, int kk) {
      const char* tb = ta + symk::A_BYTES;
      const int c = kk * 2 + fchunk;
      if (q == 0) fa[buf][0] = read_frag(ta, wm * 128 + frow, c);
      if (q == 1) fb[buf][0] = read_frag(tb, wn * 64 + frow, c);
      if (q == 2) fb[buf][1] = read_frag(tb, wn * 64 + 32 + frow, c);
      if (q >= 3) fa[buf][q - 2] = read_frag(ta, wm * 128 + (q - 2) * 32 + frow, c);
    };
    auto mma = [&](int buf, int q) {
      const int i = q >> 1, j = q & 1;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
    };
#pragma unroll
    for (int q = 0; q < 6; ++q) rd(0, q, smem, 0);
    __builtin_amdgcn_sched_barrier(0);
    int cur = 0;
    for (int kt = 0; kt < nk; ++kt) {
      const char* ta = smem + cur * symk::STAGE;
      const int nxt = cur == symk::NSTAGE - 1 ? 0 : cur + 1;
      const int prv = nxt == symk::NSTAGE - 1 ? 0 : nxt + 1;   // tile kt + 2's stage
      const int k2 = min(kt + 2, nk - 1);
      const char* ba2 = base_a(k2);
      const char* bb2 = base_b(k2);
#pragma unroll
      for (int kk = 0; kk < 3; ++kk) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          if (q < 6) rd((kk + 1) & 1, q, ta, kk + 1);
          if (q % 3 == 0 && 4 + 3 * kk + q / 3 < 12) dma_c(4 + 3 * kk + q / 3, ba2, bb2, prv);
          mma(kk & 1, q);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      tile_barrier();
      const int k3 = min(kt + 3, nk - 1);
      const char* ba3 = base_a(k3);
      const char* bb3 = base_b(k3);
      const char* na = smem + nxt * symk::STAGE;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (q < 6) rd(0, q, na, 0);
        if (q < 4) dma_c(q, ba3, bb3, cur);
        mma(1, q);
        __builtin_amdgcn_sched_barrier(0);
      }
      cur = nxt;
    }
    symk::wait_vm<0>();   // the reloads past the last tile land before the LDS is reused
    __syncthreads();   // every wave is done with the operand stages
    floatx16 blk[8];
    int r0[8], c0[8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        blk[i * 2 + j] = acc[i][j];
        r0[i * 2 + j] = m0 + wm * 128 + i * 32;
        c0[i * 2 + j] = n0 + wn * 64 + j * 32;
      }
    symk::blocks_pre(epi, blk, r0, c0, lane);
#pragma unroll
    for (int b = 0; b < 8; ++b) symk::block_out(epi, blk[b], r0[b], c0[b], true, stage_out, lane);
    return;
  }

  // ---- diagonal tile: wave W owns block rows W and 7 - W of the upper blocks
  auto diag_wave = [&](auto w_c) {
    constexpr int W = decltype(w_c)::value;
    constexpr int NF = 8 - W;          // fragments of block rows W .. 7
    constexpr int N0 = 8 - W;          // blocks (W, W .. 7)
    constexpr int N1 = W + 1;          // blocks (7 - W, 7 - W .. 7)
    floatx16 acc[N0 + N1];
#pragma unroll
    for (int b = 0; b < N0 + N1; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[b][e] = 0.f;
    // the same slot order as the half tiles: nine products per step, slots
    // 0 .. NF - 1 read the next step's fragments (row W + q); slots 0 and 4
    // of the first three steps carry copies 2 .. 7 of tile kt + 2, those of
    // the fourth step copies 0 and 1 of tile kt + 3
    bf16x8 f[2][NF];
    auto rd = [&](int buf, int q, const char* ta, int kk) {
      f[buf][q] = read_frag(ta, (W + q) * 32 + frow, kk * 2 + fchunk);
    };
    auto mma = [&](int buf, int b) {
      if (b < N0)
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[buf][0], f[buf][b], acc[b], 0, 0, 0);
      else
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[buf][7 - 2 * W], f[buf][7 - 2 * W + b - N0],
                                                         acc[b], 0, 0, 0);
    };
#pragma unroll
    for (int q = 0; q < NF; ++q) rd(0, q, smem, 0);
    __builtin_amdgcn_sched_barrier(0);
    int cur = 0;
    for (int kt = 0; kt < nk; ++kt) {
      const char* ta = smem + cur * symk::STAGE;
      const int nxt = cur == symk::NSTAGE - 1 ? 0 : cur + 1;
      const int prv = nxt == symk::NSTAGE - 1 ? 0 : nxt + 1;   // tile kt + 2's stage
      const char* ba2 = base_a(min(kt + 2, nk - 1));
#pragma unroll
      for (int kk = 0; kk < 3; ++kk) {
#pragma unroll
        for (int q = 0; q < N0 + N1; ++q) {
          if (q < NF) rd((kk + 1) & 1, q, ta, kk + 1);
          if (q % 4 == 0 && q < 8) dma_a(2 + 2 * kk + q / 4, ba2, prv);
          mma(kk & 1, q);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      tile_barrier();
      const char* ba3 = base_a(min(kt + 3, nk - 1));
      const char* na = smem + nxt * symk::STAGE;
#pragma unroll
      for (int q = 0; q < N0 + N1; ++q) {
        if (q < NF) rd(0, q, na, 0);
        if (q % 4 == 0 && q < 8) dma_a(q / 4, ba3, cur);
        mma(1, q);
        __builtin_amdgcn_sched_barrier(0);
      }
      cur = nxt;
    }
    symk::wait_vm<0>();
    __syncthreads();
    int r0[N0 + N1], c0[N0 + N1];
#pragma unroll
    for (int b = 0; b < N0; ++b) {
      r0[b] = m0 + W * 32;
      c0[b] = m0 + (W + b) * 32;
    }
#pragma unroll
    for (int b = 0; b < N1; ++b) {
      r0[N0 + b] = m0 + (7 - W) * 32;
      c0[N0 + b] = m0 + (7 - W + b) * 32;
    }
    symk::blocks_pre(epi, acc, r0, c0, lane);
#pragma unroll
    for (int b = 0; b < N0; ++b) symk::block_out(epi, acc[b], r0[b], c0[b], b > 0, stage_out, lane);
#pragma unroll
    for (int b = 0; b < N1; ++b)
      symk::block_out(epi, acc[N0 + b], r0[N0 + b], c0[N0 + b], b > 0, stage_out, lane);
  };
  switch (wave) {
    case 0: diag_wave(std::integral_constant<int, 0>{}); break;
    case 1: diag_wave(std::integral_constant<int, 1>{}); break;
    case 2: diag_wave(std::integral_constant<int, 2>{}); break;
    default: diag_wave(std::integral_constant<int, 3>{}); break;
  }
}

}  // namespace ortho
