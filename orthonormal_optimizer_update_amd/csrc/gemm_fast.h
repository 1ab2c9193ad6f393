// Large bf16 "NT" GEMM for the Newton-Schulz products on gfx950:
//   C[i, j] = sum_k A[i, k] * B[j, k],  A: M x K, B: N x K, both row-major bf16
// (k contiguous), fp32 accumulation, result handed to an epilogue policy with
// the same interface as gemm_kernel's.
//
// 256 x 256 x 64 block tile, 4 waves in a 2 x 2 grid, 128 x 128 per wave
// (4 x 4 v_mfma_f32_32x32x16_bf16 accumulators).  Operand tiles go straight
// from HBM/L2 into LDS with global_load_lds_dwordx4 (each lane's 16 bytes land
// at M0 + 16 * lane), two stages, one barrier per 64-wide k step.  The LDS row
// of a tile is 8 chunks of 16 bytes; chunk c of row r is stored at position
// c ^ ((r >> 1) & 7), which each lane realises by choosing which global chunk
// it fetches, so that the fragment reads of 16 consecutive rows hit 64
// distinct banks.
//
// Issue order inside a k tile is fixed by hand (scheduling fences): each of
// the 8 slots of a 16-wide k step holds one fragment read for the next step,
// in the order the next step's products consume them (a0 b0 b1 b2 b3 a1 a2
// a3), and two products; the 16 tile loads of the next tile ride in the slots
// of the first step.  The barrier sits before the last step's products, so the
// first fragment reads of the next tile overlap them.  The tile loads are
// written as inline assembly with a scalar base address and a per-lane 32-bit
// offset: the compiler treats the LDS-DMA builtin as an unordered LDS event
// and would then wait for every outstanding fragment read before each product
// step; with the loads hidden from it, its LDS waits count exactly, and the
// kernel waits for the loads itself (s_waitcnt before the barrier).
//
// Requirements (checked by the launcher): M, N multiples of 256, K a multiple
// of 64, 16-byte aligned rows, 256 rows of an operand within 4 GiB of bytes;
// every split-K slice holds at least one k tile.
#pragma once

#include "gemm_core.h"

namespace ortho {

namespace fast {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int TILE_BYTES = BM * BK * 2;  // 32 KB per operand per stage
// row of the transposed bf16 tile staged in LDS: 256 elements + 8 of padding
// (528 bytes: 16-byte aligned, and the 32 columns written by one instruction
// fall two to a bank pair)
constexpr int kTRow = 264;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// 16 bytes per lane from global memory into LDS at lds + 16 * lane.  lds must
// be wave-uniform.  The compiler does not look inside the assembly for
// hazards, so it carries its own wait states: five before anything in it (a
// vector instruction that wrote an SGPR the load reads, e.g. a readfirstlane
// of the base, needs five before a vector memory instruction), and one between
// the M0 write and the load.  The caller waits (vmcnt) before the LDS is read.
__device__ __forceinline__ void dma16(unsigned voff, const char* sbase, unsigned lds) {
  asm volatile("s_nop 4\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds) : "memory");
}
__device__ __forceinline__ void dma16_flat(const void* addr, unsigned lds) {
  asm volatile("s_nop 4\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(addr), "s"(lds) : "memory");
}

// A pointer the caller knows to be wave-uniform, in scalar registers.
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const char*>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ unsigned lds_addr(const char* p) {
  // address-space cast (generic -> local) needs a C-style cast
  return __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(lds_ptr_t)(p));
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
  const unsigned lds0 = lds_addr(smem);
#pragma unroll
  for (int pass = 0; pass < 256 / kRowsPerPass; ++pass) {
#pragma unroll 8
    for (int q = 0; q < kInstrPerWave; ++q) {
      const int ins = wave * kInstrPerWave + q;
      const int rl = ins * kRowsPerInstr + lrow;  // LDS row
      const int row = m0 + (kBf ? rl : (rl >> 6) * 128 + pass * 64 + (rl & 63));
      const char* g = src + ((int64_t)row * ldp + n0 + lcol) * kEsz;
      dma16_flat(g, lds0 + ins * 1024);
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
  // (policies with a transposed output also stage that tile, 256 x kTRow
  // bf16, in the same memory after the loop)
  constexpr int kLds = Epi::kFastT ? (256 * kTRow * 2 > 4 * TILE_BYTES ? 256 * kTRow * 2 : 4 * TILE_BYTES)
                                   : 4 * TILE_BYTES;
  __shared__ __attribute__((aligned(1024))) char smem_fast[kLds];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // Tile order: each XCD (workgroup id mod 8) gets a contiguous run of
  // logical tiles, walked in groups of 4 tile rows so that a run shares A row
  // blocks and B column blocks in that XCD's L2.
  const int nwg = gridDim.x;
  int t = blockIdx.x;
  if ((nwg & 7) == 0) t = (t & 7) * (nwg >> 3) + (t >> 3);
  const int tiles_n = p.tiles_n;
  int tm, tn;
  if (Epi::kFastSym && p.sym) {
    // symmetric result: tiles on and above the diagonal, row by row
    int rem = t;
    tm = 0;
    while (rem >= tiles_n - tm) {
      rem -= tiles_n - tm;
      ++tm;
    }
    tn = tm + rem;
  } else {
    const int tiles_m = nwg / tiles_n;
    const int group = 4 * tiles_n;
    const int first_m = (t / group) * 4;
    const int gsize = min(tiles_m - first_m, 4);
    tm = first_m + (t % group) % gsize;
    tn = (t % group) / gsize;
  }
  // blockIdx.y = member * splits + split (split-K over the k tiles)
  const int bi = blockIdx.y / p.splits, split = blockIdx.y % p.splits;
  const int m0 = tm * BM, n0 = tn * BN;

  // Epi::kSegs > 1: the reduction runs over segments of length K, each the
  // product of one piece of A and one piece of B (bf16 pieces of fp32 data,
  // x = p0 + p1 (+ p2)), in the order
  //   kSegs == 3: p0 q0, p0 q1, p1 q0                        (bf16x3)
  //   kSegs == 6: p0 q0, p0 q1, p1 q0, p0 q2, p1 q1, p2 q0   (bf16x6)
  // with p0..p2 = a, a2, a3 and q0..q2 = b0, b0s, b0t.
  static_assert(Epi::kSegs == 1 || Epi::kSegs == 3 || Epi::kSegs == 6, "segment count");
  const uint16_t* A = static_cast<const uint16_t*>(p.a.p[bi]);
  const uint16_t* B = static_cast<const uint16_t*>(p.b0.p[bi]);
  const uint16_t* A2 = Epi::kSegs > 1 ? static_cast<const uint16_t*>(p.a2.p[bi]) : A;
  const uint16_t* B2 = Epi::kSegs > 1 ? static_cast<const uint16_t*>(p.b0s.p[bi]) : B;
  const uint16_t* A3 = Epi::kSegs == 6 ? static_cast<const uint16_t*>(p.a3.p[bi]) : A;
  const uint16_t* B3 = Epi::kSegs == 6 ? static_cast<const uint16_t*>(p.b0t.p[bi]) : B;
  const int64_t lda = p.a.ld, ldb = p.b0.ld;
  const int nks = p.K / BK;                       // k tiles per segment
  const int kt_begin = split * p.kchunk;          // this split's k tiles
  const int kt_end = min(kt_begin + p.kchunk, nks * Epi::kSegs);
  auto seg_of = [&](int kt) {  // segment of k tile kt (no division)
    int sg = 0;
#pragma unroll
    for (int t = 1; t < Epi::kSegs; ++t) sg += kt >= t * nks;
    return sg;
  };
  // byte address of row m0 / n0 of tile kt (uniform: scalar registers)
  auto base_a = [&](int kt) {
    const int sg = seg_of(kt);
    const uint16_t* src = sg == 5 ? A3 : (sg == 2 || sg == 4 ? A2 : A);
    return uniform_ptr(reinterpret_cast<const char*>(src + (int64_t)m0 * lda + (kt - sg * nks) * BK));
  };
  auto base_b = [&](int kt) {
    const int sg = seg_of(kt);
    const uint16_t* src = sg == 3 ? B3 : (sg == 1 || sg == 4 ? B2 : B);
    return uniform_ptr(reinterpret_cast<const char*>(src + (int64_t)n0 * ldb + (kt - sg * nks) * BK));
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  Epi epi(p.e, bi, split);

  auto sa = [&](int st) { return smem_fast + st * 2 * TILE_BYTES; };
  auto sb = [&](int st) { return smem_fast + st * 2 * TILE_BYTES + TILE_BYTES; };
  const unsigned lds0 = lds_addr(smem_fast);

  // Tile loads: instruction q (0..7 rows of A, 8..15 rows of B) of wave w
  // fills rows (8w + q % 8) * 8 .. + 7 of its operand tile; lane = 8 * (row
  // within the group) + stored chunk position.  Per-lane byte offsets from
  // the tile's first row are loop-invariant.
  const int sub = lane >> 3, pos = lane & 7;
  unsigned offa[8], offb[8];
#pragma unroll
  for (int qq = 0; qq < 8; ++qq) {
    const int row = (wave * 8 + qq) * 8 + sub;
    const int chunk = swz(row, pos);  // logical chunk this lane fetches
    offa[qq] = static_cast<unsigned>((row * lda + chunk * 8) * 2);
    offb[qq] = static_cast<unsigned>((row * ldb + chunk * 8) * 2);
  }
  auto load_one = [&](int q, const char* ba, const char* bb, int st) {
    const int qq = q & 7;
    if (q < 8) dma16(offa[qq], ba, lds0 + st * 2 * TILE_BYTES + (wave * 8 + qq) * 1024);
    else dma16(offb[qq], bb, lds0 + st * 2 * TILE_BYTES + TILE_BYTES + (wave * 8 + qq) * 1024);
  };

  const int frow = lane & 31, fchunk = lane >> 5;
  // Fragments of two consecutive 16-wide k steps: read q of step kk goes to
  // buffer kk & 1 in consumption order a0 b0 b1 b2 b3 a1 a2 a3.
  bf16x8 fa[2][4], fb[2][4];
  auto read_one = [&](int buf, int q, const char* ta, const char* tb, int kk) {
    if (q == 0) fa[buf][0] = read_frag(ta, wm * 128 + frow, kk * 2 + fchunk);
    else if (q <= 4) fb[buf][q - 1] = read_frag(tb, wn * 128 + (q - 1) * 32 + frow, kk * 2 + fchunk);
    else fa[buf][q - 4] = read_frag(ta, wm * 128 + (q - 4) * 32 + frow, kk * 2 + fchunk);
  };
  // product pair q: accumulators (q / 2, 2 (q % 2)) and (q / 2, 2 (q % 2) + 1)
  auto mfma_pair = [&](int buf, int q) {
    const int i = q >> 1, j0 = (q & 1) * 2;
    acc[i][j0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j0], acc[i][j0], 0, 0, 0);
    acc[i][j0 + 1] =
        __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j0 + 1], acc[i][j0 + 1], 0, 0, 0);
  };

  {
    const char* ba = base_a(kt_begin);
    const char* bb = base_b(kt_begin);
#pragma unroll
    for (int q = 0; q < 16; ++q) load_one(q, ba, bb, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 8; ++q) read_one(0, q, sa(0), sb(0), 0);
  __builtin_amdgcn_sched_barrier(0);

  // One 64-wide k tile on stage cur while the next tile streams into the other
  // stage.  The last tile reloads itself into the free stage (no branch; the
  // copy is never read), and the fragment reads of the "next" tile after the
  // last barrier likewise go unused.
  auto k_tile = [&](int kt) {
    const int cur = (kt - kt_begin) & 1;
    const int kn = kt + 1 < kt_end ? kt + 1 : kt;
    const char* ba = base_a(kn);
    const char* bb = base_b(kn);
    const char* ta = sa(cur);
    const char* tb = sb(cur);
#pragma unroll
    for (int kk = 0; kk < 3; ++kk) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (kk == 0) {
          load_one(2 * q, ba, bb, cur ^ 1);
          load_one(2 * q + 1, ba, bb, cur ^ 1);
        }
        read_one((kk + 1) & 1, q, ta, tb, kk + 1);
        mfma_pair(kk & 1, q);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // The last step's fragments are in registers: wait for this wave's tile
    // loads and fragment reads, then the barrier hands stage cur over to the
    // next tile's loads and stage cur ^ 1 to the fragment reads.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      read_one(0, q, sa(cur ^ 1), sb(cur ^ 1), 0);
      mfma_pair(1, q);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int kt = kt_begin; kt < kt_end; ++kt) k_tile(kt);

  // Memory terms of the policy (scale * S) join the products after the loop:
  // accumulators that start at zero keep the loop free of live-in values.
  // The loop's last barrier has released the tile stages (what is still read
  // after it is never used).
  if constexpr (Epi::kFastPre != 0)
    fast_preload<Epi::kFastPre == 1, true>(acc, epi.fast_pre_src(), epi.fast_pre_ld(),
                                           epi.fast_pre_scale(), m0, n0, smem_fast, wave, lane);
  if constexpr (Epi::kFastPre2 != 0)
    fast_preload<true, true>(acc, epi.fast_pre2_src(), epi.fast_pre2_ld(), epi.fast_pre2_scale(),
                             m0, n0, smem_fast, wave, lane);

  // A transposed bf16 output with a 16-byte-aligned destination goes through
  // LDS: each lane writes its four consecutive rows of one column as 8 bytes
  // of one row of the transposed tile, then every half-wave stores one whole
  // 512-byte row piece (the per-lane stores below write 8 bytes at 32
  // addresses 8 KB apart per instruction, and took 13 us of a 4096^2 apply).
  bool t_done = false;
  if constexpr (Epi::kFastT) {
    int64_t tld = 0;
    uint16_t* tdst = epi.fast_t_rows(tld);
    if (tdst != nullptr) {
      uint16_t* tt = reinterpret_cast<uint16_t*>(smem_fast);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int r0 = wm * 128 + i * 32 + g * 8 + (lane >> 5) * 4;
            const int c = wn * 128 + j * 32 + (lane & 31);
            const floatx4 v = {acc[i][j][g * 4 + 0], acc[i][j][g * 4 + 1], acc[i][j][g * 4 + 2],
                               acc[i][j][g * 4 + 3]};
            *reinterpret_cast<uint2*>(tt + c * kTRow + r0) = pack_bf16x4(v);
          }
      __syncthreads();
#pragma unroll 8
      for (int q = 0; q < 32; ++q) {
        const int c = wave * 64 + q * 2 + (lane >> 5);
        const uint4 v = *reinterpret_cast<const uint4*>(tt + c * kTRow + (lane & 31) * 8);
        *reinterpret_cast<uint4*>(tdst + (int64_t)(n0 + c) * tld + m0 + (lane & 31) * 8) = v;
      }
      __syncthreads();
      t_done = true;
    } else if (!epi.fast_t_any()) {
      t_done = true;
    }
  }
  // Transposed outputs straight from the accumulators (four consecutive rows
  // of one column per lane): a transposed copy, or the mirror tile (tn, tm)
  // of a symmetric result.
  if (!t_done && (Epi::kFastT || (Epi::kFastSym && p.sym && tm != tn))) {
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
