// Dion's third sweep as an HBM-streaming kernel (bf16 weights, fp32 momentum):
//
//   M' = (M + G) - P (c1 R)^T          error feedback (paper page: the
//                                       momentum keeps what the low-rank
//                                       update did not apply; MSR talk)
//   X' = X - P (c2 Q')^T               SGD-form weight step, rounded to bf16
//
// The factors arrive as bf16 copies with the scales already applied, so both
// products are single bf16 products with fp32 accumulation.  The sweep moves
// 14 bytes per element of X (read M, G, X; write M, X) and does 4r flops per
// element, so below the bf16 ridge it is bound by HBM, not by the matrix cores.
//
// Layout of the work:
// - A workgroup owns a 128 x 32 tile of M and X: four waves, each a 32 x 32
//   block (one 32-row strip).
// - The products are formed transposed, C^T = R P^T, so the fp32 accumulator of
//   lane l, element e is C[i0 + l%32][j0 + 8*(e/4) + 4*(l/32) + e%4]: four
//   consecutive columns of one row.  After the products each wave passes its
//   two accumulator blocks through LDS (the factor staging buffer, free by
//   then) so that lane l holds columns 4 (l % 8) .. + 3 of rows l / 8 + 8 q:
//   every memory term and store is then one access per four elements that
//   covers 8 whole 32-column row segments per instruction (the accumulator
//   layout itself touched 32 rows per instruction, four times per line).
// - The R and Q' rows of the tile go through LDS in chunks of 256 k, shared by
//   the four waves; P fragments come straight from global memory (each wave
//   reads only its own rows), from a copy of P stored in fragment order when
//   one is given (one contiguous 1 KB per fragment instead of 32 rows of 32
//   bytes: a quarter of the cache-line requests).  A chunk's factor loads are issued first, then
//   every memory term of the tile, so the products start as soon as the
//   (L2-resident) factors have arrived while the HBM reads are still in flight.
// - Small tiles let three workgroups share a CU, so one's epilogue and loads
//   overlap the others' products.
#include "launch.h"

namespace ortho {

namespace {

constexpr int kUpdRows = 128;   // tile rows (4 waves x 32)
constexpr int kUpdCols = 32;    // tile columns
constexpr int kUpdKc = 256;     // k per chunk staged in LDS
constexpr int kUpdLds = kUpdKc + 8;  // bf16 per LDS row; +16 B spreads rows over the banks
constexpr int kUpdStage = kUpdCols * (kUpdKc / 8) / 256;  // 16-byte pieces per thread per factor
constexpr int kUpdTp = 36;   // floats per row of a wave's 32 x 32 transposition block
constexpr int kUpdLdsBytes = 2 * kUpdCols * kUpdLds * 2;  // sR and sQ
constexpr int kUpdTBytes = 4 * 2 * 32 * kUpdTp * 4;       // 4 waves x (M, X) blocks
constexpr int kUpdShared = kUpdLdsBytes > kUpdTBytes ? kUpdLdsBytes : kUpdTBytes;

struct UpdStreamParams {
  MatArg m, g, x;      // fp32 momentum, bf16 gradient, bf16 weight
  MatArg pb, rb, qb;   // bf16 P (m x r), c1 R (n x r), c2 Q' (n x r)
  MatArg pf;           // bf16 P in fragment order (has_pf)
  int has_pf;
  int M, N, K;         // K = r = 256 or 512
  int tiles_j;         // N / 32
};

typedef uint32_t uint2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ floatx4 bf16x4_bits_to_f32(uint2v u) {
  floatx4 v;
  v[0] = __uint_as_float(u[0] << 16);
  v[1] = __uint_as_float(u[0] & 0xffff0000u);
  v[2] = __uint_as_float(u[1] << 16);
  v[3] = __uint_as_float(u[1] & 0xffff0000u);
  return v;
}

__device__ __forceinline__ uint2v f32x4_to_bf16_bits(floatx4 v) {
  const uint32_t a = to_bf16_bits(v[0]), b = to_bf16_bits(v[1]);
  const uint32_t c = to_bf16_bits(v[2]), d = to_bf16_bits(v[3]);
  uint2v r;
  r[0] = a | (b << 16);
  r[1] = c | (d << 16);
  return r;
}

// Loads of one 256-k chunk: thread t stages 16-byte pieces t, t + 256, ... of
// the 32 x 32 grid of pieces that covers factor rows 0..31 (from r0 and q0),
// k in [kc, kc + 256), and takes its own 16 P fragments: from its row of P
// (prow, pstep = 1: k steps 16 elements apart) or from the fragment-order
// copy (prow at the lane's 8 elements of the block's first k step, pstep =
// 512: k steps 64 lanes x 8 apart).
__device__ __forceinline__ void upd_chunk_load(uint4 (&stR)[kUpdStage], uint4 (&stQ)[kUpdStage],
                                               bf16x8 (&pf)[kUpdKc / 16], const uint16_t* r0,
                                               int64_t ldr, const uint16_t* q0, int64_t ldq,
                                               const uint16_t* prow, int pstep, int kc, int tid) {
#pragma unroll
  for (int u = 0; u < kUpdStage; ++u) {
    const int idx = tid + u * 256;
    const int64_t r = idx >> 5;
    const int c = kc + (idx & 31) * 8;
    stR[u] = *reinterpret_cast<const uint4*>(r0 + r * ldr + c);
    stQ[u] = *reinterpret_cast<const uint4*>(q0 + r * ldq + c);
  }
#pragma unroll
  for (int s = 0; s < kUpdKc / 16; ++s)
    pf[s] = *reinterpret_cast<const bf16x8*>(prow + (int64_t)(kc / 16 + s) * 16 * pstep);
}

// NCH chunks of 256 k (r = 256 NCH).  Every loop is unrolled, so the code is
// straight-line and each wait for a load names exactly that load: the memory
// terms issued after a chunk's factor loads stay in flight under its products.
template <int NCH>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(NCH == 1 ? 3 : 2, NCH == 1 ? 3 : 2)))
void dion_update_stream_kernel(UpdStreamParams p) {
  __shared__ __attribute__((aligned(16))) char smem[kUpdShared];
  uint16_t* sR = reinterpret_cast<uint16_t*>(smem);
  uint16_t* sQ = sR + kUpdCols * kUpdLds;
  constexpr int kSteps = kUpdKc / 16;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bi = blockIdx.y;

  // Consecutive workgroup ids go round-robin over the 8 XCDs.  When the tile
  // grid splits into 2 x 4 blocks, XCD x takes block (x / 4, x % 4), column
  // tile innermost: its P rows and its c1 R, c2 Q' rows (a quarter of the
  // columns) then both stay in its L2.  Walking all columns per row band
  // instead re-fetched all of R and Q' for every band, about as many bytes as
  // the sweep's own reads.
  const int tiles_i = p.M / kUpdRows;
  int ti, tj;
  if ((gridDim.x & 7) == 0 && (tiles_i & 1) == 0 && (p.tiles_j & 3) == 0) {
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    const int bj = p.tiles_j >> 2;
    ti = (xcd >> 2) * (tiles_i >> 1) + local / bj;
    tj = (xcd & 3) * bj + local % bj;
  } else {
    ti = blockIdx.x / p.tiles_j;
    tj = blockIdx.x % p.tiles_j;
  }
  const int i0 = ti * kUpdRows + wave * 32;
  const int j0 = tj * kUpdCols;
  const int row = i0 + (lane & 31);
  const int h = lane >> 5;

  float* mp = static_cast<float*>(const_cast<void*>(p.m.p[bi]));
  const uint16_t* gp = static_cast<const uint16_t*>(p.g.p[bi]);
  uint16_t* xp = static_cast<uint16_t*>(const_cast<void*>(p.x.p[bi]));
  const uint16_t* pbp = static_cast<const uint16_t*>(p.pb.p[bi]);
  const uint16_t* rbp = static_cast<const uint16_t*>(p.rb.p[bi]);
  const uint16_t* qbp = static_cast<const uint16_t*>(p.qb.p[bi]);

  // memory terms: lane l, rows i0 + l / 8 + 8 q, columns j0 + 4 (l % 8) .. + 3
  const int mr0 = i0 + (lane >> 3), mc = j0 + 4 * (lane & 7);
  // P fragments: 16 k steps of 16 per chunk
  const uint16_t* prow;
  int pstep;
  if (p.has_pf) {
    // block of 32 rows i0 / 32, lane's 8 elements; k step s at s * 512
    prow = static_cast<const uint16_t*>(p.pf.p[bi]) +
           ((static_cast<int64_t>(i0 >> 5) * (p.K >> 4)) * 64 + lane) * 8;
    pstep = 32;
  } else {
    prow = pbp + static_cast<int64_t>(row) * p.pb.ld + 8 * h;
    pstep = 1;
  }
  const int frag = (lane & 31) * kUpdLds + 8 * h;

  uint4 stR[kUpdStage], stQ[kUpdStage];
  bf16x8 pf[kSteps];
  upd_chunk_load(stR, stQ, pf, rbp + static_cast<int64_t>(j0) * p.rb.ld, p.rb.ld,
                 qbp + static_cast<int64_t>(j0) * p.qb.ld, p.qb.ld, prow, pstep, 0, tid);

  floatx4 mv[4];
  uint2v gv[4], xv[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t rq = mr0 + 8 * q;
    mv[q] = *reinterpret_cast<const floatx4*>(mp + rq * p.m.ld + mc);
    gv[q] = *reinterpret_cast<const uint2v*>(gp + rq * p.g.ld + mc);
    xv[q] = *reinterpret_cast<const uint2v*>(xp + rq * p.x.ld + mc);
  }

  floatx16 accM, accX;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    accM[e] = 0.f;
    accX[e] = 0.f;
  }

#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    if (ch > 0) {
      __syncthreads();  // every wave is done with the last chunk
    }
#pragma unroll
    for (int u = 0; u < kUpdStage; ++u) {
      const int idx = tid + u * 256;
      const int r = idx >> 5, c = (idx & 31) * 8;
      *reinterpret_cast<uint4*>(sR + r * kUpdLds + c) = stR[u];
      *reinterpret_cast<uint4*>(sQ + r * kUpdLds + c) = stQ[u];
    }
    __syncthreads();
    bf16x8 pc[kSteps];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) pc[s] = pf[s];
    if (ch + 1 < NCH)
      upd_chunk_load(stR, stQ, pf, rbp + static_cast<int64_t>(j0) * p.rb.ld, p.rb.ld,
                     qbp + static_cast<int64_t>(j0) * p.qb.ld, p.qb.ld, prow, pstep,
                     (ch + 1) * kUpdKc, tid);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const bf16x8 r0 = *reinterpret_cast<const bf16x8*>(sR + frag + 16 * s);
      const bf16x8 q0 = *reinterpret_cast<const bf16x8*>(sQ + frag + 16 * s);
      accM = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r0, pc[s], accM, 0, 0, 0);
      accX = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q0, pc[s], accX, 0, 0, 0);
    }
  }

  // accumulators to row-contiguous order through this wave's LDS blocks
  __syncthreads();  // every wave is done with sR and sQ
  float* tM = reinterpret_cast<float*>(smem) + wave * (2 * 32 * kUpdTp);
  float* tX = tM + 32 * kUpdTp;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int c = 8 * g + 4 * h;
    floatx4 a, b;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      a[t] = accM[4 * g + t];
      b[t] = accX[4 * g + t];
    }
    *reinterpret_cast<floatx4*>(tM + (lane & 31) * kUpdTp + c) = a;
    *reinterpret_cast<floatx4*>(tX + (lane & 31) * kUpdTp + c) = b;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int rl = (lane >> 3) + 8 * q, cl = 4 * (lane & 7);
    const floatx4 am = *reinterpret_cast<const floatx4*>(tM + rl * kUpdTp + cl);
    const floatx4 ax = *reinterpret_cast<const floatx4*>(tX + rl * kUpdTp + cl);
    const floatx4 gf = bf16x4_bits_to_f32(gv[q]);
    const floatx4 xf = bf16x4_bits_to_f32(xv[q]);
    floatx4 mo, xo;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      mo[t] = (mv[q][t] + gf[t]) - am[t];
      xo[t] = xf[t] - ax[t];
    }
    const int64_t rq = mr0 + 8 * q;
    *reinterpret_cast<floatx4*>(mp + rq * p.m.ld + mc) = mo;
    *reinterpret_cast<uint2v*>(xp + rq * p.x.ld + mc) = f32x4_to_bf16_bits(xo);
  }
}

bool aligned_rows(const MatArg& t, int members, size_t esz, size_t bytes) {
  if ((static_cast<size_t>(t.ld) * esz) % bytes != 0) return false;
  for (int i = 0; i < members; ++i)
    if (reinterpret_cast<uintptr_t>(t.p[i]) % bytes != 0) return false;
  return true;
}

}  // namespace

bool dion_update_stream_ok(const DionUpdateArgs& a, int members) {
  return a.M % kUpdRows == 0 && a.N % kUpdCols == 0 && (a.rank == 256 || a.rank == 512) &&
         aligned_rows(a.m, members, 4, 16) && aligned_rows(a.g, members, 2, 8) &&
         aligned_rows(a.x, members, 2, 8) && aligned_rows(a.pb, members, 2, 16) &&
         aligned_rows(a.rb, members, 2, 16) && aligned_rows(a.qb, members, 2, 16);
}

hipError_t launch_dion_update_stream(const DionUpdateArgs& a, int members, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0 || members <= 0) return hipSuccess;
  if (!dion_update_stream_ok(a, members)) return hipErrorInvalidValue;
  UpdStreamParams p{};
  p.m = a.m; p.g = a.g; p.x = a.x;
  p.pb = a.pb; p.rb = a.rb; p.qb = a.qb;
  p.pf = a.pf; p.has_pf = a.has_pf;
  p.M = a.M; p.N = a.N; p.K = a.rank;
  p.tiles_j = a.N / kUpdCols;
  dim3 grid((a.M / kUpdRows) * p.tiles_j, members);
  if (a.rank == 256)
    hipLaunchKernelGGL(dion_update_stream_kernel<1>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(dion_update_stream_kernel<2>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace ortho
