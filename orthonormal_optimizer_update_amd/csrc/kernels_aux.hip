// Reductions, normalisations and the small dense r x r linear algebra of the
// Dion orthonormalisation, for gfx950.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace ortho {

// ---------------------------------------------------------------------------
// Split-K reduction:  out[i][j] = sum_s part[s][i][j], summed in slice order
// (deterministic).  With colsq != nullptr the kernel also writes, per 64-row
// block, the sum of squares of each output column (for the column norms).
// grid (ceil(cols/64), ceil(rows/64), members); 256 threads = 64 cols x 4.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void reduce_splits_kernel(RedArgs a) {
  __shared__ float red[4][64];
  const int bi = blockIdx.z;
  const float* part = a.part + bi * a.part_member_stride;
  float* out = static_cast<float*>(const_cast<void*>(a.out.p[bi]));
  const int c = blockIdx.x * 64 + (threadIdx.x & 63);
  const int rg = threadIdx.x >> 6;
  const int rbase = blockIdx.y * 64;
  float sq = 0.f;
  if (c < a.cols) {
    for (int rr = rg; rr < 64; rr += 4) {
      const int r = rbase + rr;
      if (r >= a.rows) break;
      float s = 0.f;
      for (int k = 0; k < a.splits; ++k) s += part[k * a.slice + (int64_t)r * a.cols + c];
      if (!a.no_store) out[(int64_t)r * a.out.ld + c] = s;
      sq += s * s;
    }
  }
  if (a.colsq) {
    red[rg][threadIdx.x & 63] = sq;
    __syncthreads();
    if (rg == 0 && c < a.cols) {
      const float t = red[0][threadIdx.x] + red[1][threadIdx.x] + red[2][threadIdx.x] + red[3][threadIdx.x];
      a.colsq[bi * a.colsq_member_stride + (int64_t)blockIdx.y * a.cols + c] = t;
    }
  }
}

// The same reduction with four consecutive columns per thread (16-byte loads
// and stores) for column counts and strides that allow it.  A block covers 64
// columns x 64 rows: 16 column quads x 16 row groups of 4 rows each; splits
// are summed in slice order as above.  grid (ceil(cols/64), ceil(rows/64),
// members).
__global__ __launch_bounds__(256) void reduce_splits_vec_kernel(RedArgs a) {
  __shared__ float red[16][65];
  const int bi = blockIdx.z;
  const float* part = a.part + bi * a.part_member_stride;
  float* out = static_cast<float*>(const_cast<void*>(a.out.p[bi]));
  const int cq = threadIdx.x & 15, rg = threadIdx.x >> 4;
  const int c = blockIdx.x * 64 + cq * 4;
  const int rbase = blockIdx.y * 64;
  floatx4 sq = {0.f, 0.f, 0.f, 0.f};
  if (c < a.cols) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = rbase + rg + 16 * j;
      if (r >= a.rows) break;
      const float* src = part + (int64_t)r * a.cols + c;
      floatx4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
      for (int k = 0; k < a.splits; ++k) s += *reinterpret_cast<const floatx4*>(src + k * a.slice);
      if (!a.no_store) *reinterpret_cast<floatx4*>(out + (int64_t)r * a.out.ld + c) = s;
      if (a.has_bf16) {
        uint16_t* ob = static_cast<uint16_t*>(const_cast<void*>(a.out_bf16.p[bi]));
        const uint16_t h[4] = {to_bf16_bits(s[0]), to_bf16_bits(s[1]), to_bf16_bits(s[2]),
                               to_bf16_bits(s[3])};
        *reinterpret_cast<uint2*>(ob + (int64_t)r * a.out_bf16.ld + c) =
            make_uint2(h[0] | (uint32_t(h[1]) << 16), h[2] | (uint32_t(h[3]) << 16));
      }
      sq += s * s;
    }
  }
  if (a.colsq) {
#pragma unroll
    for (int t = 0; t < 4; ++t) red[rg][cq * 4 + t] = sq[t];
    __syncthreads();
    const int cc = blockIdx.x * 64 + threadIdx.x;
    if (threadIdx.x < 64 && cc < a.cols) {
      float tot = 0.f;
#pragma unroll
      for (int g = 0; g < 16; ++g) tot += red[g][threadIdx.x];
      a.colsq[bi * a.colsq_member_stride + (int64_t)blockIdx.y * a.cols + cc] = tot;
    }
  }
}

// NP bf16 pieces of an fp32 matrix (x = p0 + p1 (+ p2)); 64 x 64 tiles, each
// thread four consecutive columns of four rows (ragged edges elementwise).
template <int NP>
__global__ __launch_bounds__(256) void split_rows_kernel(SplitRowsArgs a) {
  const int bi = blockIdx.z;
  const float* src = static_cast<const float*>(a.src.p[bi]);
  const int c = blockIdx.x * 64 + (threadIdx.x & 15) * 4;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = blockIdx.y * 64 + (threadIdx.x >> 4) + 16 * q;
    if (r >= a.rows) break;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (c + t >= a.cols) break;
      float x = src[(int64_t)r * a.src.ld + c + t];
#pragma unroll
      for (int k = 0; k < NP; ++k) {
        const uint16_t h = to_bf16_bits(x);
        static_cast<uint16_t*>(const_cast<void*>(a.piece[k].p[bi]))[(int64_t)r * a.piece[k].ld + c + t] = h;
        x -= bf16_bits_to_f32(h);
      }
    }
  }
}

// bf16x2 pieces of B = M + G (row-major and transposed) and of the transpose
// of an fp32 matrix, for the 256 x 256 product kernel.  64 x 64 tiles of 256
// threads; thread t handles columns 4 (t & 15) .. + 3 of rows (t >> 4) + 16 q;
// the transposed pieces are staged in LDS and written 4 elements per lane.
// grid (cols / 64, rows / 64, members).
__device__ __forceinline__ uint2 pack4(const uint16_t (&h)[4]) {
  return make_uint2(h[0] | (uint32_t(h[1]) << 16), h[2] | (uint32_t(h[3]) << 16));
}

// With blk16 > 0 the transposed pieces are written k-blocked instead of with
// leading dimension ldt: element (j, k) of the cols x rows transpose at
// (k / 16) * blk16 * 16 + j * 16 + k % 16 (blk16 = cols), so every 16-deep k
// block of all cols rows is one contiguous run.
template <bool kSum>
__device__ __forceinline__ void split_tile(const float* src, int64_t lds_, const uint16_t* g,
                                           int64_t ldg, uint16_t* hi, uint16_t* lo, int64_t ldo,
                                           uint16_t* hit, uint16_t* lot, int64_t ldt, int r0,
                                           int c0, int blk16 = 0) {
  __shared__ uint16_t th[64][68];
  __shared__ uint16_t tl[64][68];
  const int cl = (threadIdx.x & 15) * 4;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int rl = (threadIdx.x >> 4) + 16 * q;
    const int64_t row = r0 + rl;
    floatx4 v = *reinterpret_cast<const floatx4*>(src + row * lds_ + c0 + cl);
    if constexpr (kSum) {
      const uint2 gv = *reinterpret_cast<const uint2*>(g + row * ldg + c0 + cl);
      v[0] += bf16_bits_to_f32(gv.x & 0xFFFF);
      v[1] += bf16_bits_to_f32(gv.x >> 16);
      v[2] += bf16_bits_to_f32(gv.y & 0xFFFF);
      v[3] += bf16_bits_to_f32(gv.y >> 16);
    }
    uint16_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bf16 bh, bl;
      split_bf16(v[e], bh, bl);
      h[e] = __builtin_bit_cast(uint16_t, bh);
      l[e] = __builtin_bit_cast(uint16_t, bl);
      th[cl + e][rl] = h[e];
      tl[cl + e][rl] = l[e];
    }
    if constexpr (kSum) {
      *reinterpret_cast<uint2*>(hi + row * ldo + c0 + cl) = pack4(h);
      *reinterpret_cast<uint2*>(lo + row * ldo + c0 + cl) = pack4(l);
    }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int j = (threadIdx.x >> 4) + 16 * q;  // row of the transposed tile
    const int i4 = (threadIdx.x & 15) * 4;
    uint16_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[e] = th[j][i4 + e];
      l[e] = tl[j][i4 + e];
    }
    const int64_t o = blk16 > 0 ? (int64_t)((r0 + i4) >> 4) * blk16 * 16 + (c0 + j) * 16 + ((r0 + i4) & 15)
                                : (int64_t)(c0 + j) * ldt + r0 + i4;
    *reinterpret_cast<uint2*>(hit + o) = pack4(h);
    *reinterpret_cast<uint2*>(lot + o) = pack4(l);
  }
}

// Split-K sum of a 64 x 64 tile, then its bf16 forms (see RedPiecesArgs).
// Thread t: columns 4 (t & 15) .. + 3 of rows (t >> 4) + 16 q; the transposed
// pieces are staged in LDS and written 4 elements per lane.
__global__ __launch_bounds__(256) void reduce_pieces_kernel(RedPiecesArgs a) {
  __shared__ uint16_t th[64][68];
  __shared__ uint16_t tl[64][68];
  const int bi = blockIdx.z;
  const float* part = a.part + bi * a.part_member_stride;
  const int cl = (threadIdx.x & 15) * 4;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int rl = (threadIdx.x >> 4) + 16 * q;
    const int64_t row = r0 + rl;
    const float* src = part + row * a.cols + c0 + cl;
    floatx4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int k = 0; k < a.splits; ++k) v += *reinterpret_cast<const floatx4*>(src + k * a.slice);
    if (a.has_out)
      *reinterpret_cast<floatx4*>(static_cast<float*>(const_cast<void*>(a.out.p[bi])) + row * a.out.ld + c0 + cl) = v;
    if (a.has_bf16 || a.has_frag) {
      const uint16_t h[4] = {to_bf16_bits(v[0]), to_bf16_bits(v[1]), to_bf16_bits(v[2]), to_bf16_bits(v[3])};
      if (a.has_bf16)
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(const_cast<void*>(a.out_bf16.p[bi])) + row * a.out_bf16.ld + c0 + cl) = pack4(h);
      if (a.has_frag) {
        // element (row, k): (((row / 32) * cols / 16 + k / 16) * 64 + row % 32 +
        // 32 * (k / 8 % 2)) * 8 + k % 8; k = c0 + cl .. + 3 share one 8-group
        const int k = c0 + cl;
        const int64_t o = (((row >> 5) * (a.cols >> 4) + (k >> 4)) * 64 + (row & 31) + 32 * ((k >> 3) & 1)) * 8 + (k & 7);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(const_cast<void*>(a.frag.p[bi])) + o) = pack4(h);
      }
    }
    floatx4 x = v;
    for (int pc = 0; pc < a.np; ++pc) {
      uint16_t h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        h[e] = to_bf16_bits(x[e]);
        x[e] -= bf16_bits_to_f32(h[e]);
      }
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(const_cast<void*>(a.piece[pc].p[bi])) + row * a.piece[pc].ld + c0 + cl) = pack4(h);
    }
    if (a.has_t) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bf16 bh, bl;
        split_bf16(v[e], bh, bl);
        th[cl + e][rl] = __builtin_bit_cast(uint16_t, bh);
        tl[cl + e][rl] = __builtin_bit_cast(uint16_t, bl);
      }
    }
  }
  if (!a.has_t) return;  // uniform over the grid
  __syncthreads();
  uint16_t* hit = static_cast<uint16_t*>(const_cast<void*>(a.tpiece[0].p[bi]));
  uint16_t* lot = static_cast<uint16_t*>(const_cast<void*>(a.tpiece[1].p[bi]));
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int j = (threadIdx.x >> 4) + 16 * q;  // row of the transposed tile
    const int i4 = (threadIdx.x & 15) * 4;
    uint16_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[e] = th[j][i4 + e];
      l[e] = tl[j][i4 + e];
    }
    // four consecutive rows r0 + i4 .. + 3 of column c0 + j: contiguous in both
    // layouts (i4 % 4 == 0, so they share one 16-row block)
    const int64_t ot = a.t_blocked
        ? (int64_t)((r0 + i4) >> 4) * a.cols * 16 + (int64_t)(c0 + j) * 16 + ((r0 + i4) & 15)
        : (int64_t)(c0 + j) * a.tpiece[0].ld + r0 + i4;
    *reinterpret_cast<uint2*>(hit + ot) = pack4(h);
    *reinterpret_cast<uint2*>(lot + ot) = pack4(l);
  }
}

__global__ __launch_bounds__(256) void split_sum_kernel(SplitSumArgs a) {
  const int bi = blockIdx.z;
  split_tile<true>(static_cast<const float*>(a.m.p[bi]), a.m.ld,
                   static_cast<const uint16_t*>(a.g.p[bi]), a.g.ld,
                   static_cast<uint16_t*>(const_cast<void*>(a.hi.p[bi])),
                   static_cast<uint16_t*>(const_cast<void*>(a.lo.p[bi])), a.hi.ld,
                   static_cast<uint16_t*>(const_cast<void*>(a.hit.p[bi])),
                   static_cast<uint16_t*>(const_cast<void*>(a.lot.p[bi])), a.hit.ld,
                   blockIdx.y * 64, blockIdx.x * 64);
}

__global__ __launch_bounds__(256) void split_t_kernel(SplitTArgs a) {
  const int bi = blockIdx.z;
  split_tile<false>(static_cast<const float*>(a.src.p[bi]), a.src.ld, nullptr, 0, nullptr, nullptr,
                    0, static_cast<uint16_t*>(const_cast<void*>(a.hit.p[bi])),
                    static_cast<uint16_t*>(const_cast<void*>(a.lot.p[bi])), a.hit.ld,
                    blockIdx.y * 64, blockIdx.x * 64, a.blocked ? a.cols : 0);
}

// Column normalisation Q'[:, j] = R[:, j] / |R[:, j]|, in two launches.
// colnorm_inv_kernel sums the per-row-block column sums of squares in block
// order (four thread groups take every fourth block, combined in a fixed order)
// and writes 1/|R[:, j]| over row block 0's sums.  A zero column gives a zero
// column and sets ORTHO_DEV_ZERO_COLUMN; NaN propagates.
__global__ __launch_bounds__(256) void colnorm_inv_kernel(ColnormArgs a) {
  __shared__ float part[4][64];
  const int bi = blockIdx.y;
  const int g = threadIdx.x >> 6, cc = threadIdx.x & 63, c = blockIdx.x * 64 + cc;
  float* cs = a.colsq + bi * a.colsq_member_stride;
  float s = 0.f;
  if (c < a.cols) {
#pragma unroll 8
    for (int b = g; b < a.nrb; b += 4) s += cs[(int64_t)b * a.cols + c];
  }
  part[g][cc] = s;
  __syncthreads();  // every read of row block 0 is done before it is overwritten
  if (threadIdx.x < 64 && c < a.cols) {
    const float t = (part[0][cc] + part[1][cc]) + (part[2][cc] + part[3][cc]);
    float v;
    if (t > 0.f) {
      v = 1.0f / sqrtf(t);
    } else if (!(t != t)) {
      v = 0.f;
      if (a.status) atomicOr(a.status, 2);
    } else {
      v = t;
    }
    cs[c] = v;
  }
}

// Q' = R diag(inv), and the bf16 operands of the last sweep; 64 x 64 tiles,
// four consecutive columns per thread (16-byte fp32 and 8-byte bf16 accesses
// where the row has them).
__global__ __launch_bounds__(256) void colnorm_kernel(ColnormArgs a) {
  const int bi = blockIdx.z;
  const float* inv = a.colsq + bi * a.colsq_member_stride;
  const float* r = static_cast<const float*>(a.r.p[bi]);
  float* q = static_cast<float*>(const_cast<void*>(a.q.p[bi]));
  uint16_t* rb = a.has_bf16 ? static_cast<uint16_t*>(const_cast<void*>(a.rb.p[bi])) : nullptr;
  uint16_t* qb = a.has_bf16 ? static_cast<uint16_t*>(const_cast<void*>(a.qb.p[bi])) : nullptr;
  const int c = blockIdx.x * 64 + (threadIdx.x & 15) * 4;
  if (c >= a.cols) return;
  const bool full = c + 4 <= a.cols;
  float iv[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) iv[t] = c + t < a.cols ? inv[c + t] : 0.f;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const int row = blockIdx.y * 64 + (threadIdx.x >> 4) + 16 * q4;
    if (row >= a.rows) break;
    const float* rrow = r + (int64_t)row * a.r.ld;
    floatx4 rv, qv;
    if (full && a.r.vec) {
      rv = *reinterpret_cast<const floatx4*>(rrow + c);
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) rv[t] = c + t < a.cols ? rrow[c + t] : 0.f;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) qv[t] = rv[t] * iv[t];
    float* qrow = q + (int64_t)row * a.q.ld;
    if (full && a.q.vec) {
      *reinterpret_cast<floatx4*>(qrow + c) = qv;
    } else {
      for (int t = 0; t < 4 && c + t < a.cols; ++t) qrow[c + t] = qv[t];
    }
    if (rb) {
      const floatx4 rs = a.c1 * rv, qs = a.c2 * qv;
      uint16_t* rbrow = rb + (int64_t)row * a.rb.ld;
      uint16_t* qbrow = qb + (int64_t)row * a.qb.ld;
      if (full) {
        *reinterpret_cast<uint2*>(rbrow + c) = pack_bf16x4(rs);
        *reinterpret_cast<uint2*>(qbrow + c) = pack_bf16x4(qs);
      } else {
        for (int t = 0; t < 4 && c + t < a.cols; ++t) {
          rbrow[c + t] = to_bf16_bits(rs[t]);
          qbrow[c + t] = to_bf16_bits(qs[t]);
        }
      }
    }
  }
}

// The split-K reduce of a short R (rows <= kFusedColnormRows = 512) fused with its
// column normalisation: one workgroup of 1024 threads per 64 columns per
// member; thread (rg, cq) holds four columns of rows rg, rg + 64, ... (at most
// 8).  Every slice load of a thread is issued before the sums are used; each
// row's slices are added in slice order (the bits reduce_splits_vec_kernel
// stores).  R is written, the squares go into per-thread column sums, the 64
// row groups are added in order and 1/|R[:, j]| formed as in
// colnorm_inv_kernel (zero column: 0 and ORTHO_DEV_ZERO_COLUMN; NaN
// propagates); then Q' = R diag(inv) and the bf16 operands from the rows
// still in registers, as colnorm_kernel.  cols % 4 == 0 and 16-byte aligned
// slices (the launcher checks); RPT = rows per thread, rows <= 64 RPT (a
// compile-time count: the loads of every row are unconditional, at clamped
// addresses, so that they are all in flight before the first add).
// grid (ceil(cols / 64), members).
template <int RPT>
__global__ __launch_bounds__(1024) void reduce_colnorm_kernel(RedArgs a, ColnormArgs cn) {
  constexpr int kRowsPerThread = RPT;
  __shared__ float red[64][65];
  __shared__ float inv[64];
  const int bi = blockIdx.y;
  const float* part = a.part + bi * a.part_member_stride;
  float* out = static_cast<float*>(const_cast<void*>(a.out.p[bi]));
  const int cq = threadIdx.x & 15, rg = threadIdx.x >> 4;
  const int c = blockIdx.x * 64 + cq * 4;
  const bool act = c < a.cols;
  const int cl = min(c, a.cols - 4);   // clamped: every load stays inside a row
  floatx4 v[kRowsPerThread];
#pragma unroll
  for (int j = 0; j < kRowsPerThread; ++j) v[j] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < a.splits; ++k) {
    const float* src = part + k * a.slice + cl;
#pragma unroll
    for (int j = 0; j < kRowsPerThread; ++j)
      v[j] += *reinterpret_cast<const floatx4*>(src + (int64_t)min(rg + 64 * j, a.rows - 1) * a.cols);
  }
  floatx4 sq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kRowsPerThread; ++j) {
    const int row = rg + 64 * j;
    if (act && row < a.rows) {
      if (!a.no_store) *reinterpret_cast<floatx4*>(out + (int64_t)row * a.out.ld + c) = v[j];
      sq += v[j] * v[j];
    }
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) red[rg][cq * 4 + t] = sq[t];
  __syncthreads();
  if (threadIdx.x < 64) {
    const int cc = blockIdx.x * 64 + threadIdx.x;
    float w = 0.f;
    if (cc < a.cols) {
      float t = 0.f;
      for (int g = 0; g < 64; ++g) t += red[g][threadIdx.x];
      if (t > 0.f) {
        w = 1.0f / sqrtf(t);
      } else if (!(t != t)) {
        w = 0.f;
        if (cn.status) atomicOr(cn.status, 2);
      } else {
        w = t;
      }
    }
    inv[threadIdx.x] = w;
  }
  __syncthreads();
  if (!act) return;
  float* q = static_cast<float*>(const_cast<void*>(cn.q.p[bi]));
  uint16_t* rb = cn.has_bf16 ? static_cast<uint16_t*>(const_cast<void*>(cn.rb.p[bi])) : nullptr;
  uint16_t* qb = cn.has_bf16 ? static_cast<uint16_t*>(const_cast<void*>(cn.qb.p[bi])) : nullptr;
  const floatx4 iv = {inv[cq * 4 + 0], inv[cq * 4 + 1], inv[cq * 4 + 2], inv[cq * 4 + 3]};
#pragma unroll
  for (int j = 0; j < kRowsPerThread; ++j) {
    const int row = rg + 64 * j;
    if (row >= a.rows) break;
    const floatx4 qv = v[j] * iv;
    float* qrow = q + (int64_t)row * cn.q.ld;
    if (cn.q.vec) {
      *reinterpret_cast<floatx4*>(qrow + c) = qv;
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) qrow[c + t] = qv[t];
    }
    if (rb) {
      const floatx4 rs = cn.c1 * v[j], qs = cn.c2 * qv;
      *reinterpret_cast<uint2*>(rb + (int64_t)row * cn.rb.ld + c) = pack_bf16x4(rs);
      *reinterpret_cast<uint2*>(qb + (int64_t)row * cn.qb.ld + c) = pack_bf16x4(qs);
    }
  }
}

// Newton-Schulz polynomial for a Gram side of M = 64 or 128 rows, fused with the
// reduction of the split Gram.  One workgroup per member: A = the sum of the
// k-split partials in slice order, rounded to bf16 into LDS (the value the
// separate reduce would store); then Bp = c ((b/c) A + A A) on the matrix cores
// with A read from LDS for both operands (A is symmetric).  The 2 x 2 wave
// layout, the preloaded (b/c) A term and the k order of the products are those
// of the 128 x 128 product kernel, so the result has the same bits.
template <int M>
__global__ __launch_bounds__(256) void ns_small_poly_kernel(NsSmallPolyArgs a) {
  constexpr int LD = M + 8;           // bf16 per LDS row; +16 B spreads rows over the banks
  constexpr int WT = M / 2, NB = WT / 32;
  __shared__ __attribute__((aligned(16))) uint16_t sA[M * LD];
  const int bi = blockIdx.x;
  const float* part = a.part + bi * a.part_member_stride;
  // each thread owns PER groups of four; all PER loads of one slice are issued
  // before any is summed, so the slices cost a few load latencies, not M * M / 1024
  constexpr int PER = M * M / 4 / 256;
  floatx4 v[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) v[q] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
  for (int sl = 0; sl < a.splits; ++sl) {
    const float* src = part + sl * a.slice;
    floatx4 t[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q)
      t[q] = *reinterpret_cast<const floatx4*>(src + (threadIdx.x + q * 256) * 4);
#pragma unroll
    for (int q = 0; q < PER; ++q) v[q] += t[q];
  }
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int e4 = threadIdx.x + q * 256;
    const int i = e4 / (M / 4), j = (e4 % (M / 4)) * 4;
    *reinterpret_cast<uint2*>(sA + i * LD + j) = pack_bf16x4(v[q]);
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const float boc = a.b / a.c;
  floatx16 acc[NB][NB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int row = wm * WT + i * 32 + g * 8 + (lane >> 5) * 4 + t;
          const int col = wn * WT + j * 32 + (lane & 31);
          acc[i][j][g * 4 + t] = boc * bf16_bits_to_f32(sA[row * LD + col]);
        }
  const int fk = (lane >> 5) * 8;
#pragma unroll
  for (int k0 = 0; k0 < M; k0 += 16) {
    bf16x8 af[NB], bfr[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i)
      af[i] = *reinterpret_cast<const bf16x8*>(sA + (wm * WT + i * 32 + (lane & 31)) * LD + k0 + fk);
#pragma unroll
    for (int j = 0; j < NB; ++j)
      bfr[j] = *reinterpret_cast<const bf16x8*>(sA + (wn * WT + j * 32 + (lane & 31)) * LD + k0 + fk);
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
  }
  uint16_t* bp = static_cast<uint16_t*>(const_cast<void*>(a.bp.p[bi]));
  float* bp32 = static_cast<float*>(const_cast<void*>(a.bp32.p[bi]));
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int row = wm * WT + i * 32 + g * 8 + (lane >> 5) * 4 + t;
          const int col = wn * WT + j * 32 + (lane & 31);
          const float y = a.c * acc[i][j][g * 4 + t];
          bp[(int64_t)row * a.bp.ld + col] = to_bf16_bits(y);
          bp32[(int64_t)row * a.bp32.ld + col] = y;
        }
}

// ---------------------------------------------------------------------------
// Muon step around Newton-Schulz: momentum buffer and SGD-form update
// ---------------------------------------------------------------------------

// M = mu M + G (heavy-ball momentum buffer, fp32), four columns of a row per
// thread; blockIdx.y = row, blockIdx.z = member.
template <typename GT>
__global__ __launch_bounds__(256) void muon_momentum_kernel(MuonArgs a) {
  const int bi = blockIdx.z;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= a.cols) return;
  for (int row = blockIdx.y; row < a.rows; row += gridDim.y) {
  float* m = static_cast<float*>(const_cast<void*>(a.m.p[bi])) + (int64_t)row * a.m.ld;
  const GT* g = static_cast<const GT*>(a.g.p[bi]) + (int64_t)row * a.g.ld;
  const float4 gv = load4<GT>(g, c, a.cols, a.g.vec);
  const float4 mv = load4<float>(m, c, a.cols, a.m.vec);
  const float4 r = make_float4(a.mu * mv.x + gv.x, a.mu * mv.y + gv.y, a.mu * mv.z + gv.z,
                               a.mu * mv.w + gv.w);
  if (a.m.vec && c + 4 <= a.cols) {
    *reinterpret_cast<float4*>(m + c) = r;
  } else {
    for (int t = 0; t < 4 && c + t < a.cols; ++t) m[c + t] = f4_get(r, t);
  }
  }
}

// X = X - c U (U the fp32 orthogonalised momentum), rounded to X's dtype.
template <typename XT>
__global__ __launch_bounds__(256) void muon_update_kernel(MuonArgs a) {
  const int bi = blockIdx.z;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= a.cols) return;
  for (int row = blockIdx.y; row < a.rows; row += gridDim.y) {
  XT* x = static_cast<XT*>(const_cast<void*>(a.x.p[bi])) + (int64_t)row * a.x.ld;
  const float* u = static_cast<const float*>(a.u.p[bi]) + (int64_t)row * a.u.ld;
  const float4 uv = load4<float>(u, c, a.cols, a.u.vec);
  const float4 xv = load4<XT>(x, c, a.cols, a.x.vec);
  const float cc = a.rowf ? a.c * a.rowf[bi * a.rowf_stride + row] : a.c;
  const floatx4 r = {xv.x - cc * uv.x, xv.y - cc * uv.y, xv.z - cc * uv.z, xv.w - cc * uv.w};
  if (a.x.vec && c + 4 <= a.cols) {
    if constexpr (sizeof(XT) == 2)
      *reinterpret_cast<uint2*>(x + c) = pack_bf16x4(r);
    else
      *reinterpret_cast<floatx4*>(x + c) = r;
  } else {
    for (int t = 0; t < 4 && c + t < a.cols; ++t) store_from_f32<XT>(x, c + t, r[t]);
  }
  }
}

// Sum over the 256 threads of a workgroup in a fixed order (butterfly within
// each wave, then the four wave sums pairwise); every thread gets the total.
__device__ __forceinline__ float block_sum256(float v, float* part4) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) part4[threadIdx.x >> 6] = v;
  __syncthreads();
  const float t = (part4[0] + part4[1]) + (part4[2] + part4[3]);
  __syncthreads();
  return t;
}

// Neuron-wise normalisation, first pass: the sum of squares of row blockIdx.x
// of U, four consecutive columns per thread.
__global__ __launch_bounds__(256) void row_sumsq_kernel(RowNormArgs a) {
  __shared__ float part4[4];
  const int bi = blockIdx.y, row = blockIdx.x;
  const float* u = static_cast<const float*>(a.u.p[bi]) + (int64_t)row * a.u.ld;
  // four 16-byte loads in flight per thread per step (zeros past the row end)
  float s = 0.f;
  for (int c = threadIdx.x * 4; c < a.cols; c += 4096) {
    float4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = load4<float>(u, c + k * 1024, a.cols, a.u.vec);
#pragma unroll
    for (int k = 0; k < 4; ++k) s += (v[k].x * v[k].x + v[k].y * v[k].y) + (v[k].z * v[k].z + v[k].w * v[k].w);
  }
  const float t = block_sum256(s, part4);
  if (threadIdx.x == 0) a.rowf[bi * a.rowf_stride + row] = t;
}

// Second pass, one workgroup per member: t^2 = (sum of the row sums) / rows,
// then each row sum q becomes t / sqrt(q) (0 when q = 0).  Each thread
// rewrites only the entries it summed, after the total is formed.
__global__ __launch_bounds__(256) void row_factor_kernel(RowNormArgs a) {
  __shared__ float part4[4];
  float* f = a.rowf + blockIdx.x * a.rowf_stride;
  float s = 0.f;
  // eight loads in flight per thread per step
  for (int i0 = threadIdx.x; i0 < a.rows; i0 += 2048) {
    float q[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) q[k] = i0 + k * 256 < a.rows ? f[i0 + k * 256] : 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += q[k];
  }
  const float total = block_sum256(s, part4);
  const float t = sqrtf(total / static_cast<float>(a.rows));
  for (int i0 = threadIdx.x; i0 < a.rows; i0 += 2048) {
    float q[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) q[k] = i0 + k * 256 < a.rows ? f[i0 + k * 256] : 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (i0 + k * 256 < a.rows)
        f[i0 + k * 256] = q[k] > 0.f ? t / sqrtf(q[k]) : (q[k] == 0.f ? 0.f : q[k]);
  }
}

// ---------------------------------------------------------------------------
// Newton-Schulz normalisation
// ---------------------------------------------------------------------------

// Partial sums of squares of G: block b of member bi covers rows
// [b*rows, (b+1)*rows) of the m x n input; threads stride along the row.
// kVec: rows 16-byte aligned and cols a multiple of 16 bytes; each thread then
// reads 16 bytes (8 bf16 or 4 fp32) per step.
template <typename T, bool kVec>
__global__ __launch_bounds__(256) void sumsq_kernel(SumsqArgs a) {
  __shared__ float red[256];
  const int bi = blockIdx.y;
  const T* g = static_cast<const T*>(a.g.p[bi]);
  const int r0 = blockIdx.x * a.chunk;
  const int r1 = min(a.g.rows, r0 + static_cast<int>(a.chunk));
  float s = 0.f;
  if constexpr (kVec) {
    constexpr int kE = 16 / sizeof(T);
    for (int r = r0; r < r1; ++r) {
      const T* row = g + (int64_t)r * a.g.ld;
      for (int c = threadIdx.x * kE; c < a.g.cols; c += 256 * kE) {
        const uint4 w = *reinterpret_cast<const uint4*>(row + c);
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if constexpr (sizeof(T) == 2) {
            const float lo = __uint_as_float(u[q] << 16), hi = __uint_as_float(u[q] & 0xffff0000u);
            s += lo * lo;
            s += hi * hi;
          } else {
            const float v = __uint_as_float(u[q]);
            s += v * v;
          }
        }
      }
    }
  } else {
    for (int r = r0; r < r1; ++r) {
      const T* row = g + (int64_t)r * a.g.ld;
      for (int c = threadIdx.x; c < a.g.cols; c += 256) {
        const float v = load_as_f32<T>(row, c);
        s += v * v;
      }
    }
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.partial[bi * a.partial_stride + blockIdx.x] = red[0];
}

// scale = 1 / (sqrt(sum of partials) + eps), summed in fp64: each of 64 threads
// takes a fixed strided subset, then a fixed-order tree (deterministic).
__global__ __launch_bounds__(64) void ns_scale_kernel(const float* partial, int64_t partial_stride,
                                                      int nparts, float* scale, int64_t scale_stride,
                                                      float eps) {
  __shared__ double red[64];
  const int bi = blockIdx.x;
  double s = 0.0;
  for (int i = threadIdx.x; i < nparts; i += 64) s += partial[bi * partial_stride + i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 32; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) scale[bi * scale_stride] = static_cast<float>(1.0 / (sqrt(red[0]) + (double)eps));
}

// X0 = scale * G (wide orientation: rows <= cols, transposing a tall G), into
// the fp32 iterate and its two bf16 copies.  64 x 64 tiles through LDS; each
// thread moves four consecutive elements of a row per access (16-byte fp32 and
// 8-byte bf16 accesses where the row has them, element by element at the
// matrix edge).
template <typename T>
__device__ __forceinline__ void load4_scaled(const T* row, int c, int limit, bool vec, float sc,
                                             float v[4]) {
  const float4 f = load4<T>(row, c, limit, vec);
  v[0] = f.x * sc; v[1] = f.y * sc; v[2] = f.z * sc; v[3] = f.w * sc;
}

template <typename T>
__global__ __launch_bounds__(256) void ns_init_kernel(NsInitArgs a) {
  __shared__ float tile[64][65];
  const int bi = blockIdx.z;
  const T* g = static_cast<const T*>(a.g.p[bi]);
  float* x32 = static_cast<float*>(const_cast<void*>(a.x32.p[bi]));
  uint16_t* xb = static_cast<uint16_t*>(const_cast<void*>(a.xb.p[bi]));
  uint16_t* xbt = static_cast<uint16_t*>(const_cast<void*>(a.xbt.p[bi]));
  const float sc = a.scale[bi * a.scale_stride];
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;  // tile of X (M x N)
  const int c4 = (threadIdx.x & 15) * 4, r16 = threadIdx.x >> 4;
  // tile[ii][jj] = X[i0+ii][j0+jj], reading G four elements of a row at a time
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int rr = r16 + 16 * q;
    float v[4];
    if (!a.transposed) {
      const int i = i0 + rr;
      if (i < a.M) {
        load4_scaled<T>(g + (int64_t)i * a.g.ld, j0 + c4, a.N, a.g.vec, sc, v);
      } else {
        v[0] = v[1] = v[2] = v[3] = 0.f;
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) tile[rr][c4 + t] = v[t];
    } else {
      const int j = j0 + rr;  // X[i][j] = G[j][i]: row j of G holds column j of X
      if (j < a.N) {
        load4_scaled<T>(g + (int64_t)j * a.g.ld, i0 + c4, a.M, a.g.vec, sc, v);
      } else {
        v[0] = v[1] = v[2] = v[3] = 0.f;
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) tile[c4 + t][rr] = v[t];
    }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int rr = r16 + 16 * q;
    // row-major copies: X[i0 + rr][j0 + c4 ..]
    // (xb is NULL when the products take fp32 operands)
    const int i = i0 + rr, j = j0 + c4;
    if (i < a.M) {
      const floatx4 v = {tile[rr][c4], tile[rr][c4 + 1], tile[rr][c4 + 2], tile[rr][c4 + 3]};
      if (j + 4 <= a.N) {
        *reinterpret_cast<floatx4*>(x32 + (int64_t)i * a.x32.ld + j) = v;
        if (xb != nullptr) *reinterpret_cast<uint2*>(xb + (int64_t)i * a.xb.ld + j) = pack_bf16x4(v);
      } else {
        for (int t = 0; t < 4 && j + t < a.N; ++t) {
          x32[(int64_t)i * a.x32.ld + j + t] = v[t];
          if (xb != nullptr) xb[(int64_t)i * a.xb.ld + j + t] = to_bf16_bits(v[t]);
        }
      }
    }
    // transposed copy: X^T[j0 + rr][i0 + c4 ..] = X[i0 + c4 ..][j0 + rr]
    // (not kept when no product reads it: xbt is NULL then)
    const int jt = j0 + rr, it = i0 + c4;
    if (xbt != nullptr && jt < a.N) {
      const floatx4 v = {tile[c4][rr], tile[c4 + 1][rr], tile[c4 + 2][rr], tile[c4 + 3][rr]};
      if (it + 4 <= a.M) {
        *reinterpret_cast<uint2*>(xbt + (int64_t)jt * a.xbt.ld + it) = pack_bf16x4(v);
      } else {
        for (int t = 0; t < 4 && it + t < a.M; ++t) xbt[(int64_t)jt * a.xbt.ld + it + t] = to_bf16_bits(v[t]);
      }
    }
  }
}

// Out = X (the normalised input) when no iteration is requested, in the
// caller's dtype and orientation.
template <typename T>
__global__ __launch_bounds__(256) void ns_store_kernel(NsInitArgs a, MatArg out) {
  const int bi = blockIdx.z;
  const float* x32 = static_cast<const float*>(a.x32.p[bi]);
  T* o = static_cast<T*>(const_cast<void*>(out.p[bi]));
  const int i = blockIdx.y * 16 + (threadIdx.x >> 4);
  const int j = blockIdx.x * 16 + (threadIdx.x & 15);
  if (i >= a.M || j >= a.N) return;
  const float v = x32[(int64_t)i * a.x32.ld + j];
  if (a.transposed) store_from_f32<T>(o, (int64_t)j * out.ld + i, v);
  else store_from_f32<T>(o, (int64_t)i * out.ld + j, v);
}

// Bp = b A when the quintic coefficient c is zero (no product needed).
__global__ __launch_bounds__(256) void ns_linear_kernel(NsPolyArgs a) {
  const int bi = blockIdx.z;
  const int i = blockIdx.y * 16 + (threadIdx.x >> 4);
  const int j = blockIdx.x * 16 + (threadIdx.x & 15);
  if (i >= a.M || j >= a.M) return;
  const uint16_t* A = static_cast<const uint16_t*>(a.a.p[bi]);
  uint16_t* bp = static_cast<uint16_t*>(const_cast<void*>(a.bp.p[bi]));
  const float y = a.b * bf16_bits_to_f32(A[(int64_t)i * a.a.ld + j]);
  bp[(int64_t)i * a.bp.ld + j] = to_bf16_bits(y);
  if (a.M <= kNsSplitRows) {
    float* b32 = static_cast<float*>(const_cast<void*>(a.bp32.p[bi]));
    b32[(int64_t)i * a.bp32.ld + j] = y;
  }
}

// ---------------------------------------------------------------------------
// fp64 Gram  W = P^T P  over rows [kbeg, kend) of P (m x r, fp32), lower
// 64 x 64 tiles only, one split-K slice per blockIdx.y.  v_mfma_f64_16x16x4_f64:
// lane l supplies row (l%16) and k = l/16 of each operand; result element e of
// lane l is row l/16 + 4*e, column l%16 of the 16 x 16 tile (rows interleave
// across the four result registers, unlike the fp32-result instructions).
// ---------------------------------------------------------------------------
// FULL: r a multiple of 64 and every k slice a whole number of 32-row tiles,
// so no load needs a bounds check (the checked loads' selects let the compiler
// sink each load into a branch of its own and wait for it there).
template <bool FULL>
__global__ __launch_bounds__(256) void gram64_kernel(Gram64Args a) {
  __shared__ double sa[2][32][66];
  __shared__ double sb[2][32][66];
  const int member = blockIdx.z;
  const float* P = static_cast<const float*>(a.p.p[member]);
  double* part = a.part + member * a.part_member_stride + blockIdx.y * a.slice;
  // lower-triangular tile decode: t -> (ta, tb), tb <= ta
  const int t = blockIdx.x;
  int ta = static_cast<int>((sqrt(8.0 * t + 1.0) - 1.0) * 0.5);
  while ((ta + 1) * (ta + 2) / 2 <= t) ++ta;
  while (ta * (ta + 1) / 2 > t) --ta;
  const int tb = t - ta * (ta + 1) / 2;
  const bool diag = ta == tb;
  const int a0 = ta * 64, b0 = tb * 64;
  const int r = a.r;
  const int kbeg = blockIdx.y * a.kchunk;
  const int kend = min(a.m, kbeg + a.kchunk);
  const int nk = kend > kbeg ? (kend - kbeg + 31) / 32 : 0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wa = wave >> 1, wb = wave & 1;
  // each thread moves 8 elements of each 32 x 64 operand tile.  Loads are
  // branch-free (addresses clamped into P, out-of-range values selected to
  // zero) and run two k tiles ahead, into alternating register sets.
  float va[2][8], vb[2][8];
  auto load = [&](auto buf_c, int k0) {
    constexpr int buf = decltype(buf_c)::value;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int e = threadIdx.x + q * 256;
      const int kr = e >> 6, cc = e & 63;
      const int gk = k0 + kr;
      if constexpr (FULL) {
        const float* row = P + (int64_t)gk * a.p.ld;
        va[buf][q] = row[a0 + cc];
        vb[buf][q] = row[b0 + cc];
      } else {
        const bool ok = gk < kend;
        const float* row = P + (int64_t)min(gk, kend - 1) * a.p.ld;
        const float x = row[min(a0 + cc, r - 1)];
        va[buf][q] = (ok && a0 + cc < r) ? x : 0.f;
        if (!diag) {
          const float y = row[min(b0 + cc, r - 1)];
          vb[buf][q] = (ok && b0 + cc < r) ? y : 0.f;
        }
      }
    }
  };
  auto store = [&](int st, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int e = threadIdx.x + q * 256;
      sa[st][e >> 6][e & 63] = static_cast<double>(va[buf][q]);
      if (FULL || !diag) sb[st][e >> 6][e & 63] = static_cast<double>(vb[buf][q]);
    }
  };
  doublex4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = doublex4{0.0, 0.0, 0.0, 0.0};
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  if (nk > 0) {
    load(B0{}, kbeg);
    if (nk > 1) load(B1{}, kbeg + 32);
    store(0, B0{});
  }
  // k tile kt from LDS stage kt & 1; register set kt & 1 is free on entry and
  // set (kt + 1) & 1 holds tile kt + 1 (or has it in flight)
  auto step = [&](int kt, auto set_c) {
    constexpr int SET = decltype(set_c)::value;
    const int cur = kt & 1;
    __syncthreads();
    if (kt + 2 < nk) load(set_c, kbeg + (kt + 2) * 32);
    double (*A)[66] = sa[cur];
    double (*B)[66] = diag ? sa[cur] : sb[cur];
    // fragments of the next 4-deep k step read while this step's products run
    double af[2][2], bf[2][2];
    auto frags = [&](int buf, int kk) {
#pragma unroll
      for (int i = 0; i < 2; ++i) af[buf][i] = A[kk + (lane >> 4)][wa * 32 + i * 16 + (lane & 15)];
#pragma unroll
      for (int j = 0; j < 2; ++j) bf[buf][j] = B[kk + (lane >> 4)][wb * 32 + j * 16 + (lane & 15)];
    };
    frags(0, 0);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (ks + 1 < 8) frags((ks + 1) & 1, (ks + 1) * 4);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(af[ks & 1][i], bf[ks & 1][j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store(cur ^ 1, std::integral_constant<int, SET ^ 1>{});
  };
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, B0{});
    if (kt + 1 < nk) step(kt + 1, B1{});
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = a0 + wa * 32 + i * 16 + (lane >> 4) + 4 * e;
        const int col = b0 + wb * 32 + j * 16 + (lane & 15);
        if (row < r && col < r) part[(int64_t)row * r + col] = acc[i][j][e];
      }
}

// fp64 Gram slices of P (m x r fp32) for r a multiple of 128: 128 x 128 lower
// tiles (tb <= ta) of r x r, four waves of 64 x 64 (4 x 4 fp64 16 x 16 x 4
// products), k in tiles of 32 rows of P.  Operand tiles are staged in LDS as
// fp32 (row pitch 144 floats: the fragment reads of four consecutive k rows
// fall on distinct banks) and widened to fp64 as fragments are read; the next
// k step's fragments are read while this step's products run.  Same output as
// gram64_kernel: slice blockIdx.y of part, element (row, col) at row * r + col.
// grid (T (T + 1) / 2 tiles, splits, members), T = r / 128.
__global__ __launch_bounds__(512) void gram64_big_kernel(Gram64Args a) {
  constexpr int kPitch = 144;
  __shared__ __attribute__((aligned(16))) float sa[2][32 * kPitch];
  __shared__ __attribute__((aligned(16))) float sb[2][32 * kPitch];
  const int member = blockIdx.z;
  const float* P = static_cast<const float*>(a.p.p[member]);
  double* part = a.part + member * a.part_member_stride + blockIdx.y * a.slice;
  const int t = blockIdx.x;
  int ta = static_cast<int>((sqrt(8.0 * t + 1.0) - 1.0) * 0.5);
  while ((ta + 1) * (ta + 2) / 2 <= t) ++ta;
  while (ta * (ta + 1) / 2 > t) --ta;
  const int tb = t - ta * (ta + 1) / 2;
  const bool diag = ta == tb;
  const int a0 = ta * 128, b0 = tb * 128;
  const int r = a.r;
  const int kbeg = blockIdx.y * a.kchunk;
  const int kend = min(a.m, kbeg + a.kchunk);
  const int nk = kend > kbeg ? (kend - kbeg + 31) / 32 : 0;
  // eight waves, two per SIMD: wave (wa, wb) owns rows 32 wa .. + 31 and
  // columns 64 wb .. + 63 of the tile
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wa = wave >> 1, wb = wave & 1;
  // thread: float4 at column 4 (tid & 31) of k rows (tid >> 5) + 16 q
  const int lc = (threadIdx.x & 31) * 4, lk = threadIdx.x >> 5;
  floatx4 va[2], vb[2];
  auto load = [&](int k0) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int gk = k0 + lk + 16 * q;
      const bool ok = gk < kend;
      const float* row = P + (int64_t)(ok ? gk : kbeg) * a.p.ld;
      const floatx4 x = *reinterpret_cast<const floatx4*>(row + a0 + lc);
      va[q] = ok ? x : floatx4{0.f, 0.f, 0.f, 0.f};
      if (!diag) {
        const floatx4 y = *reinterpret_cast<const floatx4*>(row + b0 + lc);
        vb[q] = ok ? y : floatx4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  auto store = [&](int st) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      *reinterpret_cast<floatx4*>(&sa[st][(lk + 16 * q) * kPitch + lc]) = va[q];
      if (!diag) *reinterpret_cast<floatx4*>(&sb[st][(lk + 16 * q) * kPitch + lc]) = vb[q];
    }
  };
  doublex4 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = doublex4{0.0, 0.0, 0.0, 0.0};
  if (nk > 0) {
    load(kbeg);
    store(0);
  }
  const int fk = lane >> 4, fc = lane & 15;
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) load(kbeg + (kt + 1) * 32);
    const float* A = sa[cur];
    const float* B = diag ? sa[cur] : sb[cur];
    double af[2][2], bf[2][4];
    auto frags = [&](int buf, int kk) {
#pragma unroll
      for (int i = 0; i < 2; ++i) af[buf][i] = static_cast<double>(A[(kk + fk) * kPitch + wa * 32 + i * 16 + fc]);
#pragma unroll
      for (int j = 0; j < 4; ++j) bf[buf][j] = static_cast<double>(B[(kk + fk) * kPitch + wb * 64 + j * 16 + fc]);
    };
    frags(0, 0);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s < 7) frags((s + 1) & 1, (s + 1) * 4);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(af[s & 1][i], bf[s & 1][j], acc[i][j], 0, 0, 0);
    }
    if (more) store(cur ^ 1);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = a0 + wa * 32 + i * 16 + fk + 4 * e;
        const int col = b0 + wb * 64 + j * 16 + fc;
        part[(int64_t)row * r + col] = acc[i][j][e];
      }
}

// Sum the Gram slices and scale to unit diagonal: S = D W D with
// d_i = 1 / sqrt(W_ii) (lower triangle), zero the inverse buffer, write d.
// A workgroup owns a 16 x 16 block: 32 of its threads first sum the W_ii of
// its 16 rows and 16 columns into LDS (slice order, as for every element),
// then every thread sums and scales its own element.
__global__ __launch_bounds__(256) void chol_prep_kernel(CholArgs a) {
  __shared__ double dd[2][16];
  const int member = blockIdx.z;
  const double* part = a.part + member * a.part_member_stride;
  double* S = a.s + member * a.mat_stride;
  double* X = a.x + member * a.mat_stride;
  double* d = a.d + member * a.vec_stride;
  const int r = a.r;
  const int i = blockIdx.y * 16 + (threadIdx.x >> 4);
  const int j = blockIdx.x * 16 + (threadIdx.x & 15);
  if (i < r && j < r) X[(int64_t)i * r + j] = 0.0;
  if (blockIdx.x > blockIdx.y) return;   // strictly upper block: uniform exit
  auto sum = [&](int u, int v) {
    double s = 0.0;
#pragma unroll 8
    for (int k = 0; k < a.splits; ++k) s += part[k * a.slice + (int64_t)u * r + v];
    return s;
  };
  if (threadIdx.x < 32) {
    const int t = threadIdx.x & 15;
    const int q = (threadIdx.x >> 4) ? blockIdx.x * 16 + t : blockIdx.y * 16 + t;
    double v = 1.0;
    if (q < r) {
      const double w = sum(q, q);
      v = w > 0.0 ? 1.0 / sqrt(w) : 1.0;
    }
    dd[threadIdx.x >> 4][t] = v;
  }
  __syncthreads();
  if (i >= r || j >= r || j > i) return;
  const double di = dd[0][threadIdx.x >> 4], dj = dd[1][threadIdx.x & 15];
  S[(int64_t)i * r + j] = sum(i, j) * di * dj;
  if (i == j) d[i] = di;
}

// Pivots below this (the scaled Gram has unit diagonal) are treated as a
// numerical rank deficiency and replaced by it.
constexpr double kPivMin = 1e-14;

// Pitch (doubles) of the 64 x 64 fp64 LDS tiles of the Cholesky kernels: rows
// start 16-byte aligned.
constexpr int kCP = 66;

// Broadcast lane `lane` (wave-uniform) of a double to the whole wave.
__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t bits = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(bits)), lane);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(bits >> 32)), lane);
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

// 1/x and 1/sqrt(x) for x > 0: hardware estimate and one Newton step (relative
// error about the square of the estimate's, far below what the Gram's
// conditioning can use).
__device__ __forceinline__ double rcp_f64(double x) {
  const double y = __builtin_amdgcn_rcp(x);
  return y * fma(-x, y, 2.0);
}
__device__ __forceinline__ double rsqrt_f64(double x) {
  const double y = __builtin_amdgcn_rsq(x);
  return y * (1.5 - 0.5 * x * y * y);
}

// One 16 x 16 tile of a phase's rank-8 update in chol_diag_factor: y = 0 for
// the factor L, 1 for the inverse Y; tile row and column.
struct CholTile {
  int y, tr, tc;
};

// Tiles of phase p: the L-tiles tc0 <= tc <= tr (tc0 = (8p + 8) / 16, the
// tile column holding the first column past panel p) in row order, then the
// Y-tiles on tile rows 8p/16..3 and tile columns 0..(8p - 1)/16.  At most ten.
__host__ __device__ constexpr int chol_ntile(int p) {
  const int tl = 4 - ((8 * p + 8) >> 4);
  const int ncy = p > 0 ? ((8 * p - 1) >> 4) + 1 : 0;
  return tl * (tl + 1) / 2 + (4 - ((8 * p) >> 4)) * ncy;
}
__host__ __device__ constexpr CholTile chol_tile(int p, int s) {
  const int tc0 = (8 * p + 8) >> 4, tl = 4 - tc0, nl = tl * (tl + 1) / 2;
  if (s < nl) {
    int ta = 0;
    while ((ta + 1) * (ta + 2) / 2 <= s) ++ta;
    return CholTile{0, tc0 + ta, tc0 + s - ta * (ta + 1) / 2};
  }
  const int ncy = ((8 * p - 1) >> 4) + 1, u = s - nl;
  return CholTile{1, ((8 * p) >> 4) + u / ncy, u % ncy};
}

// Operands of tile S of phase P (lane: (lane & 15, lane >> 4) is (row, k) of
// the left operand and (column, row) of the target):
//   L-tile: L[i][c] -= sum over k in panel P of L[i][k] L[c][k]
//   Y-tile: Y[i][c] -= sum over k in panel P - 1 of L[i][k] X[k][c]
// (ly: L at 0, Y at 64 rows; pitch kCP.)  Every offset is a constant.
template <int P, int S>
__device__ __forceinline__ void chol_tile_load(const double* ly, int lane_a, int lane_t, double* av,
                                               double* bv, double* old) {
  constexpr CholTile t = chol_tile(P, S);
  constexpr int kb = 8 * P - 8 * t.y;
  constexpr int offa = t.tr * 16 * kCP + kb;
  av[0] = ly[lane_a + offa];
  av[1] = ly[lane_a + offa + 4];
  if constexpr (t.y != 0) {
    constexpr int offb = (64 + kb) * kCP + t.tc * 16;
    bv[0] = ly[lane_t + offb];
    bv[1] = ly[lane_t + offb + 4 * kCP];
  } else {
    constexpr int offb = t.tc * 16 * kCP + kb;
    bv[0] = ly[lane_a + offb];
    bv[1] = ly[lane_a + offb + 4];
  }
  constexpr int offt = (t.y * 64 + t.tr * 16) * kCP + t.tc * 16;
#pragma unroll
  for (int e = 0; e < 4; ++e) old[e] = ly[lane_t + offt + e * 4 * kCP];
}

// Product and masked write-back of tile S of phase P: an element changes
// where the update applies (L: row >= pe, pe + 8 <= col <= row -- the columns
// pe .. pe + 7 of panel P + 1 are updated in registers by the wave that
// factors it; Y: row >= 8P, col < 8P), so no element outside the update is
// written.
template <int P, int S>
__device__ __forceinline__ void chol_tile_apply(double* ly, int lane, int lane_t, const double* av,
                                                const double* bv, const double* old) {
  constexpr CholTile t = chol_tile(P, S);
  constexpr int j0 = 8 * P, pe = j0 + 8;
  constexpr int offt = (t.y * 64 + t.tr * 16) * kCP + t.tc * 16;
  doublex4 acc = {0.0, 0.0, 0.0, 0.0};
  acc = __builtin_amdgcn_mfma_f64_16x16x4f64(av[0], bv[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f64_16x16x4f64(av[1], bv[1], acc, 0, 0, 0);
  const int col = t.tc * 16 + (lane & 15);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = t.tr * 16 + (lane >> 4) + 4 * e;
    const bool ok = t.y != 0 ? (row >= j0 && col < j0) : (row >= pe && col >= pe + 8 && col <= row);
    if (ok) ly[lane_t + offt + e * 4 * kCP] = old[e] - acc[e];
  }
}

// Tiles of phase P by wave, for the factorisation in which wave 0 updates and
// factors panel P + 1 in registers during phase P: wave 1 every Y-tile, waves
// 2 and 3 the L-tiles alternately (none for wave 0).  chol_pick gives the
// index (as in chol_tile) of the n-th tile of wave W, or -1.
__host__ __device__ constexpr int chol_pick(int p, int w, int n) {
  int seen = 0, rest = 0;
  for (int s = 0; s < chol_ntile(p); ++s) {
    const CholTile t = chol_tile(p, s);
    int owner = 0;
    if (t.y != 0) {
      owner = 1;
    } else {
      owner = 2 + (rest & 1);
      ++rest;
    }
    if (owner == w) {
      if (seen == n) return s;
      ++seen;
    }
  }
  return -1;
}

template <int P, int W, int N>
__device__ __forceinline__ void chol_tiles2_n(double* ly, int lane, int lane_a, int lane_t) {
  constexpr int s0 = chol_pick(P, W, N), s1 = chol_pick(P, W, N + 1), s2 = chol_pick(P, W, N + 2);
  double av[3][2], bv[3][2], old[3][4];
  if constexpr (s0 >= 0) chol_tile_load<P, (s0 >= 0 ? s0 : 0)>(ly, lane_a, lane_t, av[0], bv[0], old[0]);
  if constexpr (s1 >= 0) chol_tile_load<P, (s1 >= 0 ? s1 : 0)>(ly, lane_a, lane_t, av[1], bv[1], old[1]);
  if constexpr (s2 >= 0) chol_tile_load<P, (s2 >= 0 ? s2 : 0)>(ly, lane_a, lane_t, av[2], bv[2], old[2]);
  if constexpr (s0 >= 0) chol_tile_apply<P, (s0 >= 0 ? s0 : 0)>(ly, lane, lane_t, av[0], bv[0], old[0]);
  if constexpr (s1 >= 0) chol_tile_apply<P, (s1 >= 0 ? s1 : 0)>(ly, lane, lane_t, av[1], bv[1], old[1]);
  if constexpr (s2 >= 0) chol_tile_apply<P, (s2 >= 0 ? s2 : 0)>(ly, lane, lane_t, av[2], bv[2], old[2]);
}

// Wave W's tiles of phase P, three loads in flight at a time (at most six
// tiles per wave).
template <int P, int W>
__device__ __forceinline__ void chol_tiles2(double* ly, int lane) {
  const int lane_a = (lane & 15) * kCP + (lane >> 4), lane_t = (lane >> 4) * kCP + (lane & 15);
  static_assert(chol_pick(P, W, 6) < 0, "more than six tiles for one wave");
  chol_tiles2_n<P, W, 0>(ly, lane, lane_a, lane_t);
  if constexpr (chol_pick(P, W, 3) >= 0) chol_tiles2_n<P, W, 3>(ly, lane, lane_a, lane_t);
}

template <int P>
__device__ __forceinline__ void chol_tiles2_wave(double* ly, int lane, int wave) {
  if (wave == 1) chol_tiles2<P, 1>(ly, lane);
  else if (wave == 2) chol_tiles2<P, 2>(ly, lane);
  else chol_tiles2<P, 3>(ly, lane);
}

// Factor the nb x nb diagonal block kb of S (S_kk = L_kk L_kk^T) and invert
// L_kk in LDS (LY[0] = L, LY[1] = Y, dinv: 64 doubles), then write L_kk into S
// and L_kk^{-1} into block (kb, kb) of X.  A block smaller than 64 is padded
// with the identity, which factors to itself.  Right-looking over 8-column
// panels p, one phase each:
//   wave 0 factors panel p in registers (lane i holds row i; pivots and column
//   entries move by readlane) while wave 1 solves block row p - 1 of the
//   inverse, X_{p-1} = L_{p-1,p-1}^{-1} Y_{p-1} (lane c holds column c);
//   then the four waves apply the rank-8 updates as 16 x 16 fp64 MFMA tiles
//   (chol_tile_load): of L by panel p beyond it, and of Y by X_{p-1} below
//   it, Y starting as the identity.  The tile work of each (phase, wave) is
//   compiled with constant offsets.
// chol_diag_load fills L (lower triangle of S_kk, identity padding) and Y = I
// from global memory; chol_diag_factor then works from LDS alone, so a caller
// that already holds the block can fill L itself.
__device__ void chol_diag_load(const CholArgs& a, int kb, int member, double (*LY)[64][kCP]) {
  const double* S = a.s + member * a.mat_stride;
  const int r = a.r;
  const int o = kb * 64;
  const int nb = min(64, r - o);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  double (*L)[kCP] = LY[0];
  double (*Y)[kCP] = LY[1];
  // element (gi, gj) = (q * 4 + wave, lane): each wave moves whole 64-wide
  // rows.  Every load is issued before any is used (clamped addresses; the
  // triangle is cut with a select, so stale words in the upper triangle, NaN
  // patterns included, never reach the arithmetic).
  uint64_t v[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int gi = q * 4 + wave, gj = lane;
    v[q] = reinterpret_cast<const uint64_t*>(S)[(int64_t)(o + min(gi, nb - 1)) * r + o + min(gj, nb - 1)];
  }
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int gi = q * 4 + wave, gj = lane;
    const double id = gi == gj ? 1.0 : 0.0;
    L[gi][gj] = (gi < nb && gj <= gi) ? __longlong_as_double(static_cast<long long>(v[q])) : id;
    Y[gi][gj] = id;
  }
}

__device__ void chol_diag_factor(const CholArgs& a, int kb, int member, double (*LY)[64][kCP],
                                 double* dinv) {
  double* S = a.s + member * a.mat_stride;
  double* X = a.x + member * a.mat_stride;
  const int r = a.r;
  const int o = kb * 64;
  const int nb = min(64, r - o);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  double (*L)[kCP] = LY[0];
  double (*Y)[kCP] = LY[1];
  double* ly = &LY[0][0][0];
  bool shifted = false;
  // block row q of the inverse, by wave 1 (lane c: column c)
  auto solve_rows = [&](int q) {
    const int jq = q * 8;
    double y[8], lq[8][8], dq[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      y[t] = Y[jq + t][lane];
      dq[t] = dinv[jq + t];
#pragma unroll
      for (int u = 0; u < t; ++u) lq[t][u] = L[jq + t][jq + u];
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      double acc = y[t];
#pragma unroll
      for (int u = 0; u < t; ++u) acc = fma(-lq[t][u], y[u], acc);
      y[t] = acc * dq[t];
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) Y[jq + t][lane] = y[t];
  };
  // panel p of L (pc: its 8 columns, lane i holding row i, with every
  // earlier panel's update applied), factored in registers by wave 0
  auto panel = [&](int p, double (&pc)[8]) {
    const int j0 = p * 8;
    double invd[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int jc = j0 + c;
      const double a0 = readlane_f64(pc[c], jc);
      shifted |= !(a0 > kPivMin);
      // maxNum: a NaN pivot is replaced too (and flagged)
      const double piv = fmax(a0, kPivMin);
      const double rs = rsqrt_f64(piv);
      invd[c] = rs;
      // scaled column; rows above jc hold entries above the diagonal: zeroed
      const double x = lane == jc ? piv : pc[c];
      pc[c] = lane >= jc ? x * rs : 0.0;
#pragma unroll
      for (int c2 = c + 1; c2 < 8; ++c2) pc[c2] = fma(-pc[c], readlane_f64(pc[c], j0 + c2), pc[c2]);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) L[lane][j0 + c] = pc[c];
    if (lane == 0) {
#pragma unroll
      for (int c = 0; c < 8; ++c) dinv[j0 + c] = invd[c];
    }
  };
  // Phase p: wave 0 applies panel p's rank-8 update to the 8 columns of
  // panel p + 1 in registers (rows by lane, the 8 x 8 block of panel p on
  // those rows read as broadcasts) and factors panel p + 1 at once, which
  // needs nothing else; wave 1 solves block row p - 1 of the inverse and
  // applies every Y-tile of the phase with it; waves 2 and 3 apply the
  // L-tiles (outside panel p + 1).  One barrier per phase.
  __syncthreads();
  if (wave == 0) {
    double pc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) pc[c] = L[lane][c];
    panel(0, pc);
  }
  for (int p = 0; p < 8; ++p) {
    __syncthreads();
    if (wave == 0) {
      if (p < 7) {
        const int j0 = p * 8, pe = j0 + 8;
        double pc[8], lp[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) pc[c] = L[lane][pe + c];
#pragma unroll
        for (int k = 0; k < 8; ++k) lp[k] = L[lane][j0 + k];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          // L[pe + c][j0 .. j0 + 7], the same address in every lane
          double b[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) b[k] = L[pe + c][j0 + k];
#pragma unroll
          for (int k = 0; k < 8; ++k) pc[c] = fma(-lp[k], b[k], pc[c]);
        }
        panel(p + 1, pc);
      }
    } else {
      if (wave == 1 && p > 0) solve_rows(p - 1);
      switch (p) {
        case 0: chol_tiles2_wave<0>(ly, lane, wave); break;
        case 1: chol_tiles2_wave<1>(ly, lane, wave); break;
        case 2: chol_tiles2_wave<2>(ly, lane, wave); break;
        case 3: chol_tiles2_wave<3>(ly, lane, wave); break;
        case 4: chol_tiles2_wave<4>(ly, lane, wave); break;
        case 5: chol_tiles2_wave<5>(ly, lane, wave); break;
        case 6: chol_tiles2_wave<6>(ly, lane, wave); break;
        default: chol_tiles2_wave<7>(ly, lane, wave); break;
      }
    }
  }
  __syncthreads();
  if (wave == 1) solve_rows(7);
  __syncthreads();
  if (shifted && threadIdx.x == 0 && a.status) atomicOr(a.status, 1);
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int gi = q * 4 + wave, gj = lane;
    if (gi < nb && gj <= gi) {
      S[(int64_t)(o + gi) * r + o + gj] = L[gi][gj];
      X[(int64_t)(o + gi) * r + o + gj] = Y[gi][gj];
    }
  }
}

__global__ __launch_bounds__(256) void chol_diag_kernel(CholArgs a, int kb) {
  __shared__ double LY[2][64][kCP];
  __shared__ double dinv[64];
  chol_diag_load(a, kb, blockIdx.x, LY);
  chol_diag_factor(a, kb, blockIdx.x, LY, dinv);
}

// The whole orthonormalisation of a rank of at most 64 in one workgroup per
// member, for short P~ (m <= 256; the small-problem chain of separate launches
// is latency, not work): P~ is read once into LDS (fp32, every load in flight
// together), then the fp64 Gram W = P~^T P~ (2 x 2 waves of 32 x 32 fp64
// 16x16x4 products, operands widened as they are read), the column scaling
// d = diag(W)^-1/2, the 64 x 64 Cholesky and inverse in LDS
// (chol_diag_factor), T1^T = L^-1 D in place, and P = P~ T1 in fp64 (the
// products of a wave stop at its last column: T1 is upper triangular).  Same
// steps, in the same precisions, as the multi-launch chain with the fp64
// apply.  grid (members).
constexpr int kSoPitch = 68;   // floats per LDS row of P~: 16 consecutive rows at one k on distinct banks
__global__ __launch_bounds__(256) void small_ortho_kernel(SmallOrthoArgs a) {
  __shared__ double LY[2][64][kCP];
  __shared__ float sp[256 * kSoPitch];
  __shared__ double dinv[64], dsc[64];
  const int member = blockIdx.x;
  const float* P = static_cast<const float*>(a.pt.p[member]);
  const int64_t ldp = a.pt.ld;
  const int m = a.m, r = a.ca.r;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  double (*L)[kCP] = LY[0];
  double (*Y)[kCP] = LY[1];

  // 0. P~ (m x r, zero-padded to 64 columns and to a multiple of 16 rows) into
  // LDS, every load of a thread issued before any store: float4 loads when the
  // rows allow them (a uniform test), else element-wise in passes of 64 rows;
  // or, with split-K slices, their sum in slice order (16-byte aligned)
  const int mp = (m + 15) & ~15;
  if (a.splits > 0) {
    const float* part = a.part + member * a.part_member_stride;
    float4 v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) v[q] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < a.splits; ++k) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int e = threadIdx.x + q * 256;
        const int i = e >> 4, c4 = (e & 15) * 4;
        // unconditional load and add (rows and columns past the end are
        // clamped here and zeroed at the store): a conditional add would let
        // the compiler move the load under the condition and wait on each
        const float4 x = *reinterpret_cast<const float4*>(part + k * a.slice + (int64_t)min(i, m - 1) * r +
                                                          min(c4, r - 4));
        v[q].x += x.x; v[q].y += x.y; v[q].z += x.z; v[q].w += x.w;
      }
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int e = threadIdx.x + q * 256;
      const int i = e >> 4, c4 = (e & 15) * 4;
      const float4 z = (i < m && c4 < r) ? v[q] : make_float4(0.f, 0.f, 0.f, 0.f);
      if (i < mp) *reinterpret_cast<float4*>(sp + i * kSoPitch + c4) = z;
    }
  } else if (a.pt.vec && (r & 3) == 0 && (ldp & 3) == 0) {
    float4 v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int e = threadIdx.x + q * 256;
      const int i = e >> 4, c4 = (e & 15) * 4;
      const float4 x = *reinterpret_cast<const float4*>(P + (int64_t)min(i, m - 1) * ldp + min(c4, r - 4));
      v[q] = (i < m && c4 < r) ? x : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int e = threadIdx.x + q * 256;
      const int i = e >> 4, c4 = (e & 15) * 4;
      if (i < mp) *reinterpret_cast<float4*>(sp + i * kSoPitch + c4) = v[q];
    }
  } else {
    for (int r0 = 0; r0 < mp; r0 += 64) {
      float v[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int e = threadIdx.x + q * 256;
        const int i = r0 + (e >> 6), c = e & 63;
        const float x = P[(int64_t)min(i, m - 1) * ldp + min(c, r - 1)];
        v[q] = (i < m && c < r) ? x : 0.f;
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int e = threadIdx.x + q * 256;
        const int i = r0 + (e >> 6);
        if (i < mp) sp[i * kSoPitch + (e & 63)] = v[q];
      }
    }
  }
  __syncthreads();

  // 1. W = P~^T P~, the 10 lower 16 x 16 blocks: each wave over a quarter of
  // the rows of P~ (fragments of the next 4-deep k step read under the current
  // products), then the four partial sums added into L in wave order
  {
    constexpr int kBI[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
    constexpr int kBJ[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};
    doublex4 w[10];
#pragma unroll
    for (int b = 0; b < 10; ++b) w[b] = doublex4{0.0, 0.0, 0.0, 0.0};
    const int quarter = mp / 4;   // a multiple of 4
    const int kb0 = wave * quarter;
    double f[2][4];
    auto frags = [&](int buf, int kk) {
      const float* row = sp + (kb0 + kk + (lane >> 4)) * kSoPitch + (lane & 15);
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) f[buf][bi] = static_cast<double>(row[bi * 16]);
    };
    if (quarter > 0) frags(0, 0);
    for (int kk = 0; kk < quarter; kk += 8) {
      if (kk + 4 < quarter) frags(1, kk + 4);
#pragma unroll
      for (int b = 0; b < 10; ++b)
        w[b] = __builtin_amdgcn_mfma_f64_16x16x4f64(f[0][kBI[b]], f[0][kBJ[b]], w[b], 0, 0, 0);
      if (kk + 4 >= quarter) break;
      if (kk + 8 < quarter) frags(0, kk + 8);
#pragma unroll
      for (int b = 0; b < 10; ++b)
        w[b] = __builtin_amdgcn_mfma_f64_16x16x4f64(f[1][kBI[b]], f[1][kBJ[b]], w[b], 0, 0, 0);
    }
    for (int src = 0; src < 4; ++src) {
      if (wave == src) {
#pragma unroll
        for (int b = 0; b < 10; ++b)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            double& dst = L[kBI[b] * 16 + (lane >> 4) + 4 * e][kBJ[b] * 16 + (lane & 15)];
            dst = src == 0 ? w[b][e] : dst + w[b][e];
          }
      }
      __syncthreads();
    }
  }
  // 2. d_i = W_ii^-1/2 (1 for a zero column or padding); L = the scaled lower
  // triangle with identity padding, Y = I (as chol_prep and chol_diag_load)
  if (threadIdx.x < 64) {
    const int t = threadIdx.x;
    const double w = L[t][t];
    dsc[t] = (t < r && w > 0.0) ? 1.0 / sqrt(w) : 1.0;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int gi = q * 4 + wave, gj = lane;
    const double id = gi == gj ? 1.0 : 0.0;
    L[gi][gj] = (gi < r && gj <= gi) ? L[gi][gj] * dsc[gi] * dsc[gj] : id;
    Y[gi][gj] = id;
  }
  __syncthreads();
  // 3. L and Y = L^-1 in LDS
  chol_diag_factor(a.ca, 0, member, LY, dinv);
  __syncthreads();
  // 4. T1^T[j][k] = Y[j][k] d_k
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int gi = q * 4 + wave, gj = lane;
    Y[gi][gj] *= dsc[gj];
  }
  __syncthreads();
  // 5. P = P~ T1 over 64-row tiles of the resident P~: wave w owns rows
  // 16 w .. + 15 of each tile and all four 16-column blocks; block jb needs
  // k < 16 (jb + 1) (T1 is upper triangular), 40 products per tile
  float* out = static_cast<float*>(const_cast<void*>(a.out.p[member]));
  uint16_t* ob = a.has_bf16 ? static_cast<uint16_t*>(const_cast<void*>(a.out_bf16.p[member])) : nullptr;
  for (int i0 = 0; i0 < m; i0 += 64) {
    doublex4 acc4[4];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) acc4[jb] = doublex4{0.0, 0.0, 0.0, 0.0};
    const float* arow = sp + min(i0 + wave * 16 + (lane & 15), mp - 1) * kSoPitch + (lane >> 4);
#pragma unroll
    for (int k0 = 0; k0 < 64; k0 += 4) {
      const double af = static_cast<double>(arow[k0]);
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        if (k0 < 16 * (jb + 1)) {
          const double bf = Y[jb * 16 + (lane & 15)][k0 + (lane >> 4)];
          acc4[jb] = __builtin_amdgcn_mfma_f64_16x16x4f64(af, bf, acc4[jb], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = i0 + wave * 16 + (lane >> 4) + 4 * e;
        const int col = jb * 16 + (lane & 15);
        if (row < m && col < r) {
          const float x = static_cast<float>(acc4[jb][e]);
          out[(int64_t)row * a.out.ld + col] = x;
          if (ob) ob[(int64_t)row * a.out_bf16.ld + col] = to_bf16_bits(x);
        }
      }
  }
}

// 64 x 64 fp64 tiles of row-major r x r matrices through LDS (pitch kCP),
// four waves of 32 x 32 on v_mfma_f64_16x16x4f64.  Element e of acc[i][j] in
// lane l is row wa * 32 + i * 16 + l / 16 + 4 e, column wb * 32 + j * 16 +
// l % 16 (wa, wb: the wave's quadrant).

// Tile at (row0, col0) into registers, zero outside the matrix.
__device__ __forceinline__ void tile_fetch64(const double* A, int r, int row0, int col0, double v[16]) {
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int e = threadIdx.x + q * 256;
    const int i = e >> 6, j = e & 63;
    v[q] = (row0 + i < r && col0 + j < r) ? A[(int64_t)(row0 + i) * r + col0 + j] : 0.0;
  }
}
__device__ __forceinline__ void tile_put_regs(const double v[16], double (*sT)[kCP]) {
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int e = threadIdx.x + q * 256;
    sT[e >> 6][e & 63] = v[q];
  }
}

// acc = A B^T (TRANS_B) or A B, K = 64, both operands in LDS.
template <bool TRANS_B>
__device__ __forceinline__ void tile_mma64(const double (*sA)[kCP], const double (*sB)[kCP],
                                           doublex4 acc[2][2]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wa = wave >> 1, wb = wave & 1;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = doublex4{0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
  for (int kk = 0; kk < 64; kk += 4) {
    double af[2], bf[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) af[i] = sA[wa * 32 + i * 16 + (lane & 15)][kk + (lane >> 4)];
#pragma unroll
    for (int j = 0; j < 2; ++j)
      bf[j] = TRANS_B ? sB[wb * 32 + j * 16 + (lane & 15)][kk + (lane >> 4)]
                      : sB[kk + (lane >> 4)][wb * 32 + j * 16 + (lane & 15)];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(af[i], bf[j], acc[i][j], 0, 0, 0);
  }
}

// acc into an LDS tile.
__device__ __forceinline__ void tile_put_acc(const doublex4 acc[2][2], double (*sT)[kCP]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wa = wave >> 1, wb = wave & 1;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sT[wa * 32 + i * 16 + (lane >> 4) + 4 * e][wb * 32 + j * 16 + (lane & 15)] = acc[i][j][e];
}

// Subtract acc from the tile at (orow, ocol) of an r x r matrix; lower_only
// keeps the strictly-upper part of a diagonal tile untouched.
__device__ __forceinline__ void tile_sub64(double* out, int r, int orow, int ocol,
                                           const doublex4 acc[2][2], bool lower_only) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wa = wave >> 1, wb = wave & 1;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rr = orow + wa * 32 + i * 16 + (lane >> 4) + 4 * e;
        const int cc = ocol + wb * 32 + j * 16 + (lane & 15);
        if (rr < r && cc < r && (!lower_only || cc <= rr)) {
          double* dst = out + (int64_t)rr * r + cc;
          *dst = *dst - acc[i][j][e];
        }
      }
}

// L_ik = S_ik X_kk^T with X_kk lower triangular: output tile column tj (16
// wide) only needs k < 16 (tj + 1).  Wave w takes tile rows 2 (w & 1) and
// 2 (w & 1) + 1 and tile columns {0, 3} (w < 2) or {1, 2} (w >= 2), 40 k steps
// each instead of 64 for the plain 32 x 32 quadrants.
__device__ __forceinline__ int lt_col_tile(int wave, int j) {
  return (wave >> 1) == 0 ? (j == 0 ? 0 : 3) : (j == 0 ? 1 : 2);
}
template <int TJ0, int TJ1>
__device__ __forceinline__ void tile_mma64_lt_w(const double (*sA)[kCP], const double (*sB)[kCP],
                                                doublex4 acc[2][2], int lane, int wa) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = doublex4{0.0, 0.0, 0.0, 0.0};
  // k steps of 4 over the longer range; tile column TJ0 stops at 16 (TJ0 + 1)
#pragma unroll
  for (int kk = 0; kk < 16 * TJ1 + 16; kk += 4) {
    const double a0 = sA[wa * 32 + (lane & 15)][kk + (lane >> 4)];
    const double a1 = sA[wa * 32 + 16 + (lane & 15)][kk + (lane >> 4)];
    const double b1 = sB[TJ1 * 16 + (lane & 15)][kk + (lane >> 4)];
    if (kk < 16 * TJ0 + 16) {
      const double b0 = sB[TJ0 * 16 + (lane & 15)][kk + (lane >> 4)];
      acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc[0][0], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, acc[1][0], 0, 0, 0);
    }
    acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, acc[0][1], 0, 0, 0);
    acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc[1][1], 0, 0, 0);
  }
}
__device__ __forceinline__ void tile_mma64_lt(const double (*sA)[kCP], const double (*sB)[kCP],
                                              doublex4 acc[2][2]) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  if ((wave >> 1) == 0) tile_mma64_lt_w<0, 3>(sA, sB, acc, lane, wave & 1);
  else tile_mma64_lt_w<1, 2>(sA, sB, acc, lane, wave & 1);
}
__device__ __forceinline__ void tile_put_acc_lt(const doublex4 acc[2][2], double (*sT)[kCP]) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int wa = wave & 1;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sT[wa * 32 + i * 16 + (lane >> 4) + 4 * e][lt_col_tile(wave, j) * 16 + (lane & 15)] = acc[i][j][e];
}

// The lower 16 x 16 tiles (ti >= tj) of A A^T, K = 64, spread 3, 3, 2, 2 over
// the waves; tile n of wave w is (lower_tile_row, lower_tile_col).
__device__ __forceinline__ int lower_ntiles(int wave) { return wave < 2 ? 3 : 2; }
__device__ __forceinline__ int lower_tile(int wave, int n) {   // ti * 4 + tj
  constexpr int list[4][3] = {{0, 12, 15}, {4, 5, 13}, {8, 9, 9}, {10, 14, 14}};
  return list[wave][n];
}
__device__ __forceinline__ void tile_mma64_lower(const double (*sA)[kCP], doublex4 acc[3]) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int nt = lower_ntiles(wave);
#pragma unroll
  for (int n = 0; n < 3; ++n) acc[n] = doublex4{0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
  for (int kk = 0; kk < 64; kk += 4) {
#pragma unroll
    for (int n = 0; n < 3; ++n) {
      if (n < nt) {
        const int t = lower_tile(wave, n), ti = t >> 2, tj = t & 3;
        const double av = sA[ti * 16 + (lane & 15)][kk + (lane >> 4)];
        const double bv = sA[tj * 16 + (lane & 15)][kk + (lane >> 4)];
        acc[n] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc[n], 0, 0, 0);
      }
    }
  }
}

// Trailing update after block column kb.  The panel is formed in LDS by the
// workgroups that use it: L_ik = S_ik Linv_kk^T for i > kb, and X_kj =
// Linv_kk Y_kj for j < kb (X_kk = Linv_kk); block row kb of X keeps Y_kj
// (make_t_kernel forms X_kj from it), and block column kb of S keeps S_ik.
//   t <  T(T+1)/2:  S_ij -= L_ik L_jk^T   for kb < j <= i
//   otherwise:      Y_ij -= L_ik X_kj     for i > kb, j <= kb
// Workgroup 0 then factors diagonal block kb + 1, whose tile it has just
// finished (no other workgroup writes it).
__global__ __launch_bounds__(256) void chol_update_kernel(CholArgs a, int kb) {
  __shared__ double sT[3][64][kCP];
  __shared__ double dinv[64];
  const int member = blockIdx.y;
  double* S = a.s + member * a.mat_stride;
  double* X = a.x + member * a.mat_stride;
  const int r = a.r, nblk = (r + 63) / 64;
  const int T = nblk - kb - 1;
  const int ntri = T * (T + 1) / 2;
  const int k0 = kb * 64;
  int t = blockIdx.x;
  doublex4 acc[2][2], acc2[2][2];
  double v0[16], v1[16], v2[16];
  if (t < ntri) {
    int ti = static_cast<int>((sqrt(8.0 * t + 1.0) - 1.0) * 0.5);
    while ((ti + 1) * (ti + 2) / 2 <= t) ++ti;
    while (ti * (ti + 1) / 2 > t) --ti;
    const int tj = t - ti * (ti + 1) / 2;
    const int ib = kb + 1 + ti, jb = kb + 1 + tj;
    const bool two = ib != jb;
    tile_fetch64(S, r, ib * 64, k0, v0);
    tile_fetch64(X, r, k0, k0, v1);
    if (two) tile_fetch64(S, r, jb * 64, k0, v2);
    tile_put_regs(v0, sT[0]);
    tile_put_regs(v1, sT[1]);
    if (two) tile_put_regs(v2, sT[2]);
    // workgroup 0: the diagonal tile it factors, in flight during L_ik
    if (t == 0) tile_fetch64(S, r, ib * 64, ib * 64, v2);
    __syncthreads();
    tile_mma64_lt(sT[0], sT[1], acc);              // L_ik
    if (two) tile_mma64_lt(sT[2], sT[1], acc2);    // L_jk
    __syncthreads();
    tile_put_acc_lt(acc, sT[0]);
    if (t != 0) {
      if (two) tile_put_acc_lt(acc2, sT[2]);
      __syncthreads();
      tile_mma64<true>(sT[0], two ? sT[2] : sT[0], acc);
      tile_sub64(S, r, ib * 64, jb * 64, acc, !two);
    } else {
      // Diagonal tile (kb + 1, kb + 1), which this workgroup then factors:
      // L = S_ii - L_ik L_ik^T is formed in LDS (sT[1], Y = I in sT[2]) and
      // never goes through global memory.  Lower triangle, identity padding.
      const int nb = min(64, r - ib * 64);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int e = threadIdx.x + q * 256;
        const int gi = e >> 6, gj = e & 63;
        const double id = gi == gj ? 1.0 : 0.0;
        sT[1][gi][gj] = (gi < nb && gj <= gi) ? v2[q] : id;
        sT[2][gi][gj] = id;
      }
      __syncthreads();
      doublex4 accd[3];
      tile_mma64_lower(sT[0], accd);
      const int lane = threadIdx.x & 63;
      const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
      const int nt = lower_ntiles(wave);
#pragma unroll
      for (int n = 0; n < 3; ++n) {
        if (n < nt) {
          const int tt = lower_tile(wave, n), ti2 = tt >> 2, tj2 = tt & 3;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int row = ti2 * 16 + (lane >> 4) + 4 * e, col = tj2 * 16 + (lane & 15);
            if (row < nb && col <= row) sT[1][row][col] -= accd[n][e];
          }
        }
      }
      chol_diag_factor(a, kb + 1, member, sT + 1, dinv);
    }
  } else {
    t -= ntri;
    const int ib = kb + 1 + t / (kb + 1), jb = t % (kb + 1);
    const bool below = jb < kb;
    tile_fetch64(S, r, ib * 64, k0, v0);
    tile_fetch64(X, r, k0, k0, v1);
    if (below) tile_fetch64(X, r, k0, jb * 64, v2);
    tile_put_regs(v0, sT[0]);
    tile_put_regs(v1, sT[1]);
    if (below) tile_put_regs(v2, sT[2]);
    __syncthreads();
    tile_mma64_lt(sT[0], sT[1], acc);                    // L_ik
    if (below) tile_mma64<false>(sT[1], sT[2], acc2);    // X_kj
    __syncthreads();
    tile_put_acc_lt(acc, sT[0]);
    if (below) tile_put_acc(acc2, sT[2]);
    __syncthreads();
    tile_mma64<false>(sT[0], below ? sT[2] : sT[1], acc);
    tile_sub64(X, r, ib * 64, jb * 64, acc, false);
  }
}

// T^T[j][k] = X[j][k] d[k] for k <= j, else 0, as fp32, on 64 x 64 tiles:
// the right factor of P1 = P_tilde T with T = D L^{-T} upper triangular.
// Diagonal tiles of X are L_jj^{-1}; a tile below the diagonal is formed as
// X_jk = L_jj^{-1} Y_jk from the Y block the factorisation left there.
// T1^T = (D L^-T)^T, lower triangular r x r (ld r, zeros above the diagonal):
// into tt as fp32 and / or into ttd as fp64 (either may be null).
__global__ __launch_bounds__(256) void make_t_kernel(CholArgs a, float* tt, int64_t tt_stride,
                                                     double* ttd, int64_t ttd_stride) {
  __shared__ double sT[2][64][kCP];
  const int member = blockIdx.z;
  const double* X = a.x + member * a.mat_stride;
  const double* d = a.d + member * a.vec_stride;
  float* out = tt ? tt + member * tt_stride : nullptr;
  double* outd = ttd ? ttd + member * ttd_stride : nullptr;
  const int r = a.r;
  const int jb = blockIdx.y, kb = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (kb >= jb) {
    for (int q = 0; q < 16; ++q) {
      const int j = jb * 64 + q * 4 + wave, k = kb * 64 + lane;
      if (j < r && k < r) {
        const double v = (kb == jb && k <= j) ? X[(int64_t)j * r + k] * d[k] : 0.0;
        if (out) out[(int64_t)j * r + k] = static_cast<float>(v);
        if (outd) outd[(int64_t)j * r + k] = v;
      }
    }
    return;
  }
  double v0[16], v1[16];
  tile_fetch64(X, r, jb * 64, jb * 64, v0);
  tile_fetch64(X, r, jb * 64, kb * 64, v1);
  tile_put_regs(v0, sT[0]);
  tile_put_regs(v1, sT[1]);
  __syncthreads();
  doublex4 acc[2][2];
  tile_mma64<false>(sT[0], sT[1], acc);
  const int wa = wave >> 1, wb = wave & 1;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = jb * 64 + wa * 32 + i * 16 + (lane >> 4) + 4 * e;
        const int k = kb * 64 + wb * 32 + jj * 16 + (lane & 15);
        if (j < r && k < r) {
          const double v = acc[i][jj][e] * d[k];
          if (out) out[(int64_t)j * r + k] = static_cast<float>(v);
          if (outd) outd[(int64_t)j * r + k] = v;
        }
      }
}

// P = P~ T1 with fp64 products, T1 given as T1^T (lower triangular, fp64, ld r):
// P[i][j] = sum over k <= j of P~[i][k] T1^T[j][k].  With T1 from the fp64
// Cholesky of the fp64 Gram and the products in fp64, the columns of P are
// orthonormal to about cond(P~)^2 2^-53 before the final rounding to fp32, so
// no correction pass follows.  64 x 64 output tiles, four waves of 32 x 32
// (2 x 2 fp64 16x16x4 products), k in tiles of 32 up to the tile's last
// column (T1 is upper triangular); both operands staged in LDS k-major as
// fp64 (P~ widened on the way), the next k tile loaded into registers while
// this one's products run.  Tiles of the last column block first: they carry
// the longest k range.  grid (tiles_i * tiles_j, members).
__global__ __launch_bounds__(256) void apply64_kernel(Apply64Args a) {
  __shared__ double sa[2][32][66];
  __shared__ double sb[2][32][66];
  const int member = blockIdx.y;
  const float* P = static_cast<const float*>(a.pt.p[member]);
  const double* T = a.t + member * a.t_member_stride;
  const int m = a.m, r = a.r;
  const int tiles_i = (m + 63) / 64, tiles_j = (r + 63) / 64;
  const int jt = tiles_j - 1 - static_cast<int>(blockIdx.x) / tiles_i;
  const int it = static_cast<int>(blockIdx.x) % tiles_i;
  const int i0 = it * 64, j0 = jt * 64;
  const int kend = min(r, j0 + 64);
  const int nk = (kend + 31) / 32;
  const int64_t ldp = a.pt.ld;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wa = wave >> 1, wb = wave & 1;
  // thread: elements e = tid + 256 q of each 64 x 32 operand tile, row e / 32,
  // k e % 32 (a row's 32 k contiguous in global memory).  Loads are
  // branch-free (addresses clamped into the operands, out-of-range values
  // selected to zero) and run two k tiles ahead, into alternating register sets.
  float va[2][8];
  double vb[2][8];
  auto load = [&](auto buf_c, int k0) {
    constexpr int buf = decltype(buf_c)::value;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int e = threadIdx.x + q * 256;
      const int row = e >> 5, k = k0 + (e & 31);
      const int kc = min(k, kend - 1);
      const float x = P[(int64_t)min(i0 + row, m - 1) * ldp + kc];
      const double y = T[(int64_t)min(j0 + row, r - 1) * r + kc];
      va[buf][q] = (k < kend && i0 + row < m) ? x : 0.f;
      vb[buf][q] = (k < kend && j0 + row < r) ? y : 0.0;
    }
  };
  auto store = [&](int st, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int e = threadIdx.x + q * 256;
      sa[st][e & 31][e >> 5] = static_cast<double>(va[buf][q]);
      sb[st][e & 31][e >> 5] = vb[buf][q];
    }
  };
  doublex4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = doublex4{0.0, 0.0, 0.0, 0.0};
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  load(B0{}, 0);
  if (nk > 1) load(B1{}, 32);
  store(0, B0{});
  // k tile kt from LDS stage kt & 1; on entry its registers (set kt & 1) are
  // in LDS, and set (kt + 1) & 1 holds tile kt + 1 (or is in flight)
  auto step = [&](int kt, auto set_c) {
    constexpr int SET = decltype(set_c)::value;
    const int cur = kt & 1;
    __syncthreads();
    if (kt + 2 < nk) load(set_c, (kt + 2) * 32);
    // fragments of the next 4-deep k step read while this step's products run
    double af[2][2], bf[2][2];
    auto frags = [&](int buf, int kk) {
#pragma unroll
      for (int i = 0; i < 2; ++i) af[buf][i] = sa[cur][kk + (lane >> 4)][wa * 32 + i * 16 + (lane & 15)];
#pragma unroll
      for (int j = 0; j < 2; ++j) bf[buf][j] = sb[cur][kk + (lane >> 4)][wb * 32 + j * 16 + (lane & 15)];
    };
    frags(0, 0);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (ks + 1 < 8) frags((ks + 1) & 1, (ks + 1) * 4);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(af[ks & 1][i], bf[ks & 1][j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store(cur ^ 1, std::integral_constant<int, SET ^ 1>{});
  };
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, B0{});
    if (kt + 1 < nk) step(kt + 1, B1{});
  }
  float* out = static_cast<float*>(const_cast<void*>(a.out.p[member]));
  uint16_t* ob = a.has_bf16 ? static_cast<uint16_t*>(const_cast<void*>(a.out_bf16.p[member])) : nullptr;
  if (i0 + 64 > m || j0 + 64 > r || !a.out.vec || (ob && !a.out_bf16.vec)) {
    // a ragged tile (or rows without 16-byte alignment): element by element
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = i0 + wa * 32 + i * 16 + (lane >> 4) + 4 * e;
          const int col = j0 + wb * 32 + j * 16 + (lane & 15);
          if (row < m && col < r) {
            const float v = static_cast<float>(acc[i][j][e]);
            out[(int64_t)row * a.out.ld + col] = v;
            if (ob) ob[(int64_t)row * a.out_bf16.ld + col] = to_bf16_bits(v);
          }
        }
    return;
  }
  // A whole tile goes through LDS (the operand stages, free now) as fp32, so
  // that each thread stores four consecutive columns of four rows: P, its bf16
  // copy, and (has_frag, has_t) the layouts the update and sweep 2 read, which
  // a separate pass over P would otherwise write (reduce_pieces_kernel).
  __syncthreads();   // every wave is done with sa and sb
  float (*tile)[68] = reinterpret_cast<float (*)[68]>(&sa[0][0][0]);
  uint16_t (*th)[68] = reinterpret_cast<uint16_t (*)[68]>(&sb[0][0][0]);
  uint16_t (*tl)[68] = th + 64;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        tile[wa * 32 + i * 16 + (lane >> 4) + 4 * e][wb * 32 + j * 16 + (lane & 15)] =
            static_cast<float>(acc[i][j][e]);
  __syncthreads();
  const int cl = (threadIdx.x & 15) * 4;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int rl = (threadIdx.x >> 4) + 16 * q;
    const int64_t row = i0 + rl;
    const floatx4 v = *reinterpret_cast<const floatx4*>(&tile[rl][cl]);
    *reinterpret_cast<floatx4*>(out + row * a.out.ld + j0 + cl) = v;
    const uint16_t h[4] = {to_bf16_bits(v[0]), to_bf16_bits(v[1]), to_bf16_bits(v[2]), to_bf16_bits(v[3])};
    if (ob) *reinterpret_cast<uint2*>(ob + row * a.out_bf16.ld + j0 + cl) = pack4(h);
    if (a.has_frag) {
      // element (row, k): (((row / 32) * r / 16 + k / 16) * 64 + row % 32 +
      // 32 * (k / 8 % 2)) * 8 + k % 8; k = j0 + cl .. + 3 share one 8-group
      const int k = j0 + cl;
      const int64_t o = (((row >> 5) * (r >> 4) + (k >> 4)) * 64 + (row & 31) + 32 * ((k >> 3) & 1)) * 8 + (k & 7);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(const_cast<void*>(a.frag.p[member])) + o) = pack4(h);
    }
    if (a.has_t) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bf16 bh, bl;
        split_bf16(v[e], bh, bl);
        th[cl + e][rl] = __builtin_bit_cast(uint16_t, bh);
        tl[cl + e][rl] = __builtin_bit_cast(uint16_t, bl);
      }
    }
  }
  if (!a.has_t) return;   // uniform over the grid
  __syncthreads();
  uint16_t* hit = static_cast<uint16_t*>(const_cast<void*>(a.tpiece[0].p[member]));
  uint16_t* lot = static_cast<uint16_t*>(const_cast<void*>(a.tpiece[1].p[member]));
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int j = (threadIdx.x >> 4) + 16 * q;   // row of the transposed tile
    const int i4 = (threadIdx.x & 15) * 4;
    uint16_t hh[4], ll[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      hh[e] = th[j][i4 + e];
      ll[e] = tl[j][i4 + e];
    }
    const int64_t ot = a.t_blocked
        ? (int64_t)((i0 + i4) >> 4) * r * 16 + (int64_t)(j0 + j) * 16 + ((i0 + i4) & 15)
        : (int64_t)(j0 + j) * a.tpiece[0].ld + i0 + i4;
    *reinterpret_cast<uint2*>(hit + ot) = pack4(hh);
    *reinterpret_cast<uint2*>(lot + ot) = pack4(ll);
  }
}

// First-order correction of a nearly orthonormal basis P1: with
// E = P1^T P1 - I (summed from split-K slices), T2 = I - Phi(E)^T where Phi(E)
// is the lower triangle of E with its diagonal halved; T2^T is written (lower
// triangular) so that P = P1 T2 has orthonormal columns up to O(|E|^2) and the
// same positive-diagonal QR basis.
__global__ __launch_bounds__(256) void correction_kernel(const float* part, int64_t part_member_stride,
                                                         int64_t slice, int splits, int r, float* tt,
                                                         int64_t tt_stride) {
  const int member = blockIdx.z;
  const int j = blockIdx.y * 16 + (threadIdx.x >> 4);
  const int k = blockIdx.x * 16 + (threadIdx.x & 15);
  if (j >= r || k >= r) return;
  float v = 0.f;
  if (k <= j) {
    const float* p = part + member * part_member_stride + (int64_t)j * r + k;
    double w = 0.0;
#pragma unroll 8
    for (int s = 0; s < splits; ++s) w += p[s * slice];
    v = k == j ? static_cast<float>(1.0 - 0.5 * (w - 1.0)) : static_cast<float>(-w);
  }
  tt[member * tt_stride + (int64_t)j * r + k] = v;
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
static inline int cdiv(int64_t a, int64_t b) { return static_cast<int>((a + b - 1) / b); }

hipError_t launch_reduce_splits(const RedArgs& a, int members, hipStream_t s) {
  dim3 grid(cdiv(a.cols, 64), cdiv(a.rows, 64), members);
  const bool vec = a.cols % 4 == 0 && a.slice % 4 == 0 && a.part_member_stride % 4 == 0 &&
                   a.out.vec && (reinterpret_cast<uintptr_t>(a.part) & 15) == 0;
  if (vec) hipLaunchKernelGGL(reduce_splits_vec_kernel, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(reduce_splits_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_reduce_pieces(const RedPiecesArgs& a, int members, hipStream_t s) {
  if (a.rows % 64 != 0 || a.cols % 64 != 0 || a.np < 0 || a.np > 3) return hipErrorInvalidValue;
  // (cols % 64 == 0 also covers the fragment order's cols % 16)
  hipLaunchKernelGGL(reduce_pieces_kernel, dim3(a.cols / 64, a.rows / 64, members), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_split_rows(const SplitRowsArgs& a, int members, hipStream_t s) {
  if (a.np != 2 && a.np != 3) return hipErrorInvalidValue;
  dim3 grid(cdiv(a.cols, 64), cdiv(a.rows, 64), members);
  if (a.np == 2) hipLaunchKernelGGL(split_rows_kernel<2>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(split_rows_kernel<3>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_ns_small_poly(const NsSmallPolyArgs& a, int members, hipStream_t s) {
  if (a.M == 128)
    hipLaunchKernelGGL(ns_small_poly_kernel<128>, dim3(members), dim3(256), 0, s, a);
  else if (a.M == 64)
    hipLaunchKernelGGL(ns_small_poly_kernel<64>, dim3(members), dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_muon_momentum(const MuonArgs& a, bool g_bf16, int members, hipStream_t s) {
  dim3 grid(cdiv(a.cols, 1024), a.rows < 65535 ? a.rows : 65535, members);
  if (g_bf16)
    hipLaunchKernelGGL(muon_momentum_kernel<uint16_t>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(muon_momentum_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_muon_update(const MuonArgs& a, bool x_bf16, int members, hipStream_t s) {
  dim3 grid(cdiv(a.cols, 1024), a.rows < 65535 ? a.rows : 65535, members);
  if (x_bf16)
    hipLaunchKernelGGL(muon_update_kernel<uint16_t>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(muon_update_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_row_factors(const RowNormArgs& a, int members, hipStream_t s) {
  if (a.rows < 1) return hipSuccess;
  hipLaunchKernelGGL(row_sumsq_kernel, dim3(a.rows, members), dim3(256), 0, s, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(row_factor_kernel, dim3(members), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_split_sum(const SplitSumArgs& a, int members, hipStream_t s) {
  hipLaunchKernelGGL(split_sum_kernel, dim3(a.cols / 64, a.rows / 64, members), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_split_t(const SplitTArgs& a, int members, hipStream_t s) {
  hipLaunchKernelGGL(split_t_kernel, dim3(a.cols / 64, a.rows / 64, members), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_reduce_colnorm(const RedArgs& a, const ColnormArgs& cn, int members, hipStream_t s) {
  // one workgroup per 64 columns reads all of its slices: only while that is a
  // few loads per thread (at 1024 x 64 with 16 slices it took 40 us longer
  // than the three launches)
  const bool fused = a.rows <= kFusedColnormRows && cdiv(a.rows, 64) * a.splits <= 16 &&
                     a.cols % 4 == 0 && a.slice % 4 == 0 &&
                     a.part_member_stride % 4 == 0 && a.out.vec &&
                     (reinterpret_cast<uintptr_t>(a.part) & 15) == 0 && cn.rows == a.rows &&
                     cn.cols == a.cols && (!cn.has_bf16 || (cn.rb.vec && cn.qb.vec));
  if (!fused) {
    const hipError_t e = launch_reduce_splits(a, members, s);
    if (e != hipSuccess) return e;
    return launch_colnorm(cn, members, s);
  }
  const dim3 grid(cdiv(a.cols, 64), members);
  const int rpt = cdiv(a.rows, 64);
  if (rpt <= 1) hipLaunchKernelGGL(reduce_colnorm_kernel<1>, grid, dim3(1024), 0, s, a, cn);
  else if (rpt <= 2) hipLaunchKernelGGL(reduce_colnorm_kernel<2>, grid, dim3(1024), 0, s, a, cn);
  else if (rpt <= 4) hipLaunchKernelGGL(reduce_colnorm_kernel<4>, grid, dim3(1024), 0, s, a, cn);
  else hipLaunchKernelGGL(reduce_colnorm_kernel<kFusedColnormRows / 64>, grid, dim3(1024), 0, s, a, cn);
  return hipGetLastError();
}

bool small_ortho_reduce_ok(const RedArgs& a) {
  return a.splits > 0 && a.cols % 4 == 0 && a.slice % 4 == 0 && a.part_member_stride % 4 == 0 &&
         (reinterpret_cast<uintptr_t>(a.part) & 15) == 0;
}

hipError_t launch_colnorm(const ColnormArgs& a, int members, hipStream_t s) {
  hipLaunchKernelGGL(colnorm_inv_kernel, dim3(cdiv(a.cols, 64), members), dim3(256), 0, s, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid(cdiv(a.cols, 64), cdiv(a.rows, 64), members);
  hipLaunchKernelGGL(colnorm_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sumsq(const SumsqArgs& a, int nblocks, int members, bool bf16, hipStream_t s) {
  dim3 grid(nblocks, members);
  // 16-byte loads need every row of every member on a 16-byte boundary
  const size_t esz = bf16 ? 2 : 4;
  bool vec = (static_cast<size_t>(a.g.cols) * esz) % 16 == 0 &&
             (static_cast<size_t>(a.g.ld) * esz) % 16 == 0;
  for (int i = 0; i < members && vec; ++i)
    vec = (reinterpret_cast<uintptr_t>(a.g.p[i]) & 15) == 0;
  if (bf16) {
    if (vec) hipLaunchKernelGGL((sumsq_kernel<uint16_t, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((sumsq_kernel<uint16_t, false>), grid, dim3(256), 0, s, a);
  } else {
    if (vec) hipLaunchKernelGGL((sumsq_kernel<float, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((sumsq_kernel<float, false>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_ns_scale(const float* partial, int64_t partial_stride, int nparts, float* scale,
                           int64_t scale_stride, float eps, int members, hipStream_t s) {
  hipLaunchKernelGGL(ns_scale_kernel, dim3(members), dim3(64), 0, s, partial, partial_stride, nparts,
                     scale, scale_stride, eps);
  return hipGetLastError();
}

hipError_t launch_ns_init(const NsInitArgs& a, int members, bool bf16, hipStream_t s) {
  dim3 grid(cdiv(a.N, 64), cdiv(a.M, 64), members);
  if (bf16) hipLaunchKernelGGL(ns_init_kernel<uint16_t>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(ns_init_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_ns_store(const NsInitArgs& a, const MatArg& out, int members, bool bf16,
                           hipStream_t s) {
  dim3 grid(cdiv(a.N, 16), cdiv(a.M, 16), members);
  if (bf16) hipLaunchKernelGGL(ns_store_kernel<uint16_t>, grid, dim3(256), 0, s, a, out);
  else hipLaunchKernelGGL(ns_store_kernel<float>, grid, dim3(256), 0, s, a, out);
  return hipGetLastError();
}

hipError_t launch_correction(const float* part, int64_t part_member_stride, int64_t slice, int splits,
                             int r, float* tt, int64_t tt_stride, int members, hipStream_t s) {
  hipLaunchKernelGGL(correction_kernel, dim3(cdiv(r, 16), cdiv(r, 16), members), dim3(256), 0, s, part,
                     part_member_stride, slice, splits, r, tt, tt_stride);
  return hipGetLastError();
}

hipError_t launch_ns_linear(const NsPolyArgs& a, int members, hipStream_t s) {
  dim3 grid(cdiv(a.M, 16), cdiv(a.M, 16), members);
  hipLaunchKernelGGL(ns_linear_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gram64(const Gram64Args& a, int splits, int members, hipStream_t s) {
  // 128 x 128 tiles where the plan chose them (and split k for them)
  if (a.big && a.r % 128 == 0 && a.kchunk % 32 == 0 && a.p.vec && a.p.ld % 4 == 0) {
    const int tb = a.r / 128;
    dim3 grid(tb * (tb + 1) / 2, splits, members);
    hipLaunchKernelGGL(gram64_big_kernel, grid, dim3(512), 0, s, a);
    return hipGetLastError();
  }
  const int tb = cdiv(a.r, 64);
  dim3 grid(tb * (tb + 1) / 2, splits, members);
  // every tile and k slice whole: m and the slice length multiples of 32
  const bool full = a.r % 64 == 0 && a.kchunk % 32 == 0 && a.m % 32 == 0;
  if (full) hipLaunchKernelGGL(gram64_kernel<true>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(gram64_kernel<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// Cholesky of the scaled Gram, its inverse, and T^T, for every member.
hipError_t launch_cholesky_inverse(const CholArgs& a, float* tt, int64_t tt_stride, int members,
                                   hipStream_t s, double* ttd, int64_t ttd_stride) {
  const int r = a.r, nblk = cdiv(r, 64);
  hipLaunchKernelGGL(chol_prep_kernel, dim3(cdiv(r, 16), cdiv(r, 16), members), dim3(256), 0, s, a);
  // Block 0 is factored on its own; block kb + 1 is factored by the update
  // launch of step kb (its workgroup 0), so each later step is one launch.
  hipLaunchKernelGGL(chol_diag_kernel, dim3(members), dim3(256), 0, s, a, 0);
  for (int kb = 0; kb + 1 < nblk; ++kb) {
    const int T = nblk - kb - 1;
    const int nupd = T * (T + 1) / 2 + T * (kb + 1);
    hipLaunchKernelGGL(chol_update_kernel, dim3(nupd, members), dim3(256), 0, s, a, kb);
  }
  hipLaunchKernelGGL(make_t_kernel, dim3(nblk, nblk, members), dim3(256), 0, s, a, tt, tt_stride,
                     ttd, ttd_stride);
  return hipGetLastError();
}

hipError_t launch_small_ortho(const SmallOrthoArgs& a, int members, hipStream_t s) {
  if (a.ca.r < 1 || a.ca.r > 64 || a.m < 1 || a.m > 256) return hipErrorInvalidValue;
  if (a.splits > 0 && (a.ca.r % 4 != 0 || a.slice % 4 != 0 || a.part_member_stride % 4 != 0 ||
                       (reinterpret_cast<uintptr_t>(a.part) & 15) != 0))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(small_ortho_kernel, dim3(members), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_apply64(const Apply64Args& a, int members, hipStream_t s) {
  if (a.m < 1 || a.r < 1 || a.t == nullptr) return hipErrorInvalidValue;
  // the extra layouts come from whole 64 x 64 tiles, 16-byte aligned rows
  if ((a.has_frag || a.has_t) && (a.m % 64 != 0 || a.r % 64 != 0 || !a.out.vec ||
                                  (a.has_bf16 && !a.out_bf16.vec)))
    return hipErrorInvalidValue;
  const int tiles = cdiv(a.m, 64) * cdiv(a.r, 64);
  hipLaunchKernelGGL(apply64_kernel, dim3(tiles, members), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ortho
