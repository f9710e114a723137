// Distributed-mode ("tensor-parallel") Newton-Schulz on one GPU: the matrix X
// (m x n) is split by columns into P shards X_p (m x n/P). Every shard forms
// its partial Gram X_p X_p^T with the Gram kernel; the partials are summed
// over the shards (an all-reduce of m x m after the first matrix product of
// each iteration) and every shard continues with the full A: B from A
// redundantly, then X_p' = a X_p + B X_p locally. Advancing Emerging
// Optimizers (zh translation, wiki.whaty.org), sections "Distributed mode"
// and "SYRK 和融合的 all-reduce" (a symmetric A needs only its upper triangle
// exchanged, and the exchange can follow the SYRK tile by tile).
//
// On one GPU the exchange is simulated. bf16 path: the Gram kernel's
// epilogue writes each shard's partial as float32 upper-triangle tiles
// (tile-packed, layout.h), the message a rank would send, straight from its
// accumulators; tile_sum sums the P messages of a matrix tile by tile in
// shard order (the all-reduce, in a fixed order) with 16-byte loads and
// writes the sum as the bf16 A (hi, and lo when A*A needs it) of the
// matrix's first shard, mirrored, which every shard's A*A then reads (on P
// ranks each would hold the same A). float32 path: tri_pack writes each
// shard's upper triangle as packed rows (row i holds columns i .. mp - 1,
// starting at i mp - i (i - 1) / 2) and tri_reduce sums them into every
// shard's A in 64 x 64 tiles.
#include <hip/hip_runtime.h>

#include "kernels.h"
#include "layout.h"

namespace muon {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline int64_t tri_row(int64_t i, int64_t mp) { return i * mp - i * (i - 1) / 2; }

// upper-triangle tile t, column by column: t = J (J + 1) / 2 + I, I <= J
__device__ inline void upper_tile(int t, int *I, int *J) {
  int j = int((sqrtf(8.f * float(t) + 1.f) - 1.f) * 0.5f);
  while ((j + 1) * (j + 2) / 2 <= t) ++j;
  while (j * (j + 1) / 2 > t) --j;
  *J = j;
  *I = t - j * (j + 1) / 2;
}

__device__ inline void locate(const GemmArgs &a, int b, int *seg, int *view, int *row) {
  int s = 0;
  while (s + 1 < a.nseg && b >= a.seg[s + 1].tile_begin) ++s;
  const int u = b - a.seg[s].tile_begin;
  *seg = s;
  *view = u / a.seg[s].tiles_per_view;
  *row = u - *view * a.seg[s].tiles_per_view;
}

// float32: one workgroup per (view, row i): T[i][j] for j >= i
__global__ __launch_bounds__(256) void tri_pack_kernel(const GemmArgs args) {
  int s, v, i;
  locate(args, int(blockIdx.x), &s, &v, &i);
  const GemmSeg &S = args.seg[s];
  char *blk = S.base + int64_t(v) * S.stride;
  const int mp = S.mp;
  float *tri = reinterpret_cast<float *>(blk + S.off_tri) + tri_row(i, mp) - i;
  const float *a = reinterpret_cast<const float *>(blk + S.off_ahi) + int64_t(i) * mp;
  for (int j = i + int(threadIdx.x); j < mp; j += 256) tri[j] = a[j];
}

// float32: one workgroup per 64 x 64 tile (I <= J) of a matrix's upper
// triangle: the packed tiles of its `group` shards are summed in shard order,
// written to every shard's A at (I, J) row by row, and through an LDS
// transpose at (J, I), so that every global write is a contiguous row run.
__global__ __launch_bounds__(256) void tri_reduce_kernel(const GemmArgs args) {
  __shared__ float tile[64][65];
  const int G = args.group, b = int(blockIdx.x), tid = int(threadIdx.x);
  int s = 0;
  while (s + 1 < args.nseg && b >= args.seg[s + 1].tile_begin) ++s;
  const GemmSeg &S = args.seg[s];
  const int mp = S.mp;
  const int u = b - S.tile_begin, mat = u / S.tiles_per_view;
  int I, J;
  upper_tile(u - mat * S.tiles_per_view, &I, &J);
  const int i0 = I * 64, j0 = J * 64;
  char *blk0 = S.base + int64_t(mat) * G * S.stride;
  const int c = tid & 63;
#pragma unroll 4
  for (int k = 0; k < 16; ++k) {
    const int r = (tid >> 6) + 4 * k, i = i0 + r, j = j0 + c;
    float x = 0.f;
    if (j >= i) {
      const int64_t idx = tri_row(i, mp) + (j - i);
      for (int g = 0; g < G; ++g) x += reinterpret_cast<const float *>(blk0 + int64_t(g) * S.stride + S.off_tri)[idx];
      for (int g = 0; g < G; ++g)
        reinterpret_cast<float *>(blk0 + int64_t(g) * S.stride + S.off_ahi)[int64_t(i) * mp + j] = x;
    }
    tile[r][c] = x;
  }
  __syncthreads();
  // mirror: A[j][i] for j > i, rows j of the tile (J, I)
#pragma unroll 4
  for (int k = 0; k < 16; ++k) {
    const int rj = (tid >> 6) + 4 * k, j = j0 + rj, i = i0 + c;
    if (j <= i) continue;
    const float x = tile[c][rj];
    for (int g = 0; g < G; ++g)
      reinterpret_cast<float *>(blk0 + int64_t(g) * S.stride + S.off_ahi)[int64_t(j) * mp + i] = x;
  }
}

// bf16: one workgroup per quarter (64 rows) of an upper 256 x 256 tile
// (I <= J) of a matrix. Its `group` shards' float32 partials (tile-packed:
// the quarter is 64 KiB in one piece) are summed in shard order, 16 bytes
// per load, and staged in LDS as bf16 hi and lo; then the quarter's rows of
// tile (I, J) and its columns of the mirror tile (J, I) leave as 16-byte
// runs of the first shard's k-blocked A (consecutive threads: consecutive
// 16-byte pieces of one 256 x 32 block). A diagonal tile is symmetrized:
// element (r, c) takes the sum at (min(r, c), max(r, c)); the quarter's row
// runs cover the upper part and the runs that cross the diagonal, its
// column runs the lower part below them.
constexpr int kSumPitch = 264;  // bf16 per staged row: 256 + 8, rows stay 16-byte aligned

// TWO: A's lo half too (the A*A from hi + lo); otherwise hi alone, and half
// the LDS.
template <bool TWO>
__global__ __launch_bounds__(256) void tile_sum_kernel(const GemmArgs args) {
  __shared__ __attribute__((aligned(16))) __bf16 hi[64 * kSumPitch];
  __shared__ __attribute__((aligned(16))) __bf16 lo[TWO ? 64 * kSumPitch : 8];
  const int G = args.group, b = int(blockIdx.x), tid = int(threadIdx.x);
  int s = 0;
  while (s + 1 < args.nseg && b >= args.seg[s + 1].tile_begin) ++s;
  const GemmSeg &S = args.seg[s];
  const int mp = S.mp;
  const int u = b - S.tile_begin, mat = u / S.tiles_per_view;
  const int t = u - mat * S.tiles_per_view, quarter = t & 3;
  int I, J;
  upper_tile(t >> 2, &I, &J);
  const int i0 = I * 256, j0 = J * 256, q0 = quarter * 64;
  char *blk0 = S.base + int64_t(mat) * G * S.stride;

  // sum: float4 f of the quarter (16 per thread) holds rows 4 .. 4 + 3 of a
  // column, at float offset 4 f from the quarter's start
  const float *src = reinterpret_cast<const float *>(blk0 + S.off_tri) + int64_t(t >> 2) * kTriTileFloats + q0 * 256;
  f32x4 acc[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int g = 0; g < G; ++g) {
    const f32x4 *p = reinterpret_cast<const f32x4 *>(src + int64_t(g) * (S.stride / 4));
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] += p[tid + 256 * k];
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int f = tid + 256 * k;
    const int blk = f >> 8, w = f & 255;  // block of the quarter (2 x 8), quad and column within it
    const int r = (blk >> 3) * 32 + (w >> 5) * 4, c = (blk & 7) * 32 + (w & 31);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const __bf16 h = __bf16(acc[k][e]);
      hi[(r + e) * kSumPitch + c] = h;
      if (TWO) lo[(r + e) * kSumPitch + c] = __bf16(acc[k][e] - float(h));
    }
  }
  __syncthreads();

  const bool diag = I == J;
  __bf16 *Ah = reinterpret_cast<__bf16 *>(blk0 + S.off_ahi);
  __bf16 *Al = reinterpret_cast<__bf16 *>(blk0 + S.off_alo);
  // rows q0 + rl of tile (I, J): thread -> (32-column block k, row tid / 4, 8-column piece tid % 4)
  const int rl = tid >> 2, piece = tid & 3;
#pragma unroll 2
  for (int k = 0; k < 8; ++k) {
    const int r = q0 + rl, c0 = k * 32 + piece * 8;
    if (diag && c0 + 7 < r) continue;  // below the diagonal: a column run's
    const int64_t o = kblk(i0 + r, j0 + c0, mp);
    if (!diag || c0 >= r) {
      *reinterpret_cast<u32x4 *>(Ah + o) = *reinterpret_cast<const u32x4 *>(hi + rl * kSumPitch + c0);
      if (TWO) *reinterpret_cast<u32x4 *>(Al + o) = *reinterpret_cast<const u32x4 *>(lo + rl * kSumPitch + c0);
    } else {  // the run that crosses the diagonal: columns c < r come from row c of this quarter
      bf16x8 vh, vl;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = c0 + e;
        const int at = c >= r ? rl * kSumPitch + c : (c - q0) * kSumPitch + r;
        vh[e] = hi[at];
        if (TWO) vl[e] = lo[at];
      }
      *reinterpret_cast<bf16x8 *>(Ah + o) = vh;
      if (TWO) *reinterpret_cast<bf16x8 *>(Al + o) = vl;
    }
  }
  // columns q0 + 8 a .. + 7 of the mirror tile (J, I), row j0 + c:
  // thread -> (32-column block k / 4, row (k mod 4) 64 + tid / 4, piece tid % 4)
#pragma unroll 2
  for (int k = 0; k < 8; ++k) {
    const int a = (k >> 2) * 4 + piece, c = (k & 3) * 64 + rl;
    if (diag && c < q0 + 8 * a + 8) continue;  // not entirely below the diagonal
    bf16x8 vh, vl;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      vh[e] = hi[(8 * a + e) * kSumPitch + c];
      if (TWO) vl[e] = lo[(8 * a + e) * kSumPitch + c];
    }
    const int64_t o = kblk(j0 + c, i0 + q0 + 8 * a, mp);
    *reinterpret_cast<bf16x8 *>(Ah + o) = vh;
    if (TWO) *reinterpret_cast<bf16x8 *>(Al + o) = vl;
  }
}

// workgroups of a launch with tiles_per_view per view, or per matrix
int total_rows(const GemmArgs &a) {
  int64_t t = 0;
  for (int s = 0; s < a.nseg; ++s) t += int64_t(a.seg[s].tiles_per_view) * a.seg[s].count;
  return int(t);
}
int total_per_matrix(const GemmArgs &a) {
  int64_t t = 0;
  for (int s = 0; s < a.nseg; ++s) t += int64_t(a.seg[s].tiles_per_view) * (a.seg[s].count / a.group);
  return int(t);
}

}  // namespace

hipError_t launch_tile_sum(const GemmArgs &a, hipStream_t s) {
  const int blocks = total_per_matrix(a);
  if (blocks <= 0) return hipSuccess;
  if (a.gram_halves > 1)
    hipLaunchKernelGGL(tile_sum_kernel<true>, dim3(blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(tile_sum_kernel<false>, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_tri_pack(const GemmArgs &a, hipStream_t s) {
  const int rows = total_rows(a);
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(tri_pack_kernel, dim3(rows), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_tri_reduce(const GemmArgs &a, hipStream_t s) {
  const int tiles = total_per_matrix(a);  // 64 x 64 tiles of the matrices' upper triangles
  if (tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(tri_reduce_kernel, dim3(tiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace muon
