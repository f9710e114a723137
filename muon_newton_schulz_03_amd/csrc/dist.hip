// Distributed-mode ("tensor-parallel") Newton-Schulz on one GPU: the matrix X
// (m x n) is split by columns into P shards X_p (m x n/P). Every shard forms
// its partial Gram X_p X_p^T with the Gram kernel; the partials are summed
// over the shards (an all-reduce of m x m after the first matrix product of
// each iteration) and every shard continues with the full A: B from A
// redundantly, then X_p' = a X_p + B X_p locally. Advancing Emerging
// Optimizers (zh translation, wiki.whaty.org), sections "Distributed mode"
// and "SYRK 和融合的 all-reduce" (a symmetric A needs only its upper triangle
// exchanged).
//
// On one GPU the exchange is simulated: tri_pack writes each shard's upper
// triangle as a packed float32 buffer (row i holds columns i .. mp - 1,
// starting at i mp - i (i - 1) / 2): the message a rank would send.
// tri_reduce sums the P packed buffers of a matrix in shard order (the
// all-reduce, in a fixed order) and unpacks the sum into every shard's A,
// mirrored, as bf16 hi + lo (or float32), in 64 x 64 tiles.
#include <hip/hip_runtime.h>

#include "kernels.h"
#include "layout.h"

namespace muon {
namespace {


__device__ inline int64_t tri_row(int64_t i, int64_t mp) { return i * mp - i * (i - 1) / 2; }

// Element offset of A[i][j] in the workspace: k-blocked for bf16, row-major
// for float32.
template <typename T>
__device__ inline int64_t aoff(int64_t i, int64_t j, int64_t mp) {
  return sizeof(T) == 2 ? kblk(i, j, mp) : i * mp + j;
}

__device__ inline void locate(const GemmArgs &a, int b, int *seg, int *view, int *row) {
  int s = 0;
  while (s + 1 < a.nseg && b >= a.seg[s + 1].tile_begin) ++s;
  const int u = b - a.seg[s].tile_begin;
  *seg = s;
  *view = u / a.seg[s].tiles_per_view;
  *row = u - *view * a.seg[s].tiles_per_view;
}

// one workgroup per (view, row i): T[i][j] for j >= i
template <typename T>
__global__ __launch_bounds__(256) void tri_pack_kernel(const GemmArgs args) {
  int s, v, i;
  locate(args, int(blockIdx.x), &s, &v, &i);
  const GemmSeg &S = args.seg[s];
  char *blk = S.base + int64_t(v) * S.stride;
  const int mp = S.mp;
  float *tri = reinterpret_cast<float *>(blk + S.off_tri) + tri_row(i, mp) - i;
  const T *hi = reinterpret_cast<const T *>(blk + S.off_ahi);
  const T *lo = reinterpret_cast<const T *>(blk + S.off_alo);
  for (int j = i + int(threadIdx.x); j < mp; j += 256) {
    const int64_t a = aoff<T>(i, j, mp);
    float x = float(hi[a]);
    if (sizeof(T) == 2) x += float(lo[a]);
    tri[j] = x;
  }
}

// One workgroup per 64 x 64 tile (I <= J) of a matrix's upper triangle: the
// packed tiles of its `group` shards are summed in shard order, written to
// every shard's A at (I, J) row by row, and through an LDS transpose at
// (J, I), so that every global write is a contiguous row run.
template <typename T>
__global__ __launch_bounds__(256) void tri_reduce_kernel(const GemmArgs args) {
  __shared__ float tile[64][65];
  const int G = args.group, b = int(blockIdx.x), tid = int(threadIdx.x);
  int s = 0;
  while (s + 1 < args.nseg && b >= args.seg[s + 1].tile_begin) ++s;
  const GemmSeg &S = args.seg[s];
  const int mp = S.mp;
  const int u = b - S.tile_begin, mat = u / S.tiles_per_view;
  int t = u - mat * S.tiles_per_view;
  int J = int((sqrtf(8.f * float(t) + 1.f) - 1.f) * 0.5f);
  while ((J + 1) * (J + 2) / 2 <= t) ++J;
  while (J * (J + 1) / 2 > t) --J;
  const int I = t - J * (J + 1) / 2;
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
      for (int g = 0; g < G; ++g) {
        char *blk = blk0 + int64_t(g) * S.stride;
        reinterpret_cast<T *>(blk + S.off_ahi)[aoff<T>(i, j, mp)] = T(x);
        if (sizeof(T) == 2) reinterpret_cast<T *>(blk + S.off_alo)[aoff<T>(i, j, mp)] = T(x - float(T(x)));
      }
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
    for (int g = 0; g < G; ++g) {
      char *blk = blk0 + int64_t(g) * S.stride;
      reinterpret_cast<T *>(blk + S.off_ahi)[aoff<T>(j, i, mp)] = T(x);
      if (sizeof(T) == 2) reinterpret_cast<T *>(blk + S.off_alo)[aoff<T>(j, i, mp)] = T(x - float(T(x)));
    }
  }
}

int total_rows(const GemmArgs &a) {
  int64_t t = 0;
  for (int s = 0; s < a.nseg; ++s) t += int64_t(a.seg[s].tiles_per_view) * a.seg[s].count;
  return int(t);
}

}  // namespace

hipError_t launch_tri_pack(const GemmArgs &a, bool bf16, hipStream_t s) {
  const int rows = total_rows(a);
  if (rows <= 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(tri_pack_kernel<__bf16>, dim3(rows), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(tri_pack_kernel<float>, dim3(rows), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_tri_reduce(const GemmArgs &a, bool bf16, hipStream_t s) {
  int64_t tiles = 0;  // 64 x 64 tiles of the matrices' upper triangles
  for (int k = 0; k < a.nseg; ++k) tiles += int64_t(a.seg[k].tiles_per_view) * (a.seg[k].count / a.group);
  const int rows = int(tiles);
  if (rows <= 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(tri_reduce_kernel<__bf16>, dim3(rows), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(tri_reduce_kernel<float>, dim3(rows), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace muon
