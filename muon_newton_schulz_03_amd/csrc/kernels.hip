// HIP kernels of the Muon step for CDNA4 (gfx950).
//
// Per group of views (whole matrices or column blocks), in stream order:
//   elem_kernel (prep)      momentum M <- beta M + G, Newton-Schulz source X0
//                           written zero-padded into the workspace in wide
//                           orientation (and transposed, X0^T, for the bf16
//                           B X), per-tile partial sums of squares.
//   norm_finalize_kernel    s = 1/(||X0||_F + eps) from the partial sums.
//   iters x { gemm <Gram>   A = s' X X^T (upper-triangle tiles, mirrored),
//                           stored as bf16 (hi, and lo when needed);
//             gemm <AA>     B = b A + c A A (upper tiles, mirrored), A A from
//                           bf16(A), or from hi*hi + hi*lo + lo*hi;
//             gemm <BX>     X' = s'' (a X + B X), written as X' and X'^T;
//                           the last one writes the caller's matrix instead:
//                           data <- O, or W <- W - lr O }
//   elem_kernel (finish)    only for zero iterations: data <- s X0, or
//                           W <- W - lr s X0.
// s' = s^2 and s'' = s in the first iteration (the normalization is folded
// into the first Gram and the first B X), 1 afterwards.
//
// Three products per iteration, the first two symmetric rank-k products
// (SYRK) with only upper-triangle tiles computed and the diagonal tiles in
// full, the result stored as a full matrix: Advancing Emerging Optimizers
// (zh translation, wiki.whaty.org), sections "Distributed mode" and
// "SYRK 和融合的 all-reduce".
//
// All three are "NT" contractions C[i][j] = sum_k P[i][k] Q[j][k] over
// K-contiguous rows: of X (Gram), of the symmetric A (A*A), of the symmetric
// B and of X^T (B X). X is kept in both orientations, each written once per
// iteration, so no product needs transposing LDS reads (in a probe of the K
// loop on gfx950 they took it from 68% to 51% of the clock-scaled peak). The
// bf16 operands are stored k-blocked (layout.h), so each K step of an operand
// tile is one contiguous 16 KiB block.
#include <hip/hip_runtime.h>

#include <utility>

#include "kernels.h"
#include "layout.h"

namespace muon {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// tile bookkeeping
// ---------------------------------------------------------------------------

// Workgroups are handed to the 8 XCDs round-robin (workgroup w runs on XCD
// w % 8). Give each XCD a contiguous range of tiles instead, so the tiles of
// one matrix share that XCD's L2.
__device__ inline int xcd_remap(int w, int total) {
  const int x = w & 7, j = w >> 3;
  const int q = total >> 3, r = total & 7;
  return x * q + min(x, r) + j;
}

struct TileInfo {
  int seg, view, I, J;
};

__device__ inline TileInfo decode_tile(const GemmArgs &a, int tile, bool syrk) {
  int s = 0;
  while (s + 1 < a.nseg && tile >= a.seg[s + 1].tile_begin) ++s;
  const GemmSeg &S = a.seg[s];
  int u = tile - S.tile_begin;
  const int view = u / S.tiles_per_view;
  u -= view * S.tiles_per_view;
  int I, J;
  if (syrk) {
    // upper-triangle tiles (I <= J) of the t x t grid. Up to 8 panels (36
    // tiles, about one XCD's worth): column by column, u = J (J + 1) / 2 + I.
    // Beyond: in bands of 8 column panels (band b: J in [8 b, 8 b + w)),
    // within a band row by row, each row's J >= I ascending, so that 32
    // consecutive tiles cover about 4 row panels x 8 column panels instead
    // of up to 32 + 2 panels (Kimi dense A*A and Gram: +1.1% per step)
    const int t = S.mp / (S.np / S.tn);
    if (t <= 8) {
      J = int((sqrtf(8.f * float(u) + 1.f) - 1.f) * 0.5f);
      while ((J + 1) * (J + 2) / 2 <= u) ++J;
      while (J * (J + 1) / 2 > u) --J;
      I = u - J * (J + 1) / 2;
      return {s, view, I, J};
    }
    int c0 = 0;
    while (c0 + 8 < t && u >= (c0 + 8) * (c0 + 9) / 2) c0 += 8;
    const int w = min(8, t - c0);
    int v = u - c0 * (c0 + 1) / 2;
    if (v < c0 * w) {
      I = v / w;
      J = c0 + v % w;
    } else {
      v -= c0 * w;
      int i = 0;
      while (v >= w - i) v -= w - i++;
      I = c0 + i;
      J = I + v;
    }
  } else {
    // B X tiles go in bands of up to 8 row panels, column by column within a
    // band: 32 consecutive tiles, one XCD's worth, then cover 8 row panels x
    // 4 column panels and share 8 panels of B and 4 of X^T in that XCD's L2
    // (a matrix with at most 8 row panels is one band, column by column)
    const int tJ = S.tn, tI = S.mp / (S.np / tJ);
    const int band = u / (8 * tJ), r0 = 8 * band, rows = min(8, tI - r0);
    const int r = u - band * 8 * tJ;
    I = r0 + r % rows;
    J = r / rows;
  }
  return {s, view, I, J};
}

// ---------------------------------------------------------------------------
// element-wise kernels: prep (momentum + source + layouts + partial norms)
// and finish (write-back / weight update). 64x64 tiles, 256 threads.
// ---------------------------------------------------------------------------

template <typename T>
struct alignas(16) Vec16 {
  T e[16 / sizeof(T)];
};

template <typename T>
__device__ inline void load_row_chunk(const void *base, int64_t ld, int gr, int gc, int rows, int cols,
                                      bool vec, float *out) {
  constexpr int V = 16 / sizeof(T);
  const T *p = static_cast<const T *>(base) + int64_t(gr) * ld + gc;
  if (vec && gr < rows && gc + V <= cols) {
    const Vec16<T> v = *reinterpret_cast<const Vec16<T> *>(p);
#pragma unroll
    for (int e = 0; e < V; ++e) out[e] = float(v.e[e]);
  } else {
#pragma unroll
    for (int e = 0; e < V; ++e) out[e] = (gr < rows && gc + e < cols) ? float(p[e]) : 0.f;
  }
}

template <typename T>
__device__ inline void store_row_chunk(void *base, int64_t ld, int gr, int gc, int rows, int cols,
                                       bool vec, const float *in) {
  constexpr int V = 16 / sizeof(T);
  T *p = static_cast<T *>(base) + int64_t(gr) * ld + gc;
  if (gr >= rows) return;
  if (vec && gc + V <= cols) {
    Vec16<T> v;
#pragma unroll
    for (int e = 0; e < V; ++e) v.e[e] = T(in[e]);
    *reinterpret_cast<Vec16<T> *>(p) = v;
  } else {
#pragma unroll
    for (int e = 0; e < V; ++e)
      if (gc + e < cols) p[e] = T(in[e]);
  }
}

// Element offset of (r, c) in the workspace copy of X or X^T: k-blocked for
// bf16 (the MFMA operands), row-major for float32.
template <typename T>
__device__ inline int64_t xoff(int64_t r, int64_t c, int64_t pitch) {
  return sizeof(T) == 2 ? kblk(r, c, pitch) : r * pitch + c;
}

template <typename T>
__global__ __launch_bounds__(256) void elem_kernel(const ElemArgs args) {
  constexpr int V = 16 / sizeof(T);      // elements per 16-byte chunk
  constexpr int CPR = 64 / V;            // chunks per 64-element row
  constexpr int CPT = 64 * CPR / 256;    // chunks per thread
  __shared__ T tile[64][64 + 2];
  __shared__ float red[4];
  // kElemTilesPerGroup consecutive tiles per workgroup (a quarter of the
  // workgroups of one per tile: prep -8% on the Kimi batch)
  const int b_end = min(args.total_tiles, (int(blockIdx.x) + 1) * kElemTilesPerGroup);
  for (int b = int(blockIdx.x) * kElemTilesPerGroup; b < b_end; ++b) {
  __syncthreads();  // the previous tile's LDS readers are done
  const int tid = threadIdx.x;
  int vi = 0;
  while (vi + 1 < args.nv && b >= args.v[vi + 1].tile_begin) ++vi;
  const ElemView &Vw = args.v[vi];
  const int u = b - Vw.tile_begin;
  const int tr = u / Vw.tiles_c, tc = u - (u / Vw.tiles_c) * Vw.tiles_c;
  const int kind = args.kind;

  T *X = reinterpret_cast<T *>(Vw.blk + Vw.off_x);
  const int64_t px = Vw.pitch_x;
  if ((kind == kPrepNs || kind == kPrepStep) && u == 0 && tid == 0) {
    // where the last B X writes this view's result
    OutDesc od{};
    od.out = kind == kPrepStep ? Vw.w : Vw.m;
    od.ld = kind == kPrepStep ? Vw.ld_w : Vw.ld_m;
    od.rows = Vw.rows;
    od.cols = Vw.cols;
    od.tall = Vw.tall;
    od.update = kind == kPrepStep ? 1 : 0;
    od.vec = (reinterpret_cast<uintptr_t>(od.out) % 8 == 0 && (od.ld * int64_t(sizeof(T))) % 8 == 0) ? 1 : 0;
    *reinterpret_cast<OutDesc *>(Vw.blk + Vw.off_scale + kOutDescOffset) = od;
  }
  if (kind == kPrepNs || kind == kPrepStep) {
    // X0 in wide orientation and, when a bf16 B X will read it, X0^T: the
    // user's tile goes to one of them row by row and to the other transposed
    // through the LDS tile (wide view: X rows, X^T transposed; tall view:
    // X^T rows, X transposed)
    T *XT = Vw.off_xt >= 0 ? reinterpret_cast<T *>(Vw.blk + Vw.off_xt) : nullptr;
    T *Dd = Vw.tall ? XT : X, *Dt = Vw.tall ? X : XT;
    const int64_t pd = Vw.tall ? int64_t(Vw.pitch_xt) : px, pt = Vw.tall ? px : int64_t(Vw.pitch_xt);
    float ss = 0.f;
    // every chunk's loads first (the M stores below may alias them as far as
    // the compiler knows, so it would not move a later chunk's loads above
    // them): CPT chunks of G and of M in flight per thread
    float g[CPT][V], m[CPT][V];
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int c = tid + 256 * q, row = c / CPR, cc = c % CPR;
      const int gr = tr * 64 + row, gc = tc * 64 + cc * V;
      if (kind == kPrepStep) load_row_chunk<T>(Vw.g, Vw.ld_g, gr, gc, Vw.rows, Vw.cols, Vw.vec & 1, g[q]);
      load_row_chunk<T>(Vw.m, Vw.ld_m, gr, gc, Vw.rows, Vw.cols, Vw.vec & 2, m[q]);
    }
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int c = tid + 256 * q, row = c / CPR, cc = c % CPR;
      const int gr = tr * 64 + row, gc = tc * 64 + cc * V;
      float x[V];
      if (kind == kPrepStep) {
#pragma unroll
        for (int e = 0; e < V; ++e) m[q][e] = fmaf(args.beta, m[q][e], g[q][e]);
        store_row_chunk<T>(Vw.m, Vw.ld_m, gr, gc, Vw.rows, Vw.cols, Vw.vec & 2, m[q]);
#pragma unroll
        for (int e = 0; e < V; ++e) x[e] = args.nesterov ? fmaf(args.beta, m[q][e], g[q][e]) : m[q][e];
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e) x[e] = m[q][e];
      }
      Vec16<T> xv;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        xv.e[e] = T(x[e]);
        const float xf = float(xv.e[e]);
        ss = fmaf(xf, xf, ss);
        tile[row][cc * V + e] = xv.e[e];
      }
      if (Dd) *reinterpret_cast<Vec16<T> *>(Dd + xoff<T>(gr, gc, pd)) = xv;
    }
    if (Dt) {
      __syncthreads();
#pragma unroll
      for (int q = 0; q < CPT; ++q) {
        const int c = tid + 256 * q, trow = c / CPR, tcc = c % CPR;
        Vec16<T> tv;
#pragma unroll
        for (int e = 0; e < V; ++e) tv.e[e] = tile[tcc * V + e][trow];
        *reinterpret_cast<Vec16<T> *>(Dt + xoff<T>(tc * 64 + trow, tr * 64 + tcc * V, pt)) = tv;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    if (tid == 0) reinterpret_cast<float *>(Vw.blk + Vw.off_part)[u] = (red[0] + red[1]) + (red[2] + red[3]);
  } else {
    const float sf = args.final_scale ? reinterpret_cast<const float *>(Vw.blk + Vw.off_scale)[0] : 1.f;
    if (Vw.tall) {
      // the user's tile (tr, tc) is X[tc*64 .., tr*64 ..] transposed: stage
      // that block of X in LDS with coalesced row reads (inside the padded
      // extent of X, so no bounds checks)
#pragma unroll
      for (int q = 0; q < CPT; ++q) {
        const int c = tid + 256 * q, row = c / CPR, cc = c % CPR;
        const Vec16<T> v = *reinterpret_cast<const Vec16<T> *>(X + xoff<T>(tc * 64 + row, tr * 64 + cc * V, px));
#pragma unroll
        for (int e = 0; e < V; ++e) tile[row][cc * V + e] = v.e[e];
      }
      __syncthreads();
    }
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int c = tid + 256 * q, row = c / CPR, cc = c % CPR;
      const int gr = tr * 64 + row, gc = tc * 64 + cc * V;
      if (gr >= Vw.rows || gc >= Vw.cols) continue;
      float o[V];
      if (Vw.tall) {
#pragma unroll
        for (int e = 0; e < V; ++e) o[e] = float(tile[cc * V + e][row]) * sf;
      } else {
        const Vec16<T> ov = *reinterpret_cast<const Vec16<T> *>(X + xoff<T>(gr, gc, px));
#pragma unroll
        for (int e = 0; e < V; ++e) o[e] = float(ov.e[e]) * sf;
      }
      if (kind == kFinishNs) {
        store_row_chunk<T>(Vw.m, Vw.ld_m, gr, gc, Vw.rows, Vw.cols, Vw.vec & 2, o);
      } else {
        float w[V];
        load_row_chunk<T>(Vw.w, Vw.ld_w, gr, gc, Vw.rows, Vw.cols, Vw.vec & 4, w);
#pragma unroll
        for (int e = 0; e < V; ++e) w[e] = fmaf(-args.lr, o[e], w[e]);
        store_row_chunk<T>(Vw.w, Vw.ld_w, gr, gc, Vw.rows, Vw.cols, Vw.vec & 4, w);
      }
    }
  }
  }  // tiles of this workgroup
}

// s = 1 / (||X0||_F + eps) from the per-tile partial sums, summed in a fixed
// order in double precision. One workgroup per matrix: its `group`
// consecutive views (1, or the shards of a distributed matrix, whose norm is
// that of the whole matrix) all receive the same scale.
__global__ __launch_bounds__(256) void norm_finalize_kernel(const GemmArgs args) {
  __shared__ double red[256];
  const int vg = int(blockIdx.x) * args.group, tid = threadIdx.x;
  int s = 0;
  while (s + 1 < args.nseg && vg >= args.seg[s + 1].view_begin) ++s;
  const GemmSeg &S = args.seg[s];
  double acc = 0.0;
  for (int g = 0; g < args.group; ++g) {
    const float *part = reinterpret_cast<const float *>(S.base + int64_t(vg + g - S.view_begin) * S.stride + S.off_part);
    for (int i = tid; i < S.nparts; i += 256) acc += double(part[i]);
  }
  red[tid] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid < args.group) {
    const double sc = 1.0 / (sqrt(red[0]) + double(args.eps));
    float *scale = reinterpret_cast<float *>(S.base + int64_t(vg + tid - S.view_begin) * S.stride + S.off_scale);
    scale[0] = float(sc);
    scale[1] = float(sc * sc);
  }
}

// ---------------------------------------------------------------------------
// bf16 matrix-core kernel: 256x256 output tile, 8 waves (two per SIMD), wave
// w covering rows 128 wm and columns 64 wn as 4x2 blocks of
// v_mfma_f32_32x32x16_bf16 (128 accumulators: two waves per SIMD leave each
// wave 256 registers).
//
// Operands stream through a 5-stage LDS ring (stage = 256 rows x 32 k of
// both operands, 2 x 16 KiB; 160 KiB in all). Global memory goes straight to
// LDS with buffer_load_dwordx4 ... lds (each lane's 16 bytes land at LDS base
// + 16 * lane), issued by waves 0..3 only, three K steps ahead, so no
// registers hold staged data and the load latency hides behind three steps
// of matrix work. One barrier per K step: after it, stage ks is visible to
// every wave and the stage of step ks - 2 is free for the loads of step
// ks + 3. The operands are k-blocked (layout.h): each K step of an operand
// tile is one contiguous 16 KiB block.
//
// A 64-byte LDS row holds four 16-byte chunks of k, XOR-swizzled by
// ((row >> 2) & 3): the 16 lanes of a fragment-read group (16 consecutive
// rows, one logical chunk) then hit 16 distinct 4-bank groups of the 64 banks.
//
// MFMA 32x32x16 register layout: lane l supplies row (l & 31) of the A
// operand and column (l & 31) of the B operand, each as 8 consecutive k
// (k half selected by l >> 5; any k permutation shared by both operands
// gives the same sum). Accumulator register r of lane l holds
// C[8 (r >> 2) + 4 (l >> 5) + (r & 3)][l & 31].
// ---------------------------------------------------------------------------

constexpr int kBM = 256, kBK = 32, kStages = 5;
constexpr int kOpBytes = kBM * kBK * 2;          // one operand tile, one stage (16 KiB)
constexpr int kStageBytes = 2 * kOpBytes;        // both operands
constexpr int kWaves = 8;                        // two per SIMD
constexpr int kThreads = kWaves * 64;
constexpr int kBN = 2;                           // 32-column accumulator blocks per wave (wave tile 128 x 64)
constexpr int kLoaders = 4;                      // waves 0..3, one per SIMD, issue every operand load
constexpr int kBxRot = 1;                         // B X: K-loop offset per row tile, in K steps

// ---------------------------------------------------------------------------
// Epilogues. After the K loop the LDS ring holds one 256 x 256 bf16 (128 KiB)
// tile: 512-byte rows whose 16-byte chunks are XOR-swizzled by
// row ^ ((row & 3) << 2) (mod 32), which spreads both 32 consecutive rows at
// one column and 4 consecutive rows at 8 consecutive columns over the banks.
// Accumulators go to that tile in whichever orientation a pass needs, and the
// tile then leaves as coalesced 16-byte row stores.
// ---------------------------------------------------------------------------

__device__ inline int tile_chunk(int row, int c) { return (c ^ row ^ ((row & 3) << 2)) & 31; }
__device__ inline int tile_off(int row, int col) {
  return row * 512 + (tile_chunk(row, col >> 3) << 4) + (col & 7) * 2;
}

// Calls f(acc[bi][bj], bi, bj) for the 4 x kBN accumulator blocks of a wave
// with compile-time indices, so the accumulators stay in registers.
template <class F, int... N>
__device__ inline void for_blocks(f32x16 (&acc)[4][kBN], F &&f, std::integer_sequence<int, N...>) {
  (f(acc[N / kBN][N % kBN], N / kBN, N % kBN), ...);
}
template <class F>
__device__ inline void for_blocks(f32x16 (&acc)[4][kBN], F &&f) {
  for_blocks(acc, f, std::make_integer_sequence<int, 4 * kBN>{});
}

// The LDS tile -> the 256 x 256 tile at (row0, col0) of a k-blocked matrix
// with `cols` columns: 8 consecutive 16 KiB blocks, written in order (each
// wave instruction stores 1 KiB: 16 rows x 64 bytes of one block). Within a
// 16-lane group the 4 rows x 4 chunks read from LDS fall in 16 distinct
// 16-byte bank slots of the swizzle.
__device__ inline void tile_store(const char *smem, bf16 *dst, int64_t cols, int row0, int col0, int tid) {
  bf16 *d = dst + kblk(row0, col0, cols);
#pragma unroll 8
  for (int k = 0; k < 8192 / kThreads; ++k) {
    const int v = tid + kThreads * k, kb = v >> 10, row = (v >> 2) & 255, cq = v & 3;
    const u32x4 x = *reinterpret_cast<const u32x4 *>(smem + row * 512 + (tile_chunk(row, kb * 4 + cq) << 4));
    *reinterpret_cast<u32x4 *>(d + int64_t(v) * 8) = x;
  }
}
// The LDS tile holding a 256 x 256 block in [j][i] order, written to rows i
// (row0 + i) of a k-blocked matrix with `cols` columns. ds_read_b64_tr_b16 (within each 16-lane
// group, lane s addresses row s >> 2, columns 4 (s & 3) .. + 3 of a 4 x 16
// block and receives column s, rows 0..3) reads it transposed: two reads
// four rows apart hand lane s the 8 consecutive j of row i = 16 ib + s, one
// 16-byte store. A wave's store covers 16 rows x 64 bytes; its 32 stores the
// whole width of 64 rows; in the k-blocked layout those 16 rows x 64 bytes
// are 1 KiB of one block. The 8 (row, chunk) pairs of 32 lanes fall in 16
// distinct 16-byte slots of the tile swizzle: no bank conflicts. The 8 waves
// take 16 of the 128 (16-row, 32-column) pieces each.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ inline s16x4 ds_read_tr(const char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
}
__device__ inline void tile_store_tr(const char *smem, bf16 *dst, int64_t cols, int row0, int col0, int tid) {
  const int w = tid >> 6, lane = tid & 63, g = lane >> 4, sl = lane & 15;
  bf16 *d = dst + kblk(row0, col0, cols);
#pragma unroll 8
  for (int k = 0; k < 128 / kWaves; ++k) {
    const int u = w * (128 / kWaves) + k, ib = u >> 3, jb = (u & 7) * 32 + g * 8;
    const int ic = ib * 16 + 4 * (sl & 3), jr = jb + (sl >> 2);
    const s16x4 x = ds_read_tr(smem + tile_off(jr, ic));
    const s16x4 y = ds_read_tr(smem + tile_off(jr + 4, ic));
    const u32x4 v = {uint32_t(uint16_t(x[0])) | (uint32_t(uint16_t(x[1])) << 16),
                     uint32_t(uint16_t(x[2])) | (uint32_t(uint16_t(x[3])) << 16),
                     uint32_t(uint16_t(y[0])) | (uint32_t(uint16_t(y[1])) << 16),
                     uint32_t(uint16_t(y[2])) | (uint32_t(uint16_t(y[3])) << 16)};
    *reinterpret_cast<u32x4 *>(d + (jb >> 5) * 8192 + (ib * 16 + sl) * 32 + (jb & 31)) = v;
  }
}
// Barrier for LDS hand-offs inside the epilogue: waits for this wave's LDS
// operations only, not for its global stores (a full __syncthreads() fence
// would wait for every store of the previous pass to land).
__device__ inline void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt unconstrained
  __builtin_amdgcn_s_barrier();
}

// The last iteration's B X writes the caller's matrix itself: out <- O, or
// W <- W - lr O with O rounded to bf16 first (bit for bit what a separate
// pass reading X' back would produce). The LDS tile holds O in the user's
// orientation (rows i for a wide view; rows j for a tall one, whose user
// matrix is X^T); each thread then updates 16-byte runs of user rows,
// skipping what lies outside the user's shape (padding).
__device__ inline void tile_update_user(const char *smem, const OutDesc &od, float lr, int row0, int col0, int tid) {
  const bool vec16 = reinterpret_cast<uintptr_t>(od.out) % 16 == 0 && (od.ld * 2) % 16 == 0;
  // 16 runs per pass, their W loads all issued before the first is used
  for (int k0 = 0; k0 < 8192 / kThreads; k0 += 16) {
    u32x4 w[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int u = tid + kThreads * (k0 + k), ur = row0 + (u >> 5), uc = col0 + (u & 31) * 8;
      w[k] = u32x4{0u, 0u, 0u, 0u};
      if (od.update && vec16 && ur < od.rows && uc + 8 <= od.cols)
        w[k] = *reinterpret_cast<const u32x4 *>(static_cast<const bf16 *>(od.out) + int64_t(ur) * od.ld + uc);
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int u = tid + kThreads * (k0 + k), row = u >> 5, c = u & 31;
      const int ur = row0 + row, uc = col0 + c * 8;
      if (ur >= od.rows || uc >= od.cols) continue;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(smem + row * 512 + (tile_chunk(row, c) << 4));
      bf16 *p = static_cast<bf16 *>(od.out) + int64_t(ur) * od.ld + uc;
      if (vec16 && uc + 8 <= od.cols) {
        u32x4 o = v;
        if (od.update) {
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const float r0 = fmaf(-lr, __uint_as_float(v[d] << 16), __uint_as_float(w[k][d] << 16));
            const float r1 = fmaf(-lr, __uint_as_float(v[d] & 0xFFFF0000u), __uint_as_float(w[k][d] & 0xFFFF0000u));
            o[d] = uint32_t(__builtin_bit_cast(uint16_t, bf16(r0))) | (uint32_t(__builtin_bit_cast(uint16_t, bf16(r1))) << 16);
          }
        }
        *reinterpret_cast<u32x4 *>(p) = o;
      } else {
        for (int e = 0; e < 8 && uc + e < od.cols; ++e) {
          bf16 x = __builtin_bit_cast(bf16, uint16_t((v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu));
          if (od.update) x = bf16(fmaf(-lr, float(x), float(p[e])));
          p[e] = x;
        }
      }
    }
  }
}

// Diagonal tile: the LDS tile holds L[c][r] = value computed at (r, c).
// Output row r takes element c from the upper-triangle computation
// (min(r, c), max(r, c)), so the stored tile is symmetric bit for bit.
// Destination: the k-blocked matrix with `cols` columns. Thread t writes
// row t mod 256, the half t / 256 of its 32 16-byte runs.
__device__ inline void tile_store_sym(const char *smem, bf16 *dst, int64_t cols, int row0, int col0, int tid) {
  const int r = tid & 255, c0 = (tid >> 8) * (32 * 256 / kThreads);
  bf16 *d = dst + kblk(row0, col0, cols) + r * 32;
#pragma unroll 4
  for (int cc = c0; cc < c0 + 32 * 256 / kThreads; ++cc) {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = 8 * cc + e;
      v[e] = *reinterpret_cast<const bf16 *>(smem + (c >= r ? tile_off(c, r) : tile_off(r, c)));
    }
    *reinterpret_cast<bf16x8 *>(d + (cc >> 2) * 8192 + (cc & 3) * 8) = v;
  }
}

// Accumulator element (r4 * 4 + q) of block (bi, bj) sits at tile row
// ti = wm*128 + bi*32 + r4*8 + fh*4 + q and tile column tj = wn*64 + bj*32 + fr.
struct EpiCoord {
  int ib, jb;  // wm*128 + fh*4, wn*64 + fr
};

// Accumulators converted once and kept bit-packed in place: the bf16 bit
// pattern sits in bits [shift, shift + 16) of each 32-bit register. Vector
// elements are reinterpreted with __float_as_uint / __uint_as_float:
// __builtin_bit_cast on a vector-element operand reads element 0.
__device__ inline uint32_t pack_bf16(float hi, float lo) {
  const bf16 h = bf16(hi), l = bf16(lo);
  return (uint32_t(__builtin_bit_cast(uint16_t, h)) << 16) | uint32_t(__builtin_bit_cast(uint16_t, l));
}
// the four bf16 of rows r4*4 .. r4*4+3 as two 32-bit words (element q in
// bits 16 (q & 1) of word q >> 1), built with integer operations only
__device__ inline u32x2 unpack4(const f32x16 &a, int r4, int shift) {
  uint32_t x[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) x[q] = (__float_as_uint(a[r4 * 4 + q]) >> shift) & 0xFFFFu;
  return u32x2{x[0] | (x[1] << 16), x[2] | (x[3] << 16)};
}
// writes block (bi, bj) of the packed accumulators into the LDS tile,
// transposed ([tj][ti], 8-byte writes) or direct ([ti][tj], 2-byte writes)
template <bool TRANS>
__device__ inline void fill_tile(char *smem, f32x16 (&acc)[4][kBN], const struct EpiCoord &e, int shift);

// [ti][tj] orientation. Within each quad of lanes (4 consecutive columns)
// the 4 x 4 block of bf16 (4 rows x 4 columns) is transposed with two DPP
// quad permutes, after which lane p of the quad holds row p of the block as
// 4 consecutive columns: one 8-byte write.
__device__ inline uint32_t quad_xor2(uint32_t v) { return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x4E, 0xF, 0xF, false)); }
__device__ inline uint32_t quad_xor1(uint32_t v) { return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0xB1, 0xF, 0xF, false)); }
__device__ inline u32x2 quad_transpose(u32x2 w, int p) {
  const bool hi2 = p & 2, odd = p & 1;
  const uint32_t y = quad_xor2(hi2 ? w[0] : w[1]);
  const uint32_t x0 = hi2 ? y : w[0], x1 = hi2 ? w[1] : y;
  const uint32_t z0 = quad_xor1(x0), z1 = quad_xor1(x1);
  return odd ? u32x2{(z0 >> 16) | (x0 & 0xFFFF0000u), (z1 >> 16) | (x1 & 0xFFFF0000u)}
             : u32x2{(x0 & 0xFFFFu) | (z0 << 16), (x1 & 0xFFFFu) | (z1 << 16)};
}
__device__ inline void put_direct(char *smem, const EpiCoord &e, int bi, int bj, int r4, u32x2 v) {
  const int p = e.jb & 3;
  const u32x2 t = quad_transpose(v, p);
  const int ti = e.ib + bi * 32 + r4 * 8 + p, tj = e.jb - p + bj * 32;
  *reinterpret_cast<u32x2 *>(smem + tile_off(ti, tj)) = t;
}
// [tj][ti .. ti+3] orientation: one 8-byte write
__device__ inline void put_trans(char *smem, const EpiCoord &e, int bi, int bj, int r4, u32x2 v) {
  const int tj = e.jb + bj * 32, ti = e.ib + bi * 32 + r4 * 8;
  *reinterpret_cast<u32x2 *>(smem + tile_off(tj, ti)) = v;
}
template <bool TRANS>
__device__ inline void fill_tile(char *smem, f32x16 (&acc)[4][kBN], const EpiCoord &e, int shift) {
  for_blocks(acc, [&](f32x16 &a, int bi, int bj) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const u32x2 v = unpack4(a, r4, shift);
      if (TRANS)
        put_trans(smem, e, bi, bj, r4, v);
      else
        put_direct(smem, e, bi, bj, r4, v);
    }
  });
}

// Block (bi, bj) of the float accumulators, rounded to bf16 on the way,
// into the LDS tile in [tj][ti] order (8-byte writes): the accumulators are
// not written back as packed bf16 first.
__device__ inline void fill_tile_trans_f32(char *smem, f32x16 (&acc)[4][kBN], const EpiCoord &e) {
  for_blocks(acc, [&](f32x16 &a, int bi, int bj) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const u32x2 v = {pack_bf16(a[r4 * 4 + 1], a[r4 * 4]), pack_bf16(a[r4 * 4 + 3], a[r4 * 4 + 2])};
      put_trans(smem, e, bi, bj, r4, v);
    }
  });
}

// A-operand fragment of a diagonal matrix v I for one 16-k half (kk) of a
// 32-k step whose k range equals the 32 output rows of an accumulator block:
// lane (m = l & 31, h = l >> 5) supplies row m at k = 16 kk + 8 h + e, so
// only the element with 16 kk + 8 h + e == m is nonzero.
__device__ inline bf16x8 diag_frag(float v, int lane, int kk) {
  const int e = (lane & 31) - 16 * kk - 8 * (lane >> 5);
  bf16x8 f;
#pragma unroll
  for (int x = 0; x < 8; ++x) f[x] = bf16(x == e ? v : 0.f);
  return f;
}

// Buffer resource over the 4 GiB from p (raw, untyped loads; the third
// dword is the gfx9 default format), and a 16-byte-per-lane load from it
// straight into LDS (lane L's bytes land at lds + 16 L).
__device__ inline __amdgpu_buffer_rsrc_t panel_rsrc(const void *p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, -1, 0x00020000);
}
__device__ inline void load_lds16(__amdgpu_buffer_rsrc_t r, char *lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voff, soff, 0, 0);
}

// Eight waves, two per SIMD (waves w and w + 4), each 128 x 64 outputs
// (4 x 2 blocks of v_mfma_f32_32x32x16_bf16). Only waves 0..3, one per SIMD,
// issue the operand loads: a wave that waits to issue a load stalls its own
// instruction stream, and the SIMD's other wave keeps the matrix core busy
// meanwhile. Loop probe (256 CUs, L2-resident operands, cycles per 32-k step
// against 1024 of matrix work): four waves of 128 x 128, every wave loading,
// 61.5%; eight waves all loading 75%; eight waves with four loading 82.8%;
// eight waves with no loads at all 86.8%. The buffer form of the LDS load
// (scalar base, 32-bit lane offset, the K step in the scalar offset) needs no
// per-load address arithmetic: 75% against 68% with 64-bit lane addresses.
// LAST (B X only): the last iteration, which writes the caller's matrices
// instead of X' and X'^T (a separate instantiation: one epilogue per kernel
// keeps the register allocation within the 256 registers of a wave).
template <int PHASE, bool LAST = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_bf16_kernel(const GemmArgs args) {
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kStageBytes];

  // the wave index goes through readfirstlane so that the compiler sees it
  // (and the K-loop bounds derived from it) as uniform
  const int wv = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
  // A*A and B X: the two waves of a SIMD (w and w + 4) take the two row
  // halves of the same 64 columns, so that the K steps that carry a
  // diagonal term (extra MFMAs in the steps whose k equal the wave's rows)
  // fall on different steps for the two and no step doubles a SIMD's extra
  // work (Qwen3 experts: B X and A*A -1.5%). The Gram, which has no such
  // steps, runs 1.3% faster with the row half w mod 2.
  const int wm = PHASE == kGram ? wv & 1 : wv >> 2;
  const int wn = PHASE == kGram ? wv >> 1 : wv & 3;
  const bool loader = wv < kLoaders;

  // Tiles of this workgroup: one (the grid covers every tile), or, in a
  // persistent launch (8 S workgroups, S per XCD), the tiles begin + slot,
  // begin + slot + S, ... of its XCD's contiguous range (the host splits
  // the tile order into 8 ranges of about equal estimated time), so that
  // the 8 XCDs each work through their own contiguous part of it.
  int t_cur, t_end, t_step;
  if (args.persistent) {
    const int x = blockIdx.x & 7, slot = blockIdx.x >> 3;
    t_cur = args.xcd_begin[x] + slot;
    t_end = args.xcd_begin[x + 1];
    t_step = int(gridDim.x) >> 3;
  } else {
    t_cur = args.remap ? xcd_remap(blockIdx.x, args.total_tiles) : int(blockIdx.x);
    t_end = t_cur + 1;
    t_step = 1;
  }
  for (; t_cur < t_end; t_cur += t_step) {
  // The thread index passes through an empty asm each tile, so the address
  // arithmetic derived from it is recomputed per tile instead of being
  // hoisted out of the tile loop (and spilled).
  int tid = int(threadIdx.x);
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const TileInfo ti = decode_tile(args, t_cur, PHASE != kBX);
  const GemmSeg &S = args.seg[ti.seg];
  char *blk = S.base + int64_t(ti.view) * S.stride;
  const int mp = S.mp, np = S.np;
  const int i0 = ti.I * kBM, j0 = ti.J * kBM;

  // P: rows i of the left operand, Q: rows j of the right one, both
  // K-contiguous: X (Gram), A (A*A), or B and X^T (B X; B is symmetric, so
  // its rows i serve as P, and X^T holds the columns of X with k contiguous).
  const bf16 *P, *Q, *P2, *Q2;
  int64_t ld;
  int K;
  if (PHASE == kGram) {
    P = Q = P2 = Q2 = reinterpret_cast<const bf16 *>(blk + S.off_xa[args.src]);
    ld = np;
    K = np;
  } else if (PHASE == kAA) {
    // distributed mode: every shard of a matrix reads the summed A held by
    // the matrix's first shard
    const char *ablk = args.tri_out ? S.base + int64_t(ti.view - ti.view % args.group) * S.stride : blk;
    P = Q = reinterpret_cast<const bf16 *>(ablk + S.off_ahi);
    P2 = Q2 = reinterpret_cast<const bf16 *>(ablk + S.off_alo);
    ld = mp;
    K = args.aa_plain ? mp : 3 * mp;
  } else {
    P = P2 = reinterpret_cast<const bf16 *>(blk + S.off_b);
    Q = Q2 = reinterpret_cast<const bf16 *>(blk + S.off_xt[args.src]);
    ld = mp;
    K = mp;
  }

  // Global -> LDS: each loader wave issues 4 loads per operand per K step.
  // Load q of wave w fills rows (4 w + q) * 16 .. + 15 of the operand tile
  // (64-byte rows, 1 KiB); lane L carries row base + L / 4 and the logical k
  // chunk that belongs in physical chunk L % 4. The operands are k-blocked:
  // the K step at k0 of the 256-row panel at i0 is the 16 KiB block at
  // i0 * ld + (k0 / 32) * 8192 elements, rows of 32 elements; the buffer
  // resource points at the panel, the K step goes in the scalar offset.
  const int lrow0 = lane >> 2;
  const int lphys = lane & 3;
  uint32_t gob[4];
  int loff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = (wv * 4 + q) * 16 + lrow0;
    const int lc = lphys ^ ((row >> 2) & 3);
    gob[q] = uint32_t(row * 32 + lc * 8) * 2u;
    loff[q] = (wv * 4 + q) * 1024;
  }
  const __amdgpu_buffer_rsrc_t rP = panel_rsrc(P + int64_t(i0) * ld), rQ = panel_rsrc(Q + int64_t(j0) * ld);
  const __amdgpu_buffer_rsrc_t rP2 = panel_rsrc(P2 + int64_t(i0) * ld), rQ2 = panel_rsrc(Q2 + int64_t(j0) * ld);
  // B X starts its K loop kBxRot K steps further on in each row tile
  // (k = kBxRot * 32 I) and wraps around: the row tiles that share a column
  // panel of X^T then read different k at any moment instead of the same 32
  // (which loads the same lines from 8 CUs at once), yet close enough
  // together that the panel's slabs are still in L2 for the next row tile.
  // Measured per row-tile offset in K steps (Kimi MoE batch, B X per step
  // and its reads per launch): 4: 325.4 ms, 44.6 GB; 2: 326.0 ms, 39.6 GB;
  // 1: 324.3 ms, 37.6 GB; 0: 328.1 ms, 36.4 GB (8, the tile's own diagonal
  // block, was 4% slower than 4 in an earlier kernel).
  const int krot = PHASE == kBX ? ti.I * kBxRot * kBK : 0;

  // B X: a + diag(B) for the row this lane supplies in each block row
  // (loaded ahead of the operand ring, so the first wait covers it)
  float coef_v[4] = {0.f, 0.f, 0.f, 0.f};
  if (PHASE == kBX) {
    const float *bdiag = reinterpret_cast<const float *>(blk + S.off_bdiag) + i0 + wm * 128 + (lane & 31);
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) coef_v[bi] = args.a + bdiag[bi * 32];
  }

  f32x16 acc[4][kBN];
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < kBN; ++bj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[bi][bj][r] = 0.f;

  const int fr = lane & 31, fh = lane >> 5;
  const int nk = K / kBK;
  // byte offset of this lane's fragment rows inside an operand tile; the
  // swizzle term (row >> 2) & 3 depends on the lane only (block bases are
  // multiples of 32 rows)
  const int fa = (wm * 128 + fr) * 64, fb = (wn * 64 + fr) * 64;
  const int fx = (fr >> 2) & 3;
  // A diagonal SYRK tile (I == J) multiplies one row panel by itself: its K
  // steps load the panel once, and both fragment sets come from that copy
  // (not in split A*A, whose hi*lo and lo*hi segments pair different halves)
  const bool dq = PHASE != kBX && __builtin_amdgcn_readfirstlane(
      int((PHASE == kGram || args.aa_plain) && ti.I == ti.J)) != 0;
  // issue the loads of K step ks_ into its stage (for A*A, K runs over three
  // segments of length mp: hi*hi, hi*lo, lo*hi)
#define MUON_GLOAD(ks_)                                                              \
  do {                                                                               \
    if (loader) {                                                                    \
      int k0_ = (ks_) * kBK;                                                         \
      if (PHASE == kBX) k0_ = k0_ + krot < K ? k0_ + krot : k0_ + krot - K;          \
      __amdgpu_buffer_rsrc_t ra_ = rP, rb_ = rQ;                                     \
      if (PHASE == kAA) {                                                            \
        const int sgm_ = k0_ / mp;                                                   \
        k0_ -= sgm_ * mp;                                                            \
        ra_ = sgm_ == 2 ? rP2 : rP;                                                  \
        rb_ = sgm_ == 1 ? rQ2 : rQ;                                                  \
      }                                                                              \
      char *st_ = smem + ((ks_) % kStages) * kStageBytes;                            \
      const uint32_t so_ = uint32_t(k0_ >> 5) * 16384u;                              \
      _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                \
        load_lds16(ra_, st_ + loff[q], gob[q], so_);                                 \
        if (!dq) load_lds16(rb_, st_ + kOpBytes + loff[q], gob[q], so_);             \
      }                                                                              \
    }                                                                                \
  } while (0)
#define MUON_FRAGS(buf_, ks_, kk_)                                                   \
  do {                                                                               \
    const char *As_ = smem + ((ks_) % kStages) * kStageBytes;                        \
    const char *Bs_ = dq ? As_ : As_ + kOpBytes;                                     \
    const int ch_ = (((kk_) * 2 + fh) ^ fx) << 4;                                    \
    _Pragma("unroll") for (int bi = 0; bi < 4; ++bi)                                 \
      af[buf_][bi] = *reinterpret_cast<const bf16x8 *>(As_ + fa + bi * 2048 + ch_);  \
    _Pragma("unroll") for (int bj = 0; bj < kBN; ++bj)                               \
      bq[buf_][bj] = *reinterpret_cast<const bf16x8 *>(Bs_ + fb + bj * 2048 + ch_);   \
  } while (0)
#define MUON_MFMA(buf_)                                                              \
  do {                                                                               \
    _Pragma("unroll") for (int bi = 0; bi < 4; ++bi)                                 \
      _Pragma("unroll") for (int bj = 0; bj < kBN; ++bj)                             \
        acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[buf_][bi], bq[buf_][bj], acc[bi][bj], 0, 0, 0); \
  } while (0)
  // s_waitcnt with vmcnt constrained (gfx9 encoding: vmcnt[3:0] and [15:14],
  // expcnt[6:4] and lgkmcnt[11:8] left at their maxima), in the loader waves
  // only: the others have no load in flight that targets LDS, and the
  // barrier after the loaders' wait publishes their stages to every wave.
  // n_ counts the loads of a full step (8 per loader wave); a diagonal tile
  // issues half of them
#define MUON_VMCNT(n_) ((((n_) & 15) | (((n_) >> 4) << 14)) | 0x0F70)
#define MUON_WAIT_VM(n_)                                                             \
  do {                                                                               \
    if (loader) {                                                                    \
      if (dq)                                                                        \
        __builtin_amdgcn_s_waitcnt(MUON_VMCNT((n_) / 2));                            \
      else                                                                           \
        __builtin_amdgcn_s_waitcnt(MUON_VMCNT(n_));                                  \
    }                                                                                \
  } while (0)
  // One K step reads stage ks only: the fragments of its k 0..15 and of its
  // k 16..31 (consumed by the MFMAs at the top of the next step). The loads
  // run three steps ahead: the wait at the top needs stage ks landed (the
  // 16 loads of ks + 1, ks + 2 stay in flight), and after the barrier the
  // loads of step ks + 3 go to the stage of step ks - 2, whose fragments
  // every wave has consumed in the MFMAs of step ks - 1, before reaching this
  // barrier; so the barrier need not wait for LDS reads. (Four steps ahead
  // with an LDS wait at the barrier measured 0.4% slower.)
  // TAIL_: the step may be one of the last three, which issue no loads (all
  // K steps are in flight already), so fewer loads may stay outstanding at
  // its top: 8 when one step remains to land after this one, 0 at the last.
#define MUON_STEP_BODY(ks_, FIRST_, CAP_, TAIL_)                                     \
  do {                                                                               \
    if (!(TAIL_) || (ks_) + 2 <= kl)                                                 \
      MUON_WAIT_VM(16);                                                              \
    else if ((ks_) + 1 == kl)                                                        \
      MUON_WAIT_VM(8);                                                               \
    else                                                                             \
      MUON_WAIT_VM(0);                                                               \
    __builtin_amdgcn_s_barrier();                                                    \
    if (!(TAIL_) || (ks_) + 3 <= kl) MUON_GLOAD((ks_) + 3);                          \
    MUON_FRAGS(0, ks_, 0);                                                           \
    if (!(FIRST_)) MUON_MFMA(1);                                                     \
    MUON_FRAGS(1, ks_, 1);                                                           \
    MUON_MFMA(0);                                                                    \
    CAP_;                                                                            \
  } while (0)
#define MUON_STEP_CORE(ks_, FIRST_, CAP_) MUON_STEP_BODY(ks_, FIRST_, CAP_, true)
  // a step with ks + 3 <= kl (no tail checks), in the compiler's order
#define MUON_STEP(ks_) MUON_STEP_BODY(ks_, false, (void)0, false)
  // The additive terms of B = b A + c A A and X' = (a + diag B) X + B' X
  // enter as products with a diagonal matrix: in the K step whose 32 k are
  // the 32 output rows of block row bi_, the Q fragments hold exactly the
  // A (or X) values of those outputs, and D Q adds D_mm Q[m][:] to row m.
  // A*A's (b / c) goes in as bf16 hi + lo parts (hi only for the small lo
  // half of A); B X's a + B_ii as its lo part only, the hi part being B's
  // stored diagonal. Both k halves are captured at the end of their step.
#define MUON_CAPTURE(buf_, bi_, dh_, dl_, lo_)                                       \
  do {                                                                               \
    _Pragma("unroll") for (int bj = 0; bj < kBN; ++bj) {                             \
      acc[bi_][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dh_[buf_], bq[buf_][bj], acc[bi_][bj], 0, 0, 0); \
      if (lo_) acc[bi_][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dl_[buf_], bq[buf_][bj], acc[bi_][bj], 0, 0, 0); \
    }                                                                                \
  } while (0)
#define MUON_CAP2(bi_, dh_, dl_, lo_)                                                \
  do {                                                                               \
    MUON_CAPTURE(0, bi_, dh_, dl_, lo_);                                             \
    MUON_CAPTURE(1, bi_, dh_, dl_, lo_);                                             \
  } while (0)

  // Every K step is loaded once; K >= 256, so nk >= 8. MUON_STEP runs the
  // steps with ks + 3 <= kl, MUON_STEP_CORE the first, the capture and the
  // last three.
  const int kl = nk - 1;
  bf16x8 af[2][4], bq[2][kBN];
  MUON_GLOAD(0);
  MUON_GLOAD(1);
  MUON_GLOAD(2);
  int ks = 0;
  if (PHASE == kGram) {
    MUON_STEP_CORE(ks, true, (void)0);
    for (++ks; ks + 3 <= kl; ++ks) MUON_STEP(ks);
    for (; ks < nk; ++ks) MUON_STEP_CORE(ks, false, (void)0);
  } else {
    if (PHASE == kAA) {
      // the K step whose k range equals this wave's first output rows
      const int c0 = ti.I * (kBM / kBK) + wm * (128 / kBK);
      const float r = args.r, rh = float(bf16(r));
      const bf16x8 dh[2] = {diag_frag(rh, lane, 0), diag_frag(rh, lane, 1)};
      const bf16x8 dl[2] = {diag_frag(r - rh, lane, 0), diag_frag(r - rh, lane, 1)};
#define MUON_CAP_STEPS(lo_, FIRST_)                                                  \
      do {                                                                           \
        MUON_STEP_CORE(ks, FIRST_, MUON_CAP2(0, dh, dl, lo_)); ++ks;                 \
        MUON_STEP_CORE(ks, false, MUON_CAP2(1, dh, dl, lo_)); ++ks;                  \
        MUON_STEP_CORE(ks, false, MUON_CAP2(2, dh, dl, lo_)); ++ks;                  \
        MUON_STEP_CORE(ks, false, MUON_CAP2(3, dh, dl, lo_)); ++ks;                  \
      } while (0)
      // segment hi*hi: r A_hi (+ its bf16 rounding remainder)
      if (c0 == 0) {
        MUON_CAP_STEPS(true, true);
      } else {
        MUON_STEP_CORE(ks, true, (void)0);
        for (++ks; ks < c0; ++ks) MUON_STEP(ks);
        MUON_CAP_STEPS(true, false);
      }
      if (!args.aa_plain) {
        // segment hi*lo: its Q fragments hold A_lo, which is symmetric too
        const int c1 = mp / kBK + c0;
        for (; ks < c1; ++ks) MUON_STEP(ks);
        MUON_CAP_STEPS(false, false);
      }
#undef MUON_CAP_STEPS
    } else {
      // K step c0 + bi (c0 = 8 I + 4 wm) is loop iteration
      // (8 - kBxRot) I + 4 wm + bi of the rotated K loop
      const int cb = ti.I * (kBM / kBK - kBxRot) + wm * (128 / kBK);
#define MUON_CAP_STEP(bi_, FIRST_)                                                   \
      do {                                                                           \
        const float cv = coef_v[bi_], ch = float(bf16(cv));                          \
        const bf16x8 dl[2] = {diag_frag(cv - ch, lane, 0), diag_frag(cv - ch, lane, 1)}; \
        MUON_STEP_CORE(ks, FIRST_, MUON_CAP2(bi_, dl, dl, false));                   \
        ++ks;                                                                        \
      } while (0)
      if (cb == 0) {
        MUON_CAP_STEP(0, true);
      } else {
        MUON_STEP_CORE(ks, true, (void)0);
        for (++ks; ks < cb; ++ks) MUON_STEP(ks);
        MUON_CAP_STEP(0, false);
      }
      MUON_CAP_STEP(1, false);
      MUON_CAP_STEP(2, false);
      MUON_CAP_STEP(3, false);
#undef MUON_CAP_STEP
    }
    for (; ks + 3 <= kl; ++ks) MUON_STEP(ks);
    for (; ks < nk; ++ks) MUON_STEP_CORE(ks, false, (void)0);
  }
  MUON_MFMA(1);  // k 16..31 of the last step
  MUON_WAIT_VM(0);  // no load may still target LDS past the K loop
#undef MUON_GLOAD
#undef MUON_FRAGS
#undef MUON_MFMA
#undef MUON_WAIT_VM
#undef MUON_VMCNT
#undef MUON_STEP_CORE
#undef MUON_STEP_BODY
#undef MUON_STEP
#undef MUON_CAPTURE
#undef MUON_CAP2

  // ---------------- epilogues ----------------
  if (PHASE != kBX) __syncthreads();  // every wave is done with the LDS ring
  const EpiCoord ec{wm * 128 + fh * 4, wn * 64 + fr};
  const bool diag = (PHASE != kBX) && ti.I == ti.J;
  float *scale_p = reinterpret_cast<float *>(blk + S.off_scale);

  if (PHASE == kGram && args.tri_out) {
    // Distributed mode: this shard's partial s' X_p X_p^T leaves in float32,
    // straight from the accumulators into its tile-packed buffer (layout.h;
    // block (bi, bj) of wave (wm, wn) is block (4 wm + bi, 2 wn + bj) of the
    // tile, its quad 2 g + fh from registers 4 g .. 4 g + 3)
    const float sg = args.first ? scale_p[1] : 1.f;
    float *dst = reinterpret_cast<float *>(blk + S.off_tri) + int64_t(ti.J * (ti.J + 1) / 2 + ti.I) * kTriTileFloats;
    for_blocks(acc, [&](f32x16 &a, int bi, int bj) {
      float *d = dst + ((wm * 4 + bi) * 8 + wn * 2 + bj) * 1024 + fh * 128 + fr * 4;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = a[4 * g + e] * sg;
        *reinterpret_cast<f32x4 *>(d + g * 256) = v;
      }
    });
  } else if (PHASE == kGram) {
    // A = s' X X^T as bf16 hi + lo. Each output tile passes through LDS once,
    // as A[j][i] (8-byte writes): its rows are the mirror tile (J, I), its
    // transposing reads the tile (I, J); a diagonal tile leaves once,
    // symmetrized.
    const float sg = args.first ? scale_p[1] : 1.f;
    for_blocks(acc, [&](f32x16 &a, int, int) {
#pragma unroll
      for (int r = 0; r < 16; ++r) a[r] *= sg;
    });
    // hi = bf16(A) first, rounded on the way into LDS; the lo half A - hi
    // (only when A*A runs on the split A) is formed in place afterwards
    const int halves = args.gram_halves;
    for (int half = 0; half < halves; ++half) {  // 0: hi, 1: lo
      bf16 *dst = reinterpret_cast<bf16 *>(blk + (half ? S.off_alo : S.off_ahi));
      if (half)
        for_blocks(acc, [&](f32x16 &a, int, int) {
#pragma unroll
          for (int r = 0; r < 16; ++r) a[r] -= float(bf16(a[r]));
        });
      fill_tile_trans_f32(smem, acc, ec);
      lds_barrier();
      if (diag) {
        tile_store_sym(smem, dst, mp, i0, j0, tid);
      } else {
        tile_store(smem, dst, mp, j0, i0, tid);     // mirror tile (J, I)
        tile_store_tr(smem, dst, mp, i0, j0, tid);  // tile (I, J)
      }
      lds_barrier();
    }
  } else if (PHASE == kAA) {
    // B = c (A A + r A), r = b / c added in the K loop
    for_blocks(acc, [&](f32x16 &a, int, int) {
#pragma unroll
      for (int r = 0; r < 16; ++r) a[r] *= args.c;
    });
    // The diagonal of B stays in float32 (bdiag); B stores bf16(a + B_ii)
    // there instead, the hi part of B X's diagonal term (a + B_ii) X, so that
    // the B X K loop adds it with the rest of the product and only the lo
    // part goes in as an extra diagonal product. In a
    // diagonal tile, block (bi, bj) of wave (wm, wn) covers rows
    // 128 wm + 32 bi and columns 64 wn + 32 bj, so the waves with
    // wn / 2 == wm hold diagonal elements, in their blocks with
    // bi == 2 (wn mod 2) + bj: row 8 r4 + 4 fh + q equals column fr for the
    // lanes with fh == (fr >> 2) & 1, in register (fr >> 3) * 4 + (fr & 3).
    float *bdiag = reinterpret_cast<float *>(blk + S.off_bdiag);
    bf16 *Bm = reinterpret_cast<bf16 *>(blk + S.off_b);
    if (diag && (wn >> 1) == wm) {
      const bool holder = fh == ((fr >> 2) & 1);
      const int rr = (fr >> 3) * 4 + (fr & 3);
      for_blocks(acc, [&](f32x16 &a, int bi, int bj) {
        if (bi != 2 * (wn & 1) + bj) return;
        float x = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) x = r == rr ? a[r] : x;
        if (holder) bdiag[i0 + wm * 128 + bi * 32 + fr] = x;
#pragma unroll
        for (int r = 0; r < 16; ++r) a[r] = (holder && r == rr) ? args.a + x : a[r];
      });
    }
    fill_tile_trans_f32(smem, acc, ec);
    lds_barrier();
    if (diag) {
      tile_store_sym(smem, Bm, mp, i0, j0, tid);
    } else {
      tile_store(smem, Bm, mp, j0, i0, tid);     // mirror tile (J, I)
      tile_store_tr(smem, Bm, mp, i0, j0, tid);  // tile (I, J)
    }
    lds_barrier();  // in a persistent launch the next tile's loads reuse the LDS
  } else {
    // X' = s'' ((a + B_ii) X + B_offdiag X), the first term added in the K
    // loop; it goes out through LDS twice: X' for the next Gram and X'^T for
    // the next B X (or, in the last iteration, into the caller's matrix)
    const float sx = args.first ? scale_p[0] : 1.f;
    bf16 *Y = reinterpret_cast<bf16 *>(blk + S.off_xa[args.src ^ 1]);
    bf16 *Yt = reinterpret_cast<bf16 *>(blk + S.off_xt[args.src ^ 1]);
    // scaled in place, ahead of the branch, so that the scaled values never
    // live beside the unscaled ones (with 256 registers per wave that spills)
    for_blocks(acc, [&](f32x16 &a, int, int) {
#pragma unroll
      for (int r = 0; r < 16; ++r) a[r] *= sx;
    });
    if (LAST) {
      for_blocks(acc, [&](f32x16 &a, int, int) {
#pragma unroll
        for (int r = 0; r < 16; ++r) a[r] = __uint_as_float(pack_bf16(0.f, a[r]));
      });
      const OutDesc od = *reinterpret_cast<const OutDesc *>(blk + S.off_scale + kOutDescOffset);
      lds_barrier();  // every wave is done with the LDS ring (its last fragment reads)
      if (od.tall)
        fill_tile<true>(smem, acc, ec, 0);
      else
        fill_tile<false>(smem, acc, ec, 0);
      lds_barrier();
      tile_update_user(smem, od, args.lr, od.tall ? j0 : i0, od.tall ? i0 : j0, tid);
    } else {
      // one pass through LDS in [j][i] order: X'^T leaves as its rows, X' as
      // the transposing reads of the same tile
      lds_barrier();  // every wave is done with the LDS ring (its last fragment reads)
      fill_tile_trans_f32(smem, acc, ec);
      lds_barrier();
      tile_store(smem, Yt, mp, j0, i0, tid);  // X'^T: tile (J, I) of an np x mp matrix
      tile_store_tr(smem, Y, np, i0, j0, tid);
    }
    lds_barrier();  // every wave is done with the LDS ring
  }
  }  // tiles of this workgroup
}

// ---------------------------------------------------------------------------
// float32 kernel (VALU FMA): 64x64 output tile, K step 16, 256 threads, each
// thread 4x4 outputs strided by 16. Same phases as above with float32
// storage everywhere (A in the hi slot, no lo half, B with its diagonal);
// the terms b A and a X come from memory in the epilogue.
// ---------------------------------------------------------------------------

template <int PHASE>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const GemmArgs args) {
  __shared__ float As[16][68], Bs[16][68];
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const TileInfo ti = decode_tile(args, int(blockIdx.x), PHASE != kBX);
  const GemmSeg &S = args.seg[ti.seg];
  char *blk = S.base + int64_t(ti.view) * S.stride;
  const int mp = S.mp, np = S.np;
  const int i0 = ti.I * 64, j0 = ti.J * 64;
  const float *P, *Q;
  int64_t ld;
  int K;
  if (PHASE == kGram) {
    P = Q = reinterpret_cast<const float *>(blk + S.off_xa[args.src]);
    ld = np;
    K = np;
  } else if (PHASE == kAA) {
    P = Q = reinterpret_cast<const float *>(blk + S.off_ahi);
    ld = mp;
    K = mp;
  } else {  // B is symmetric: its rows i serve as P; Q is X, read by rows k
    P = reinterpret_cast<const float *>(blk + S.off_b);
    Q = reinterpret_cast<const float *>(blk + S.off_xa[args.src]);
    ld = mp;
    K = mp;
  }
  float acc[4][4] = {};
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  const int kr = tid >> 4, kc = (tid & 15) * 4;
  for (int k0 = 0; k0 < K; k0 += 16) {
    const float4 pa = *reinterpret_cast<const float4 *>(P + int64_t(i0 + lr) * ld + k0 + lk);
    As[lk + 0][lr] = pa.x;
    As[lk + 1][lr] = pa.y;
    As[lk + 2][lr] = pa.z;
    As[lk + 3][lr] = pa.w;
    if (PHASE == kBX) {
      const float4 qa = *reinterpret_cast<const float4 *>(Q + int64_t(k0 + kr) * np + j0 + kc);
      Bs[kr][kc + 0] = qa.x;
      Bs[kr][kc + 1] = qa.y;
      Bs[kr][kc + 2] = qa.z;
      Bs[kr][kc + 3] = qa.w;
    } else {
      const float4 qa = *reinterpret_cast<const float4 *>(Q + int64_t(j0 + lr) * ld + k0 + lk);
      Bs[lk + 0][lr] = qa.x;
      Bs[lk + 1][lr] = qa.y;
      Bs[lk + 2][lr] = qa.z;
      Bs[lk + 3][lr] = qa.w;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) a[x] = As[k][ty + 16 * x];
#pragma unroll
      for (int y = 0; y < 4; ++y) b[y] = Bs[k][tx + 16 * y];
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = fmaf(a[x], b[y], acc[x][y]);
    }
    __syncthreads();
  }
  const bool diag = ti.I == ti.J;
  if (PHASE == kGram || PHASE == kAA) {
    const float sg = (PHASE == kGram && args.first) ? reinterpret_cast<const float *>(blk + S.off_scale)[1] : 1.f;
    const float *A = reinterpret_cast<const float *>(blk + S.off_ahi);
    float *O = reinterpret_cast<float *>(blk + (PHASE == kGram ? S.off_ahi : S.off_b));
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int i = i0 + ty + 16 * x, j = j0 + tx + 16 * y;
        float v;
        if (PHASE == kGram)
          v = acc[x][y] * sg;
        else
          v = fmaf(args.b, A[int64_t(i) * mp + j], args.c * acc[x][y]);
        if (!diag || i <= j) O[int64_t(i) * mp + j] = v;
        if (!diag || i < j) O[int64_t(j) * mp + i] = v;
      }
  } else {
    const float sx = args.first ? reinterpret_cast<const float *>(blk + S.off_scale)[0] : 1.f;
    const float *X = reinterpret_cast<const float *>(blk + S.off_xa[args.src]);
    float *Ya = reinterpret_cast<float *>(blk + S.off_xa[args.src ^ 1]);
    const OutDesc od = *reinterpret_cast<const OutDesc *>(blk + S.off_scale + kOutDescOffset);
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int i = i0 + ty + 16 * x, j = j0 + tx + 16 * y;
        const float o = sx * fmaf(args.a, X[int64_t(i) * np + j], acc[x][y]);
        if (!args.last) {
          Ya[int64_t(i) * np + j] = o;
        } else {
          // the caller's matrix directly (see store_user)
          const int ur = od.tall ? j : i, uc = od.tall ? i : j;
          if (ur < od.rows && uc < od.cols) {
            float *p = static_cast<float *>(od.out) + int64_t(ur) * od.ld + uc;
            *p = od.update ? fmaf(-args.lr, o, *p) : o;
          }
        }
      }
  }
}

}  // namespace

hipError_t launch_elem(const ElemArgs &a, bool bf16, hipStream_t s) {
  if (a.total_tiles <= 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(elem_kernel<__bf16>, dim3((a.total_tiles + kElemTilesPerGroup - 1) / kElemTilesPerGroup), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(elem_kernel<float>, dim3((a.total_tiles + kElemTilesPerGroup - 1) / kElemTilesPerGroup), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_norm_finalize(const GemmArgs &a, int views, hipStream_t s) {
  if (views <= 0) return hipSuccess;
  hipLaunchKernelGGL(norm_finalize_kernel, dim3(views / a.group), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs &a, int phase, bool bf16, hipStream_t s) {
  if (a.total_tiles <= 0) return hipSuccess;
  const dim3 grid(a.persistent ? a.persistent : a.total_tiles), block(bf16 ? kThreads : 256);
  if (bf16) {
    switch (phase) {
      case kGram: hipLaunchKernelGGL(gemm_bf16_kernel<kGram>, grid, block, 0, s, a); break;
      case kAA: hipLaunchKernelGGL(gemm_bf16_kernel<kAA>, grid, block, 0, s, a); break;
      default:
        if (a.last)
          hipLaunchKernelGGL((gemm_bf16_kernel<kBX, true>), grid, block, 0, s, a);
        else
          hipLaunchKernelGGL(gemm_bf16_kernel<kBX>, grid, block, 0, s, a);
        break;
    }
  } else {
    switch (phase) {
      case kGram: hipLaunchKernelGGL(gemm_f32_kernel<kGram>, grid, block, 0, s, a); break;
      case kAA: hipLaunchKernelGGL(gemm_f32_kernel<kAA>, grid, block, 0, s, a); break;
      default: hipLaunchKernelGGL(gemm_f32_kernel<kBX>, grid, block, 0, s, a); break;
    }
  }
  return hipGetLastError();
}

}  // namespace muon
