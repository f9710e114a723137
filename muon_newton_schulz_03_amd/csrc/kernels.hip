// HIP kernels of the Muon step for CDNA4 (gfx950).
//
// Per group of views (whole matrices or column blocks), in stream order:
//   elem_kernel (prep)      momentum M <- beta M + G, Newton-Schulz source X0,
//                           X0 and X0^T written zero-padded into the
//                           workspace, per-tile partial sums of squares.
//   norm_finalize_kernel    s = 1/(||X0||_F + eps) from the partial sums.
//   iters x { gemm <Gram>   A = s' X X^T (upper-triangle tiles, mirrored),
//                           stored as bf16 hi + lo;
//             gemm <AA>     B = b A + c A A (upper tiles, mirrored), A A from
//                           hi*hi + hi*lo + lo*hi;
//             gemm <BX>     X' = s'' (a X + B X), stored as X' and X'^T }
//   elem_kernel (finish)    data <- O, or W <- W - lr O.
// s' = s^2 and s'' = s in the first iteration (the normalization is folded
// into the first Gram and the first B X epilogue), 1 afterwards.
//
// Three products per iteration, the first two symmetric rank-k products
// (SYRK) with only upper-triangle tiles computed and the diagonal tiles in
// full, the result stored as a full matrix: Advancing Emerging Optimizers
// (zh translation, wiki.whaty.org), sections "Distributed mode" and
// "SYRK 和融合的 all-reduce".
//
// All three products are "NT" contractions C[i][j] = sum_k P[i][k] Q[j][k]
// with both operands K-contiguous: the Gram reads rows of X twice, A*A reads
// rows of the symmetric A twice, and B X reads rows of B and rows of X^T --
// which is why every B X epilogue also writes X'^T.
#include <hip/hip_runtime.h>

#include <utility>

#include "kernels.h"

namespace muon {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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
  if (syrk) {  // upper triangle, column by column: u = J (J + 1) / 2 + I
    J = int((sqrtf(8.f * float(u) + 1.f) - 1.f) * 0.5f);
    while ((J + 1) * (J + 2) / 2 <= u) ++J;
    while (J * (J + 1) / 2 > u) --J;
    I = u - J * (J + 1) / 2;
  } else {
    I = u / S.tn;
    J = u - I * S.tn;
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

template <typename T>
__global__ __launch_bounds__(256) void elem_kernel(const ElemArgs args) {
  constexpr int V = 16 / sizeof(T);      // elements per 16-byte chunk
  constexpr int CPR = 64 / V;            // chunks per 64-element row
  constexpr int CPT = 64 * CPR / 256;    // chunks per thread
  __shared__ T tile[64][64 + 2];
  __shared__ float red[4];

  const int b = blockIdx.x, tid = threadIdx.x;
  int vi = 0;
  while (vi + 1 < args.nv && b >= args.v[vi + 1].tile_begin) ++vi;
  const ElemView &Vw = args.v[vi];
  const int u = b - Vw.tile_begin;
  const int tr = u / Vw.tiles_c, tc = u - (u / Vw.tiles_c) * Vw.tiles_c;
  const int kind = args.kind;

  if (kind == kPrepNs || kind == kPrepStep) {
    T *direct = reinterpret_cast<T *>(Vw.blk + Vw.off_direct);
    T *trans = reinterpret_cast<T *>(Vw.blk + Vw.off_trans);
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int c = tid + 256 * q, row = c / CPR, cc = c % CPR;
      const int gr = tr * 64 + row, gc = tc * 64 + cc * V;
      float x[V];
      if (kind == kPrepStep) {
        float g[V], m[V];
        load_row_chunk<T>(Vw.g, Vw.ld_g, gr, gc, Vw.rows, Vw.cols, Vw.vec & 1, g);
        load_row_chunk<T>(Vw.m, Vw.ld_m, gr, gc, Vw.rows, Vw.cols, Vw.vec & 2, m);
#pragma unroll
        for (int e = 0; e < V; ++e) m[e] = fmaf(args.beta, m[e], g[e]);
        store_row_chunk<T>(Vw.m, Vw.ld_m, gr, gc, Vw.rows, Vw.cols, Vw.vec & 2, m);
#pragma unroll
        for (int e = 0; e < V; ++e) x[e] = args.nesterov ? fmaf(args.beta, m[e], g[e]) : m[e];
      } else {
        load_row_chunk<T>(Vw.m, Vw.ld_m, gr, gc, Vw.rows, Vw.cols, Vw.vec & 2, x);
      }
      Vec16<T> xv;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        xv.e[e] = T(x[e]);
        const float xf = float(xv.e[e]);
        ss = fmaf(xf, xf, ss);
        tile[row][cc * V + e] = xv.e[e];
      }
      *reinterpret_cast<Vec16<T> *>(direct + int64_t(gr) * Vw.pitch_direct + gc) = xv;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int c = tid + 256 * q, trow = c / CPR, tcc = c % CPR;
      Vec16<T> tv;
#pragma unroll
      for (int e = 0; e < V; ++e) tv.e[e] = tile[tcc * V + e][trow];
      *reinterpret_cast<Vec16<T> *>(trans + int64_t(tc * 64 + trow) * Vw.pitch_trans + tr * 64 + tcc * V) = tv;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    if (tid == 0) reinterpret_cast<float *>(Vw.blk + Vw.off_part)[u] = (red[0] + red[1]) + (red[2] + red[3]);
  } else {
    const T *O = reinterpret_cast<const T *>(Vw.blk + Vw.off_direct);
    const float sf = args.final_scale ? reinterpret_cast<const float *>(Vw.blk + Vw.off_scale)[0] : 1.f;
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int c = tid + 256 * q, row = c / CPR, cc = c % CPR;
      const int gr = tr * 64 + row, gc = tc * 64 + cc * V;
      if (gr >= Vw.rows || gc >= Vw.cols) continue;
      const Vec16<T> ov = *reinterpret_cast<const Vec16<T> *>(O + int64_t(gr) * Vw.pitch_direct + gc);
      float o[V];
#pragma unroll
      for (int e = 0; e < V; ++e) o[e] = float(ov.e[e]) * sf;
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
}

// s = 1 / (||X0||_F + eps) from the per-tile partial sums, summed in a fixed
// order in double precision. One workgroup per view.
__global__ __launch_bounds__(256) void norm_finalize_kernel(const GemmArgs args) {
  __shared__ double red[256];
  const int vg = blockIdx.x, tid = threadIdx.x;
  int s = 0;
  while (s + 1 < args.nseg && vg >= args.seg[s + 1].view_begin) ++s;
  const GemmSeg &S = args.seg[s];
  char *blk = S.base + int64_t(vg - S.view_begin) * S.stride;
  const float *part = reinterpret_cast<const float *>(blk + S.off_part);
  double acc = 0.0;
  for (int i = tid; i < S.nparts; i += 256) acc += double(part[i]);
  red[tid] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid == 0) {
    const double sc = 1.0 / (sqrt(red[0]) + double(args.eps));
    float *scale = reinterpret_cast<float *>(blk + S.off_scale);
    scale[0] = float(sc);
    scale[1] = float(sc * sc);
  }
}

// ---------------------------------------------------------------------------
// bf16 matrix-core kernel: 256x256 output tile, K step 64, 4 waves (2x2),
// each wave 128x128 = 4x4 blocks of v_mfma_f32_32x32x16_bf16.
// Operand tiles (256 rows x 64 k, bf16) are staged through LDS, double
// buffered (2 stages x 2 operands x 32 KiB); each 128-byte row keeps its
// eight 16-byte chunks XOR-swizzled by (row & 7) so that the fragment reads
// (32 rows, one chunk each) spread over the banks.
//
// MFMA 32x32x16 register layout: lane l supplies row (l & 31) of the A
// operand and column (l & 31) of the B operand, each as 8 consecutive k
// (k half selected by l >> 5; any k permutation shared by both operands
// gives the same sum). Accumulator register r of lane l holds
// C[8 (r >> 2) + 4 (l >> 5) + (r & 3)][l & 31].
// ---------------------------------------------------------------------------

constexpr int kBM = 256, kBK = 64;
constexpr int kOpBytes = kBM * kBK * 2;  // one operand tile, one stage

// Epilogue of one 32x32 accumulator block: rows ib + 8 r4 + q (q = 0..3),
// column j, for r4 = 0..3 (see the MFMA layout above).
template <int PHASE>
struct GemmEpilogue {
  int mp, np, ib, jb;
  bool diag;
  float a, b, c, scale;
  bf16 *ahi, *alo, *bm, *ya, *yt;
  const bf16 *xt;
  float *bdiag;

  __device__ inline void block(const f32x16 &acc, int i0, int j) const {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int i = i0 + r4 * 8;  // rows i .. i+3, column j
      if (PHASE == kBX) {
        // X' = s'' (a X + B X); X[i..i+3][j] = X^T[j][i..i+3]
        // B's diagonal is kept in float32 (bdiag) and is zero in the bf16 B
        // operand, so the diagonal part of B X is (a + B_ii) X[i][j] here
        const bf16x4 x4 = *reinterpret_cast<const bf16x4 *>(xt + int64_t(j) * mp + i);
        const float4 d4 = *reinterpret_cast<const float4 *>(bdiag + i);
        const float dd[4] = {d4.x, d4.y, d4.z, d4.w};
        bf16x4 o4;
#pragma unroll
        for (int q = 0; q < 4; ++q) o4[q] = bf16(scale * fmaf(a + dd[q], float(x4[q]), acc[r4 * 4 + q]));
        *reinterpret_cast<bf16x4 *>(yt + int64_t(j) * mp + i) = o4;
#pragma unroll
        for (int q = 0; q < 4; ++q) ya[int64_t(i + q) * np + j] = o4[q];
        continue;
      }
      bf16x4 v1, v2;
      if (PHASE == kGram) {
        // A = s' X X^T, kept as bf16 hi + lo
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float v = acc[r4 * 4 + q] * scale;
          v1[q] = bf16(v);
          v2[q] = bf16(v - float(v1[q]));
        }
      } else {
        // B = b A + c A A; A[i..i+3][j] = A[j][i..i+3] (A is symmetric).
        // The diagonal goes to bdiag in float32 and is stored as zero in B.
        const bf16x4 h4 = *reinterpret_cast<const bf16x4 *>(ahi + int64_t(j) * mp + i);
        const bf16x4 l4 = *reinterpret_cast<const bf16x4 *>(alo + int64_t(j) * mp + i);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float bv = fmaf(b, float(h4[q]) + float(l4[q]), c * acc[r4 * 4 + q]);
          v1[q] = bf16(bv);
          if (diag && i + q == j) {
            bdiag[j] = bv;
            v1[q] = bf16(0.f);
          }
        }
      }
      bf16 *o1 = PHASE == kGram ? ahi : bm;
      bf16 *o2 = alo;
      if (!diag) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          o1[int64_t(i + q) * mp + j] = v1[q];
          if (PHASE == kGram) o2[int64_t(i + q) * mp + j] = v2[q];
        }
        *reinterpret_cast<bf16x4 *>(o1 + int64_t(j) * mp + i) = v1;
        if (PHASE == kGram) *reinterpret_cast<bf16x4 *>(o2 + int64_t(j) * mp + i) = v2;
      } else {
        // diagonal tile: keep the upper element and mirror it, so the stored
        // matrix is symmetric bit for bit
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ii = i + q;
          if (ii <= j) {
            o1[int64_t(ii) * mp + j] = v1[q];
            if (PHASE == kGram) o2[int64_t(ii) * mp + j] = v2[q];
          }
          if (ii < j) {
            o1[int64_t(j) * mp + ii] = v1[q];
            if (PHASE == kGram) o2[int64_t(j) * mp + ii] = v2[q];
          }
        }
      }
    }
  }
};

// Applies the epilogue to the 16 accumulator blocks with compile-time
// indices, so the accumulators stay in registers.
template <int PHASE, int... N>
__device__ inline void run_epilogue(const f32x16 (&acc)[4][4], const GemmEpilogue<PHASE> &ep,
                                    std::integer_sequence<int, N...>) {
  (ep.block(acc[N / 4][N % 4], ep.ib + (N / 4) * 32, ep.jb + (N % 4) * 32), ...);
}

template <int PHASE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_kernel(const GemmArgs args) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * 2 * kOpBytes];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int tile = args.remap ? xcd_remap(blockIdx.x, args.total_tiles) : int(blockIdx.x);
  const TileInfo ti = decode_tile(args, tile, PHASE != kBX);
  const GemmSeg &S = args.seg[ti.seg];
  char *blk = S.base + int64_t(ti.view) * S.stride;
  const int mp = S.mp, np = S.np;
  const int i0 = ti.I * kBM, j0 = ti.J * kBM;

  const bf16 *P, *Q, *P2, *Q2;
  int64_t ld;
  int K;
  if (PHASE == kGram) {
    P = Q = P2 = Q2 = reinterpret_cast<const bf16 *>(blk + S.off_xa[args.src]);
    ld = np;
    K = np;
  } else if (PHASE == kAA) {
    P = Q = reinterpret_cast<const bf16 *>(blk + S.off_ahi);
    P2 = Q2 = reinterpret_cast<const bf16 *>(blk + S.off_alo);
    ld = mp;
    K = args.aa_plain ? mp : 3 * mp;
  } else {
    P = P2 = reinterpret_cast<const bf16 *>(blk + S.off_b);
    Q = Q2 = reinterpret_cast<const bf16 *>(blk + S.off_xt[args.src]);
    ld = mp;
    K = mp;
  }

  // global -> register -> LDS staging: thread t moves 16-byte chunk (t & 7)
  // of rows (t >> 3) + 32 q, q = 0..7, of both operand tiles.
  const int lrow = tid >> 3, lkc = tid & 7;
  const int64_t prow = int64_t(i0 + lrow) * ld + lkc * 8;
  const int64_t qrow = int64_t(j0 + lrow) * ld + lkc * 8;
  const int sw_off = lrow * 128 + ((lkc ^ (lrow & 7)) << 4);
  u32x4 ra[8], rb[8];

  f32x16 acc[4][4];
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[bi][bj][r] = 0.f;

  const int fr = lane & 31, fh = lane >> 5, fx = lane & 7;
  const int nk = K / kBK;
  for (int ks = -1; ks < nk; ++ks) {
    // prefetch K step ks + 1 into registers (for AA: K runs over three
    // segments of length mp -- hi*hi, hi*lo, lo*hi)
    if (ks + 1 < nk) {
      int k0 = (ks + 1) * kBK;
      const bf16 *pa = P, *qa = Q;
      if (PHASE == kAA) {
        const int sgm = k0 / mp;
        k0 -= sgm * mp;
        if (sgm == 2) pa = P2;
        if (sgm == 1) qa = Q2;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        ra[q] = *reinterpret_cast<const u32x4 *>(pa + prow + int64_t(q) * 32 * ld + k0);
        rb[q] = *reinterpret_cast<const u32x4 *>(qa + qrow + int64_t(q) * 32 * ld + k0);
      }
    }
    if (ks >= 0) {
      const char *A = smem + (ks & 1) * 2 * kOpBytes;
      const char *B = A + kOpBytes;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int ch = ((kk * 2 + fh) ^ fx) << 4;
        bf16x8 af[4], bfr[4];
#pragma unroll
        for (int bi = 0; bi < 4; ++bi)
          af[bi] = *reinterpret_cast<const bf16x8 *>(A + (wm * 128 + bi * 32 + fr) * 128 + ch);
#pragma unroll
        for (int bj = 0; bj < 4; ++bj)
          bfr[bj] = *reinterpret_cast<const bf16x8 *>(B + (wn * 128 + bj * 32 + fr) * 128 + ch);
#pragma unroll
        for (int bi = 0; bi < 4; ++bi)
#pragma unroll
          for (int bj = 0; bj < 4; ++bj)
            acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[bi], bfr[bj], acc[bi][bj], 0, 0, 0);
      }
    }
    if (ks + 1 < nk) {
      // stage ks + 1 lives in buffer (ks + 1) & 1; its previous contents
      // (step ks - 1) were consumed before the barrier that ended step ks - 1
      char *A = smem + ((ks + 1) & 1) * 2 * kOpBytes;
      char *B = A + kOpBytes;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        *reinterpret_cast<u32x4 *>(A + q * 4096 + sw_off) = ra[q];
        *reinterpret_cast<u32x4 *>(B + q * 4096 + sw_off) = rb[q];
      }
    }
    __syncthreads();
  }

  // ---------------- epilogues ----------------
  GemmEpilogue<PHASE> ep;
  ep.mp = mp;
  ep.np = np;
  ep.ib = i0 + wm * 128 + fh * 4;
  ep.jb = j0 + wn * 128 + fr;
  ep.diag = ti.I == ti.J;
  ep.a = args.a;
  ep.b = args.b;
  ep.c = args.c;
  ep.ahi = reinterpret_cast<bf16 *>(blk + S.off_ahi);
  ep.alo = reinterpret_cast<bf16 *>(blk + S.off_alo);
  ep.bm = reinterpret_cast<bf16 *>(blk + S.off_b);
  ep.xt = reinterpret_cast<const bf16 *>(blk + S.off_xt[args.src]);
  ep.ya = reinterpret_cast<bf16 *>(blk + S.off_xa[args.src ^ 1]);
  ep.yt = reinterpret_cast<bf16 *>(blk + S.off_xt[args.src ^ 1]);
  ep.bdiag = reinterpret_cast<float *>(blk + S.off_bdiag);
  ep.scale = 1.f;
  if (args.first) {
    const float *sc = reinterpret_cast<const float *>(blk + S.off_scale);
    ep.scale = PHASE == kGram ? sc[1] : (PHASE == kBX ? sc[0] : 1.f);
  }
  run_epilogue(acc, ep, std::make_integer_sequence<int, 16>{});
}

// ---------------------------------------------------------------------------
// float32 kernel (VALU FMA): 64x64 output tile, K step 16, 256 threads, each
// thread 4x4 outputs strided by 16. Same phases and epilogues as above, with
// float32 storage everywhere (A in the hi slot, no lo half).
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
  } else {
    P = reinterpret_cast<const float *>(blk + S.off_b);
    Q = reinterpret_cast<const float *>(blk + S.off_xt[args.src]);
    ld = mp;
    K = mp;
  }
  float acc[4][4] = {};
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  for (int k0 = 0; k0 < K; k0 += 16) {
    const float4 pa = *reinterpret_cast<const float4 *>(P + int64_t(i0 + lr) * ld + k0 + lk);
    const float4 qa = *reinterpret_cast<const float4 *>(Q + int64_t(j0 + lr) * ld + k0 + lk);
    As[lk + 0][lr] = pa.x;
    As[lk + 1][lr] = pa.y;
    As[lk + 2][lr] = pa.z;
    As[lk + 3][lr] = pa.w;
    Bs[lk + 0][lr] = qa.x;
    Bs[lk + 1][lr] = qa.y;
    Bs[lk + 2][lr] = qa.z;
    Bs[lk + 3][lr] = qa.w;
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
    float *Yt = reinterpret_cast<float *>(blk + S.off_xt[args.src ^ 1]);
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int i = i0 + ty + 16 * x, j = j0 + tx + 16 * y;
        const float o = sx * fmaf(args.a, X[int64_t(i) * np + j], acc[x][y]);
        Ya[int64_t(i) * np + j] = o;
        Yt[int64_t(j) * mp + i] = o;
      }
  }
}

}  // namespace

hipError_t launch_elem(const ElemArgs &a, bool bf16, hipStream_t s) {
  if (a.total_tiles <= 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(elem_kernel<__bf16>, dim3(a.total_tiles), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(elem_kernel<float>, dim3(a.total_tiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_norm_finalize(const GemmArgs &a, int views, hipStream_t s) {
  if (views <= 0) return hipSuccess;
  hipLaunchKernelGGL(norm_finalize_kernel, dim3(views), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs &a, int phase, bool bf16, hipStream_t s) {
  if (a.total_tiles <= 0) return hipSuccess;
  const dim3 grid(a.total_tiles), block(256);
  if (bf16) {
    switch (phase) {
      case kGram: hipLaunchKernelGGL(gemm_bf16_kernel<kGram>, grid, block, 0, s, a); break;
      case kAA: hipLaunchKernelGGL(gemm_bf16_kernel<kAA>, grid, block, 0, s, a); break;
      default: hipLaunchKernelGGL(gemm_bf16_kernel<kBX>, grid, block, 0, s, a); break;
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
