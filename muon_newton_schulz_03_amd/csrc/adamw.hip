// AdamW step for CDNA4 (gfx950): the optimizer the pages compare Muon with
// (Advancing Emerging Optimizers for Accelerated LLM Training, Table 1).
// The pages do not restate it; this is the published algorithm (Adam's
// bias-corrected moments, Kingma and Ba, Algorithm 1; decoupled weight decay,
// Loshchilov and Hutter, Algorithm 2):
//   m <- b1 m + (1 - b1) g,  v <- b2 v + (1 - b2) g^2,
//   W <- W (1 - lr wd) - lr/(1 - b1^t) * m / (sqrt(v) / sqrt(1 - b2^t) + eps).
// Purely element-wise and HBM bound: per element it reads W, g, m, v and
// writes W, m, v (22 bytes for bf16 parameters with float32 moments), so each
// thread moves whole 16/32-byte runs of 8 elements.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace muon {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct alignas(16) Run8 {
  T e[8];
};

template <typename T>
__global__ __launch_bounds__(256) void adamw_kernel(const AdamArgs args) {
  const int c = int(blockIdx.x) * 256 + int(threadIdx.x);
  if (c >= args.total_chunks) return;
  int vi = 0;
  while (vi + 1 < args.nv && c >= args.v[vi + 1].chunk_begin) ++vi;
  const AdamView &V = args.v[vi];
  const int u = c - V.chunk_begin;
  const int row = u / V.chunks_per_row, col = (u - row * V.chunks_per_row) * 8;
  T *w = static_cast<T *>(V.w) + int64_t(row) * V.ld_w + col;
  const T *g = static_cast<const T *>(V.g) + int64_t(row) * V.ld_g + col;
  float *m = V.m + int64_t(row) * V.ld_m + col;
  float *v = V.v + int64_t(row) * V.ld_v + col;
  const float b1 = args.beta1, b2 = args.beta2;
  auto update = [&](float &wv, float gv, float &mv, float &vv) {
    mv = fmaf(b1, mv, (1.f - b1) * gv);
    vv = fmaf(b2, vv, (1.f - b2) * (gv * gv));
    const float denom = fmaf(sqrtf(vv), args.inv_sqrt_bc2, args.eps);
    wv = fmaf(-args.step_size, mv / denom, wv * args.decay);
  };
  if (V.vec) {
    Run8<T> wr = *reinterpret_cast<const Run8<T> *>(w);
    const Run8<T> gr = *reinterpret_cast<const Run8<T> *>(g);
    f32x4 m0 = *reinterpret_cast<const f32x4 *>(m), m1 = *reinterpret_cast<const f32x4 *>(m + 4);
    f32x4 v0 = *reinterpret_cast<const f32x4 *>(v), v1 = *reinterpret_cast<const f32x4 *>(v + 4);
    float mm[8] = {m0[0], m0[1], m0[2], m0[3], m1[0], m1[1], m1[2], m1[3]};
    float vv[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float wv = float(wr.e[e]);
      update(wv, float(gr.e[e]), mm[e], vv[e]);
      wr.e[e] = T(wv);
    }
    *reinterpret_cast<Run8<T> *>(w) = wr;
    *reinterpret_cast<f32x4 *>(m) = f32x4{mm[0], mm[1], mm[2], mm[3]};
    *reinterpret_cast<f32x4 *>(m + 4) = f32x4{mm[4], mm[5], mm[6], mm[7]};
    *reinterpret_cast<f32x4 *>(v) = f32x4{vv[0], vv[1], vv[2], vv[3]};
    *reinterpret_cast<f32x4 *>(v + 4) = f32x4{vv[4], vv[5], vv[6], vv[7]};
  } else {
    const int n = V.cols - col < 8 ? V.cols - col : 8;
    for (int e = 0; e < n; ++e) {
      float wv = float(w[e]), mv = m[e], vv = v[e];
      update(wv, float(g[e]), mv, vv);
      w[e] = T(wv);
      m[e] = mv;
      v[e] = vv;
    }
  }
}

}  // namespace

hipError_t launch_adamw(const AdamArgs &a, bool bf16, hipStream_t s) {
  if (a.total_chunks <= 0) return hipSuccess;
  const dim3 grid((a.total_chunks + 255) / 256), block(256);
  if (bf16)
    hipLaunchKernelGGL(adamw_kernel<__bf16>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(adamw_kernel<float>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace muon
