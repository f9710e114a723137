// Launch arguments shared by the host runtime and the HIP kernels.
//
// Workspace: every view (a whole matrix, or a column block in blockwise mode)
// owns one block of the caller's workspace holding X (wide orientation,
// ping-pong), on the bf16 path also X^T (ping-pong: the right
// operand of B X with k contiguous), the Gram matrix A (bf16 hi/lo halves,
// or float32), B = b A + c A A, the per-tile partial sums of squares and its
// scale s = 1/(||X||_F + eps).
// The float32 path stores them row-major, the bf16 path k-blocked (layout.h).
// Views of one padded shape sit at a uniform stride ("segment"), so a grouped
// launch needs only a handful of segment descriptors in its kernel arguments.
#pragma once

#include <cstdint>

#include <hip/hip_runtime_api.h>

namespace muon {

constexpr int kSegsMax = 8;
constexpr int kAdamViewsMax = 32;     // matrices per AdamW launch (AdamArgs within 4 KiB)
// views per prep / finish launch: 32 of 120 bytes keep ElemArgs within 4 KiB
// of kernel arguments (against 16: Kimi prep 30.7 -> 29.3 ms per step, the
// Qwen3 experts' 0.94 -> 0.89 ms, fewer launch tails)
constexpr int kPrepViewsMax = 32;
constexpr int kElemTilesPerGroup = 4;  // element-wise launches: 64x64 tiles per workgroup

enum ElemKind : int32_t {
  kPrepNs = 0,    // X0 = data
  kPrepStep = 1,  // M <- beta M + G, X0 = M (or G + beta M)
  kFinishNs = 2,  // data <- O
  kFinishStep = 3 // W <- W - lr O
};

enum Phase : int32_t { kGram = 0, kAA = 1, kBX = 2 };

struct ElemView {
  const void *g;  // gradient view (prep step)
  void *m;        // momentum view (step) or data view (ns)
  void *w;        // weight view (finish step)
  int64_t ld_g, ld_m, ld_w;  // elements
  char *blk;                 // workspace block of the view
  int64_t off_x;             // X (wide orientation: X^T of the user's view if tall)
  int64_t off_xt;            // prep: X^T as well (np x mp), or -1
  int64_t off_part, off_scale;
  int32_t rows, cols;        // view shape, user orientation
  int32_t pitch_x;           // row pitch (elements) of X
  int32_t tall;              // user view is X^T: prep and finish transpose through LDS
  int32_t tiles_c;           // 64-wide tiles along the user's columns
  int32_t tile_begin;        // first tile of this view in the launch
  int32_t vec;               // bit 0/1/2: g/m/w rows start on 16-byte boundaries
  int32_t pitch_xt;          // row pitch (elements) of X^T
};

// Where the result of a view goes, recorded by the prep kernel in the view's
// workspace block (kOutDescOffset bytes into its scale region) and read by
// the last B X, which then writes the caller's matrix itself: data <- O
// (muon_ns_batched) or W <- W - lr O (muon_step), in the user's orientation.
struct OutDesc {
  void *out;       // caller's matrix at the view's first column (W, or the data)
  int64_t ld;      // its row pitch (elements)
  int32_t rows, cols;  // view shape in the user's orientation
  int32_t tall;    // the user's view is X^T (wide X = user transposed)
  int32_t update;  // 1: W <- W - lr O; 0: out <- O
  int32_t vec;     // rows start on 8-byte boundaries (4-element runs)
  int32_t pad_;
};
constexpr int kOutDescOffset = 64;

struct ElemArgs {
  ElemView v[kPrepViewsMax];
  int32_t nv;
  int32_t total_tiles;
  int32_t kind;
  int32_t nesterov;
  int32_t final_scale;  // finish: multiply O by s (iters == 0)
  float beta, lr;
};
static_assert(sizeof(ElemArgs) <= 4096, "prep kernel arguments within 4 KiB");

struct GemmSeg {
  char *base;
  int64_t stride;
  int64_t off_xa[2], off_xt[2], off_ahi, off_alo, off_b, off_bdiag, off_part, off_scale, off_tri;
  int32_t mp, np;
  int32_t count;
  int32_t tiles_per_view;
  int32_t tile_begin;
  int32_t tn;      // tiles along n (B X phase)
  int32_t nparts;  // partial sums per view
  int32_t view_begin;
};

struct GemmArgs {
  GemmSeg seg[kSegsMax];
  int32_t nseg;
  int32_t total_tiles;
  int32_t src;      // X (and X^T) buffer read this iteration; the product goes to src ^ 1
  int32_t first;    // first iteration: apply the normalization scale
  int32_t aa_plain; // A*A and b A from bf16(A) only (no lo half of A)
  int32_t remap;    // XCD-aware tile order
  int32_t persistent; // > 0: grid of this many workgroups (a multiple of 8),
                      // each looping over tiles of its XCD's range
  int32_t xcd_begin[9]; // persistent: XCD x takes tiles [xcd_begin[x], xcd_begin[x + 1])
  int32_t last;       // B X of the last iteration: write the caller's matrices
                      // through each view's OutDesc instead of X'
  float lr;           // muon_step's learning rate (for last)
  int32_t group;      // views per matrix that share one norm and one Gram
                      // (distributed mode: the shards), else 1
  int32_t gram_halves;// bf16 A: 1 writes A hi only, 2 also A lo
  int32_t tri_out;    // bf16 distributed mode: the Gram writes the shard's
                      // float32 partial (tile-packed) instead of A, and A*A
                      // reads the A of the matrix's first shard
  float a, b, c;
  float r;          // b / c: the A*A kernel adds r A inside its K loop, then scales by c
  float eps;
};

// AdamW (the comparator): one element-wise launch over up to kAdamViewsMax
// matrices; each thread updates one run of 8 consecutive elements of a row.
struct AdamView {
  void *w;                     // parameters (T)
  const void *g;               // gradients (T)
  float *m, *v;                // first and second moments (float32)
  int64_t ld_w, ld_g, ld_m, ld_v;
  int32_t rows, cols;
  int32_t chunks_per_row;      // ceil(cols / 8)
  int32_t chunk_begin;         // first chunk of this matrix in the launch
  int32_t vec;                 // every row of every buffer holds whole aligned runs of 8
  int32_t pad_;
};

struct AdamArgs {
  AdamView v[kAdamViewsMax];
  int32_t nv;
  int32_t total_chunks;
  float beta1, beta2, eps;
  float decay;                 // 1 - lr * weight_decay
  float step_size;             // lr / (1 - beta1^t)
  float inv_sqrt_bc2;          // 1 / sqrt(1 - beta2^t)
};
static_assert(sizeof(AdamArgs) <= 4096, "AdamW kernel arguments within 4 KiB");

// Launchers (kernels.hip, adamw.hip). Each returns the HIP error of the launch.
hipError_t launch_elem(const ElemArgs &a, bool bf16, hipStream_t s);
hipError_t launch_norm_finalize(const GemmArgs &a, int views, hipStream_t s);
hipError_t launch_gemm(const GemmArgs &a, int phase, bool bf16, hipStream_t s);
hipError_t launch_adamw(const AdamArgs &a, bool bf16, hipStream_t s);
// Distributed mode (dist.hip).
// bf16: the Gram kernel (tri_out) writes each shard's float32 partial into
// its tile-packed buffer; launch_tile_sum sums the `group` partials of every
// matrix in shard order into the first shard's A (tiles_per_view =
// 4 t (t + 1) / 2 per matrix: a quarter of an upper 256 x 256 tile per
// workgroup, t = mp / 256, count / group matrices per segment).
// float32: pack each shard's Gram into its row-packed upper triangle
// (tiles_per_view = mp: one workgroup per row of a view); sum the packed
// buffers of every matrix's shards in shard order and unpack the sum into
// every shard's A (tiles_per_view = t (t + 1) / 2 upper 64 x 64 tiles per
// matrix, t = mp / 64, with count / group matrices per segment).
// tile_begin holds the prefix over segments in every case.
hipError_t launch_tile_sum(const GemmArgs &a, hipStream_t s);
hipError_t launch_tri_pack(const GemmArgs &a, hipStream_t s);
hipError_t launch_tri_reduce(const GemmArgs &a, hipStream_t s);

// Allocation-free entry point (scratch.hip): the device address of this
// device's scratch array of kNoAllocScratchBytes, looked up on the first call
// per device (with that device current) and cached.
constexpr size_t kNoAllocScratchBytes = size_t(256) << 20;
hipError_t noalloc_scratch(void **ptr);

}  // namespace muon
