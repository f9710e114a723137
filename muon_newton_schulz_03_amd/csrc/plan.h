// Host-side validation and scheduling for the Muon library. Plain C++ with no
// HIP dependency, so it builds and runs on a machine without a GPU.
//
// The unit of work is a "view": one whole matrix, or one column block of it
// in blockwise mode. A view of rows x cols is oriented wide (m = min, n = max;
// transposed when rows > cols) and padded to (mp, np), multiples of the
// kernel tile. Zero padding is exact for the iteration: padded rows and
// columns of X stay zero through A = X X^T, B = b A + c A A and a X + B X.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "muon.h"

namespace muon {

constexpr int kMaxSegs = 8;          // uniform-shape segments per grouped launch
constexpr int kMaxElemViews = 16;    // views per element-wise launch
constexpr int64_t kMaxMinDim = 32768;
constexpr int64_t kMaxMaxDim = 4194304;
constexpr int kMaxIters = 64;
// Above this many iterations A*A always runs from A as bf16 hi + lo: from
// bf16(A) alone the error of O grows with the iteration count (measured on
// 300x520, 768x2048 and 2048x7168: relative Frobenius error 0.6e-2 at 5
// iterations, 1.3-1.4e-2 at 10, 1.7-1.8e-2 at 15, 1.9-2.4e-2 at 20, against
// 1.1e-2 at 15 and 1.9-2.0e-2 at 64 with the split).
constexpr int kPlainMaxIters = 12;
constexpr int32_t kMaxMats = 1 << 20;
constexpr int kPadBf16 = 256;        // bf16 matrix-core tile
constexpr int kPadF32 = 64;          // float32 tile
constexpr int kElemTile = 64;        // element-wise kernels work on 64x64 tiles
constexpr int kGemmTile = 256;

// Byte offsets of the buffers of one view inside its workspace block.
struct Layout {
  size_t xa[2];     // X, mp x np (ping-pong; row-major for float32, k-blocked for bf16)
  size_t xt[2];     // bf16 path: X^T, np x mp k-blocked (ping-pong), read by B X
  size_t ahi, alo;  // A = X X^T (bf16 hi/lo halves; float32 path uses ahi only)
  size_t b;         // B = b A + c A A (bf16 path: diagonal stored as zero)
  size_t bdiag;     // bf16 path: diagonal of B in float32
  size_t partials;  // per-64x64-tile sums of squares (float)
  size_t scale;     // s = 1/(||X||_F + eps), s^2 (float)
  size_t tri;       // distributed mode: this shard's Gram, upper triangle packed
                    // row by row as float32 (mp (mp + 1) / 2 entries)
  size_t total;
  int64_t nparts;
};

Layout view_layout(int64_t mp, int64_t np, bool bf16, bool distributed = false);

struct View {
  int32_t mat = 0, block = 0;  // block: column block (blockwise) or shard (distributed)
  int64_t rows = 0, cols = 0;  // user orientation
  int64_t col_off = 0;         // first column of the block inside the matrix
  bool tall = false;
  int64_t m = 0, n = 0;        // wide
  int64_t mp = 0, np = 0;      // padded wide
  double cost = 0;             // nominal flops iters * (4 m^2 n + 2 m^3)
  size_t bytes = 0;            // workspace block size
};

struct Segment {
  int32_t first = 0, count = 0;  // views [first, first+count) of the plan order
  int64_t mp = 0, np = 0;
  size_t base = 0;               // workspace offset of the first view's block
  size_t stride = 0;             // bytes between consecutive blocks
  int64_t tiles_syrk = 0, tiles_gemm = 0, tiles_elem = 0;  // per view
};

struct Chunk {
  int32_t first = 0, count = 0;
  std::vector<Segment> segs;
  size_t bytes = 0;
};

struct Plan {
  bool bf16 = true;
  bool distributed = false;
  int32_t shards = 1;  // distributed mode: views per matrix, consecutive in every chunk
  int pad = kPadBf16;
  int iters = 5;
  uint32_t mode = 0;
  std::vector<View> views;  // processing order
  std::vector<Chunk> chunks;
  size_t full_bytes = 0, min_bytes = 0;
};

struct Error {
  muon_status status = MUON_OK;
  std::string msg;
  bool set(muon_status s, const std::string &m) {
    status = s;
    msg = m;
    return false;
  }
};

size_t dtype_size(int32_t dtype);

// Checks one descriptor array (shapes, dtype, alignment, blocks).
bool validate_descs(const muon_mat *d, int32_t n, uint32_t mode, const char *what, Error *err);
// muon_step: params/grads/moms agree per matrix.
bool validate_step_triplets(const muon_mat *w, const muon_mat *g, const muon_mat *m, int32_t n,
                            Error *err);
// Written buffers must not overlap any other buffer of the call. `writable`
// flags which of the arrays are written.
bool check_alias(const muon_mat *const *arrays, const bool *writable, int narrays, int32_t n,
                 Error *err);
// No matrix of the call may reach into the workspace [ws, ws + ws_bytes)
// (extent test: the first to the last byte of each matrix).
bool check_workspace_alias(const muon_mat *const *arrays, const char *const *names, int narrays, int32_t n,
                           const void *ws, size_t ws_bytes, Error *err);
bool validate_mode(uint32_t mode, Error *err);

// Orders the views, groups them into chunks that fit `ws_bytes` (0 = as
// many as needed to hold everything at once) and into uniform segments.
bool build_plan(const muon_mat *d, int32_t n, int32_t iters, uint32_t mode, size_t ws_bytes,
                Plan *plan, Error *err);

std::string plan_json(const Plan &p);

// Persistent launches: the tile order (segment by segment, tiles[s] tiles of
// ksteps[s] K steps each) split into 8 contiguous ranges, one per XCD, of
// about equal estimated time, a tile costing its K steps plus a fixed
// kTileOverheadSteps (prologue and epilogue). out[x] .. out[x + 1] is XCD
// x's range; out[0] = 0, out[8] = the total. With mixed K (a group of long
// and short matrices) a split by tile count leaves the XCD that gets the
// long tiles last.
constexpr double kTileOverheadSteps = 16.0;
void xcd_ranges(const int64_t *tiles, const int64_t *ksteps, int nseg, int32_t out[9]);

// Placement of n costs on `ranks` ranks (policy 0: round robin, 1: LPT);
// writes owner[n] and load[ranks]. Arguments are validated by the caller.
void place(const double *costs, int32_t n, int32_t ranks, uint32_t policy, int32_t *owner,
           double *load);

// Exact element-overlap test of two strided matrices (byte addresses).
bool matrices_overlap(const muon_mat &a, const muon_mat &b);

// Upper-triangle tile index u -> (I, J), I <= J, enumerated column by column.
inline void syrk_tile(int64_t u, int64_t *I, int64_t *J) {
  int64_t j = 0;
  while ((j + 1) * (j + 2) / 2 <= u) ++j;
  *J = j;
  *I = u - j * (j + 1) / 2;
}

}  // namespace muon
