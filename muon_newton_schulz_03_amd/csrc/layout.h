// Layout of the bf16 Newton-Schulz operands in the workspace (X, X^T, A, B).
//
// "k-blocked": a matrix with C columns (C a multiple of 32; rows padded to a
// multiple of 256) is stored as blocks of 256 rows x 32 columns, each block
// row-major (16 KiB), ordered by 256-row panel and, within a panel, by
// 32-column block. One K step of a GEMM operand tile (256 rows x 32 k) is then
// a single contiguous 16 KiB block, so the global->LDS loads of the K loop
// read whole 128-byte lines (with plain row-major rows every load instruction
// reads 64 bytes from each of 16 rows: half lines, and half the load rate).
// A 256 x 256 output tile is 8 consecutive blocks (128 KiB).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace muon {

__device__ inline int64_t kblk(int64_t r, int64_t c, int64_t cols) {
  return ((r >> 8) * (cols >> 5) + (c >> 5)) * 8192 + (r & 255) * 32 + (c & 31);
}

// "tile-packed" float32 upper triangle: the message of one shard in the
// distributed mode (bf16 path). The upper 256 x 256 tiles (I <= J) of an
// mp x mp symmetric matrix, tile (I, J) at index J (J + 1) / 2 + I, 65536
// floats each. Inside a tile, 8 x 8 blocks of 32 x 32 in row-major block
// order (1024 floats each); inside a block, 8 quads of rows (4 q .. 4 q + 3),
// each stored column by column (32 columns x 4 rows). That is the order in
// which a wave's 32 x 32 MFMA accumulators leave with 16-byte stores: lane l
// holds, in registers 4 g .. 4 g + 3, rows 8 g + 4 (l / 32) .. + 3 of column
// l mod 32, so every store instruction writes 1 KiB contiguously.
constexpr int kTriTileFloats = 65536;
__device__ inline int tri_tile_elem(int r, int c) {
  return ((r >> 5) * 8 + (c >> 5)) * 1024 + ((r & 31) >> 2) * 128 + (c & 31) * 4 + (r & 3);
}

}  // namespace muon
