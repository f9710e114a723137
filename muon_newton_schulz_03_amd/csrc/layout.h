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

}  // namespace muon
