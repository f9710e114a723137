"""The k-blocked workspace layout of the bf16 operands, as the GPU tests read
it back (gpu_util.unblock), against the element-offset formula the kernels use:
(r, c) of a matrix with C columns sits at
((r // 256) * (C // 32) + c // 32) * 8192 + (r % 256) * 32 + c % 32."""
import numpy as np
import torch

from gpu_util import unblock


def kblk_offsets(rows, cols):
    r, c = np.meshgrid(np.arange(rows), np.arange(cols), indexing="ij")
    return ((r // 256) * (cols // 32) + c // 32) * 8192 + (r % 256) * 32 + c % 32


def test_kblk_offsets_are_a_permutation():
    for rows, cols in [(256, 32), (512, 96), (768, 2048)]:
        off = kblk_offsets(rows, cols).ravel()
        assert np.array_equal(np.sort(off), np.arange(rows * cols))


def test_unblock_inverts_the_kblk_layout():
    for rows, cols in [(256, 32), (512, 96), (768, 256)]:
        want = torch.arange(rows * cols, dtype=torch.float64).reshape(rows, cols)
        flat = torch.empty(rows * cols, dtype=torch.float64)
        flat[torch.from_numpy(kblk_offsets(rows, cols).ravel())] = want.ravel()
        assert torch.equal(unblock(flat, rows, cols), want)


def test_one_k_step_of_a_panel_is_contiguous():
    # rows i0 .. i0 + 255 and k0 .. k0 + 31 (i0 a multiple of 256, k0 of 32):
    # one 16 KiB block, starting at i0 * cols + (k0 // 32) * 8192 elements
    rows, cols = 768, 2048
    off = kblk_offsets(rows, cols)
    for i0, k0 in [(0, 0), (256, 64), (512, 2016)]:
        blk = off[i0:i0 + 256, k0:k0 + 32].ravel()
        base = i0 * cols + (k0 // 32) * 8192
        assert np.array_equal(blk, base + np.arange(8192))
