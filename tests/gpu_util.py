"""Helpers shared by the GPU tests (comparison metrics and buffers)."""
import numpy as np
import torch


def np64(t):
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def relF(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    n = np.linalg.norm(ref)
    d = np.linalg.norm(x - ref)
    return d / n if n > 0 else d


def bf16_round(a):
    """Round float64 values to bf16 (nearest even), returned as float64."""
    t = torch.tensor(np.asarray(a, np.float64), dtype=torch.float64)
    return t.to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()


def bf16_ulp_diff(a, b):
    """Per-element distance in bf16 ulps between two bf16-representable arrays
    (measured by bit pattern; sign changes count through zero)."""
    ta = torch.tensor(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).to(torch.int64)
    tb = torch.tensor(np.asarray(b, np.float32)).to(torch.bfloat16).view(torch.int16).to(torch.int64)

    def ordered(x):  # map sign-magnitude bf16 bits onto a monotone integer line
        mag = x & 0x7FFF
        return torch.where(x < 0, -mag, mag)
    return (ordered(ta) - ordered(tb)).abs().numpy()


def padded(rows, cols, dtype, ld=None, device="cuda", fill=None):
    """A rows x cols view with row pitch ld inside a larger buffer whose
    padding holds `fill` (NaN by default, so stray reads or writes show)."""
    ld = cols if ld is None else ld
    base = torch.full((rows, ld), float("nan") if fill is None else fill, dtype=dtype, device=device)
    return base, base[:, :cols]


def unblock(t, rows, cols):
    """Row-major copy of a bf16 workspace operand (X, X^T, A or B), which the
    library keeps k-blocked: blocks of 256 rows x 32 columns, row-major inside,
    ordered by 256-row panel and then by 32-column block."""
    return t.reshape(rows // 256, cols // 32, 256, 32).permute(0, 2, 1, 3).reshape(rows, cols).contiguous()
