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


GUARD_ROWS = 4
_guarded = []  # (base, rows, cols, fill) of every buffer padded() made since the last check


def padded(rows, cols, dtype, ld=None, device="cuda", fill=None):
    """A rows x cols view with row pitch ld inside a larger buffer whose
    padding holds `fill` (NaN by default, so stray reads or writes show): the
    pitch padding of every row, and GUARD_ROWS whole rows before the first
    row and after the last. Returns (base, view); base[:, cols:] is the pitch
    padding. Every such buffer is recorded, and check_guards() (run after each
    GPU test by the conftest fixture) verifies that its padding is untouched."""
    ld = cols if ld is None else ld
    g = GUARD_ROWS
    full = torch.full((rows + 2 * g, ld), float("nan") if fill is None else fill, dtype=dtype, device=device)
    _guarded.append((full, rows, cols, fill))
    base = full[g:g + rows]
    return base, base[:, :cols]


def check_guards(release=None):
    """Asserts that nothing wrote outside the views padded() handed out: the
    guard rows before and after each view and the pitch padding of its rows
    still hold their fill. Without `release` the record is cleared; with it,
    only the buffers of the listed tensors are dropped from the record (so
    that they can be freed) and the others stay recorded."""
    items = list(_guarded)
    if release is None:
        _guarded.clear()
    else:
        gone = {t.untyped_storage().data_ptr() for t in release}
        _guarded[:] = [x for x in _guarded if x[0].untyped_storage().data_ptr() not in gone]
    g = GUARD_ROWS
    for full, rows, cols, fill in items:
        pad = [full[:g], full[g + rows:], full[g:g + rows, cols:]]
        for t in pad:
            if t.numel() == 0:
                continue
            t = t.float()
            ok = torch.isnan(t).all() if fill is None else (t == fill).all()
            assert bool(ok), f"a write landed outside a {rows} x {cols} view (pitch {full.shape[1]})"


def clear_guards():
    _guarded.clear()


def unblock(t, rows, cols):
    """Row-major copy of a bf16 workspace operand (X, X^T, A or B), which the
    library keeps k-blocked: blocks of 256 rows x 32 columns, row-major inside,
    ordered by 256-row panel and then by 32-column block."""
    return t.reshape(rows // 256, cols // 32, 256, 32).permute(0, 2, 1, 3).reshape(rows, cols).contiguous()


def guarded_copy(t):
    """A copy of a 2-D device tensor inside a padded() buffer (guard rows and
    their check included)."""
    _, v = padded(t.shape[0], t.shape[1], t.dtype, device=t.device)
    v.copy_(t)
    return v
