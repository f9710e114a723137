"""FLOP and byte accounting for the Muon step (host arithmetic on shapes only).

Per view (a matrix, or a column block in blockwise mode) of wide shape m x n
(m = min, n = max) and `iters` iterations of A = X X^T, B = b A + c A A,
X = a X + B X:

* nominal FLOPs:      iters * (2 m^2 n + 2 m^3 + 2 m^2 n)   -- three full products
* algorithmic FLOPs:  iters * (m (m+1) n + m^2 (m+1) + 2 m^2 n)
  -- the upper triangle (diagonal included) of both symmetric products plus
  the full B X: the work the method needs once the mirrored half is skipped.

Element-wise traffic of the step, algorithmic: momentum reads G and M and
writes M; the update reads W and O and writes W -- 6 element accesses.
"""


def wide(rows, cols):
    return (rows, cols) if rows <= cols else (cols, rows)


def views(shapes, col_blocks=1):
    out = []
    for (r, c) in shapes:
        k = col_blocks if col_blocks and col_blocks > 1 else 1
        if c % k:
            raise ValueError("col_blocks must divide cols")
        out.extend([(r, c // k)] * k)
    return out


def flops_nominal(m, n, iters):
    return iters * (4 * m * m * n + 2 * m ** 3)


def flops_algorithmic(m, n, iters):
    return iters * (m * (m + 1) * n + m * m * (m + 1) + 2 * m * m * n)


def phase_flops_algorithmic(m, n):
    """Per iteration: (Gram, A*A, B*X)."""
    return m * (m + 1) * n, m * m * (m + 1), 2 * m * m * n


def syrk_tiles(m, tile):
    t = -(-m // tile)
    return t * (t + 1) // 2


def syrk_executed_fraction(m, tile):
    t = -(-m // tile)
    return t * (t + 1) / (2 * t * t)


def workload_flops(shapes, iters, col_blocks=1):
    nom = alg = 0
    for (r, c) in views(shapes, col_blocks):
        m, n = wide(r, c)
        nom += flops_nominal(m, n, iters)
        alg += flops_algorithmic(m, n, iters)
    return nom, alg


def workload_phase_flops(shapes, col_blocks=1):
    g = a = b = 0
    for (r, c) in views(shapes, col_blocks):
        m, n = wide(r, c)
        x, y, z = phase_flops_algorithmic(m, n)
        g, a, b = g + x, a + y, b + z
    return g, a, b


def elementwise_bytes(shapes, elem_size):
    """Algorithmic HBM bytes of momentum + update for one step."""
    n = sum(r * c for (r, c) in shapes)
    return 6 * n * elem_size


def prep_bytes(shapes, elem_size, transposed=True):
    """HBM bytes of the prep pass: read G and M, write M and the
    Newton-Schulz source X0, and X0^T as well when `transposed` (the bf16
    path with iterations, whose B X reads X with k contiguous). The update
    itself runs inside the last B X."""
    n = sum(r * c for (r, c) in shapes)
    return (5 if transposed else 4) * n * elem_size
