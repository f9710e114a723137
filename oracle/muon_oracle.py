"""Plain, slow, obviously correct CPU oracle for the Muon optimizer step.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg call this module; the library never does.

Everything runs in numpy at the precision the caller asks for (float64 for
parity checks, float32 only when the benchmark times the CPU). The one
library primitive used is the matrix product (``@``); there is no blocking,
fusion or reordering beyond the steps written here.

Sources (the pages are web reports of NVIDIA's blog post "Advancing Emerging
Optimizers for Accelerated LLM Training"):

* [zh] wiki.whaty.org, "使用 NVIDIA Megatron 推进新兴优化器以加速 LLM 训练"
  (Chinese translation of the blog post), sections "分布式 Newton-Schulz",
  "Duplicated mode", "Distributed mode" (blockwise paragraph),
  "SYRK 和融合的 all-reduce".
* [de] ki-news-radar.de news summary (running text, no headings).
* [pt] cafecomtech.com, "NVIDIA Megatron ganha suporte a Muon ...",
  section "2. Newton-Schulz distribuído".

What the pages fix: Muon orthogonalizes the whole momentum-buffer matrix of a
layer ([zh] "分布式 Newton-Schulz"); each Newton-Schulz iteration performs three
matrix multiplications, an all-reduce follows the first when the matrix is
column-sharded ([zh] "Distributed mode"; [de]), and the first two are
symmetric rank-k products ([zh] "SYRK 和融合的 all-reduce"); the iteration
count is usually five ([zh] "Duplicated mode"); each GPU then updates its
weights with the orthogonalized momentum ([zh] "Duplicated mode"); blockwise
mode orthogonalizes only the locally held part and is not equivalent to the
whole-matrix result ([zh] "Distributed mode", blockwise paragraph; [pt]).

What the pages leave open, and the reading taken here (each one is also
listed with its reason in the design notes):

* momentum rule ``M <- beta*M + G`` (no dampening, no (1-beta) factor);
* Nesterov source ``G + beta*M_new``;
* the three products of one iteration are ``A = X X^T``, ``B = b A + c A A``,
  ``X <- a X + B X`` -- the only three-product form whose first two products
  are symmetric and whose first product, summed over column shards, is what a
  column-sharded run must all-reduce; it maps every singular value s to
  ``p(s) = a s + b s^3 + c s^5``;
* default coefficients (a, b, c) = (3.4445, -4.7750, 2.0315), used unchanged
  in every iteration;
* Frobenius normalization ``X / (||X||_F + eps)`` with eps = 1e-7 added to
  the norm (not to its square);
* a matrix with more rows than columns is transposed before the iteration and
  transposed back after it (square: no transpose);
* blockwise mode splits the columns into equal blocks; each block is
  oriented and normalized on its own;
* update ``W <- W - lr * O`` with no shape factor and no weight decay.

Parity pins: none of these functions is trusted on its own. The CPU test
suite checks them against the singular-value closed form of the iteration,
exact rational values of the scalar quintic, orthonormal and diagonal special
cases, and the transpose, orthogonal-conjugation, scale and blockwise
invariants.
"""
import numpy as np

DEFAULT_COEFFS = (3.4445, -4.7750, 2.0315)
DEFAULT_EPS = 1e-7


def momentum_update(M, G, beta, dtype=np.float64):
    """Momentum buffer update ``M_new = beta * M + G``.

    The pages only name the momentum buffer that Muon orthogonalizes ([zh]
    "分布式 Newton-Schulz"); the heavy-ball form without dampening is the
    reading taken.
    """
    M = np.asarray(M, dtype=dtype)
    G = np.asarray(G, dtype=dtype)
    return dtype(beta) * M + G


def ns_source(M_new, G, beta, nesterov, dtype=np.float64):
    """Matrix handed to Newton-Schulz: the new momentum, or with Nesterov
    look-ahead ``G + beta * M_new`` (reading; the pages do not mention
    Nesterov)."""
    M_new = np.asarray(M_new, dtype=dtype)
    if not nesterov:
        return M_new
    return np.asarray(G, dtype=dtype) + dtype(beta) * M_new


def orient_wide(X):
    """Return ``(X_wide, transposed)``: a matrix with more rows than columns is
    transposed so that the Gram matrix X X^T is the smaller of the two."""
    if X.shape[0] > X.shape[1]:
        return X.T, True
    return X, False


def frobenius_normalize(X, eps):
    """``X / (||X||_F + eps)`` with the Frobenius norm written out."""
    norm = np.sqrt(np.sum(X * X))
    return X / (norm + X.dtype.type(eps))


def newton_schulz(X, iters=5, coeffs=DEFAULT_COEFFS, eps=DEFAULT_EPS,
                  dtype=np.float64):
    """Newton-Schulz orthogonalization of one whole matrix.

    Steps, in order: orient wide; Frobenius-normalize; ``iters`` times the
    three products ``A = X X^T`` (symmetric), ``B = b A + c A A`` (symmetric),
    ``X = a X + B X``; undo the orientation. Three products per iteration
    ([zh] "Distributed mode"; [de]), the first two symmetric ([zh]
    "SYRK 和融合的 all-reduce"), usually five iterations ([zh]
    "Duplicated mode").
    """
    X = np.array(X, dtype=dtype)
    if X.ndim != 2:
        raise ValueError("newton_schulz expects a matrix")
    a, b, c = (dtype(v) for v in coeffs)
    X, transposed = orient_wide(X)
    X = frobenius_normalize(X, eps)
    for _ in range(iters):
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X.T if transposed else X


def newton_schulz_blockwise(X, col_blocks, iters=5, coeffs=DEFAULT_COEFFS,
                            eps=DEFAULT_EPS, dtype=np.float64):
    """Blockwise mode: split the columns into ``col_blocks`` equal blocks and
    orthogonalize each one on its own, as a GPU holding only its block would
    ([zh] "Distributed mode", blockwise paragraph; [pt] "Blockwise mode").
    Ragged splits are rejected."""
    X = np.asarray(X, dtype=dtype)
    cols = X.shape[1]
    if col_blocks < 1 or cols % col_blocks:
        raise ValueError("col_blocks must divide the column count")
    w = cols // col_blocks
    parts = [newton_schulz(X[:, k * w:(k + 1) * w], iters, coeffs, eps, dtype)
             for k in range(col_blocks)]
    return np.concatenate(parts, axis=1)


def newton_schulz_distributed(X, shards, iters=5, coeffs=DEFAULT_COEFFS,
                              eps=DEFAULT_EPS, dtype=np.float64):
    """Distributed (tensor-parallel) mode: the wide matrix X is split by
    columns into ``shards`` pieces X_p, as P GPUs would hold it ([zh]
    "Distributed mode"; [pt] "2. Newton-Schulz distribuído"). Each iteration
    sums the shards' partial Grams X_p X_p^T in shard order (the all-reduce
    after the first product), forms B from the full A on every shard, and
    updates each shard with its own columns: X_p <- a X_p + B X_p. The norm is
    that of the whole matrix (sum of the shards' squared norms). The result
    equals ``newton_schulz(X)`` up to rounding order; X must be wide
    (rows <= cols) and ``shards`` must divide its column count."""
    X = np.array(X, dtype=dtype)
    rows, cols = X.shape
    if rows > cols or shards < 1 or cols % shards:
        raise ValueError("distributed mode needs a wide matrix and equal column shards")
    a, b, c = (dtype(v) for v in coeffs)
    w = cols // shards
    parts = [X[:, p * w:(p + 1) * w] for p in range(shards)]
    nrm = np.sqrt(sum(np.sum(P * P) for P in parts))
    parts = [P / (nrm + eps) for P in parts]
    for _ in range(iters):
        A = np.zeros((rows, rows), dtype=dtype)
        for P in parts:
            A = A + P @ P.T
        B = b * A + c * (A @ A)
        parts = [a * P + B @ P for P in parts]
    return np.concatenate(parts, axis=1)


def muon_step(W, G, M, lr, beta, nesterov=False, iters=5,
              coeffs=DEFAULT_COEFFS, eps=DEFAULT_EPS, col_blocks=1,
              dtype=np.float64):
    """One Muon step for one layer matrix: momentum, Newton-Schulz on the
    whole matrix (or per column block), weight update with the
    orthogonalized momentum ([zh] "Duplicated mode": each GPU updates the
    weights it owns with the orthogonalized momentum).

    Returns ``(O, M_new, W_new)``.
    """
    M_new = momentum_update(M, G, beta, dtype)
    X = ns_source(M_new, G, beta, nesterov, dtype)
    if col_blocks > 1:
        O = newton_schulz_blockwise(X, col_blocks, iters, coeffs, eps, dtype)
    else:
        O = newton_schulz(X, iters, coeffs, eps, dtype)
    W_new = np.asarray(W, dtype=dtype) - dtype(lr) * O
    return O, M_new, W_new


def newton_schulz_iteration_rows(X, rows, coeffs=DEFAULT_COEFFS, scale=1.0,
                                 dtype=np.float64):
    """Selected rows of one Newton-Schulz iteration applied to ``scale * X``
    (X already oriented wide): rows of ``a Y + (b A + c A A) Y`` with
    ``Y = scale * X`` and ``A = Y Y^T``.

    Row i needs only matrix-vector products: ``A[i,:] = Y Y[i]``,
    ``(A A)[i,:] = Y (Y^T A[i,:])`` and ``(B Y)[i] = Y^T B[i,:]``. This lets a
    check recompute one iteration exactly for a few rows of a matrix too large
    for the whole-matrix oracle.
    """
    a, b, c = (dtype(v) for v in coeffs)
    Y = np.asarray(X, dtype=dtype) * dtype(scale)
    out = []
    for i in rows:
        y = Y[i]
        Ai = Y @ y
        AAi = Y @ (Y.T @ Ai)
        Bi = b * Ai + c * AAi
        out.append(a * y + Y.T @ Bi)
    return np.array(out)
