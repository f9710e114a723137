"""Pins for the CPU oracle (no GPU).

Nothing here re-types the oracle's own iteration. Each check comes from a
different route to the same mathematics:

* the singular-value closed form: for X = U diag(s) V^T the iteration maps
  every singular value through the scalar quintic p(s) = a s + b s^3 + c s^5
  and keeps U and V (computed with LAPACK's SVD, not with the matrix products
  the oracle uses);
* exact rational values of p composed k times (Python fractions);
* special cases whose answer is known without any matrix product: a single
  row, orthonormal rows, a diagonal matrix, zero iterations, the zero matrix;
* invariants: transpose, orthogonal conjugation, positive scaling;
* blockwise mode against the closed form applied block by block;
* the momentum rule's special cases.

A final test plants plausible mistakes in a copy of the oracle and checks
that these pins catch every one of them.
"""
import inspect
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import muon_oracle as om

COEFFS = (3.4445, -4.7750, 2.0315)
EPS = 1e-7


# ---------------------------------------------------------------------------
# independent references
# ---------------------------------------------------------------------------

def quintic_exact(t, iters, coeffs=COEFFS):
    """p composed ``iters`` times at t, in exact rational arithmetic on the
    binary values of t and of the coefficients."""
    a, b, c = (Fraction(v) for v in coeffs)
    x = Fraction(t)
    for _ in range(iters):
        x2 = x * x
        x = x * (a + x2 * (b + c * x2))
    return float(x)


def quintic_float(s, iters, coeffs=COEFFS):
    a, b, c = coeffs
    s = np.array(s, dtype=np.float64)
    for _ in range(iters):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def closed_form(X, iters, coeffs=COEFFS, eps=EPS):
    """U diag(p^k(s / (||X||_F + eps))) V^T via LAPACK's SVD."""
    U, s, Vt = np.linalg.svd(np.asarray(X, np.float64), full_matrices=False)
    fro = math.sqrt(float(np.sum(s * s)))
    t = s / (fro + eps)
    return (U * quintic_float(t, iters, coeffs)) @ Vt


def relF(x, ref):
    d = np.linalg.norm(np.asarray(x, np.float64) - ref)
    n = np.linalg.norm(ref)
    return d / n if n > 0 else d


# ---------------------------------------------------------------------------
# scalar quintic
# ---------------------------------------------------------------------------

def test_quintic_at_one_is_coefficient_sum():
    # p(1) = a + b + c
    assert quintic_exact(1.0, 1) == pytest.approx(3.4445 - 4.7750 + 2.0315, abs=1e-15)
    assert quintic_exact(1.0, 1) == pytest.approx(0.701, abs=1e-15)


def test_quintic_float_matches_exact():
    for t in (1.0, 0.5, 0.125, 0.01, 0.9, 1.1):
        for k in range(6):
            assert quintic_float(t, k) == pytest.approx(quintic_exact(t, k), rel=1e-14)


# ---------------------------------------------------------------------------
# closed form
# ---------------------------------------------------------------------------

SHAPES = [(1, 7), (7, 1), (4, 4), (5, 9), (9, 5), (64, 128), (128, 64), (33, 70), (70, 33)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("iters", [0, 1, 2, 5, 7])
def test_svd_closed_form(shape, iters):
    rng = np.random.default_rng(hash((shape, iters)) % (2 ** 32))
    X = rng.standard_normal(shape)
    O = oracle.newton_schulz(X, iters=iters)
    assert O.shape == X.shape
    assert relF(O, closed_form(X, iters)) < 1e-12


def test_svd_closed_form_other_coefficients():
    # the classic cubic (1.5, -0.5, 0) and an arbitrary quintic
    rng = np.random.default_rng(11)
    X = rng.standard_normal((12, 20))
    for coeffs in [(1.5, -0.5, 0.0), (2.0, -1.5, 0.5)]:
        O = oracle.newton_schulz(X, iters=4, coeffs=coeffs)
        assert relF(O, closed_form(X, 4, coeffs)) < 1e-12


def test_rank_deficient_closed_form():
    rng = np.random.default_rng(5)
    X = rng.standard_normal((20, 3)) @ rng.standard_normal((3, 30))  # rank 3
    O = oracle.newton_schulz(X)
    assert relF(O, closed_form(X, 5)) < 1e-11
    assert np.linalg.matrix_rank(O, tol=1e-8) == 3


def test_singular_vectors_preserved():
    rng = np.random.default_rng(3)
    X = rng.standard_normal((24, 40))
    U, s, Vt = np.linalg.svd(X, full_matrices=False)
    O = oracle.newton_schulz(X)
    D = U.T @ O @ Vt.T
    off = D - np.diag(np.diag(D))
    assert np.abs(off).max() < 1e-13
    expect = quintic_float(s / (np.sqrt(np.sum(s * s)) + EPS), 5)
    assert np.allclose(np.diag(D), expect, rtol=0, atol=1e-13)


def test_output_singular_values_in_band():
    # p^5 maps [0.01, 1] into roughly [0.68, 1.14]; Gaussian inputs with not
    # too small singular values land in that band.
    rng = np.random.default_rng(9)
    X = rng.standard_normal((32, 256))
    s = np.linalg.svd(oracle.newton_schulz(X), compute_uv=False)
    assert s.min() > 0.6 and s.max() < 1.2


# ---------------------------------------------------------------------------
# special cases
# ---------------------------------------------------------------------------

def test_single_row():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((1, 50))
    nx = float(np.sqrt(np.sum(x * x)))
    O = oracle.newton_schulz(x)
    expect = quintic_exact(nx / (nx + EPS), 5) * x / nx
    assert np.allclose(O, expect, rtol=1e-14, atol=1e-16)
    # eps is negligible here, so the scalar is p^5(1)
    assert float(np.sqrt(np.sum(O * O))) == pytest.approx(quintic_exact(1.0, 5), rel=1e-6)


@pytest.mark.parametrize("m,n,c", [(4, 9, 1.0), (4, 9, 3.0), (64, 100, 0.25), (1, 5, 2.0)])
def test_orthonormal_rows(m, n, c):
    rng = np.random.default_rng(m * n)
    Q, _ = np.linalg.qr(rng.standard_normal((n, m)))
    Q = Q.T  # m x n with orthonormal rows
    O = oracle.newton_schulz(c * Q)
    t = c / (c * math.sqrt(m) + EPS)
    assert np.allclose(O, quintic_exact(t, 5) * Q, rtol=0, atol=1e-13)


def test_orthonormal_values():
    # with eps negligible: m = 4 -> p^5(1/2), m = 64 -> p^5(1/8)
    assert quintic_exact(0.5, 5) == pytest.approx(0.7654385304543396, rel=1e-12)
    assert quintic_exact(0.125, 5) == pytest.approx(0.6881398557760554, rel=1e-12)


def test_diagonal():
    d = np.array([3.0, -1.0, 0.5, 2.0, 0.0])
    X = np.zeros((5, 8))
    X[np.arange(5), np.arange(5)] = d
    O = oracle.newton_schulz(X)
    nd = float(np.sqrt(np.sum(d * d)))
    expect = np.zeros_like(X)
    for i, di in enumerate(d):
        expect[i, i] = quintic_exact(di / (nd + EPS), 5)
    assert np.allclose(O, expect, rtol=0, atol=1e-14)


def test_iters_zero_is_normalization():
    rng = np.random.default_rng(1)
    X = rng.standard_normal((6, 10))
    O = oracle.newton_schulz(X, iters=0)
    assert np.allclose(O, X / (np.linalg.norm(X, "fro") + EPS), rtol=1e-15, atol=0)


def test_zero_matrix():
    O = oracle.newton_schulz(np.zeros((3, 7)))
    assert np.all(O == 0) and np.all(np.isfinite(O))


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def test_transpose_invariance():
    rng = np.random.default_rng(2)
    X = rng.standard_normal((13, 29))
    assert relF(oracle.newton_schulz(X.T), oracle.newton_schulz(X).T) < 1e-13


def test_orthogonal_conjugation():
    rng = np.random.default_rng(4)
    X = rng.standard_normal((10, 17))
    P, _ = np.linalg.qr(rng.standard_normal((10, 10)))
    Q, _ = np.linalg.qr(rng.standard_normal((17, 17)))
    lhs = oracle.newton_schulz(P @ X @ Q)
    rhs = P @ oracle.newton_schulz(X) @ Q
    assert relF(lhs, rhs) < 1e-12


def test_scale_invariance():
    rng = np.random.default_rng(6)
    X = rng.standard_normal((10, 17))
    for alpha in (1e-3, 2.0, 1e3):
        assert relF(oracle.newton_schulz(alpha * X, eps=0.0),
                    oracle.newton_schulz(X, eps=0.0)) < 1e-12


def test_gram_symmetric():
    # the first two products of an iteration are symmetric
    rng = np.random.default_rng(8)
    X = om.frobenius_normalize(rng.standard_normal((9, 21)), EPS)
    A = X @ X.T
    B = -4.775 * A + 2.0315 * (A @ A)
    assert np.array_equal(A, A.T) or np.abs(A - A.T).max() < 1e-16
    assert np.abs(B - B.T).max() < 1e-15


# ---------------------------------------------------------------------------
# blockwise
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape,k", [((8, 24), 3), ((16, 12), 4), ((6, 6), 2)])
def test_blockwise_closed_form(shape, k):
    rng = np.random.default_rng(shape[0] * 100 + k)
    X = rng.standard_normal(shape)
    O = oracle.newton_schulz_blockwise(X, k)
    w = shape[1] // k
    for j in range(k):
        blk = X[:, j * w:(j + 1) * w]
        assert relF(O[:, j * w:(j + 1) * w], closed_form(blk, 5)) < 1e-12


def test_blockwise_not_equivalent_to_full():
    rng = np.random.default_rng(12)
    X = rng.standard_normal((8, 32))
    full = oracle.newton_schulz(X)
    blk = oracle.newton_schulz_blockwise(X, 4)
    assert relF(blk, full) > 1e-2
    assert relF(oracle.newton_schulz_blockwise(X, 1), full) < 1e-15


def test_blockwise_rejects_ragged():
    with pytest.raises(ValueError):
        oracle.newton_schulz_blockwise(np.ones((3, 10)), 3)


# ---------------------------------------------------------------------------
# momentum and the whole step
# ---------------------------------------------------------------------------

def test_momentum_special_cases():
    rng = np.random.default_rng(7)
    M, G = rng.standard_normal((2, 5, 6))
    assert np.array_equal(oracle.momentum_update(M, G, 0.0), G)
    assert np.allclose(oracle.momentum_update(M, np.zeros_like(G), 0.95), 0.95 * M, rtol=0, atol=0)
    # linear in (M, G)
    M2, G2 = rng.standard_normal((2, 5, 6))
    lhs = oracle.momentum_update(M + 2 * M2, G + 2 * G2, 0.9)
    rhs = oracle.momentum_update(M, G, 0.9) + 2 * oracle.momentum_update(M2, G2, 0.9)
    assert np.allclose(lhs, rhs, rtol=1e-14, atol=1e-14)
    # nesterov source with beta = 0 is the gradient
    assert np.array_equal(oracle.ns_source(M, G, 0.0, True), G)
    assert np.array_equal(oracle.ns_source(M, G, 0.5, False), M)


def test_muon_step_closed_form():
    # diagonal momentum: O is known entrywise, so the update is too
    G = np.zeros((4, 6))
    M = np.zeros((4, 6))
    M[np.arange(4), np.arange(4)] = [1.0, 2.0, -3.0, 0.5]
    W = np.full((4, 6), 0.25)
    O, M_new, W_new = oracle.muon_step(W, G, M, lr=0.02, beta=0.95)
    assert np.allclose(M_new, 0.95 * M, rtol=0, atol=0)
    d = 0.95 * np.array([1.0, 2.0, -3.0, 0.5])
    nd = float(np.sqrt(np.sum(d * d)))
    expect_O = np.zeros((4, 6))
    for i in range(4):
        expect_O[i, i] = quintic_exact(d[i] / (nd + EPS), 5)
    assert np.allclose(O, expect_O, rtol=0, atol=1e-14)
    assert np.allclose(W_new, W - 0.02 * expect_O, rtol=0, atol=1e-15)


def test_muon_step_blockwise_uses_blocks():
    rng = np.random.default_rng(10)
    W, G, M = rng.standard_normal((3, 6, 12))
    O, M_new, _ = oracle.muon_step(W, G, M, lr=0.02, beta=0.9, col_blocks=3)
    for j in range(3):
        assert relF(O[:, 4 * j:4 * j + 4], closed_form(M_new[:, 4 * j:4 * j + 4], 5)) < 1e-12


# ---------------------------------------------------------------------------
# row-sampled single iteration
# ---------------------------------------------------------------------------

def test_iteration_rows_match_closed_form():
    # one iteration of the normalized matrix is the closed form with k = 1
    rng = np.random.default_rng(21)
    X = rng.standard_normal((12, 30))
    s = 1.0 / (np.linalg.norm(X) + EPS)
    rows = [0, 5, 11]
    got = oracle.newton_schulz_iteration_rows(X, rows, scale=s)
    assert relF(got, closed_form(X, 1)[rows]) < 1e-13


def test_iteration_rows_second_iteration():
    # applied to the first iterate it gives rows of the second (closed form)
    rng = np.random.default_rng(22)
    X = rng.standard_normal((9, 20))
    X1 = closed_form(X, 1)
    got = oracle.newton_schulz_iteration_rows(X1, [0, 8])
    assert relF(got, closed_form(X, 2)[[0, 8]]) < 1e-12


# ---------------------------------------------------------------------------
# the pins catch planted mistakes
# ---------------------------------------------------------------------------

MUTATIONS = [
    ("B = b * A + c * (A @ A)", "B = b * A + c * A"),           # dropped product
    ("B = b * A + c * (A @ A)", "B = c * A + b * (A @ A)"),     # swapped b, c
    ("X = a * X + B @ X", "X = a * X - B @ X"),                 # sign
    ("X = a * X + B @ X", "X = B @ X"),                         # dropped term
    ("A = X @ X.T", "A = X.T @ X"),                             # transposed Gram
    ("a, b, c = (dtype(v) for v in coeffs)", "c, b, a = (dtype(v) for v in coeffs)"),
    ("X = frobenius_normalize(X, eps)", "X = X / (np.sum(X * X) + eps)"),  # norm squared
    ("X = frobenius_normalize(X, eps)", "X = X / (np.abs(X).max() + eps)"),  # wrong norm
    ("return X.T if transposed else X", "return X"),            # orientation not undone
]


def _pins_pass(ns):
    try:
        rng = np.random.default_rng(99)
        for shape in [(5, 9), (9, 5), (6, 6)]:
            X = rng.standard_normal(shape)
            if relF(ns(X, iters=5), closed_form(X, 5)) > 1e-10:
                return False
        x = rng.standard_normal((1, 8))
        nx = float(np.sqrt(np.sum(x * x)))
        if not np.allclose(ns(x, iters=5), quintic_exact(nx / (nx + EPS), 5) * x / nx, atol=1e-13):
            return False
        return True
    except Exception:
        return False


def test_pins_pass_on_oracle():
    assert _pins_pass(oracle.newton_schulz)


@pytest.mark.parametrize("old,new", MUTATIONS)
def test_pins_catch_planted_mistake(old, new):
    src = inspect.getsource(om.newton_schulz)
    assert old in src
    ns_ns = dict(vars(om))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns_ns)
    assert not _pins_pass(ns_ns["newton_schulz"])


# ---------------------------------------------------------------------------
# distributed (column-sharded) mode: the sum of the shards' partial Grams is
# the Gram of the whole matrix, so the result must be the full-matrix one
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape,shards", [((12, 40), 1), ((12, 40), 4), ((16, 48), 8), ((20, 20), 5)])
def test_distributed_equals_full(shape, shards):
    X = np.random.default_rng(11).standard_normal(shape)
    full = oracle.newton_schulz(X)
    dist = oracle.newton_schulz_distributed(X, shards)
    assert relF(dist, full) < 1e-13
    assert relF(dist, closed_form(X, 5)) < 1e-12


def test_distributed_is_not_blockwise():
    """With several shards the shared Gram makes the result differ from
    orthogonalizing each column block alone."""
    X = np.random.default_rng(12).standard_normal((12, 48))
    assert relF(oracle.newton_schulz_distributed(X, 4), oracle.newton_schulz_blockwise(X, 4)) > 1e-2


def test_distributed_rejects_tall_and_ragged():
    with pytest.raises(ValueError):
        oracle.newton_schulz_distributed(np.ones((8, 4)), 2)
    with pytest.raises(ValueError):
        oracle.newton_schulz_distributed(np.ones((4, 9)), 2)


DIST_MUTATIONS = [
    ("            A = A + P @ P.T", "            A = P @ P.T"),
    ("    nrm = np.sqrt(sum(np.sum(P * P) for P in parts))", "    nrm = np.sqrt(np.sum(parts[0] * parts[0]))"),
    ("        parts = [a * P + B @ P for P in parts]", "        parts = [a * P + B @ P.T.T * 0 + B @ parts[0] * 0 + B @ P * (P is parts[0]) for P in parts]"),
]


@pytest.mark.parametrize("old,new", DIST_MUTATIONS)
def test_distributed_pins_catch_planted_mistake(old, new):
    import inspect
    from oracle import muon_oracle
    src = inspect.getsource(muon_oracle.newton_schulz_distributed)
    assert old in src
    ns = dict(vars(muon_oracle))
    exec(src.replace(old, new), ns)
    orig = oracle.newton_schulz_distributed
    oracle.newton_schulz_distributed = ns["newton_schulz_distributed"]
    try:
        with pytest.raises(AssertionError):
            test_distributed_equals_full((16, 48), 8)
    finally:
        oracle.newton_schulz_distributed = orig
