"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Small and ragged shapes that span several tiles and leave ragged tails, both
precision paths, every mode bit, and the edge cases (zero iterations, zero
matrix, NaN input, empty batch, single row/column). Tolerances: relative
Frobenius error <= 1e-4 on the float32 path and <= 2e-2 on the bf16 path
(per matrix, against the float64 oracle on the same stored inputs); the
element-wise kernels within 1 bf16 ulp.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import bf16_round, bf16_ulp_diff, np64, padded, relF, unblock

pytestmark = pytest.mark.gpu

F32_TOL = 1e-4
BF16_TOL = 2e-2


def rand(shape, dtype, seed, std=1.0, ld=None):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    base, view = padded(shape[0], shape[1], dtype, ld)
    view.copy_(torch.randn(shape, generator=g, device="cuda", dtype=torch.float32) * std)
    return base, view


# ---------------------------------------------------------------------------
# float32 path
# ---------------------------------------------------------------------------

def test_f32_step_64x128(gpu_lib):
    from muon_newton_schulz_03_amd.workloads import WORKLOADS, make_inputs
    wl = WORKLOADS["fp32_64x128"]
    W, G, M = make_inputs(wl)
    W0, G0, M0 = np64(W[0]), np64(G[0]), np64(M[0])
    gpu_lib.muon_step(W, G, M, lr=wl.lr, beta=wl.beta, nesterov=wl.nesterov, iters=wl.iters)
    torch.cuda.synchronize()
    O_ref, M_ref, W_ref = oracle.muon_step(W0, G0, M0, lr=wl.lr, beta=wl.beta)
    assert relF(np64(M[0]), M_ref) <= F32_TOL
    assert relF(W0 - np64(W[0]), W0 - W_ref) <= F32_TOL


# (600, 700) and (1100, 577): 10 row panels of 64, so the SYRK tiles run in
# bands of 8 column panels, the last one 2 wide
@pytest.mark.parametrize("shape,ld", [((100, 37), 40), ((37, 100), 103), ((1, 50), 50), ((64, 64), 64),
                                      ((130, 260), 264), ((300, 7), 7), ((65, 65), 66),
                                      ((600, 700), 704), ((1100, 577), 580)])
def test_f32_ns_ragged(gpu_lib, shape, ld):
    base, X = rand(shape, torch.float32, 7, ld=ld)
    X0 = np64(X)
    gpu_lib.muon_ns_batched([X], iters=5)
    torch.cuda.synchronize()
    assert relF(np64(X), oracle.newton_schulz(X0)) <= F32_TOL
    if ld > shape[1]:
        assert torch.isnan(base[:, shape[1]:]).all()  # pitch padding untouched


@pytest.mark.parametrize("iters", [0, 1, 3])
def test_f32_iters(gpu_lib, iters):
    _, X = rand((40, 90), torch.float32, 3)
    X0 = np64(X)
    gpu_lib.muon_ns_batched([X], iters=iters)
    torch.cuda.synchronize()
    assert relF(np64(X), oracle.newton_schulz(X0, iters=iters)) <= F32_TOL


# ---------------------------------------------------------------------------
# bf16 path
# ---------------------------------------------------------------------------

# (2100, 2400): 9 row panels of 256 (B X in a band of 8 row panels and one
# of 1, the SYRK tiles in a band of 8 column panels and one of 1);
# (2600, 2305), tall: 10 (last bands 2 wide)
BF16_SHAPES = [((300, 520), 520), ((520, 300), 304), ((256, 256), 256), ((1, 64), 64), ((64, 1), 8),
               ((1, 96), 96), ((2, 300), 304),
               ((777, 1030), 1032), ((512, 2048), 2048), ((1030, 777), 777),
               ((2100, 2400), 2400), ((2600, 2305), 2312)]


@pytest.mark.parametrize("shape,ld", BF16_SHAPES)
def test_bf16_ns_ragged(gpu_lib, shape, ld):
    base, X = rand(shape, torch.bfloat16, 11, std=0.01, ld=ld)
    X0 = np64(X)
    gpu_lib.muon_ns_batched([X], iters=5)
    torch.cuda.synchronize()
    err = relF(np64(X), oracle.newton_schulz(X0))
    print(f"shape {shape} relF {err:.3e}")
    assert err <= BF16_TOL
    if ld > shape[1]:
        assert torch.isnan(base[:, shape[1]:].float()).all()


@pytest.mark.parametrize("nesterov", [False, True])
def test_bf16_step_batch(gpu_lib, nesterov):
    shapes = [(300, 520), (520, 300), (256, 768), (64, 64), (1, 96)]
    G = [rand(s, torch.bfloat16, 100 + i, std=1e-3)[1] for i, s in enumerate(shapes)]
    M = [rand(s, torch.bfloat16, 200 + i, std=1e-2)[1] for i, s in enumerate(shapes)]
    W = [rand(s, torch.bfloat16, 300 + i, std=0.02)[1] for i, s in enumerate(shapes)]
    G0, M0, W0 = [np64(t) for t in G], [np64(t) for t in M], [np64(t) for t in W]
    # the ABI takes lr and beta as float32; the oracle gets those same values
    lr, beta = float(np.float32(0.02)), float(np.float32(0.95))
    # run 1: W = 0 and lr = -1 make W_new = O exactly (O is bf16 already)
    Wz = [torch.zeros_like(t) for t in W]
    Mc = [t.clone() for t in M]
    gpu_lib.muon_step(Wz, G, Mc, lr=-1.0, beta=beta, nesterov=nesterov)
    torch.cuda.synchronize()
    O_gpu = [np64(t) for t in Wz]
    for i in range(len(shapes)):
        O_ref, M_ref, _ = oracle.muon_step(W0[i], G0[i], M0[i], lr=lr, beta=beta, nesterov=nesterov)
        err = relF(O_gpu[i], O_ref)
        print(f"{shapes[i]} O relF {err:.3e}")
        assert err <= BF16_TOL
        assert bf16_ulp_diff(np64(Mc[i]), bf16_round(M_ref)).max() <= 1
    # run 2: real weights; the update is pinned given the O of run 1
    Mc2 = [t.clone() for t in M]
    gpu_lib.muon_step(W, G, Mc2, lr=lr, beta=beta, nesterov=nesterov)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        assert torch.equal(Mc2[i], Mc[i])
        expect = bf16_round(W0[i] - lr * O_gpu[i])
        assert bf16_ulp_diff(np64(W[i]), expect).max() <= 1


@pytest.mark.parametrize("iters,coeffs", [(1, None), (2, None), (7, None), (3, (2.0, -1.5, 0.5)),
                                          (10, None), (12, None), (13, None), (20, None), (40, None)])
def test_bf16_step_iters_and_coeffs(gpu_lib, iters, coeffs):
    """muon_step with other iteration counts (iters = 1: the first B X, which
    applies the normalization, is also the one that writes the weights) and
    user coefficients, against the oracle with the same (float32-rounded)
    coefficients. Up to 12 iterations A*A runs from bf16(A) (the default
    mode); from 13 on the library switches to the split A (hi + lo), whose
    error stays inside the bound up to the 64-iteration limit."""
    import muon_newton_schulz_03_amd as mu
    c = mu.DEFAULT_COEFFS if coeffs is None else coeffs
    c32 = tuple(float(np.float32(x)) for x in c)
    shapes = [(300, 520), (520, 300), (256, 768)]
    G = [rand(s, torch.bfloat16, 400 + i, std=1e-3)[1] for i, s in enumerate(shapes)]
    M = [rand(s, torch.bfloat16, 500 + i, std=1e-2)[1] for i, s in enumerate(shapes)]
    G0, M0 = [np64(t) for t in G], [np64(t) for t in M]
    beta = float(np.float32(0.95))
    Wz = [torch.zeros_like(t) for t in G]
    gpu_lib.muon_step(Wz, G, M, lr=-1.0, beta=beta, iters=iters, coeffs=c)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        O_ref, _, _ = oracle.muon_step(np.zeros(shapes[i]), G0[i], M0[i], lr=-1.0, beta=beta,
                                       iters=iters, coeffs=c32)
        err = relF(np64(Wz[i]), O_ref)
        print(f"{shapes[i]} iters {iters} coeffs {c} O relF {err:.3e}")
        assert err <= BF16_TOL


@pytest.mark.parametrize("shape,k", [((512, 1536), 3), ((1024, 768), 4), ((300, 520), 2)])
def test_bf16_blockwise(gpu_lib, shape, k):
    import muon_newton_schulz_03_amd as mu
    _, X = rand(shape, torch.bfloat16, 21, std=0.01)
    X0 = np64(X)
    Y = X.clone()
    gpu_lib.muon_ns_batched([X], iters=5, mode=mu.MUON_NS_BLOCKWISE | mu.MUON_PACK_COST, col_blocks=k)
    # the same blocks as separate (strided) matrices in one call
    w = shape[1] // k
    gpu_lib.muon_ns_batched([Y[:, j * w:(j + 1) * w] for j in range(k)], iters=5)
    torch.cuda.synchronize()
    assert torch.equal(X, Y)
    ref = oracle.newton_schulz_blockwise(X0, k)
    for j in range(k):
        assert relF(np64(X[:, j * w:(j + 1) * w]), ref[:, j * w:(j + 1) * w]) <= BF16_TOL
    assert relF(np64(X), oracle.newton_schulz(X0)) > 5e-2  # not the whole-matrix result


@pytest.mark.parametrize("split", [False, True])
def test_bf16_symmetric_intermediates(gpu_lib, split):
    """After one iteration the workspace holds A (hi, and lo in split mode)
    and B of it: bitwise symmetric (mirrored), A equal to s^2 X0 X0^T, zero
    padding, B = b A + c A A with its diagonal in float32, and X1 (in the
    caller's matrix)."""
    import muon_newton_schulz_03_amd as mu
    shape = (300, 520)
    _, X = rand(shape, torch.bfloat16, 5, std=0.01)
    X0 = np64(X)
    mode = mu.MUON_PACK_RR | (mu.MUON_AA_SPLIT if split else mu.MUON_AA_PLAIN)
    gpu_lib.muon_ns_batched([X], iters=1, mode=mode)
    torch.cuda.synchronize()
    plan = mu.muon_plan_info([mu.mat_of(X)], iters=1, mode=mode, workspace_bytes=mu._ws.nbytes)
    seg = plan["chunks"][0]["segments"][0]
    L = seg["layout"]
    mp, np_ = seg["mp"], seg["np"]
    buf = mu._ws.buf

    def mat(off, rows, cols):  # the workspace operands are k-blocked
        return unblock(buf[seg["base"] + off: seg["base"] + off + rows * cols * 2].view(torch.bfloat16), rows, cols)
    Ah, Al, B = mat(L["ahi"], mp, mp), mat(L["alo"], mp, mp), mat(L["b"], mp, mp)
    s = 1.0 / (np.linalg.norm(X0) + 1e-7)
    m, n = shape
    # prep wrote X0 and X0^T (the right operand of B X), zero-padded, exactly
    Xa, Xt = np64(mat(L["xa"][0], mp, np_)), np64(mat(L["xt"][0], np_, mp))
    assert np.array_equal(Xa[:m, :n], X0) and np.array_equal(Xt, Xa.T)
    assert not Xa[m:, :].any() and not Xa[:, n:].any()
    Aref = s * s * (X0 @ X0.T)
    if split:
        A = np64(Ah) + np64(Al)
        assert torch.equal(Al, Al.t())
        assert relF(A[:m, :m], Aref) < 1e-4
    else:
        A = np64(Ah)                        # bf16(A): within half an ulp per element
        assert relF(A[:m, :m], Aref) < 2.0 ** -8
    print(f"A relF {relF(A[:m, :m], Aref):.3e}")
    for T in (Ah, B):
        assert torch.equal(T, T.t())
    assert np.all(A[m:, :] == 0) and np.all(A[:, m:] == 0)
    # B's diagonal is kept in float32 (bdiag); B itself stores bf16(a + B_ii)
    # there, the hi part of B X's diagonal term (a + B_ii) X
    off = seg["base"] + L["bdiag"]
    bd32 = buf[off: off + mp * 4].view(torch.float32).cpu()
    a32 = torch.tensor(3.4445, dtype=torch.float32)
    assert torch.equal(torch.diagonal(B).cpu().view(torch.int16), (a32 + bd32).to(torch.bfloat16).view(torch.int16))
    bdiag = bd32.numpy().astype(np.float64)
    Bfull = np64(B) - np.diag(np.diag(np64(B))) + np.diag(bdiag)
    Bdev = -4.7750 * A + 2.0315 * (A @ A)   # from the device's own A
    Bref = -4.7750 * Aref + 2.0315 * (Aref @ Aref)
    print(f"B relF vs device A {relF(Bfull[:m, :m], Bdev[:m, :m]):.3e}, vs exact {relF(Bfull[:m, :m], Bref):.3e}")
    assert relF(Bfull[:m, :m], Bdev[:m, :m]) < 1e-2
    assert np.allclose(bdiag, np.diag(Bdev), rtol=1e-4, atol=1e-6)
    # the last B X writes X1 straight into the caller's matrix
    X1 = np64(X)
    X1ref = s * (3.4445 * X0 + Bref @ X0)
    print(f"X1 relF {relF(X1, X1ref):.3e}")
    assert relF(X1, X1ref) < 1e-2


def test_bf16_deterministic_and_packing_invariant(gpu_lib):
    import muon_newton_schulz_03_amd as mu
    shapes = [(256, 768), (520, 300), (512, 1024), (300, 520), (256, 768)]
    src = [rand(s, torch.bfloat16, 40 + i, std=0.01)[1] for i, s in enumerate(shapes)]
    outs = []
    for mode, cap in [(mu.MUON_PACK_COST, None), (mu.MUON_PACK_COST, None), (mu.MUON_PACK_RR, None),
                      (mu.MUON_PACK_RR, 1)]:
        xs = [t.clone() for t in src]
        if cap is not None:  # a workspace of one matrix: one group per matrix
            mu._ws = None
            cap = mu.muon_workspace_min_size([mu.mat_of(t) for t in xs], mode)
        gpu_lib.muon_ns_batched(xs, iters=5, mode=mode, max_workspace_bytes=cap)
        torch.cuda.synchronize()
        outs.append(xs)
        mu._ws = None
    for other in outs[1:]:
        for a, b in zip(outs[0], other):
            assert torch.equal(a, b)


@pytest.mark.parametrize("dtype,tol", [(torch.bfloat16, BF16_TOL), (torch.float32, F32_TOL)])
def test_iters_zero_normalizes(gpu_lib, dtype, tol):
    _, X = rand((300, 520), dtype, 8, std=0.3)
    X0 = np64(X)
    gpu_lib.muon_ns_batched([X], iters=0)
    torch.cuda.synchronize()
    assert relF(np64(X), oracle.newton_schulz(X0, iters=0)) <= (5e-3 if dtype == torch.bfloat16 else tol)


def test_zero_and_nan_matrices(gpu_lib):
    Z = torch.zeros((130, 300), dtype=torch.bfloat16, device="cuda")
    _, N = rand((130, 300), torch.bfloat16, 9, std=0.01)
    N[5, 7] = float("nan")
    _, X = rand((130, 300), torch.bfloat16, 10, std=0.01)
    X0 = np64(X)
    gpu_lib.muon_ns_batched([Z, N, X], iters=5)
    torch.cuda.synchronize()
    assert torch.all(Z == 0)
    assert torch.isnan(N.float()).all()       # the norm is NaN, so every entry is
    assert torch.isfinite(X.float()).all()    # neighbours in the batch are unaffected
    assert relF(np64(X), oracle.newton_schulz(X0)) <= BF16_TOL


def test_empty_batch(gpu_lib):
    gpu_lib.muon_ns_batched([], iters=5)
    gpu_lib.muon_step([], [], [], lr=0.02, beta=0.95)


def test_aa_modes(gpu_lib):
    """bf16(A) (the default) and the hi + lo split both meet the bar; the
    split is the more accurate of the two."""
    import muon_newton_schulz_03_amd as mu
    _, X = rand((512, 2048), torch.bfloat16, 12, std=0.01)
    X0 = np64(X)
    ref = oracle.newton_schulz(X0)
    err = {}
    for name, aa in [("plain", mu.MUON_AA_PLAIN), ("split", mu.MUON_AA_SPLIT)]:
        Y = X.clone()
        gpu_lib.muon_ns_batched([Y], iters=5, mode=aa)
        torch.cuda.synchronize()
        err[name] = relF(np64(Y), ref)
    print(f"A*A modes relF {err}")
    assert err["plain"] <= BF16_TOL and err["split"] <= BF16_TOL
    assert err["split"] < err["plain"]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_checkpoint_resume_bitwise(gpu_lib, dtype):
    """The library carries no state between steps beyond W and M: two steps
    in a row equal, bit for bit, one step, a checkpoint of W and M through
    host memory, a workspace overwritten with NaN, and the second step from
    the restored buffers."""
    import muon_newton_schulz_03_amd as mu
    shapes = [(300, 520), (520, 300), (768, 2048)] if dtype == torch.bfloat16 else [(64, 128), (100, 37)]
    G1 = [rand(s, dtype, 600 + i, std=1e-3)[1] for i, s in enumerate(shapes)]
    G2 = [rand(s, dtype, 700 + i, std=1e-3)[1] for i, s in enumerate(shapes)]
    M0 = [rand(s, dtype, 800 + i, std=1e-2)[1] for i, s in enumerate(shapes)]
    W0 = [rand(s, dtype, 900 + i, std=0.02)[1] for i, s in enumerate(shapes)]
    W, M = [t.clone() for t in W0], [t.clone() for t in M0]
    gpu_lib.muon_step(W, G1, M)
    gpu_lib.muon_step(W, G2, M)
    Wr, Mr = [t.clone() for t in W0], [t.clone() for t in M0]
    gpu_lib.muon_step(Wr, G1, Mr)
    torch.cuda.synchronize()
    ckW, ckM = [t.cpu() for t in Wr], [t.cpu() for t in Mr]
    del Wr, Mr
    mu._ws.buf.fill_(0xFF)  # all-ones bytes: NaN in bf16 and float32
    Wr, Mr = [t.cuda() for t in ckW], [t.cuda() for t in ckM]
    gpu_lib.muon_step(Wr, G2, Mr)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        assert torch.equal(W[i], Wr[i]), shapes[i]
        assert torch.equal(M[i], Mr[i]), shapes[i]
