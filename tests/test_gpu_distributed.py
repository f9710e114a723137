"""GPU parity of the distributed (column-sharded) mode simulated on one GPU,
through the C ABI: the result against the float64 oracle of the whole matrix
(which the sharded computation must equal up to rounding order), the packed
upper-triangle partial Grams each shard would send, and the summed Gram every
shard receives."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import np64, padded, relF, unblock

pytestmark = pytest.mark.gpu

F32_TOL = 1e-4
BF16_TOL = 2e-2


def rand(shape, dtype, seed, std=0.01):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    _, v = padded(shape[0], shape[1], dtype)
    v.copy_(torch.randn(shape, generator=g, device="cuda") * std)
    return v


@pytest.mark.parametrize("shape,shards", [((256, 1024), 1), ((256, 1024), 4), ((300, 1000), 4),
                                          ((512, 512), 4), ((128, 2048), 8)])
def test_distributed_bf16_matches_whole_matrix(gpu_lib, shape, shards):
    import muon_newton_schulz_03_amd as mu
    X = rand(shape, torch.bfloat16, 21 + shards)
    X0 = np64(X)
    ref = oracle.newton_schulz(X0)
    assert relF(oracle.newton_schulz_distributed(X0, shards), ref) < 1e-12
    Y = X.clone()
    gpu_lib.muon_ns_batched([Y], iters=5, mode=mu.MUON_NS_DISTRIBUTED, col_blocks=shards)
    torch.cuda.synchronize()
    err = relF(np64(Y), ref)
    print(f"{shape} x{shards} shards: relF {err:.3e}")
    assert err <= BF16_TOL


def test_distributed_full_size(gpu_lib):
    """The tensor-parallel benchmark's shape: two 2048 x 7168 MoE matrices,
    each in 8 column shards of 2048 x 896 (a persistent Gram, the packed
    exchange of 8 partials and B X per shard), against the float64 oracle of
    the whole matrix."""
    import muon_newton_schulz_03_amd as mu
    xs = [rand((2048, 7168), torch.bfloat16, 70 + i) for i in range(2)]
    refs = [oracle.newton_schulz(np64(x)) for x in xs]
    ys = [x.clone() for x in xs]
    gpu_lib.muon_ns_batched(ys, iters=5, mode=mu.MUON_NS_DISTRIBUTED | mu.MUON_PACK_COST,
                            col_blocks=[8, 8])
    torch.cuda.synchronize()
    for y, ref in zip(ys, refs):
        err = relF(np64(y), ref)
        print(f"2048x7168 x8 shards: relF {err:.3e}")
        assert err <= BF16_TOL


def test_distributed_f32(gpu_lib):
    import muon_newton_schulz_03_amd as mu
    X = rand((64, 384), torch.float32, 5, std=1.0)
    X0 = np64(X)
    gpu_lib.muon_ns_batched([X], iters=5, mode=mu.MUON_NS_DISTRIBUTED, col_blocks=3)
    torch.cuda.synchronize()
    assert relF(np64(X), oracle.newton_schulz(X0)) <= F32_TOL


def test_distributed_batch_and_step(gpu_lib):
    """Several matrices (grouped launches, cost order) and the full Muon step."""
    import muon_newton_schulz_03_amd as mu
    shapes = [(256, 1024), (128, 512), (256, 1024), (64, 1024)]
    W = [rand(s, torch.bfloat16, 40 + i, std=0.02) for i, s in enumerate(shapes)]
    G = [rand(s, torch.bfloat16, 50 + i, std=1e-3) for i, s in enumerate(shapes)]
    M = [rand(s, torch.bfloat16, 60 + i, std=1e-2) for i, s in enumerate(shapes)]
    W0, G0, M0 = [np64(t) for t in W], [np64(t) for t in G], [np64(t) for t in M]
    Wz = [torch.zeros_like(t) for t in W]
    gpu_lib.muon_step(Wz, G, M, lr=-1.0, beta=float(np.float32(0.95)),
                      mode=mu.MUON_NS_DISTRIBUTED | mu.MUON_PACK_COST, col_blocks=4)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        O_ref, _, _ = oracle.muon_step(W0[i], G0[i], M0[i], lr=0.0, beta=float(np.float32(0.95)))
        assert relF(np64(Wz[i]), O_ref) <= BF16_TOL


def untile_upper(buf, mp):
    """The tile-packed float32 upper triangle of an mp x mp matrix (upper
    256 x 256 tiles, tile (I, J) at index J (J + 1) / 2 + I; in a tile, 32 x 32
    blocks in row-major order; in a block, quads of 4 rows stored column by
    column) as a full matrix whose lower tiles hold NaN."""
    t = mp // 256
    out = np.full((mp, mp), np.nan, np.float32)
    tiles = buf.reshape(-1, 8, 8, 8, 32, 4)  # tile, block row, block col, quad, column, row in quad
    for J in range(t):
        for I in range(J + 1):
            x = tiles[J * (J + 1) // 2 + I]
            # -> block row, quad, row in quad, block col, column
            out[I * 256:(I + 1) * 256, J * 256:(J + 1) * 256] = x.transpose(0, 2, 4, 1, 3).reshape(256, 256)
    return out


@pytest.mark.parametrize("split", [False, True])
def test_packed_partial_grams(gpu_lib, split):
    """After one iteration each shard's buffer holds its partial Gram
    s^2 X_p X_p^T as tile-packed float32 upper tiles (the message a rank
    sends), and the matrix's first shard holds A = the sum of the partials in
    shard order, rounded to bf16 (hi, and lo = the rest when A*A uses both),
    bit for bit, symmetric, mirrored from the upper tiles."""
    import muon_newton_schulz_03_amd as mu
    shape, P = (300, 1000), 4
    X = rand(shape, torch.bfloat16, 7)
    X0 = np64(X)
    mode = mu.MUON_NS_DISTRIBUTED | mu.MUON_PACK_RR | (mu.MUON_AA_SPLIT if split else 0)
    gpu_lib.muon_ns_batched([X], iters=1, mode=mode, col_blocks=P)
    torch.cuda.synchronize()
    desc = mu.mat_of(X, P)
    plan = mu.muon_plan_info([desc], iters=1, mode=mode, workspace_bytes=mu._ws.nbytes)
    seg = plan["chunks"][0]["segments"][0]
    L, mp, stride, base = seg["layout"], seg["mp"], seg["stride"], seg["base"]
    assert mp == 512  # two tile rows: a diagonal and an off-diagonal tile
    buf = mu._ws.buf
    m, w = shape[0], shape[1] // P
    s = 1.0 / (np.linalg.norm(X0) + 1e-7)
    t = mp // 256
    nfl = t * (t + 1) // 2 * 65536
    parts = []
    for p in range(P):
        blk = base + p * stride
        tri = buf[blk + L["tri"]: blk + L["tri"] + nfl * 4].view(torch.float32).cpu().numpy()
        up = untile_upper(tri, mp)
        Xp = np.zeros((mp, w))
        Xp[:m] = X0[:, p * w:(p + 1) * w]
        part = s * s * (Xp @ Xp.T)
        iu = np.triu_indices(mp)
        assert relF(up[iu].astype(np.float64), part[iu]) < 1e-5
        parts.append(up)
    # the sum in shard order, in float32, then rounded as the kernel rounds
    tot = np.zeros((mp, mp), np.float32)
    for up in parts:
        tot = tot + up
    tot = np.triu(tot) + np.triu(tot, 1).T  # symmetrized from the upper triangle
    hi_ref = torch.from_numpy(tot).to(torch.bfloat16)
    lo_ref = torch.from_numpy(tot - hi_ref.float().numpy()).to(torch.bfloat16)
    blk = base
    Ah = unblock(buf[blk + L["ahi"]: blk + L["ahi"] + mp * mp * 2].view(torch.bfloat16), mp, mp).cpu()
    assert torch.equal(Ah, Ah.t())
    assert torch.equal(Ah.view(torch.int16), hi_ref.view(torch.int16))
    if split:
        Al = unblock(buf[blk + L["alo"]: blk + L["alo"] + mp * mp * 2].view(torch.bfloat16), mp, mp).cpu()
        assert torch.equal(Al.view(torch.int16), lo_ref.view(torch.int16))
        A = np64(Ah) + np64(Al)
        assert relF(A[:m, :m], s * s * (X0 @ X0.T)) < 1e-5
    else:
        assert relF(np64(Ah)[:m, :m], s * s * (X0 @ X0.T)) < 4e-3
