"""C ABI checks that need no GPU: the library loads and exports every symbol
the header declares; validation rejects bad calls with the documented status
before anything is launched; the planner's orientation, padding, ordering,
grouping and tile counts; the FLOP accounting.

Device pointers here are fake and are never dereferenced: every call either
fails validation or is a host-only planner query, and no workspace is set, so
no call can reach a kernel launch.
"""
import ctypes
import os
import re

import pytest

import muon_newton_schulz_03_amd as mu
from muon_newton_schulz_03_amd import accounting as acc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 32  # 256-byte aligned, never dereferenced


def header_functions():
    txt = open(os.path.join(ROOT, "include", "muon.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(muon_[a-z_]+)\s*\(", txt)))


def desc(rows, cols, dtype=mu.MUON_BF16, ld=None, ptr=FAKE, col_blocks=1):
    return mu.muon_mat(ctypes.c_void_p(ptr), rows, cols, cols if ld is None else ld, dtype, col_blocks)


@pytest.fixture(scope="module")
def lib():
    return mu.load_library()


def test_exports_every_header_symbol(lib):
    names = header_functions()
    assert set(names) == set(mu.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def status_of(fn, *args):
    return fn(*args)


def test_ns_validation_codes(lib):
    mu.muon_set_workspace(None, 0)
    call = lambda ds, n=None, iters=5, mode=0: lib.muon_ns_batched(
        mu.mats(ds), len(ds) if n is None else n, iters, None, mode)
    assert call([], 0) == mu.MUON_OK                                   # no-op
    assert lib.muon_ns_batched(None, 1, 5, None, 0) == mu.MUON_ERR_INVALID_ARG
    assert call([desc(4, 8)], n=-1) == mu.MUON_ERR_INVALID_ARG
    assert call([desc(4, 8)], iters=-1) == mu.MUON_ERR_INVALID_ARG
    assert call([desc(4, 8)], iters=65) == mu.MUON_ERR_INVALID_ARG
    assert call([desc(4, 8)], mode=0x4) == mu.MUON_ERR_INVALID_ARG
    both = mu.MUON_NS_BLOCKWISE | mu.MUON_NS_DISTRIBUTED
    assert call([desc(4, 8, col_blocks=2)], mode=both) == mu.MUON_ERR_INVALID_ARG
    dist = mu.MUON_NS_DISTRIBUTED
    assert call([desc(9, 8, col_blocks=2)], mode=dist) == mu.MUON_ERR_SHAPE      # tall
    assert call([desc(4, 9, col_blocks=2)], mode=dist) == mu.MUON_ERR_SHAPE      # 2 does not divide 9
    assert call([desc(4, 8, col_blocks=2), desc(4, 8, col_blocks=4, ptr=FAKE * 2)],
                mode=dist) == mu.MUON_ERR_SHAPE                                    # unequal shard counts
    assert call([desc(4, 8, ptr=0)]) == mu.MUON_ERR_INVALID_ARG
    assert call([desc(0, 8)]) == mu.MUON_ERR_SHAPE
    assert call([desc(4, -1)]) == mu.MUON_ERR_SHAPE
    assert call([desc(4, 8, ld=7)]) == mu.MUON_ERR_SHAPE
    assert call([desc(40000, 40000)]) == mu.MUON_ERR_SHAPE
    assert call([desc(4, 9, col_blocks=2)], mode=mu.MUON_NS_BLOCKWISE) == mu.MUON_ERR_SHAPE
    assert call([desc(4, 8, dtype=7)]) == mu.MUON_ERR_DTYPE
    assert call([desc(4, 8), desc(4, 8, dtype=mu.MUON_F32, ptr=FAKE * 2)]) == mu.MUON_ERR_DTYPE
    assert call([desc(4, 8, ptr=FAKE + 1)]) == mu.MUON_ERR_ALIGN
    assert call([desc(4, 8), desc(4, 8, ptr=FAKE + 32)]) == mu.MUON_ERR_ALIAS
    assert call([desc(4, 8)]) == mu.MUON_ERR_WORKSPACE                 # valid, but no workspace
    assert "workspace" in mu.muon_last_error()
    nan = (ctypes.c_float * 3)(float("nan"), 0, 0)
    assert lib.muon_ns_batched(mu.mats([desc(4, 8)]), 1, 5, nan, 0) == mu.MUON_ERR_INVALID_ARG
    # B is formed as c (A A + (b / c) A): c == 0 (a cubic iteration) and an
    # overflowing b / c are rejected before anything else
    for bad in [(1.5, -0.5, 0.0), (3.0, -3e38, 1e-3)]:
        cf = (ctypes.c_float * 3)(*bad)
        assert lib.muon_ns_batched(mu.mats([desc(4, 8)]), 1, 5, cf, 0) == mu.MUON_ERR_INVALID_ARG
        assert "c != 0" in mu.muon_last_error()
        assert lib.muon_set_step_options(5, cf, 1e-7, 0) == mu.MUON_ERR_INVALID_ARG


def test_adamw_validation_codes(lib):
    """Every invalid AdamW call is rejected on the host, before any launch."""
    def call(W, G, Mo, V, lr=1e-3, b1=0.9, b2=0.95, eps=1e-8, wd=0.0, step=1, n=None):
        k = len(W) if n is None else n
        return lib.muon_adamw_step(mu.mats(W), mu.mats(G), mu.mats(Mo), mu.mats(V), k, lr, b1, b2, eps, wd, step)
    bf, f32 = mu.MUON_BF16, mu.MUON_F32
    W = [desc(4, 8, dtype=bf, ptr=FAKE)]
    G = [desc(4, 8, dtype=bf, ptr=FAKE * 2)]
    Mo = [desc(4, 8, dtype=f32, ptr=FAKE * 3)]
    V = [desc(4, 8, dtype=f32, ptr=FAKE * 4)]
    assert call([], [], [], [], n=0) == mu.MUON_OK
    assert call(W, G, Mo, V, n=-1) == mu.MUON_ERR_INVALID_ARG
    assert call(W, G, Mo, V, b1=1.0) == mu.MUON_ERR_INVALID_ARG
    assert call(W, G, Mo, V, b2=-0.1) == mu.MUON_ERR_INVALID_ARG
    assert call(W, G, Mo, V, eps=0.0) == mu.MUON_ERR_INVALID_ARG
    assert call(W, G, Mo, V, lr=float("nan")) == mu.MUON_ERR_INVALID_ARG
    assert call(W, G, Mo, V, step=0) == mu.MUON_ERR_INVALID_ARG
    assert call(W, G, [desc(4, 8, dtype=bf, ptr=FAKE * 3)], V) == mu.MUON_ERR_DTYPE
    assert call(W, [desc(4, 8, dtype=f32, ptr=FAKE * 2)], Mo, V) == mu.MUON_ERR_DTYPE
    assert call(W, G, Mo, [desc(4, 9, dtype=f32, ptr=FAKE * 4)]) == mu.MUON_ERR_SHAPE
    assert call(W, G, Mo, [desc(4, 8, dtype=f32, ptr=FAKE * 4 + 2)]) == mu.MUON_ERR_ALIGN
    assert call(W, G, [desc(4, 8, dtype=f32, ptr=FAKE + 16)], V) == mu.MUON_ERR_ALIAS


def test_workspace_overlap_rejected(lib):
    """A matrix that reaches into the workspace is rejected before anything is
    enqueued (the workspace is fake and never dereferenced: every call here
    fails validation)."""
    ws = FAKE * 8
    try:
        mu.muon_set_workspace(ws, 1 << 20)
        inside = desc(4, 8, ptr=ws + 4096)
        assert lib.muon_ns_batched(mu.mats([inside]), 1, 5, None, 0) == mu.MUON_ERR_ALIAS
        assert "workspace" in mu.muon_last_error()
        straddle = desc(64, 64, ptr=ws - 256)  # starts before, ends inside
        assert lib.muon_ns_batched(mu.mats([straddle]), 1, 5, None, 0) == mu.MUON_ERR_ALIAS
        W, G, M = desc(4, 8, ptr=FAKE), desc(4, 8, ptr=FAKE * 2), desc(4, 8, ptr=ws + (1 << 20) - 16)
        assert lib.muon_step(mu.mats([W]), mu.mats([G]), mu.mats([M]), 1, 0.02, 0.95, 0) == mu.MUON_ERR_ALIAS
        assert "moms[0]" in mu.muon_last_error()
        G = desc(4, 8, ptr=ws + 1024)  # read-only buffers may not sit there either
        M = desc(4, 8, ptr=FAKE * 3)
        assert lib.muon_step(mu.mats([W]), mu.mats([G]), mu.mats([M]), 1, 0.02, 0.95, 0) == mu.MUON_ERR_ALIAS
    finally:
        mu.muon_set_workspace(None, 0)


def test_noalloc_rejects_what_the_scratch_cannot_hold(lib):
    """muon_step_noalloc plans against its fixed device scratch before any HIP
    call: a matrix whose workspace alone exceeds it is rejected on the host."""
    W, G, M = desc(7168, 18432, ptr=FAKE), desc(7168, 18432, ptr=FAKE * 2), desc(7168, 18432, ptr=FAKE * 3)
    assert mu.muon_workspace_min_size([W]) > mu.MUON_NOALLOC_SCRATCH_BYTES
    st = lib.muon_step_noalloc(mu.mats([W]), mu.mats([G]), mu.mats([M]), 1, 0.02, 0.95, 0)
    assert st == mu.MUON_ERR_WORKSPACE
    assert "scratch" in mu.muon_last_error()
    # the other host-side checks come first, as in muon_step
    assert lib.muon_step_noalloc(mu.mats([W]), mu.mats([G]), mu.mats([M]), 1, float("nan"), 0.95, 0) \
        == mu.MUON_ERR_INVALID_ARG
    assert lib.muon_step_noalloc(mu.mats([W]), mu.mats([W]), mu.mats([M]), 1, 0.02, 0.95, 0) == mu.MUON_ERR_ALIAS


def test_alias_exact_for_interleaved_views(lib):
    # two column blocks of one 8 x 64 bf16 buffer do not overlap element-wise
    left = desc(8, 32, ld=64)
    right = desc(8, 32, ld=64, ptr=FAKE + 64)
    # they pass alias checking and stop at the missing workspace
    assert lib.muon_ns_batched(mu.mats([left, right]), 2, 5, None, 0) == mu.MUON_ERR_WORKSPACE
    shifted = desc(8, 32, ld=64, ptr=FAKE + 62)  # overlaps one column
    assert lib.muon_ns_batched(mu.mats([left, shifted]), 2, 5, None, 0) == mu.MUON_ERR_ALIAS
    below = desc(8, 32, ld=64, ptr=FAKE + 8 * 64 * 2)  # starts after left ends
    assert lib.muon_ns_batched(mu.mats([left, below]), 2, 5, None, 0) == mu.MUON_ERR_WORKSPACE


def test_step_validation_codes(lib):
    mu.muon_set_workspace(None, 0)
    W, G, M = desc(4, 8), desc(4, 8, ptr=FAKE * 2), desc(4, 8, ptr=FAKE * 3)
    step = lambda w, g, m, lr=0.02, beta=0.95, nest=0: lib.muon_step(
        mu.mats([w]), mu.mats([g]), mu.mats([m]), 1, lr, beta, nest)
    assert step(W, G, M) == mu.MUON_ERR_WORKSPACE
    assert step(W, G, desc(4, 9, ptr=FAKE * 3)) == mu.MUON_ERR_SHAPE
    assert step(W, desc(4, 8, dtype=mu.MUON_F32, ptr=FAKE * 2), M) == mu.MUON_ERR_DTYPE
    assert step(W, G, M, lr=float("inf")) == mu.MUON_ERR_INVALID_ARG
    assert step(W, G, M, nest=2) == mu.MUON_ERR_INVALID_ARG
    assert step(W, G, W) == mu.MUON_ERR_ALIAS                      # moms == params
    assert step(W, W, M) == mu.MUON_ERR_ALIAS                      # grads overlap params (written)
    # two matrices may share one read-only gradient
    assert lib.muon_step(mu.mats([W, desc(4, 8, ptr=FAKE * 4)]), mu.mats([G, G]),
                         mu.mats([M, desc(4, 8, ptr=FAKE * 5)]), 2, 0.02, 0.95, 0) == mu.MUON_ERR_WORKSPACE


def test_options_and_workspace_args(lib):
    assert lib.muon_set_step_options(-1, None, 1e-7, 0) == mu.MUON_ERR_INVALID_ARG
    assert lib.muon_set_step_options(5, None, -1.0, 0) == mu.MUON_ERR_INVALID_ARG
    assert lib.muon_set_step_options(5, None, 1e-7, 0x1000) == mu.MUON_ERR_INVALID_ARG
    assert lib.muon_set_step_options(5, None, 1e-7, mu.DEFAULT_MODE) == mu.MUON_OK
    assert lib.muon_set_workspace(ctypes.c_void_p(FAKE + 16), 1024) == mu.MUON_ERR_ALIGN
    assert lib.muon_set_workspace(ctypes.c_void_p(FAKE), 0) == mu.MUON_ERR_INVALID_ARG
    assert lib.muon_set_workspace(None, 0) == mu.MUON_OK


def test_workspace_too_small_is_rejected(lib):
    d = [desc(300, 520)]
    need = mu.muon_workspace_min_size(d)
    assert lib.muon_set_workspace(ctypes.c_void_p(FAKE * 8), need - 256) == mu.MUON_OK
    try:
        assert lib.muon_ns_batched(mu.mats(d), 1, 5, None, 0) == mu.MUON_ERR_WORKSPACE
    finally:
        assert lib.muon_set_workspace(None, 0) == mu.MUON_OK


# ---------------------------------------------------------------------------
# planner
# ---------------------------------------------------------------------------

def shapes_descs(shapes, dtype=mu.MUON_BF16, col_blocks=1):
    out = []
    for i, (r, c) in enumerate(shapes):
        out.append(desc(r, c, dtype=dtype, ptr=FAKE * (i + 1), col_blocks=col_blocks))
    return out


def test_plan_orientation_and_padding():
    p = mu.muon_plan_info(shapes_descs([(300, 520), (520, 300), (256, 256), (1, 7)]), mode=mu.MUON_PACK_RR)
    v = p["views"]
    assert [(x["m"], x["n"], x["tall"]) for x in v] == [(300, 520, False), (300, 520, True),
                                                         (256, 256, False), (1, 7, False)]
    assert [(x["mp"], x["np"]) for x in v] == [(512, 768), (512, 768), (256, 256), (256, 256)]
    f = mu.muon_plan_info(shapes_descs([(100, 37)], dtype=mu.MUON_F32))
    assert f["views"][0]["mp"] == 64 and f["views"][0]["np"] == 128 and f["pad"] == 64


def test_plan_rr_vs_cost_order_block_workload():
    from muon_newton_schulz_03_amd.workloads import WORKLOADS
    shapes = WORKLOADS["qwen3_block"].shapes
    rr = mu.muon_plan_info(shapes_descs(shapes), mode=mu.MUON_PACK_RR)
    cost = mu.muon_plan_info(shapes_descs(shapes), mode=mu.MUON_PACK_COST)
    assert [x["mat"] for x in rr["views"]] == list(range(len(shapes)))
    costs = [x["cost"] for x in cost["views"]]
    assert costs == sorted(costs, reverse=True)
    # stable: equal costs keep the input order
    assert [x["mat"] for x in cost["views"]][:2] == [0, 3]
    # one group each; RR has 4 uniform-shape segments, COST 3
    assert len(rr["chunks"]) == 1 and len(cost["chunks"]) == 1
    assert [(s["mp"], s["np"], s["count"]) for s in rr["chunks"][0]["segments"]] == [
        (2048, 4096, 1), (512, 2048, 2), (2048, 4096, 1), (768, 2048, 384)]
    assert [(s["mp"], s["np"], s["count"]) for s in cost["chunks"][0]["segments"]] == [
        (2048, 4096, 2), (768, 2048, 384), (512, 2048, 2)]


def test_plan_tile_counts_and_syrk_fraction():
    p = mu.muon_plan_info(shapes_descs([(2048, 7168)] * 3))
    s = p["chunks"][0]["segments"][0]
    t = 2048 // 256
    assert s["tiles_syrk"] == t * (t + 1) // 2 == acc.syrk_tiles(2048, 256)
    assert s["tiles_gemm"] == 8 * 28
    assert p["chunks"][0]["launch_tiles"]["gram"] == 3 * 36
    assert acc.syrk_executed_fraction(2048, 256) == pytest.approx(0.5625)
    assert acc.syrk_executed_fraction(7168, 256) == pytest.approx(0.5179, abs=1e-4)
    assert acc.syrk_executed_fraction(7168, 128) == pytest.approx(0.5089, abs=1e-4)


def test_plan_groups_fit_workspace():
    ds = shapes_descs([(768, 2048)] * 10)
    full = mu.muon_workspace_size(ds)
    one = mu.muon_workspace_min_size(ds)
    assert full == 10 * one
    p = mu.muon_plan_info(ds, workspace_bytes=3 * one + 5)
    assert [c["count"] for c in p["chunks"]] == [3, 3, 3, 1]
    assert all(c["bytes"] <= 3 * one + 5 for c in p["chunks"])
    with pytest.raises(mu.MuonError):
        mu.muon_plan_info(ds, workspace_bytes=one - 1)


def test_plan_segment_limit_splits_groups():
    shapes = [(256 * (i + 1), 2048) for i in range(8)] + [(256, 4096)]
    p = mu.muon_plan_info(shapes_descs(shapes), mode=mu.MUON_PACK_RR)
    assert [len(c["segments"]) for c in p["chunks"]] == [8, 1]


def test_plan_blockwise_expansion():
    ds = shapes_descs([(7168, 18432)], col_blocks=8)
    p = mu.muon_plan_info(ds, mode=mu.MUON_NS_BLOCKWISE)
    v = p["views"]
    assert len(v) == 8
    assert [x["col_off"] for x in v] == [2304 * k for k in range(8)]
    assert all(x["tall"] and (x["m"], x["n"]) == (2304, 7168) for x in v)
    # without the blockwise bit col_blocks is ignored
    assert len(mu.muon_plan_info(ds)["views"]) == 1


def test_plan_distributed_shards():
    """Distributed mode: P shards per matrix, each m x n/P in the matrix's
    own orientation (even when n/P < m), consecutive, never split across
    groups, with a buffer for the shard's tile-packed upper triangle."""
    ds = [desc(300, 1000, col_blocks=4), desc(200, 400, col_blocks=4, ptr=FAKE * 2),
          desc(300, 1000, col_blocks=4, ptr=FAKE * 3)]
    p = mu.muon_plan_info(ds, mode=mu.MUON_NS_DISTRIBUTED | mu.MUON_PACK_COST)
    assert p["distributed"] and p["shards"] == 4
    v = p["views"]
    assert len(v) == 12
    for k in range(0, 12, 4):
        assert [x["block"] for x in v[k:k + 4]] == [0, 1, 2, 3]
        assert len({x["mat"] for x in v[k:k + 4]}) == 1
    first = v[0]
    assert (first["m"], first["n"], first["tall"]) == (300, 250, False)
    L = p["chunks"][0]["segments"][0]["layout"]
    mp = p["chunks"][0]["segments"][0]["mp"]
    t = mp // 256  # bf16: the upper 256 x 256 tiles in float32
    assert L["total"] - L["tri"] >= t * (t + 1) // 2 * 65536 * 4
    # a workspace of one matrix's shards: one matrix per group
    one = 4 * v[0]["bytes"]
    q = mu.muon_plan_info(ds, mode=mu.MUON_NS_DISTRIBUTED | mu.MUON_PACK_COST, workspace_bytes=one)
    assert [c["count"] for c in q["chunks"]] == [4, 4, 4]


@pytest.mark.parametrize("dtype", [mu.MUON_BF16, mu.MUON_F32])
def test_plan_layout_disjoint(dtype):
    """Every buffer of a view's workspace block is 256-byte aligned, inside the
    block and disjoint from the others; the bf16 path also holds X^T twice
    (np x mp, ping-pong), the float32 path no X^T and no lo half of A."""
    p = mu.muon_plan_info(shapes_descs([(300, 520)], dtype=dtype))
    seg = p["chunks"][0]["segments"][0]
    L, mp, np_ = seg["layout"], seg["mp"], seg["np"]
    es = 2 if dtype == mu.MUON_BF16 else 4
    bf = dtype == mu.MUON_BF16
    nparts = (mp // 64) * (np_ // 64)
    spans = [(L["xa"][0], mp * np_ * es), (L["xa"][1], mp * np_ * es),
             (L["ahi"], mp * mp * es), (L["b"], mp * mp * es),
             (L["partials"], nparts * 4), (L["scale"], 16)]
    if bf:
        spans += [(L["xt"][0], np_ * mp * es), (L["xt"][1], np_ * mp * es), (L["alo"], mp * mp * es),
                  (L["bdiag"], mp * 4)]
    else:
        assert L["xt"][0] == L["xt"][1] and L["alo"] == L["b"]
    spans.sort()
    assert all(off % 256 == 0 for off, _ in spans)
    assert all(a + n <= b for (a, n), (b, _) in zip(spans, spans[1:]))
    assert spans[-1][0] + spans[-1][1] <= L["total"]


# ---------------------------------------------------------------------------
# accounting
# ---------------------------------------------------------------------------

def brute_syrk_mults(m, n):
    # multiply-adds of the upper triangle (diagonal included) of an m x m
    # symmetric product with inner dimension n
    return sum(n for i in range(m) for j in range(i, m))


@pytest.mark.parametrize("m,n", [(1, 1), (3, 5), (7, 7), (4, 11)])
def test_algorithmic_flops_by_enumeration(m, n):
    gram = 2 * brute_syrk_mults(m, n)
    aa = 2 * brute_syrk_mults(m, m)
    bx = 2 * m * m * n
    assert acc.flops_algorithmic(m, n, 1) == gram + aa + bx
    assert acc.flops_nominal(m, n, 1) == 2 * m * m * n + 2 * m ** 3 + 2 * m * m * n


def test_workload_flops_match_hand_counts():
    """Per-step FLOPs of two workloads, counted by hand from the shapes: the
    Kimi MoE layer (1152 matrices, 5 iterations) and the blockwise dense
    matrix (8 column blocks of 7168 x 2304, each oriented to 2304 x 7168)."""
    from muon_newton_schulz_03_amd.workloads import WORKLOADS
    nom, alg = acc.workload_flops(WORKLOADS["kimi_moe_layer"].shapes, 5)
    assert nom / 1e12 == pytest.approx(791.648, abs=1e-3)
    assert alg / 1e12 == pytest.approx(569.106, abs=1e-3)
    nom, alg = acc.workload_flops(WORKLOADS["kimi_dense_blockwise"].shapes, 5, col_blocks=8)
    assert nom / 1e12 == pytest.approx(7.067, abs=1e-3)
