"""The allocation-free entry point, muon_step_noalloc, through the C ABI: its
results must equal muon_step's on the same inputs (same kernels, same
arithmetic per matrix; only the scratch differs, so equality is bitwise), on
two calls in a row, the second with fewer and smaller matrices than the
first, for both precision paths; its orthogonalized update must meet the
bf16 bound against the float64 oracle; and a HIP graph that records it must
replay bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import np64, relF

pytestmark = pytest.mark.gpu


def inputs(shapes, dtype, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    out = []
    for std in (0.02, 1e-3, 1e-2):  # W, G, M
        out.append([(torch.randn(s, generator=g, device="cuda") * std).to(dtype) for s in shapes])
    return out


def run_both(mu, shapes, dtype, seed):
    W, G, M = inputs(shapes, dtype, seed)
    Wa, Ma = [t.clone() for t in W], [t.clone() for t in M]
    Wb, Mb = [t.clone() for t in W], [t.clone() for t in M]
    mu.muon_step(Wa, G, Ma, lr=0.02, beta=0.95)
    mu.muon_step_noalloc(Wb, G, Mb, lr=0.02, beta=0.95)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        assert torch.equal(Wa[i], Wb[i]), (shapes[i], "W")
        assert torch.equal(Ma[i], Mb[i]), (shapes[i], "M")
    # the orthogonalized update itself (W = 0, lr = -1: W_new = O)
    Wz = [torch.zeros_like(t) for t in W]
    Mz = [t.clone() for t in M]
    mu.muon_step_noalloc(Wz, G, Mz, lr=-1.0, beta=0.95)
    torch.cuda.synchronize()
    beta32 = float(np.float32(0.95))
    i = len(shapes) - 1
    O_ref, _, _ = oracle.muon_step(np.zeros(shapes[i]), np64(G[i]), np64(M[i]), lr=-1.0, beta=beta32)
    err = relF(np64(Wz[i]), O_ref)
    print(f"noalloc {dtype} {shapes[i]}: O relF {err:.3e}", flush=True)
    assert err <= (2e-2 if dtype == torch.bfloat16 else 1e-4)


def test_noalloc_matches_muon_step(gpu_lib):
    import muon_newton_schulz_03_amd as mu
    # first call: more than the 256 MiB scratch holds at once (the 2048 x 7168
    # matrix alone takes ~143 MB), so it runs in several groups
    first = [(2048, 7168), (7168, 2048), (768, 2048), (2048, 768), (300, 520)]
    second = [(520, 300), (256, 256), (64, 96)]
    print("noalloc: first call", first, flush=True)
    run_both(mu, first, torch.bfloat16, 21)
    print("noalloc: second call", second, flush=True)
    run_both(mu, second, torch.bfloat16, 22)
    print("noalloc: float32", flush=True)
    run_both(mu, [(64, 128), (100, 37)], torch.float32, 23)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_graph_replays(gpu_lib, dtype):
    """The entry point's purpose: a caller that cannot allocate records the
    step into a HIP graph (torch.cuda.graph on its own stream) and replays
    it. Three replays, each after fresh inputs are copied in eagerly and the
    device synchronized, each bit for bit equal to the eager call."""
    import muon_newton_schulz_03_amd as mu
    shapes = [(300, 520), (520, 300), (256, 768)] if dtype == torch.bfloat16 else [(64, 128), (100, 37)]
    W0, G0, M0 = inputs(shapes, dtype, 31)
    We, Me = [t.clone() for t in W0], [t.clone() for t in M0]
    mu.muon_step_noalloc(We, G0, Me, lr=0.02, beta=0.95)  # eager reference (and scratch lookup)
    torch.cuda.synchronize()
    Wg, Gg, Mg = [t.clone() for t in W0], [t.clone() for t in G0], [t.clone() for t in M0]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        mu.muon_step_noalloc(Wg, Gg, Mg, lr=0.02, beta=0.95)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        mu.muon_step_noalloc(Wg, Gg, Mg, lr=0.02, beta=0.95)
    torch.cuda.synchronize()
    for rep in range(3):
        for dst, src in zip(Wg + Mg, W0 + M0):
            dst.copy_(src)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i in range(len(shapes)):
            assert torch.equal(Wg[i], We[i]), (rep, shapes[i], "W")
            assert torch.equal(Mg[i], Me[i]), (rep, shapes[i], "M")
    mu.muon_set_stream(None)
