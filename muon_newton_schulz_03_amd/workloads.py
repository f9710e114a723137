"""Seeded synthetic workloads shaped like the layers of the models the pages
measure (Qwen3 30B-A3B, Kimi K2), and the generators that fill them.

This module holds no part of the method's arithmetic: it only names shapes,
value distributions and seeds, and draws the random inputs that both the HIP
path and the CPU oracle consume. Weights and data of the real models are not
used (none are available); values are i.i.d. Gaussians of the stated standard
deviation.
"""
from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np


@dataclass
class Workload:
    name: str
    description: str
    shapes: List[Tuple[int, int]]   # stored (rows, cols) of every matrix
    dtype: str                      # "f32" or "bf16"
    std_g: float
    std_m: float
    std_w: float = 0.02
    seed: int = 0
    lr: float = 0.02
    beta: float = 0.95
    nesterov: bool = False
    iters: int = 5
    col_blocks: int = 1             # > 1: blockwise mode
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "fp32_64x128": Workload(
        "fp32_64x128", "single float32 matrix 64x128", [(64, 128)], "f32",
        std_g=1.0, std_m=1.0, seed=1),
    "qwen3_moe_experts": Workload(
        "qwen3_moe_experts",
        "Qwen3-30B-A3B-shaped expert batch: 128 x 768x2048 (up/gate) + 128 x 2048x768 (down)",
        [(768, 2048)] * 128 + [(2048, 768)] * 128, "bf16", std_g=1e-3, std_m=1e-2, seed=2),
    "qwen3_block": Workload(
        "qwen3_block",
        "one Qwen3-30B-A3B-shaped block: q 4096x2048, k/v 512x2048, o 2048x4096, "
        "128 experts x (768x2048, 768x2048, 2048x768)",
        [(4096, 2048), (512, 2048), (512, 2048), (2048, 4096)]
        + [(768, 2048), (768, 2048), (2048, 768)] * 128, "bf16", std_g=1e-2, std_m=1e-2, seed=3),
    "kimi_dense": Workload(
        "kimi_dense", "Kimi-K2-dense-shaped MLP: 7168x18432 (gate, up) + 18432x7168 (down)",
        [(7168, 18432), (7168, 18432), (18432, 7168)], "bf16", std_g=1e-2, std_m=1e-2, seed=4),
    "kimi_dense_blockwise": Workload(
        "kimi_dense_blockwise", "one 7168x18432 matrix in 8 column blocks of 7168x2304",
        [(7168, 18432)], "bf16", std_g=1e-2, std_m=1e-2, seed=4, col_blocks=8),
    "kimi_moe_layer": Workload(
        "kimi_moe_layer",
        "Kimi-K2-MoE-layer-shaped batch: 384 experts x (2048x7168 gate, 2048x7168 up, 7168x2048 down)",
        [(2048, 7168), (2048, 7168), (7168, 2048)] * 384, "bf16", std_g=1e-3, std_m=1e-2, seed=5),
}


def torch_dtype(name):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def make_inputs(wl: Workload, device="cuda", shapes=None, seed=None):
    """Draw (W, G, M) lists of device tensors. Draw order per matrix, by
    matrix index: G, M, W. The float32 workload draws on the host with numpy's
    PCG64 (so it is the same on every machine); the bf16 workloads draw on the
    device with torch's generator and round to bf16."""
    import torch
    shapes = wl.shapes if shapes is None else shapes
    seed = wl.seed if seed is None else seed
    dt = torch_dtype(wl.dtype)
    W, G, M = [], [], []
    if wl.dtype == "f32":
        rng = np.random.default_rng(seed)
        for (r, c) in shapes:
            g = rng.standard_normal((r, c)) * wl.std_g
            m = rng.standard_normal((r, c)) * wl.std_m
            w = rng.standard_normal((r, c)) * wl.std_w
            G.append(torch.tensor(g, dtype=dt, device=device))
            M.append(torch.tensor(m, dtype=dt, device=device))
            W.append(torch.tensor(w, dtype=dt, device=device))
        return W, G, M
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    for (r, c) in shapes:
        for lst, std in ((G, wl.std_g), (M, wl.std_m), (W, wl.std_w)):
            t = torch.empty((r, c), dtype=dt, device=device)
            t.normal_(0.0, std, generator=gen)
            lst.append(t)
    return W, G, M


def sample_indices(n, k, seed):
    """k distinct matrix indices out of n, seeded."""
    if k >= n:
        return list(range(n))
    return sorted(int(i) for i in np.random.default_rng(seed).choice(n, k, replace=False))
