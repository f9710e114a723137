"""GPU parity of the AdamW comparator kernel against the float64 oracle,
through the C ABI: bf16 and float32 parameters, float32 moments, ragged
column counts (scalar tail path), padded pitches, several matrices in one
call, three consecutive steps (bias correction). Moments within 1e-5
relative (float32 arithmetic), parameters within 1 bf16 ulp of the rounded
oracle (bf16) or 1e-5 relative (float32); the oracle always starts from the
device's own stored inputs of the step."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import bf16_round, bf16_ulp_diff, np64, padded

pytestmark = pytest.mark.gpu

LR, B1, B2, EPS, WD = 1e-3, 0.9, 0.95, 1e-8, 0.1


def make(shape, dtype, seed, pitch_extra=0):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    ld = shape[1] + pitch_extra if pitch_extra else None
    _, W = padded(shape[0], shape[1], dtype, ld)
    _, G = padded(shape[0], shape[1], dtype, ld)
    W.copy_(torch.randn(shape, generator=g, device="cuda") * 0.02)
    G.copy_(torch.randn(shape, generator=g, device="cuda") * 1e-3)
    _, Mo = padded(shape[0], shape[1], torch.float32, ld)
    _, V = padded(shape[0], shape[1], torch.float32, ld)
    Mo.zero_()
    V.zero_()
    return W, G, Mo, V


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_adamw_three_steps(gpu_lib, dtype):
    shapes = [(64, 128), (33, 77), (256, 1000), (5, 8), (1, 3)]
    mats = [make(s, dtype, 10 + i, pitch_extra=(8 if i == 2 else 0)) for i, s in enumerate(shapes)]
    for step in (1, 2, 3):
        before = [(np64(W), np64(G), np64(Mo), np64(V)) for W, G, Mo, V in mats]
        gpu_lib.muon_adamw_step([m[0] for m in mats], [m[1] for m in mats], [m[2] for m in mats],
                                [m[3] for m in mats], lr=LR, beta1=B1, beta2=B2, eps=EPS, weight_decay=WD,
                                step=step)
        torch.cuda.synchronize()
        for (W, G, Mo, V), (W0, G0, M0, V0) in zip(mats, before):
            Wr, Mr, Vr = oracle.adamw_step(W0, G0, M0, V0, LR, B1, B2, EPS, WD, step=step)
            assert np.allclose(np64(Mo), Mr, rtol=1e-5, atol=1e-12)
            assert np.allclose(np64(V), Vr, rtol=1e-5, atol=1e-14)
            if dtype == torch.bfloat16:
                assert bf16_ulp_diff(np64(W), bf16_round(Wr)).max() <= 1
            else:
                assert np.allclose(np64(W), Wr, rtol=1e-5, atol=1e-9)
        # the next step starts from what the device stored


def test_adamw_gradient_sign_first_step(gpu_lib):
    """From zero moments the first step moves every weight by lr * sign(g)
    (up to eps), whatever the gradient's scale."""
    W, G, Mo, V = make((128, 256), torch.float32, 3)
    G.mul_(1e3)
    W0, G0 = np64(W), np64(G)
    gpu_lib.muon_adamw_step([W], [G], [Mo], [V], lr=LR, beta1=B1, beta2=B2, eps=EPS, weight_decay=0.0, step=1)
    torch.cuda.synchronize()
    assert np.allclose(np64(W), W0 - LR * np.sign(G0), rtol=0, atol=1e-6)


def test_adamw_empty(gpu_lib):
    gpu_lib.muon_adamw_step([], [], [], [], lr=LR)
