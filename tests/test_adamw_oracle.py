"""Pins of the AdamW oracle against closed forms of the published algorithm
(Adam moments with bias correction, decoupled weight decay):

* first step from zero moments: m_hat = g and v_hat = g^2 exactly, so
  W1 = W0 (1 - lr wd) - lr g / (|g| + eps);
* a constant gradient for t steps keeps m_hat = g and v_hat = g^2, so each
  step moves W by - lr g / (|g| + eps) (no weight decay);
* zero gradients from zero moments leave only the decay: W_t = W0 (1 - lr wd)^t;
* the moments after t steps of a constant gradient: m = (1 - beta1^t) g,
  v = (1 - beta2^t) g^2.
A planted mistake in the oracle (dropped bias correction, coupled decay,
eps inside the root, swapped betas) must fail at least one pin.
"""
import inspect

import numpy as np
import pytest

import oracle
from oracle import adamw_oracle

LR, B1, B2, EPS, WD = 0.01, 0.9, 0.95, 1e-8, 0.1


def rand(seed, shape=(7, 13)):
    r = np.random.default_rng(seed)
    return r.standard_normal(shape), r.standard_normal(shape) * 1e-2


def test_first_step_closed_form():
    W, G = rand(1)
    z = np.zeros_like(W)
    W1, m1, v1 = oracle.adamw_step(W, G, z, z, LR, B1, B2, EPS, WD, step=1)
    assert np.allclose(W1, W * (1 - LR * WD) - LR * G / (np.abs(G) + EPS), rtol=0, atol=1e-15)
    assert np.allclose(m1, (1 - B1) * G, rtol=1e-15, atol=0)
    assert np.allclose(v1, (1 - B2) * G * G, rtol=1e-15, atol=0)


def test_constant_gradient_steps():
    W, G = rand(2)
    W0, m, v = W.copy(), np.zeros_like(W), np.zeros_like(W)
    for t in range(1, 7):
        W, m, v = oracle.adamw_step(W, G, m, v, LR, B1, B2, EPS, 0.0, step=t)
        assert np.allclose(m, (1 - B1 ** t) * G, rtol=1e-13, atol=0)
        assert np.allclose(v, (1 - B2 ** t) * G * G, rtol=1e-13, atol=0)
        assert np.allclose(W, W0 - t * LR * G / (np.abs(G) + EPS), rtol=0, atol=1e-13)


def test_decay_only():
    W, _ = rand(3)
    W0, z = W.copy(), np.zeros_like(W)
    m, v = z.copy(), z.copy()
    for t in range(1, 5):
        W, m, v = oracle.adamw_step(W, z, m, v, LR, B1, B2, EPS, WD, step=t)
    assert np.allclose(W, W0 * (1 - LR * WD) ** 4, rtol=1e-14, atol=0)


MUTATIONS = [
    ("m_hat = m / (1 - beta1 ** step)", "m_hat = m"),
    ("W = W - lr * weight_decay * W - lr * m_hat", "W = W - weight_decay * W - lr * m_hat"),
    ("(np.sqrt(v_hat) + eps)", "np.sqrt(v_hat + eps)"),
    ("m = beta1 * m + (1 - beta1) * G", "m = beta2 * m + (1 - beta2) * G"),
    ("v = beta2 * v + (1 - beta2) * (G * G)", "v = beta2 * v + (1 - beta2) * G"),
]


@pytest.mark.parametrize("old,new", MUTATIONS)
def test_pins_catch_planted_mistake(old, new):
    src = inspect.getsource(adamw_oracle.adamw_step)
    assert old in src
    ns = {"np": np}
    exec(src.replace(old, new), ns)
    orig = oracle.adamw_step
    adamw_oracle.adamw_step = oracle.adamw_step = ns["adamw_step"]
    failed = False
    try:
        for pin in (test_first_step_closed_form, test_constant_gradient_steps, test_decay_only):
            try:
                pin()
            except AssertionError:
                failed = True
    finally:
        adamw_oracle.adamw_step = oracle.adamw_step = orig
    assert failed, f"no pin caught: {new}"
