"""Plain CPU oracle of one AdamW step -- the comparator the pages measure Muon
against (Table 1 of "Advancing Emerging Optimizers for Accelerated LLM
Training": AdamW and Muon training throughput on the same models).

TEST INFRASTRUCTURE ONLY: the tests and the benchmark call this module; the
library never does. It shares no code with the HIP path.

The pages name AdamW but do not restate it; this follows the published
algorithm: Adam's exponential moment estimates with bias correction (Kingma
and Ba, "Adam: A Method for Stochastic Optimization", Algorithm 1) and the
decoupled weight decay of AdamW (Loshchilov and Hutter, "Decoupled Weight
Decay Regularization", Algorithm 2), with the learning rate as the schedule
multiplier:

    m <- beta1 m + (1 - beta1) g
    v <- beta2 v + (1 - beta2) g^2
    m_hat = m / (1 - beta1^t),   v_hat = v / (1 - beta2^t)
    W <- W - lr * weight_decay * W - lr * m_hat / (sqrt(v_hat) + eps)

with t the 1-based step count. Every array is converted to `dtype` first.
"""
import numpy as np


def adamw_step(W, G, m, v, lr, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0, step=1,
               dtype=np.float64):
    """One AdamW step; returns (W_new, m_new, v_new)."""
    W, G, m, v = (np.asarray(x, dtype=dtype) for x in (W, G, m, v))
    m = beta1 * m + (1 - beta1) * G
    v = beta2 * v + (1 - beta2) * (G * G)
    m_hat = m / (1 - beta1 ** step)
    v_hat = v / (1 - beta2 ** step)
    W = W - lr * weight_decay * W - lr * m_hat / (np.sqrt(v_hat) + eps)
    return W, m, v
