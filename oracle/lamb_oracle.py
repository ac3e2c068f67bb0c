"""fp64 CPU oracle of the LAMB optimizer step (MegaScale reading notes,
"MegaScale：ByteDance 如何在 12,288 块 GPU 上实现 55% MFU 的大规模 LLM 训练",
section 1.1, eq (7)).

TEST INFRASTRUCTURE. Only the test-suite and the benchmark may import or run
this module; the HIP library never calls it and shares no code with it.

Eq (7) scales each layer's Adam-style step by the layer-wise trust ratio
||theta_l|| / ||r_l||, where r_l = m_hat_l / (sqrt(v_hat_l) + eps) is built
from the bias-corrected first and second moments.  Readings where the notes
are silent or inconsistent (each also a documented choice of the library):
  * the moments follow the usual exponential averages,
        m <- b1 m + (1 - b1) g,  v <- b2 v + (1 - b2) g^2,
    with bias corrections 1 - b^t at step t (the notes only name m_hat, v_hat
    "de-biased estimates");
  * the trust ratio's denominator, printed as ||m_hat / v_hat^(1/2) + eps||,
    is the norm of the same direction r the step applies (the notes' own
    description: the step of every layer is scaled relative to its parameter
    norm);
  * a "layer" is one parameter tensor; the trust ratio is 1 when either norm
    is zero; no weight decay (the notes name none);
  * theta, m and v are fp32 master copies, the gradient is the bf16 output of
    the backward (Megatron tuning post, mixed-precision section); here all of
    them are float64.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def lamb_moments(m: np.ndarray, v: np.ndarray, g: np.ndarray, step: int, beta1: float,
                 beta2: float, eps: float) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """New moments and the bias-corrected direction r of one step."""
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** step)
    v_hat = v / (1.0 - beta2 ** step)
    return m, v, m_hat / (np.sqrt(v_hat) + eps)


def lamb_step(theta: np.ndarray, m: np.ndarray, v: np.ndarray, g: np.ndarray, step: int,
              lr: float, beta1: float, beta2: float, eps: float):
    """One LAMB step of one tensor ("layer").  Returns
    (theta_new, m_new, v_new, ||theta||, ||r||), the norms over the whole
    tensor with theta taken before the update."""
    m, v, r = lamb_moments(m, v, g, step, beta1, beta2, eps)
    n_theta = float(np.linalg.norm(theta))
    n_r = float(np.linalg.norm(r))
    trust = n_theta / n_r if (n_theta > 0.0 and n_r > 0.0) else 1.0
    return theta - lr * trust * r, m, v, n_theta, n_r
