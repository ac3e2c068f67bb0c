"""Pins of the fp64 LAMB oracle (MegaScale reading notes, section 1.1, eq (7))
against facts that do not come from its own code: the step-size identity the
trust ratio exists for, a closed form at the first step, torch.optim.Adam
(the same moments and direction, without the trust ratio) over several steps,
brute-force moment sums, and scaling properties.  CPU only."""
import numpy as np
import pytest
import torch

from oracle import lamb_oracle as L

HP = dict(beta1=0.9, beta2=0.999, eps=1e-6)


def _state(rng, n, scale=0.02):
    theta = rng.standard_normal(n) * scale
    m = rng.standard_normal(n) * 1e-3
    v = np.abs(rng.standard_normal(n)) * 1e-6
    g = rng.standard_normal(n) * 1e-3
    return theta, m, v, g


@pytest.mark.parametrize("step", [1, 2, 7, 1000])
def test_each_layer_moves_lr_times_its_norm(step):
    """The trust ratio makes ||theta_new - theta|| = lr * ||theta|| exactly,
    whatever the gradient and moments (eq (7): the step of every layer is
    scaled to its parameter norm)."""
    rng = np.random.default_rng(step)
    theta, m, v, g = _state(rng, 5000)
    lr = 3e-3
    new, _, _, nt, nr = L.lamb_step(theta, m, v, g, step, lr, **HP)
    np.testing.assert_allclose(np.linalg.norm(new - theta), lr * np.linalg.norm(theta),
                               rtol=1e-12)
    assert nt == pytest.approx(np.linalg.norm(theta), rel=1e-14)


def test_first_step_closed_form():
    """Step 1 from zero moments with eps = 0: m_hat = g, v_hat = g^2, so
    r = sign(g), ||r|| = sqrt(N) and theta_new = theta - lr ||theta|| sign(g) / sqrt(N)."""
    rng = np.random.default_rng(1)
    n = 4096
    theta = rng.standard_normal(n)
    g = rng.standard_normal(n)
    new, m, v, nt, nr = L.lamb_step(theta, np.zeros(n), np.zeros(n), g, 1, 0.01, 0.9, 0.999, 0.0)
    np.testing.assert_allclose(m, 0.1 * g, rtol=1e-15)
    np.testing.assert_allclose(v, 0.001 * g * g, rtol=1e-12)
    assert nr == pytest.approx(np.sqrt(n), rel=1e-12)
    expect = theta - 0.01 * np.linalg.norm(theta) / np.sqrt(n) * np.sign(g)
    np.testing.assert_allclose(new, expect, rtol=1e-12, atol=1e-15)


def test_direction_matches_torch_adam_over_several_steps():
    """Without the trust ratio the step is Adam's: torch.optim.Adam (no weight
    decay) moves p by -lr * m_hat / (sqrt(v_hat) + eps); the oracle's r must
    equal that move / -lr at every step of a gradient sequence."""
    rng = np.random.default_rng(2)
    n, lr = 300, 1e-2
    p = torch.zeros(n, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.Adam([p], lr=lr, betas=(HP["beta1"], HP["beta2"]), eps=HP["eps"])
    m = np.zeros(n)
    v = np.zeros(n)
    for step in range(1, 8):
        g = rng.standard_normal(n) * 10.0 ** rng.integers(-4, 1)
        before = p.detach().clone()
        p.grad = torch.tensor(g)
        opt.step()
        adam_r = -(p.detach() - before).numpy() / lr
        m, v, r = L.lamb_moments(m, v, g, step, **HP)
        np.testing.assert_allclose(r, adam_r, rtol=1e-9, atol=1e-12)


def test_moments_equal_brute_force_sums():
    rng = np.random.default_rng(3)
    gs = [rng.standard_normal(50) for _ in range(6)]
    m = np.zeros(50)
    v = np.zeros(50)
    b1, b2 = 0.8, 0.95
    for t, g in enumerate(gs, start=1):
        m, v, _ = L.lamb_moments(m, v, g, t, b1, b2, 1e-8)
    t = len(gs)
    m_ref = sum((1 - b1) * b1 ** (t - s) * gs[s - 1] for s in range(1, t + 1))
    v_ref = sum((1 - b2) * b2 ** (t - s) * gs[s - 1] ** 2 for s in range(1, t + 1))
    np.testing.assert_allclose(m, m_ref, rtol=1e-13)
    np.testing.assert_allclose(v, v_ref, rtol=1e-13)


def test_scaling_properties_and_zero_weights():
    """With eps = 0 the direction ignores the gradient's scale; the update
    scales with theta (trust ratio proportional to ||theta||); an all-zero
    tensor takes the plain step (trust ratio 1)."""
    rng = np.random.default_rng(4)
    theta, m, v, g = _state(rng, 1000)
    a = L.lamb_step(theta, m, v, g, 3, 1e-2, 0.9, 0.999, 0.0)[0]
    b = L.lamb_step(theta, 7.0 * m, 49.0 * v, 7.0 * g, 3, 1e-2, 0.9, 0.999, 0.0)[0]
    np.testing.assert_allclose(a, b, rtol=1e-12)
    c = L.lamb_step(5.0 * theta, m, v, g, 3, 1e-2, 0.9, 0.999, 0.0)[0]
    np.testing.assert_allclose(c, 5.0 * a, rtol=1e-12)
    z, _, _, nt, nr = L.lamb_step(np.zeros(1000), m, v, g, 3, 1e-2, **HP)
    assert nt == 0.0
    _, _, r = L.lamb_moments(m, v, g, 3, **HP)
    np.testing.assert_allclose(z, -1e-2 * r, rtol=1e-15)
