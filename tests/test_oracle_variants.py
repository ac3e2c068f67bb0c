"""Pins of the fp64 oracle's layer variants (MegaScale reading notes, section
1.3: MegaScale's fused RMSNorm and SwiGLU kernels): RMSNorm against its closed
form, torch's rms_norm and finite differences; SiLU against torch, an odd-part
identity and finite differences; the [W1 | W3] block interleave on an explicit
example; whole layers (parallel and serial) against an independent torch fp64
autograd implementation and central finite differences; the FLOP count of the
SwiGLU layer against the closed form.  CPU only."""
import math

import numpy as np
import pytest
import torch

from oracle import ptb_oracle as O
from transformer_block_amd import flops as F


def test_rmsnorm_closed_form_and_torch():
    rng = np.random.default_rng(600)
    x = rng.standard_normal((13, 96)) * 2 + 0.7
    eps = 1e-5
    a, mu, rstd = O.rmsnorm_forward(x, np.ones(96), eps)
    ms = (x * x).mean(axis=1)
    np.testing.assert_allclose((a * a).mean(axis=1), ms / (ms + eps), rtol=1e-13)
    np.testing.assert_array_equal(mu, 0.0)
    gamma = 1 + 0.3 * rng.standard_normal(96)
    a, _, _ = O.rmsnorm_forward(x, gamma, eps)
    ref = torch.nn.functional.rms_norm(torch.tensor(x), (96,), torch.tensor(gamma), eps)
    np.testing.assert_allclose(a, ref.numpy(), rtol=1e-13, atol=1e-13)


def test_rmsnorm_backward_finite_difference():
    rng = np.random.default_rng(601)
    x = rng.standard_normal((5, 24))
    gamma = 1 + 0.2 * rng.standard_normal(24)
    da = rng.standard_normal(x.shape)
    _, _, rstd = O.rmsnorm_forward(x, gamma, 1e-5)
    dx, dg, db = O.rmsnorm_backward(da, x, gamma, rstd)
    np.testing.assert_array_equal(db, 0.0)
    e = 1e-6
    L = lambda xx, gg: (O.rmsnorm_forward(xx, gg, 1e-5)[0] * da).sum()
    vx = rng.standard_normal(x.shape)
    vg = rng.standard_normal(24)
    fd = (L(x + e * vx, gamma) - L(x - e * vx, gamma)) / (2 * e)
    assert abs(fd - (dx * vx).sum()) <= 1e-7 * max(1.0, abs(fd))
    fd = (L(x, gamma + e * vg) - L(x, gamma - e * vg)) / (2 * e)
    assert abs(fd - (dg * vg).sum()) <= 1e-7 * max(1.0, abs(fd))


def test_silu_against_torch_identity_and_derivative():
    u = np.linspace(-12, 12, 401)
    np.testing.assert_allclose(O.silu(u), torch.nn.functional.silu(torch.tensor(u)).numpy(),
                               rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(O.silu(u) - O.silu(-u), u, rtol=1e-13, atol=1e-13)
    assert O.silu(np.array([0.0]))[0] == 0.0
    e = 1e-6
    np.testing.assert_allclose(O.silu_grad(u), (O.silu(u + e) - O.silu(u - e)) / (2 * e),
                               rtol=1e-7, atol=1e-9)


def test_w13_block_interleave():
    """Block 2j of w_fc1 holds W1 columns 32j..32j+31 and block 2j+1 the same
    columns of W3."""
    f = 96
    w1 = np.arange(2 * f, dtype=float).reshape(2, f)
    w3 = -w1 - 1
    w = O.merge_w13(w1, w3)
    assert w.shape == (2, 2 * f)
    np.testing.assert_array_equal(w[:, 0:32], w1[:, 0:32])
    np.testing.assert_array_equal(w[:, 32:64], w3[:, 0:32])
    np.testing.assert_array_equal(w[:, 64:96], w1[:, 32:64])
    np.testing.assert_array_equal(w[:, 160:192], w3[:, 64:96])
    a, b = O.split_w13(w)
    np.testing.assert_array_equal(a, w1)
    np.testing.assert_array_equal(b, w3)


def _params(rng, h, n, d, f, mlp, scale):
    hl = n * d
    f1 = 2 * f if mlp == "swiglu" else f
    return dict(
        w_qkv=rng.standard_normal((h, 3 * hl)) * scale, w_o=rng.standard_normal((hl, h)) * scale,
        w_fc1=rng.standard_normal((h, f1)) * scale, w_fc2=rng.standard_normal((f, h)) * scale,
        ln_gamma=1 + 0.2 * rng.standard_normal(h), ln_beta=0.2 * rng.standard_normal(h),
        ln2_gamma=1 + 0.2 * rng.standard_normal(h), ln2_beta=0.2 * rng.standard_normal(h))


def _torch_layer(x, p, b, s, n, d, w, eps, norm, mlp, serial):
    """Independent torch implementation (autograd for the gradients); W1 and
    W3 are picked out of w_fc1 by explicit column index lists."""
    hl = n * d
    h = x.shape[1]

    def nrm(z, g, bt):
        if norm == "rmsnorm":
            return torch.nn.functional.rms_norm(z, (h,), g, eps)
        return torch.nn.functional.layer_norm(z, (h,), g, bt, eps)

    def heads(t):
        return t.reshape(b, s, n, d).permute(0, 2, 1, 3)

    def attn(a):
        qkv = a @ p["w_qkv"]
        q, k, v = heads(qkv[:, :hl]), heads(qkv[:, hl:2 * hl]), heads(qkv[:, 2 * hl:])
        i = torch.arange(s)[:, None]
        j = torch.arange(s)[None, :]
        ok = (i >= j) & (i - j < w)
        lg = ((q @ k.transpose(-1, -2)) / math.sqrt(d)).masked_fill(~ok, float("-inf"))
        return (torch.softmax(lg, -1) @ v).permute(0, 2, 1, 3).reshape(b * s, hl) @ p["w_o"]

    def mlp_(a):
        if mlp == "swiglu":
            f = p["w_fc2"].shape[0]
            cols1 = [64 * (c // 32) + c % 32 for c in range(f)]
            w1 = p["w_fc1"][:, cols1]
            w3 = p["w_fc1"][:, [c + 32 for c in cols1]]
            return (torch.nn.functional.silu(a @ w1) * (a @ w3)) @ p["w_fc2"]
        return torch.nn.functional.gelu(a @ p["w_fc1"]) @ p["w_fc2"]

    a = nrm(x, p["ln_gamma"], p["ln_beta"])
    if serial:
        x1 = x + attn(a)
        return x1 + mlp_(nrm(x1, p["ln2_gamma"], p["ln2_beta"]))
    return x + attn(a) + mlp_(a)


KEYS = ("ln_gamma", "ln_beta", "w_qkv", "w_o", "w_fc1", "w_fc2")
SKEYS = KEYS + ("ln2_gamma", "ln2_beta")
GRAD = dict(ln_gamma="d_ln_gamma", ln_beta="d_ln_beta", ln2_gamma="d_ln2_gamma",
            ln2_beta="d_ln2_beta", w_qkv="dw_qkv", w_o="dw_o", w_fc1="dw_fc1", w_fc2="dw_fc2")


@pytest.mark.parametrize("serial", [False, True])
@pytest.mark.parametrize("norm,mlp", [("rmsnorm", "gelu"), ("layernorm", "swiglu"),
                                      ("rmsnorm", "swiglu")])
def test_variant_layers_match_torch_fp64_autograd(norm, mlp, serial):
    rng = np.random.default_rng(610)
    b, s, h, n, d, f, w = 2, 23, 64, 4, 16, 96, 9
    x = rng.standard_normal((b * s, h))
    p = _params(rng, h, n, d, f, mlp, 0.15)
    dy = rng.standard_normal(x.shape)
    if serial:
        y, cache = O.serial_forward(x, p, b, s, n, d, w, 1e-5, norm=norm, mlp=mlp)
        g = O.serial_backward(dy, cache, p, w)
    else:
        y, cache = O.ptb_forward(x, p, b, s, n, d, w, 1e-5, norm=norm, mlp=mlp)
        g = O.ptb_backward(dy, cache, p, w)
    tx = torch.tensor(x, requires_grad=True)
    tp = {k: torch.tensor(v, requires_grad=True) for k, v in p.items()}
    ty = _torch_layer(tx, tp, b, s, n, d, w, 1e-5, norm, mlp, serial)
    ty.backward(torch.tensor(dy))
    np.testing.assert_allclose(y, ty.detach().numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(g["dx"], tx.grad.numpy(), rtol=1e-10, atol=1e-10)
    for k in (SKEYS if serial else KEYS):
        if norm == "rmsnorm" and k in ("ln_beta", "ln2_beta"):
            assert tp[k].grad is None      # beta takes no part in RMSNorm
            ref = np.zeros(p[k].shape)
        else:
            ref = tp[k].grad.numpy()
        np.testing.assert_allclose(g[GRAD[k]], ref, rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("window", [1, 4, 7])
def test_rmsnorm_swiglu_layer_finite_difference_every_tensor(window):
    rng = np.random.default_rng(620 + window)
    b, s, h, n, d, f = 2, 7, 16, 2, 8, 64
    x = rng.standard_normal((b * s, h))
    p = _params(rng, h, n, d, f, "swiglu", 0.3)
    dy = rng.standard_normal(x.shape)
    _, cache = O.ptb_forward(x, p, b, s, n, d, window, 1e-5, norm="rmsnorm", mlp="swiglu")
    g = O.ptb_backward(dy, cache, p, window)
    e = 1e-6

    def L(xx, pp):
        return (O.ptb_forward(xx, pp, b, s, n, d, window, 1e-5, norm="rmsnorm",
                              mlp="swiglu")[0] * dy).sum()

    for key in ("ln_gamma", "w_qkv", "w_o", "w_fc1", "w_fc2", "x"):
        vdir = rng.standard_normal(x.shape if key == "x" else p[key].shape)
        if key == "x":
            fd = (L(x + e * vdir, p) - L(x - e * vdir, p)) / (2 * e)
            an = (g["dx"] * vdir).sum()
        else:
            fd = (L(x, dict(p, **{key: p[key] + e * vdir}))
                  - L(x, dict(p, **{key: p[key] - e * vdir}))) / (2 * e)
            an = (g[GRAD[key]] * vdir).sum()
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (key, fd, an)


def test_swiglu_flop_counter_equals_closed_form():
    rng = np.random.default_rng(630)
    b, s, h, n, d, f, w = 2, 13, 32, 2, 8, 64, 5
    x = rng.standard_normal((b * s, h))
    p = _params(rng, h, n, d, f, "swiglu", 0.3)
    fc = O.FlopCounter()
    _, cache = O.ptb_forward(x, p, b, s, n, d, w, 1e-5, fc, norm="rmsnorm", mlp="swiglu")
    O.ptb_backward(rng.standard_normal(x.shape), cache, p, w, fc)
    assert fc.model == F.model_flops(b, s, h, n, d, f, w, mlp="swiglu")
    assert F.matmul_params(h, n, d, f, "swiglu") == h * (4 * n * d + 3 * f)
