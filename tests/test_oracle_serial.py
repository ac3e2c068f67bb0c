"""Pins of the fp64 oracle's serial (standard) block, MegaScale reading notes
section 1.1 eq (3), against facts that do not come from its own code path:
an exact identity that builds the block from three calls of the (separately
pinned) parallel-block oracle, reductions to the parallel block when one
sub-block is switched off, central finite differences, an independent torch
fp64 autograd implementation, and the closed-form FLOP count.  CPU only.
"""
import math

import numpy as np
import pytest
import torch

from oracle import ptb_oracle as O
from transformer_block_amd import flops as F
from transformer_block_amd import inputs as I

PARAM_KEYS = ("ln_gamma", "ln_beta", "ln2_gamma", "ln2_beta", "w_qkv", "w_o", "w_fc1",
              "w_fc2")
GRAD_OF = dict(ln_gamma="d_ln_gamma", ln_beta="d_ln_beta", ln2_gamma="d_ln2_gamma",
               ln2_beta="d_ln2_beta", w_qkv="dw_qkv", w_o="dw_o", w_fc1="dw_fc1",
               w_fc2="dw_fc2")


def _params(rng, h, n, d, f, scale=0.3):
    hl = n * d
    return dict(
        w_qkv=rng.standard_normal((h, 3 * hl)) * scale,
        w_o=rng.standard_normal((hl, h)) * scale,
        w_fc1=rng.standard_normal((h, f)) * scale,
        w_fc2=rng.standard_normal((f, h)) * scale,
        ln_gamma=1 + 0.2 * rng.standard_normal(h), ln_beta=0.2 * rng.standard_normal(h),
        ln2_gamma=1 + 0.2 * rng.standard_normal(h), ln2_beta=0.2 * rng.standard_normal(h),
    )


def _case(seed, b=2, s=11, h=32, n=2, d=8, f=64, scale=0.3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((b * s, h))
    return rng, x, _params(rng, h, n, d, f, scale)


@pytest.mark.parametrize("window", [1, 4, 11, 30])
def test_serial_block_from_three_parallel_block_calls(window):
    """x1 = x + Attn(LN1(x)) W_o is the parallel block with W_fc2 = 0;
    z -> z + MLP(LN2(z)) is the parallel block with W_o = 0 and LN2's
    parameters; the serial block is the second applied to the first."""
    rng, x, p = _case(40 + window)
    b, s, n, d = 2, 11, 2, 8
    y, cache = O.serial_forward(x, p, b, s, n, d, window, 1e-5)
    attn_only = dict(p, w_fc2=np.zeros_like(p["w_fc2"]))
    x1, _ = O.ptb_forward(x, attn_only, b, s, n, d, window, 1e-5)
    mlp_only = dict(p, w_o=np.zeros_like(p["w_o"]), ln_gamma=p["ln2_gamma"],
                    ln_beta=p["ln2_beta"])
    y_ref, _ = O.ptb_forward(x1, mlp_only, b, s, n, d, window, 1e-5)
    np.testing.assert_allclose(cache["x1"], x1, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(y, y_ref, rtol=1e-13, atol=1e-13)


def test_serial_reduces_to_parallel_attention_branch_without_mlp():
    """W_fc2 = 0: both blocks are x + Attn(LN1(x)) W_o; so are dx, dW_qkv,
    dW_o and LN1's gradients, and W_fc1 and LN2 get no gradient."""
    rng, x, p = _case(50)
    b, s, n, d, w = 2, 11, 2, 8, 5
    p["w_fc2"][:] = 0
    dy = rng.standard_normal(x.shape)
    ys, cs = O.serial_forward(x, p, b, s, n, d, w, 1e-5)
    gs = O.serial_backward(dy, cs, p, w)
    yp, cp = O.ptb_forward(x, p, b, s, n, d, w, 1e-5)
    gp = O.ptb_backward(dy, cp, p, w)
    np.testing.assert_allclose(ys, yp, rtol=1e-13, atol=1e-13)
    for k in ("dx", "dw_qkv", "dw_o", "d_ln_gamma", "d_ln_beta"):
        np.testing.assert_allclose(gs[k], gp[k], rtol=1e-12, atol=1e-12)
    for k in ("dw_fc1", "d_ln2_gamma", "d_ln2_beta"):
        np.testing.assert_array_equal(gs[k], 0.0)


def test_serial_reduces_to_parallel_mlp_branch_without_attention_output():
    """W_o = 0: x1 = x, so the serial block is x + MLP(LN2(x)), the parallel
    block with W_o = 0 and LN2's parameters; so are dx and the MLP's and
    LN2's gradients, and W_qkv and LN1 get no gradient."""
    rng, x, p = _case(51)
    b, s, n, d, w = 2, 11, 2, 8, 7
    p["w_o"][:] = 0
    dy = rng.standard_normal(x.shape)
    ys, cs = O.serial_forward(x, p, b, s, n, d, w, 1e-5)
    gs = O.serial_backward(dy, cs, p, w)
    pm = dict(p, ln_gamma=p["ln2_gamma"], ln_beta=p["ln2_beta"])
    yp, cp = O.ptb_forward(x, pm, b, s, n, d, w, 1e-5)
    gp = O.ptb_backward(dy, cp, pm, w)
    np.testing.assert_allclose(ys, yp, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(gs["dx"], gp["dx"], rtol=1e-12, atol=1e-12)
    for k in ("dw_fc1", "dw_fc2"):
        np.testing.assert_allclose(gs[k], gp[k], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gs["d_ln2_gamma"], gp["d_ln_gamma"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gs["d_ln2_beta"], gp["d_ln_beta"], rtol=1e-12, atol=1e-12)
    for k in ("dw_qkv", "d_ln_gamma", "d_ln_beta"):
        np.testing.assert_array_equal(gs[k], 0.0)


@pytest.mark.parametrize("window", [1, 3, 7, 9])
def test_serial_backward_finite_difference_every_tensor(window):
    """Central differences on b=2, s=7, h=16, n=2, d=8, f=32: one random
    direction per tensor (x and all eight parameters) and single coordinates."""
    rng, x, p = _case(60 + window, b=2, s=7, h=16, n=2, d=8, f=32)
    b, s, n, d = 2, 7, 2, 8
    dy = rng.standard_normal(x.shape)
    _, cache = O.serial_forward(x, p, b, s, n, d, window, 1e-5)
    g = O.serial_backward(dy, cache, p, window)
    e = 1e-6

    def L(xx, pp):
        return (O.serial_forward(xx, pp, b, s, n, d, window, 1e-5)[0] * dy).sum()

    for key in PARAM_KEYS + ("x",):
        vdir = rng.standard_normal(x.shape if key == "x" else p[key].shape)
        if key == "x":
            fd = (L(x + e * vdir, p) - L(x - e * vdir, p)) / (2 * e)
            an = (g["dx"] * vdir).sum()
        else:
            fd = (L(x, dict(p, **{key: p[key] + e * vdir}))
                  - L(x, dict(p, **{key: p[key] - e * vdir}))) / (2 * e)
            an = (g[GRAD_OF[key]] * vdir).sum()
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (key, fd, an)
    for key in ("w_o", "ln2_gamma", "w_qkv"):
        for _ in range(2):
            idx = tuple(rng.integers(0, dim) for dim in p[key].shape)
            pp = p[key].copy(); pp[idx] += e
            pm = p[key].copy(); pm[idx] -= e
            fd = (L(x, dict(p, **{key: pp})) - L(x, dict(p, **{key: pm}))) / (2 * e)
            assert abs(fd - g[GRAD_OF[key]][idx]) <= 1e-6 * max(1.0, abs(fd))


def _torch_serial(x, p, b, s, n, d, w, eps):
    """Independent serial block written with torch ops (autograd for grads)."""
    hl = n * d
    ln = torch.nn.functional.layer_norm
    a1 = ln(x, (x.shape[1],), p["ln_gamma"], p["ln_beta"], eps)
    qkv = a1 @ p["w_qkv"]

    def heads(t):
        return t.reshape(b, s, n, d).permute(0, 2, 1, 3)

    q, k, v = heads(qkv[:, :hl]), heads(qkv[:, hl:2 * hl]), heads(qkv[:, 2 * hl:])
    i = torch.arange(s)[:, None]
    j = torch.arange(s)[None, :]
    allowed = (i >= j) & (i - j < w)
    logits = ((q @ k.transpose(-1, -2)) / math.sqrt(d)).masked_fill(~allowed, float("-inf"))
    c = (torch.softmax(logits, dim=-1) @ v).permute(0, 2, 1, 3).reshape(b * s, hl)
    x1 = x + c @ p["w_o"]
    a2 = ln(x1, (x.shape[1],), p["ln2_gamma"], p["ln2_beta"], eps)
    return x1 + torch.nn.functional.gelu(a2 @ p["w_fc1"]) @ p["w_fc2"]


@pytest.mark.parametrize("window", [1, 5, 37, 64])
def test_serial_matches_torch_fp64_autograd(window):
    rng, x, p = _case(70 + window, b=2, s=37, h=64, n=4, d=16, f=128, scale=0.15)
    b, s, n, d = 2, 37, 4, 16
    dy = rng.standard_normal(x.shape)
    y, cache = O.serial_forward(x, p, b, s, n, d, window, 1e-5)
    g = O.serial_backward(dy, cache, p, window)
    tx = torch.tensor(x, requires_grad=True)
    tp = {k: torch.tensor(v, requires_grad=True) for k, v in p.items()}
    ty = _torch_serial(tx, tp, b, s, n, d, window, 1e-5)
    ty.backward(torch.tensor(dy))
    np.testing.assert_allclose(y, ty.detach().numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(g["dx"], tx.grad.numpy(), rtol=1e-10, atol=1e-10)
    for k in PARAM_KEYS:
        np.testing.assert_allclose(g[GRAD_OF[k]], tp[k].grad.numpy(), rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("b,s,h,n,d,f,w", [(2, 13, 32, 2, 8, 64, 5), (1, 20, 64, 4, 16, 96, 20),
                                           (3, 9, 16, 1, 8, 32, 100)])
def test_serial_flop_counter_equals_closed_form(b, s, h, n, d, f, w):
    """The serial block does the same products and attention pairs as the
    parallel one, so its counted model FLOPs equal the same closed form."""
    rng = np.random.default_rng(80)
    x = rng.standard_normal((b * s, h))
    p = _params(rng, h, n, d, f)
    fc = O.FlopCounter()
    _, cache = O.serial_forward(x, p, b, s, n, d, w, 1e-5, fc)
    O.serial_backward(rng.standard_normal(x.shape), cache, p, w, fc)
    assert fc.model == F.model_flops(b, s, h, n, d, f, w)
    assert fc.recompute == F.recompute_flops(b, s, n, d, w)


def test_inputs_carry_a_second_layernorm_without_changing_other_draws():
    wl = I.WORKLOADS["tiny_h256_s256_w64"]
    a = I.make_inputs(wl, random_ln=True)
    lay = a["layers"][0]
    assert lay["ln2_gamma"].shape == (256,) and lay["ln2_beta"].shape == (256,)
    assert not np.array_equal(lay["ln2_gamma"], lay["ln_gamma"])
    plain = I.make_inputs(wl)["layers"][0]
    np.testing.assert_array_equal(I.bf16_bits_to_f64(plain["ln2_gamma"]), 1.0)
    np.testing.assert_array_equal(I.bf16_bits_to_f64(plain["ln2_beta"]), 0.0)
    np.testing.assert_array_equal(plain["w_fc2"], lay["w_fc2"])
