"""Pins of the dropout oracle (oracle/dropout_oracle.py) and of the layer
oracle with dropout (MegaScale reading notes, section 1.3: fused dropout,
dropout activations kept for backward).  The generator is pinned to the
published known-answer values of Philox-4x32-10 and to a scalar
re-computation in Python integers; the masks to binomial keep rates and to
their documented element-to-counter mapping; the layer to the no-dropout
layer at p = 0, to central finite differences with a fixed mask and to an
independent torch fp64 autograd implementation.  CPU only."""
import math
import os

import numpy as np
import pytest
import torch

from oracle import dropout_oracle as D
from oracle import ptb_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _kat():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            w = [int(t, 16) for t in line.split()]
            rows.append((w[:4], w[4:6], w[6:10]))
    return rows


def test_philox_known_answers():
    rows = _kat()
    assert len(rows) == 3
    for ctr, key, out in rows:
        got = D.philox4x32_10(*[np.array([c], np.uint64) for c in ctr], *key)
        assert [int(g[0]) for g in got] == out


def _philox_scalar(ctr, key):
    """The same generator in Python integers, one counter at a time."""
    c = list(ctr)
    k0, k1 = key
    for r in range(10):
        if r:
            k0 = (k0 + 0x9E3779B9) & 0xFFFFFFFF
            k1 = (k1 + 0xBB67AE85) & 0xFFFFFFFF
        p0 = 0xD2511F53 * c[0]
        p1 = 0xCD9E8D57 * c[2]
        c = [(p1 >> 32) ^ c[1] ^ k0, p1 & 0xFFFFFFFF, (p0 >> 32) ^ c[3] ^ k1, p0 & 0xFFFFFFFF]
    return c


def test_vectorised_generator_equals_scalar_integers():
    rng = np.random.default_rng(1)
    ctr = rng.integers(0, 2 ** 32, size=(64, 4), dtype=np.uint64)
    key = (0x12345678, 0x9ABCDEF0)
    got = np.stack(D.philox4x32_10(ctr[:, 0], ctr[:, 1], ctr[:, 2], ctr[:, 3], *key), axis=1)
    for i in range(64):
        assert [int(v) for v in got[i]] == _philox_scalar([int(v) for v in ctr[i]], key)


def test_mask_element_mapping():
    """Element e takes word e & 3 of the output for counter (e >> 2, stream,
    0, 0) under key (seed mod 2^32, seed >> 32), kept iff >= floor(p 2^32)."""
    seed, stream, p = (7 << 32) | 12345, 5, 0.3
    n = 103   # a ragged last group
    keep = D.dropout_keep(n, seed, stream, p)
    t = D.dropout_threshold(p)
    for e in range(n):
        word = _philox_scalar([e >> 2, stream, 0, 0], (seed & 0xFFFFFFFF, seed >> 32))[e & 3]
        assert bool(keep[e]) == (word >= t)


def test_threshold_and_scale_from_the_fp32_rate():
    assert D.dropout_threshold(0.0) == 0
    assert D.dropout_threshold(0.5) == 2 ** 31
    # 0.1 in fp32 is 13421773 * 2^-27, so p * 2^32 = 13421773 * 32 exactly
    assert D.dropout_threshold(0.1) == 13421773 * 32
    assert D.dropout_scale(0.5) == 2.0
    assert D.dropout_scale(0.1) == 1.0 / (1.0 - float(np.float32(0.1)))
    for bad in (-0.1, 1.0, 1.5):
        with pytest.raises(ValueError):
            D.dropout_threshold(bad)


@pytest.mark.parametrize("p", [0.05, 0.1, 0.5, 0.9])
def test_keep_rate_within_binomial_bounds(p):
    n = 1 << 20
    keep = D.dropout_keep(n, seed=2024, stream=3, p=p)
    q = 1.0 - D.dropout_threshold(p) / 2 ** 32
    sigma = math.sqrt(n * q * (1 - q))
    assert abs(keep.sum() - n * q) <= 5 * sigma


def test_p_zero_keeps_everything_and_streams_differ():
    assert D.dropout_keep(1000, 1, 0, 0.0).all()
    np.testing.assert_array_equal(D.dropout_multiplier((10, 8), 1, 0, 0.0), 1.0)
    a = D.dropout_keep(1 << 16, 99, 0, 0.5)
    b = D.dropout_keep(1 << 16, 99, 1, 0.5)
    c = D.dropout_keep(1 << 16, 100, 0, 0.5)
    # different streams and seeds: masks agree on about half the elements
    for other in (b, c):
        agree = (a == other).mean()
        assert abs(agree - 0.5) < 5 * 0.5 / math.sqrt(1 << 16)


def test_output_bits_are_uniform():
    """Every bit of the output words is set half the time (counters 0..2^16)."""
    j = np.arange(1 << 16, dtype=np.uint64)
    words = np.concatenate(D.philox4x32_10(j, 0, 0, 0, 0xDEADBEEF, 0x01234567))
    n = words.size
    for bit in range(32):
        ones = int(((words >> np.uint32(bit)) & np.uint32(1)).sum())
        assert abs(ones - n / 2) <= 5 * math.sqrt(n / 4), bit


# ------------------------------------------------------------ layer with dropout
def _rand_params(rng, h, n, d, f, scale=0.3):
    hl = n * d
    return dict(
        w_qkv=rng.standard_normal((h, 3 * hl)) * scale,
        w_o=rng.standard_normal((hl, h)) * scale,
        w_fc1=rng.standard_normal((h, f)) * scale,
        w_fc2=rng.standard_normal((f, h)) * scale,
        ln_gamma=1 + 0.2 * rng.standard_normal(h), ln_beta=0.2 * rng.standard_normal(h),
        ln2_gamma=1 + 0.2 * rng.standard_normal(h), ln2_beta=0.2 * rng.standard_normal(h),
    )


PARAM_KEYS = ("ln_gamma", "ln_beta", "w_qkv", "w_o", "w_fc1", "w_fc2")
GRAD_OF = dict(ln_gamma="d_ln_gamma", ln_beta="d_ln_beta", w_qkv="dw_qkv", w_o="dw_o",
               w_fc1="dw_fc1", w_fc2="dw_fc2", ln2_gamma="d_ln2_gamma", ln2_beta="d_ln2_beta")


def test_rate_zero_reproduces_the_layer_exactly():
    rng = np.random.default_rng(3)
    b, s, h, n, d, f, w = 2, 9, 32, 2, 8, 64, 4
    x = rng.standard_normal((b * s, h))
    p = _rand_params(rng, h, n, d, f)
    dy = rng.standard_normal(x.shape)
    ones = D.dropout_multiplier(x.shape, 5, 0, 0.0)
    y0, c0 = O.ptb_forward(x, p, b, s, n, d, w, 1e-5)
    y1, c1 = O.ptb_forward(x, p, b, s, n, d, w, 1e-5, drop=ones)
    np.testing.assert_array_equal(y0, y1)
    g0, g1 = O.ptb_backward(dy, c0, p, w), O.ptb_backward(dy, c1, p, w)
    for k in g0:
        np.testing.assert_array_equal(g0[k], g1[k])
    ys0, cs0 = O.serial_forward(x, p, b, s, n, d, w, 1e-5)
    ys1, cs1 = O.serial_forward(x, p, b, s, n, d, w, 1e-5, drop1=ones, drop2=ones)
    np.testing.assert_array_equal(ys0, ys1)
    gs0, gs1 = O.serial_backward(dy, cs0, p, w), O.serial_backward(dy, cs1, p, w)
    for k in gs0:
        np.testing.assert_array_equal(gs0[k], gs1[k])


def test_dropped_elements_carry_the_residual_only():
    rng = np.random.default_rng(4)
    b, s, h, n, d, f, w = 1, 16, 32, 2, 8, 64, 16
    x = rng.standard_normal((b * s, h))
    p = _rand_params(rng, h, n, d, f)
    m = D.dropout_multiplier(x.shape, 77, D.layer_stream(0), 0.25)
    assert 0 < (m == 0).mean() < 0.5
    y, cache = O.ptb_forward(x, p, b, s, n, d, w, 1e-5, drop=m)
    np.testing.assert_array_equal(y[m == 0], x[m == 0])
    y_plain, _ = O.ptb_forward(x, p, b, s, n, d, w, 1e-5)
    kept = m > 0
    np.testing.assert_allclose((y - x)[kept], (y_plain - x)[kept] / (1 - np.float32(0.25)),
                               rtol=1e-12, atol=1e-12)
    # the residual's gradient is dy itself wherever the branch is dropped
    dy = rng.standard_normal(x.shape)
    g = O.ptb_backward(dy, cache, p, w)
    p0 = dict(p, w_o=np.zeros_like(p["w_o"]), w_fc2=np.zeros_like(p["w_fc2"]))
    _, c0 = O.ptb_forward(x, p0, b, s, n, d, w, 1e-5, drop=m)
    np.testing.assert_array_equal(O.ptb_backward(dy, c0, p0, w)["dx"], dy)
    assert np.isfinite(g["dx"]).all()


@pytest.mark.parametrize("window", [1, 3, 7])
def test_dropout_layer_finite_difference(window):
    rng = np.random.default_rng(40 + window)
    b, s, h, n, d, f = 2, 7, 16, 2, 8, 32
    x = rng.standard_normal((b * s, h))
    p = _rand_params(rng, h, n, d, f)
    m = D.dropout_multiplier(x.shape, 1234, D.layer_stream(1), 0.3)
    dy = rng.standard_normal(x.shape)
    _, cache = O.ptb_forward(x, p, b, s, n, d, window, 1e-5, drop=m)
    g = O.ptb_backward(dy, cache, p, window)
    e = 1e-6

    def L(xx, pp):
        return (O.ptb_forward(xx, pp, b, s, n, d, window, 1e-5, drop=m)[0] * dy).sum()

    for key in PARAM_KEYS + ("x",):
        v = rng.standard_normal(x.shape if key == "x" else p[key].shape)
        if key == "x":
            fd = (L(x + e * v, p) - L(x - e * v, p)) / (2 * e)
            an = (g["dx"] * v).sum()
        else:
            fd = (L(x, dict(p, **{key: p[key] + e * v})) - L(x, dict(p, **{key: p[key] - e * v}))) / (2 * e)
            an = (g[GRAD_OF[key]] * v).sum()
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (key, fd, an)


@pytest.mark.parametrize("window", [2, 7])
def test_dropout_serial_block_finite_difference(window):
    rng = np.random.default_rng(50 + window)
    b, s, h, n, d, f = 2, 7, 16, 2, 8, 32
    x = rng.standard_normal((b * s, h))
    p = _rand_params(rng, h, n, d, f)
    m1 = D.dropout_multiplier(x.shape, 99, D.layer_stream(0, 0), 0.2)
    m2 = D.dropout_multiplier(x.shape, 99, D.layer_stream(0, 1), 0.2)
    assert not np.array_equal(m1, m2)
    dy = rng.standard_normal(x.shape)
    _, cache = O.serial_forward(x, p, b, s, n, d, window, 1e-5, drop1=m1, drop2=m2)
    g = O.serial_backward(dy, cache, p, window)
    e = 1e-6

    def L(xx, pp):
        return (O.serial_forward(xx, pp, b, s, n, d, window, 1e-5, drop1=m1, drop2=m2)[0]
                * dy).sum()

    for key in PARAM_KEYS + ("ln2_gamma", "ln2_beta", "x"):
        v = rng.standard_normal(x.shape if key == "x" else p[key].shape)
        if key == "x":
            fd = (L(x + e * v, p) - L(x - e * v, p)) / (2 * e)
            an = (g["dx"] * v).sum()
        else:
            fd = (L(x, dict(p, **{key: p[key] + e * v})) - L(x, dict(p, **{key: p[key] - e * v}))) / (2 * e)
            an = (g[GRAD_OF[key]] * v).sum()
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (key, fd, an)


def _torch_ptb_dropout(x, p, m, b, s, n, d, w, eps):
    """Independent PTB with the dropout multiplier m on the branch output,
    written with torch ops and differentiated by autograd."""
    hl = n * d
    a = torch.nn.functional.layer_norm(x, (x.shape[1],), p["ln_gamma"], p["ln_beta"], eps)
    qkv = a @ p["w_qkv"]

    def heads(t):
        return t.reshape(b, s, n, d).permute(0, 2, 1, 3)

    q, k, v = heads(qkv[:, :hl]), heads(qkv[:, hl:2 * hl]), heads(qkv[:, 2 * hl:])
    i = torch.arange(s)[:, None]
    j = torch.arange(s)[None, :]
    allowed = (i >= j) & (i - j < w)
    logits = ((q @ k.transpose(-1, -2)) / math.sqrt(d)).masked_fill(~allowed, float("-inf"))
    c = (torch.softmax(logits, dim=-1) @ v).permute(0, 2, 1, 3).reshape(b * s, hl)
    branch = c @ p["w_o"] + torch.nn.functional.gelu(a @ p["w_fc1"]) @ p["w_fc2"]
    return x + m * branch


@pytest.mark.parametrize("window", [1, 9, 37])
def test_dropout_layer_matches_torch_fp64_autograd(window):
    rng = np.random.default_rng(60 + window)
    b, s, h, n, d, f = 2, 37, 64, 4, 16, 128
    x = rng.standard_normal((b * s, h))
    p = _rand_params(rng, h, n, d, f, scale=0.15)
    m = D.dropout_multiplier(x.shape, 4321, D.layer_stream(2), 0.15)
    dy = rng.standard_normal(x.shape)
    y, cache = O.ptb_forward(x, p, b, s, n, d, window, 1e-5, drop=m)
    g = O.ptb_backward(dy, cache, p, window)
    tx = torch.tensor(x, requires_grad=True)
    tp = {k: torch.tensor(v, requires_grad=True) for k, v in p.items() if k in PARAM_KEYS}
    ty = _torch_ptb_dropout(tx, tp, torch.tensor(m), b, s, n, d, window, 1e-5)
    ty.backward(torch.tensor(dy))
    np.testing.assert_allclose(y, ty.detach().numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(g["dx"], tx.grad.numpy(), rtol=1e-10, atol=1e-10)
    for k in PARAM_KEYS:
        np.testing.assert_allclose(g[GRAD_OF[k]], tp[k].grad.numpy(), rtol=1e-10, atol=1e-10)
