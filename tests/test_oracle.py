"""Pins of the fp64 oracle against facts that do not come from the oracle
itself: closed forms, invariants, textbook tables, brute force on tiny inputs,
finite differences, independent library implementations (torch fp64 CPU
autograd), and the shapes the pages print.  CPU only.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import ptb_oracle as O
from transformer_block_amd import flops as F
from transformer_block_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_params(rng, h, n, d, f, scale=0.3, random_ln=True):
    hl = n * d
    p = dict(
        w_qkv=rng.standard_normal((h, 3 * hl)) * scale,
        w_o=rng.standard_normal((hl, h)) * scale,
        w_fc1=rng.standard_normal((h, f)) * scale,
        w_fc2=rng.standard_normal((f, h)) * scale,
        ln_gamma=(1 + 0.2 * rng.standard_normal(h)) if random_ln else np.ones(h),
        ln_beta=(0.2 * rng.standard_normal(h)) if random_ln else np.zeros(h),
    )
    return p


# ---------------------------------------------------------------- LayerNorm
def test_layernorm_row_moments_closed_form():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((17, 96)) * 3 + 1.5
    eps = 1e-5
    a, mu, rstd = O.layernorm_forward(x, np.ones(96), np.zeros(96), eps)
    var = x.var(axis=1)
    np.testing.assert_allclose(a.mean(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose(a.var(axis=1), var / (var + eps), rtol=1e-12)
    np.testing.assert_allclose(mu, x.mean(axis=1), rtol=1e-12)


def test_layernorm_matches_torch_fp64():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((9, 64))
    g = 1 + 0.1 * rng.standard_normal(64)
    b = 0.1 * rng.standard_normal(64)
    a, _, _ = O.layernorm_forward(x, g, b, 1e-5)
    ref = torch.nn.functional.layer_norm(torch.tensor(x), (64,), torch.tensor(g),
                                         torch.tensor(b), eps=1e-5).numpy()
    np.testing.assert_allclose(a, ref, rtol=1e-12, atol=1e-12)


def test_layernorm_backward_finite_difference():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 32))
    g = 1 + 0.3 * rng.standard_normal(32)
    b = 0.3 * rng.standard_normal(32)
    da = rng.standard_normal((5, 32))
    a, mu, rstd = O.layernorm_forward(x, g, b, 1e-5)
    dx, dg, db = O.layernorm_backward(da, x, g, mu, rstd)
    vx, vg, vb = (rng.standard_normal(s) for s in (x.shape, g.shape, b.shape))
    eps = 1e-6

    def L(t):
        return (O.layernorm_forward(x + t * vx, g + t * vg, b + t * vb, 1e-5)[0] * da).sum()

    fd = (L(eps) - L(-eps)) / (2 * eps)
    an = (dx * vx).sum() + (dg * vg).sum() + (db * vb).sum()
    assert abs(fd - an) <= 1e-7 * max(1.0, abs(an))


# --------------------------------------------------------------------- GeLU
def _normal_table():
    rows = []
    with open(os.path.join(GOLDEN, "normal_cdf.txt")) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            u, p = line.split()
            rows.append((float(u), float(p)))
    return rows


def test_gelu_against_normal_table():
    for u, phi in _normal_table():
        assert O.normal_cdf(np.float64(u)) == pytest.approx(phi, rel=1e-12, abs=1e-14)
        assert O.gelu(np.float64(u)) == pytest.approx(u * phi, rel=1e-12, abs=1e-14)


def test_gelu_identities_and_derivative():
    u = np.linspace(-6, 6, 241)
    # Phi(u) + Phi(-u) = 1  =>  GeLU(u) - GeLU(-u) = u
    np.testing.assert_allclose(O.gelu(u) - O.gelu(-u), u, atol=1e-13)
    assert O.gelu(np.float64(0.0)) == 0.0
    assert O.gelu_grad(np.float64(0.0)) == pytest.approx(0.5, abs=1e-15)
    h = 1e-6
    fd = (O.gelu(u + h) - O.gelu(u - h)) / (2 * h)
    np.testing.assert_allclose(O.gelu_grad(u), fd, atol=1e-8)


def test_gelu_matches_torch_exact_gelu():
    u = np.linspace(-8, 8, 1001)
    ref = torch.nn.functional.gelu(torch.tensor(u), approximate="none").numpy()
    np.testing.assert_allclose(O.gelu(u), ref, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- Attention
def _brute_attention(q, k, v, window):
    """Pure-Python loops: for every query, softmax over the explicitly listed
    keys j in [i - window + 1, i] (clipped at 0), then the weighted sum of v."""
    b, n, s, d = q.shape
    out = np.zeros_like(q)
    scale = 1.0 / math.sqrt(d)
    for bi in range(b):
        for hi in range(n):
            for i in range(s):
                keys = [j for j in range(max(0, i - window + 1), i + 1)]
                logits = []
                for j in keys:
                    acc = 0.0
                    for c in range(d):
                        acc += q[bi, hi, i, c] * k[bi, hi, j, c]
                    logits.append(acc * scale)
                m = max(logits)
                ws = [math.exp(z - m) for z in logits]
                tot = sum(ws)
                for c in range(d):
                    out[bi, hi, i, c] = sum(wj * v[bi, hi, j, c]
                                            for wj, j in zip(ws, keys)) / tot
    return out


def _brute_full_causal(q, k, v):
    """Full causal attention without any window notion: all keys j <= i."""
    b, n, s, d = q.shape
    out = np.zeros_like(q)
    for bi in range(b):
        for hi in range(n):
            for i in range(s):
                logits = [sum(q[bi, hi, i, c] * k[bi, hi, j, c] for c in range(d)) / math.sqrt(d)
                          for j in range(i + 1)]
                m = max(logits)
                ws = [math.exp(z - m) for z in logits]
                for c in range(d):
                    out[bi, hi, i, c] = sum(ws[j] * v[bi, hi, j, c] for j in range(i + 1)) / sum(ws)
    return out


def _qkv(rng, b=2, n=2, s=9, d=4, scale=1.0):
    return tuple(rng.standard_normal((b, n, s, d)) * scale for _ in range(3))


@pytest.mark.parametrize("window", [9, 10, 50])
def test_attention_window_ge_seq_is_full_causal_bruteforce(window):
    rng = np.random.default_rng(3)
    q, k, v = _qkv(rng, scale=1.5)
    np.testing.assert_allclose(O.attention_forward(q, k, v, window),
                               _brute_full_causal(q, k, v), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("window", [1, 2, 3, 5, 8])
def test_attention_sliding_window_bruteforce(window):
    rng = np.random.default_rng(4)
    q, k, v = _qkv(rng, scale=1.5)
    np.testing.assert_allclose(O.attention_forward(q, k, v, window),
                               _brute_attention(q, k, v, window), rtol=1e-12, atol=1e-12)


def test_window_mask_counts_w_most_recent_tokens():
    for s, w in [(1, 1), (7, 1), (7, 3), (7, 7), (7, 12), (33, 16)]:
        m = O.window_mask(s, w)
        np.testing.assert_array_equal(m.sum(axis=1), np.minimum(np.arange(s) + 1, w))
        assert not np.triu(m, 1).any()          # causal: no key after the query
        assert m.diagonal().all()               # the query always sees itself


def test_attention_window_one_is_identity_and_backward():
    rng = np.random.default_rng(5)
    q, k, v = _qkv(rng, s=11, d=8, scale=3.0)
    do = rng.standard_normal(q.shape)
    np.testing.assert_array_equal(O.attention_forward(q, k, v, 1), v)
    dq, dk, dv = O.attention_backward(q, k, v, do, 1)
    np.testing.assert_array_equal(dq, 0.0)
    np.testing.assert_array_equal(dk, 0.0)
    np.testing.assert_allclose(dv, do, rtol=0, atol=0)


def test_attention_constant_values_pass_through():
    # softmax rows sum to one: if every v_j is the same vector, o_i is that vector
    rng = np.random.default_rng(6)
    q, k, _ = _qkv(rng, s=13, d=8, scale=2.0)
    vec = rng.standard_normal(8)
    v = np.broadcast_to(vec, q.shape).copy()
    for w in (1, 4, 13):
        np.testing.assert_allclose(O.attention_forward(q, k, v, w),
                                   np.broadcast_to(vec, q.shape), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("window", [1, 4, 16, 40])
def test_attention_matches_torch_sdpa_fp64(window):
    rng = np.random.default_rng(7)
    q, k, v = _qkv(rng, b=2, n=3, s=40, d=16, scale=2.0)
    mask = torch.tensor(O.window_mask(40, window))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q), torch.tensor(k), torch.tensor(v), attn_mask=mask).numpy()
    np.testing.assert_allclose(O.attention_forward(q, k, v, window), ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("window", [1, 3, 7, 9])
def test_attention_backward_finite_difference(window):
    rng = np.random.default_rng(8)
    q, k, v = _qkv(rng, b=2, n=2, s=7, d=8, scale=1.5)
    do = rng.standard_normal(q.shape)
    dq, dk, dv = O.attention_backward(q, k, v, do, window)
    vq, vk, vv = (rng.standard_normal(q.shape) for _ in range(3))
    e = 1e-6

    def L(t):
        return (O.attention_forward(q + t * vq, k + t * vk, v + t * vv, window) * do).sum()

    fd = (L(e) - L(-e)) / (2 * e)
    an = (dq * vq).sum() + (dk * vk).sum() + (dv * vv).sum()
    assert abs(fd - an) <= 1e-6 * max(1.0, abs(an))


# -------------------------------------------------------------- Whole layer
def _layer(rng, b, s, h, n, d, f, scale=0.3, random_ln=True):
    x = rng.standard_normal((b * s, h))
    return x, _rand_params(rng, h, n, d, f, scale, random_ln)


def test_zero_output_projections_give_identity():
    rng = np.random.default_rng(9)
    b, s, h, n, d, f, w = 2, 12, 32, 2, 8, 64, 5
    x, p = _layer(rng, b, s, h, n, d, f)
    p["w_o"][:] = 0
    p["w_fc2"][:] = 0
    y, cache = O.ptb_forward(x, p, b, s, n, d, w, 1e-5)
    np.testing.assert_array_equal(y, x)
    dy = rng.standard_normal(x.shape)
    g = O.ptb_backward(dy, cache, p, w)
    np.testing.assert_array_equal(g["dx"], dy)
    for key in ("dw_qkv", "dw_fc1", "d_ln_gamma", "d_ln_beta"):
        np.testing.assert_array_equal(g[key], 0.0)


PARAM_KEYS = ("ln_gamma", "ln_beta", "w_qkv", "w_o", "w_fc1", "w_fc2")
GRAD_OF = dict(ln_gamma="d_ln_gamma", ln_beta="d_ln_beta", w_qkv="dw_qkv",
               w_o="dw_o", w_fc1="dw_fc1", w_fc2="dw_fc2")


@pytest.mark.parametrize("window", [1, 3, 7, 9])
def test_ptb_backward_finite_difference_every_tensor(window):
    """Central differences on b=2, s=7, h=16, n=2, d=8, f=32, one random
    direction per tensor and a few single coordinates."""
    rng = np.random.default_rng(10 + window)
    b, s, h, n, d, f = 2, 7, 16, 2, 8, 32
    x, p = _layer(rng, b, s, h, n, d, f)
    dy = rng.standard_normal(x.shape)
    y, cache = O.ptb_forward(x, p, b, s, n, d, window, 1e-5)
    g = O.ptb_backward(dy, cache, p, window)
    e = 1e-6

    def L(xx, pp):
        return (O.ptb_forward(xx, pp, b, s, n, d, window, 1e-5)[0] * dy).sum()

    # per-tensor random directions
    for key in PARAM_KEYS + ("x",):
        vdir = rng.standard_normal(x.shape if key == "x" else p[key].shape)
        if key == "x":
            fd = (L(x + e * vdir, p) - L(x - e * vdir, p)) / (2 * e)
            an = (g["dx"] * vdir).sum()
        else:
            pp = dict(p); pm = dict(p)
            pp[key] = p[key] + e * vdir
            pm[key] = p[key] - e * vdir
            fd = (L(x, pp) - L(x, pm)) / (2 * e)
            an = (g[GRAD_OF[key]] * vdir).sum()
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (key, fd, an)
    # a few single coordinates of the weights
    for key in ("w_qkv", "w_fc1"):
        for _ in range(3):
            idx = tuple(rng.integers(0, dim) for dim in p[key].shape)
            pp = dict(p); pm = dict(p)
            pp[key] = p[key].copy(); pp[key][idx] += e
            pm[key] = p[key].copy(); pm[key][idx] -= e
            fd = (L(x, pp) - L(x, pm)) / (2 * e)
            assert abs(fd - g[GRAD_OF[key]][idx]) <= 1e-6 * max(1.0, abs(fd))


def test_ptb_stack_two_layers_finite_difference():
    rng = np.random.default_rng(20)
    b, s, h, n, d, f, w = 1, 6, 16, 2, 8, 32, 4
    x = rng.standard_normal((b * s, h))
    params = [_rand_params(rng, h, n, d, f) for _ in range(2)]
    dy = rng.standard_normal(x.shape)
    y, caches = O.ptb_stack_forward(x, params, b, s, n, d, w, 1e-5)
    dx, grads = O.ptb_stack_backward(dy, caches, params, w)
    vx = rng.standard_normal(x.shape)
    vw = rng.standard_normal(params[0]["w_fc1"].shape)
    e = 1e-6

    def L(t):
        ps = [dict(params[0]), params[1]]
        ps[0]["w_fc1"] = params[0]["w_fc1"] + t * vw
        return (O.ptb_stack_forward(x + t * vx, ps, b, s, n, d, w, 1e-5)[0] * dy).sum()

    fd = (L(e) - L(-e)) / (2 * e)
    an = (dx * vx).sum() + (grads[0]["dw_fc1"] * vw).sum()
    assert abs(fd - an) <= 1e-6 * max(1.0, abs(an))


def test_ptb_adjoint_identity_at_tiny_workload_scale():
    """<dy, J v> == <J^T dy, v> on the tiny workload's shape, J v by central
    differences along v (x and every weight perturbed at once)."""
    wl = I.WORKLOADS["tiny_h256_s256_w64"]
    rng = np.random.default_rng(21)
    x, p = _layer(rng, wl.batch, wl.seq, wl.hidden, wl.heads, wl.head_dim, wl.ffn,
                  scale=0.05)
    dy = rng.standard_normal(x.shape)
    args = (wl.batch, wl.seq, wl.heads, wl.head_dim, wl.window, wl.ln_eps)
    _, cache = O.ptb_forward(x, p, *args)
    g = O.ptb_backward(dy, cache, p, wl.window)
    vx = rng.standard_normal(x.shape)
    vp = {k: rng.standard_normal(p[k].shape) for k in PARAM_KEYS}
    e = 1e-5

    def Y(t):
        pp = {k: p[k] + t * vp[k] for k in PARAM_KEYS}
        return O.ptb_forward(x + t * vx, pp, *args)[0]

    jv = (Y(e) - Y(-e)) / (2 * e)
    lhs = (dy * jv).sum()
    rhs = (g["dx"] * vx).sum() + sum((g[GRAD_OF[k]] * vp[k]).sum() for k in PARAM_KEYS)
    assert abs(lhs - rhs) <= 1e-7 * abs(rhs)


def _torch_ptb(x, p, b, s, n, d, w, eps):
    """Independent PTB written with torch ops, differentiated by autograd."""
    hl = n * d
    a = torch.nn.functional.layer_norm(x, (x.shape[1],), p["ln_gamma"], p["ln_beta"], eps)
    qkv = a @ p["w_qkv"]

    def heads(t):
        return t.reshape(b, s, n, d).permute(0, 2, 1, 3)

    q, k, v = heads(qkv[:, :hl]), heads(qkv[:, hl:2 * hl]), heads(qkv[:, 2 * hl:])
    i = torch.arange(s)[:, None]
    j = torch.arange(s)[None, :]
    allowed = (i >= j) & (i - j < w)
    logits = (q @ k.transpose(-1, -2)) / math.sqrt(d)
    logits = logits.masked_fill(~allowed, float("-inf"))
    o = torch.softmax(logits, dim=-1) @ v
    c = o.permute(0, 2, 1, 3).reshape(b * s, hl)
    return x + c @ p["w_o"] + torch.nn.functional.gelu(a @ p["w_fc1"]) @ p["w_fc2"]


@pytest.mark.parametrize("window", [1, 5, 37, 64])
def test_ptb_matches_torch_fp64_autograd(window):
    rng = np.random.default_rng(30 + window)
    b, s, h, n, d, f = 2, 37, 64, 4, 16, 128
    x, p = _layer(rng, b, s, h, n, d, f, scale=0.15)
    dy = rng.standard_normal(x.shape)
    y, cache = O.ptb_forward(x, p, b, s, n, d, window, 1e-5)
    g = O.ptb_backward(dy, cache, p, window)
    tx = torch.tensor(x, requires_grad=True)
    tp = {k: torch.tensor(v, requires_grad=True) for k, v in p.items()}
    ty = _torch_ptb(tx, tp, b, s, n, d, window, 1e-5)
    ty.backward(torch.tensor(dy))
    np.testing.assert_allclose(y, ty.detach().numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(g["dx"], tx.grad.numpy(), rtol=1e-10, atol=1e-10)
    for k in PARAM_KEYS:
        np.testing.assert_allclose(g[GRAD_OF[k]], tp[k].grad.numpy(), rtol=1e-10, atol=1e-10)


def test_tensor_parallel_shard_sum_identity():
    """Splitting heads and FFN columns over 8 shards and summing the shards'
    partial outputs gives the unsharded layer (the TP=8 share semantics of the
    175B-shape workload; Megatron-LM explainer sections 2.1-2.2)."""
    rng = np.random.default_rng(40)
    tp = 8
    b, s, h, n, d, f, w = 1, 10, 32, 8, 4, 64, 6
    x, p = _layer(rng, b, s, h, n, d, f)
    y, _ = O.ptb_forward(x, p, b, s, n, d, w, 1e-5)
    hl = n * d
    nl, fl = n // tp, f // tp
    total = x.copy()
    for r in range(tp):
        hc = np.arange(r * nl * d, (r + 1) * nl * d)
        fc = np.arange(r * fl, (r + 1) * fl)
        ps = dict(ln_gamma=p["ln_gamma"], ln_beta=p["ln_beta"],
                  w_qkv=np.concatenate([p["w_qkv"][:, hc], p["w_qkv"][:, hl + hc],
                                        p["w_qkv"][:, 2 * hl + hc]], axis=1),
                  w_o=p["w_o"][hc], w_fc1=p["w_fc1"][:, fc], w_fc2=p["w_fc2"][fc])
        ys, _ = O.ptb_forward(x, ps, b, s, nl, d, w, 1e-5)
        total += ys - x
    np.testing.assert_allclose(total, y, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------- FLOPs
@pytest.mark.parametrize("b,s,h,n,d,f,w", [
    (2, 7, 16, 2, 8, 32, 1), (2, 7, 16, 2, 8, 32, 3), (1, 16, 32, 4, 8, 48, 16),
    (1, 16, 32, 4, 8, 48, 40), (3, 33, 64, 2, 16, 96, 10),
])
def test_flop_counter_equals_closed_form(b, s, h, n, d, f, w):
    rng = np.random.default_rng(50)
    x, p = _layer(rng, b, s, h, n, d, f)
    fc = O.FlopCounter()
    _, cache = O.ptb_forward(x, p, b, s, n, d, w, 1e-5, fc)
    O.ptb_backward(rng.standard_normal(x.shape), cache, p, w, fc)
    assert fc.model == F.model_flops(b, s, h, n, d, f, w)
    assert fc.recompute == F.recompute_flops(b, s, n, d, w)


def test_flop_counter_tiny_workload_and_pairs():
    wl = I.WORKLOADS["tiny_h256_s256_w64"]
    rng = np.random.default_rng(51)
    x, p = _layer(rng, wl.batch, wl.seq, wl.hidden, wl.heads, wl.head_dim, wl.ffn, 0.05)
    fc = O.FlopCounter()
    _, cache = O.ptb_forward(x, p, wl.batch, wl.seq, wl.heads, wl.head_dim, wl.window, 1e-5, fc)
    O.ptb_backward(rng.standard_normal(x.shape), cache, p, wl.window, fc)
    assert fc.model == F.workload_model_flops(wl) == 2_504_196_096
    for s, w in [(1, 1), (5, 1), (5, 5), (5, 9), (256, 64), (2048, 512), (8192, 1024)]:
        assert F.window_pairs(s, w) == int(O.window_mask(s, w).sum()) if s <= 2048 else True
    assert F.window_pairs(8192, 1024) == 8192 * 1024 - 1024 * 1023 // 2


# ------------------------------------------------------- Shapes on the pages
def test_175b_tp8_share_derived_from_printed_gpt3_shape():
    vals = {}
    with open(os.path.join(GOLDEN, "gpt3_175b_shape.txt")) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            k, v = line.split()
            vals[k] = int(v)
    wl = I.WORKLOADS["gpt175b_tp8_share_s2048"]
    assert wl.hidden == vals["hidden"]
    assert wl.heads == vals["heads"] // vals["tp"]
    assert wl.head_dim == vals["hidden"] // vals["heads"]
    assert wl.ffn == vals["ffn_multiplier"] * vals["hidden"] // vals["tp"]
    assert wl.seq == vals["context"] and wl.window >= wl.seq


# --------------------------------------------------------- Input generator
def test_bf16_round_to_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0,
                     1.0 + 2 ** -7 + 2 ** -9], np.float32)
    bits = I.f32_to_bf16_bits(vals)
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 tie -> even (1+2^-6); 1+2^-7+2^-9 rounds down
    assert list(bits) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x0000, 0x3F81]
    np.testing.assert_array_equal(I.bf16_bits_to_f32(bits)[[0, 3, 4]], [1.0, -2.5, 0.0])


def test_inputs_are_seeded_and_shaped():
    wl = I.WORKLOADS["tiny_h256_s256_w64"]
    a = I.make_inputs(wl)
    b = I.make_inputs(wl)
    np.testing.assert_array_equal(a["x"], b["x"])
    assert a["x"].shape == (512, 256) and a["dy"].shape == (512, 256)
    lay = a["layers"][0]
    assert lay["w_qkv"].shape == (256, 768) and lay["w_o"].shape == (256, 256)
    assert lay["w_fc1"].shape == (256, 1024) and lay["w_fc2"].shape == (1024, 256)
    std = I.bf16_bits_to_f64(lay["w_fc1"]).std()
    assert 0.019 < std < 0.021
