"""Parity of the FP8 GEMM variant (ptb_fp8_* through the C ABI) with the fp64
FP8 oracle (oracle/fp8_oracle.py) on the same seeded bf16 inputs.

* The current-scaling cast (ptb_fp8_quantize, ptb_fp8_cast_weights) is
  compared code by code: both sides decide each code in fp32 (x * s one fp32
  multiply, s = FMAX / amax one fp32 division), so the codes must be
  identical, padding included.
* The block-scaled cast (ptb_fp8_quantize_mx, and the weight cast under
  PTB_FP8_MX) is compared the same way, codes and scale words: the scale of
  a block comes from its bf16 maximum's exponent and x 2^-X is exact.
* The layer, under either recipe, is compared by relative Frobenius error
  per output tensor against
  FP8_TOL.  Where the two sides feed a cast slightly different bf16 values (an
  upstream difference of relative size delta, at most the bf16 path's bar
  1e-2), a value near an FP8 rounding boundary lands on the neighbouring code:
  with probability about delta / u per element, u the format's relative step
  (2^-3 E4M3, 2^-2 E5M2), each time one whole step.  The RMS effect is about
  sqrt(delta u) = sqrt(1e-2 * 2^-2) = 0.05, which is the bar.  The residual
  paths dominate y and dx, so y - x and dx - dy are compared with the bf16
  rounding floor of the output added, as for the bf16 layer."""
import math

import numpy as np
import pytest
import torch

from oracle import fp8_oracle as F8
from transformer_block_amd import inputs as I
from transformer_block_amd import ptb as P
from transformer_block_amd.runner import Fp8Layer, bf16_to_numpy_f64

from .helpers import log, rel_fro

pytestmark = pytest.mark.gpu

FP8_TOL = math.sqrt(1e-2 * 2.0 ** -2)

W = I.Workload


def _np(t):
    if t.dtype == torch.bfloat16:
        return bf16_to_numpy_f64(t)
    return t.detach().cpu().numpy().astype(np.float64)


def _probe_matrix(rows, cols, seed):
    """bf16 values: every significand of the binades 2^-33 .. 2^1 (both signs),
    the largest magnitude 3 exactly once, zeros, and N(0, 0.5) filler; shuffled."""
    rng = np.random.default_rng(seed)
    e = np.arange(-33, 2)
    m = 1 + np.arange(128) / 128.0
    grid = (m[None, :] * 2.0 ** e[:, None]).ravel()
    grid = grid[grid < 3.0]
    vals = np.concatenate([grid, -grid, [3.0, 0.0, 0.0]])
    n = rows * cols
    assert vals.size <= n
    fill = rng.standard_normal(n - vals.size) * 0.5
    allv = np.concatenate([vals, np.clip(fill, -2.9, 2.9)])
    rng.shuffle(allv)
    bits = I.f32_to_bf16_bits(allv.astype(np.float32)).reshape(rows, cols)
    return bits, I.bf16_bits_to_f64(bits)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("rows,cols", [(130, 264), (64, 512)])
def test_quantize_codes_match_the_oracle(fmt, rows, cols):
    log(f"fp8 quantize {fmt} {rows}x{cols}")
    bits, x = _probe_matrix(rows, cols, 900 + rows)
    dev = torch.device("cuda")
    xt = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    ldq, ldqt = (cols + 63) // 64 * 64, (rows + 63) // 64 * 64
    q = torch.full((rows, ldq), 0x55, dtype=torch.uint8, device=dev)
    qt = torch.full((cols, ldqt), 0x55, dtype=torch.uint8, device=dev)
    amax = torch.full((4,), -1.0, dtype=torch.float32, device=dev)
    P.ptb_fp8_quantize(xt, rows, cols, fmt, amax, q, qt)
    torch.cuda.synchronize()
    assert amax[0].item() == 3.0
    s = F8.current_scale(x, fmt)
    codes, _ = F8.quantize(x, s, fmt)
    got = q.cpu().numpy()
    np.testing.assert_array_equal(got[:, :cols], codes)
    assert not got[:, cols:].any()
    gott = qt.cpu().numpy()
    np.testing.assert_array_equal(gott[:, :rows], codes.T)
    assert not gott[:, rows:].any()


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("rows,cols", [(1, 8), (65, 8), (3, 200)])
def test_quantize_small_and_ragged_shapes(fmt, rows, cols):
    """One row, one 16-byte chunk per row, and a ragged row count: the codes,
    the zero padding of both copies (to multiples of 64) and the amax."""
    rng = np.random.default_rng(950 + rows)
    x = (rng.standard_normal((rows, cols)) * 1.7).astype(np.float32)
    bits = I.f32_to_bf16_bits(x)
    xv = I.bf16_bits_to_f64(bits)
    dev = torch.device("cuda")
    xt = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    ldq, ldqt = (cols + 63) // 64 * 64, (rows + 63) // 64 * 64
    q = torch.full((rows, ldq), 0x55, dtype=torch.uint8, device=dev)
    qt = torch.full((cols, ldqt), 0x55, dtype=torch.uint8, device=dev)
    amax = torch.full((4,), -1.0, dtype=torch.float32, device=dev)
    P.ptb_fp8_quantize(xt, rows, cols, fmt, amax, q, qt)
    torch.cuda.synchronize()
    assert amax[0].item() == np.abs(xv).max()
    codes, _ = F8.quantize(xv, F8.current_scale(xv, fmt), fmt)
    got, gott = q.cpu().numpy(), qt.cpu().numpy()
    np.testing.assert_array_equal(got[:, :cols], codes)
    assert not got[:, cols:].any()
    np.testing.assert_array_equal(gott[:, :rows], codes.T)
    assert not gott[:, rows:].any()


def _mx_scale_bytes(sc, kp, rows_p):
    """The scales of a block-scaled copy as the ABI lays them out, from block
    codes sc [rows, nblocks] (blocks along k), 127 where the block or the row
    is padding: [kp/128][4 rows_p] bytes; with r = 128 g + 32 i + l, the code
    of row r's block 4 j + b sits in row j at byte
    512 g + 16 l + 8 (b & 1) + 4 (b >> 1) + i."""
    rows, nb = sc.shape
    full = np.full((rows_p, kp // 32), 127, dtype=np.uint8)
    full[:rows, :nb] = sc
    r = np.arange(rows_p)[:, None]
    b = np.arange(4)[None, :]
    pos = 512 * (r // 128) + 16 * (r % 32) + 8 * (b & 1) + 4 * (b >> 1) + (r // 32) % 4
    assert np.array_equal(np.sort(pos.ravel()), np.arange(4 * rows_p))  # a permutation
    out = np.empty((kp // 128, 4 * rows_p), dtype=np.uint8)
    out[:, pos.ravel()] = full.reshape(rows_p, kp // 128, 4).transpose(1, 0, 2).reshape(kp // 128, -1)
    return out


def _check_mx_copies(q, qs, qt, qts, x, fmt):
    """Row-wise and transposed block-scaled copies (device tensors) of x
    against the oracle, padding included."""
    rows, cols = x.shape
    p128 = lambda v: (v + 127) // 128 * 128
    codes, sc, _ = F8.mx_quantize(x, fmt, axis=1)
    got = q.cpu().numpy()
    np.testing.assert_array_equal(got[:, :cols], codes)
    assert not got[:, cols:].any()
    np.testing.assert_array_equal(qs.cpu().numpy().view(np.uint8).reshape(p128(cols) // 128, -1),
                                  _mx_scale_bytes(sc, p128(cols), p128(rows)))
    codes0, sc0, _ = F8.mx_quantize(x, fmt, axis=0)
    gott = qt.cpu().numpy()
    np.testing.assert_array_equal(gott[:, :rows], codes0.T)
    assert not gott[:, rows:].any()
    np.testing.assert_array_equal(qts.cpu().numpy().view(np.uint8).reshape(p128(rows) // 128, -1),
                                  _mx_scale_bytes(sc0.T, p128(rows), p128(cols)))


def _mx_buffers(rows, cols, dev):
    p128 = lambda v: (v + 127) // 128 * 128
    fill = lambda shape, dt: torch.full(shape, 0x55, dtype=dt, device=dev)
    return (fill((rows, p128(cols)), torch.uint8), fill((p128(cols) // 128, p128(rows)), torch.int32),
            fill((cols, p128(rows)), torch.uint8), fill((p128(rows) // 128, p128(cols)), torch.int32))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("rows,cols", [(130, 264), (64, 512), (1, 8), (65, 8), (3, 200)])
def test_quantize_mx_codes_and_scales_match_the_oracle(fmt, rows, cols):
    """Every significand of 35 binades in random places (so the blocks' scales
    spread over many binades), rows scaled by 2^-20 .. 2^20, a zero block, and
    ragged shapes: codes, scale words and padding of both copies."""
    log(f"fp8 mx quantize {fmt} {rows}x{cols}")
    dev = torch.device("cuda")
    if rows * cols >= 8960:
        bits, x = _probe_matrix(rows, cols, 960 + rows)
    else:
        rng = np.random.default_rng(960 + rows)
        x32 = (rng.standard_normal((rows, cols)) * 1.7).astype(np.float32)
        bits = I.f32_to_bf16_bits(x32)
        x = I.bf16_bits_to_f64(bits)
    rng = np.random.default_rng(970 + cols)
    scale = np.exp2(rng.integers(-20, 21, (rows, 1))).astype(np.float32)
    bits = I.f32_to_bf16_bits((x * scale).astype(np.float32))
    if cols >= 64:
        bits[0, 32:64] = 0
    x = I.bf16_bits_to_f64(bits)
    xt = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    q, qs, qt, qts = _mx_buffers(rows, cols, dev)
    P.ptb_fp8_quantize_mx(xt, rows, cols, fmt, q, qs, qt, qts)
    torch.cuda.synchronize()
    _check_mx_copies(q, qs, qt, qts, x, fmt)


def test_cast_weights_mx_match_the_oracle():
    w = W("f8wmx", 1, 128, 192, 3, 64, 768, 32, seed=902)
    inp = I.make_inputs(w, random_ln=True)
    dev = torch.device("cuda")
    lay = inp["layers"][0]
    t = {k: torch.from_numpy(lay[k].view(np.int16)).to(dev).view(torch.bfloat16)
         for k in ("w_qkv", "w_o", "w_fc1", "w_fc2")}
    dims = P.dims_of(w)
    buf = torch.full((P.ptb_fp8_weights_bytes(dims, "mx"),), 0x55, dtype=torch.uint8, device=dev)
    P.ptb_fp8_cast_weights(dims, t["w_qkv"], t["w_o"], t["w_fc1"], t["w_fc2"], buf, recipe="mx")
    torch.cuda.synchronize()
    off = P.ptb_fp8_weights_layout(dims, "mx")
    f = I.bf16_bits_to_f64
    w1 = np.concatenate([f(lay["w_qkv"]), f(lay["w_fc1"])], axis=1)
    w2 = np.concatenate([f(lay["w_o"]), f(lay["w_fc2"])], axis=0)
    p128 = lambda v: (v + 127) // 128 * 128
    for name, mat, tname in (("w1", w1, "w1t"), ("w2", w2, "w2t")):
        R, C = mat.shape
        view = lambda o, shape, dt: buf[o:o + int(np.prod(shape)) * (4 if dt == torch.int32 else 1)
                                        ].view(dt).view(shape)
        q = view(off[name], (R, p128(C)), torch.uint8)
        qs = view(off[name + "_s"], (p128(C) // 128, p128(R)), torch.int32)
        qt = view(off[tname], (C, p128(R)), torch.uint8)
        qts = view(off[tname + "_s"], (p128(R) // 128, p128(C)), torch.int32)
        _check_mx_copies(q, qs, qt, qts, mat, F8.E4M3)


def test_cast_weights_match_the_oracle():
    w = W("f8w", 1, 128, 192, 3, 64, 768, 32, seed=901)
    inp = I.make_inputs(w, random_ln=True)
    dev = torch.device("cuda")
    lay = inp["layers"][0]
    t = {k: torch.from_numpy(lay[k].view(np.int16)).to(dev).view(torch.bfloat16)
         for k in ("w_qkv", "w_o", "w_fc1", "w_fc2")}
    dims = P.dims_of(w)
    buf = torch.zeros(P.ptb_fp8_weights_bytes(dims), dtype=torch.uint8, device=dev)
    P.ptb_fp8_cast_weights(dims, t["w_qkv"], t["w_o"], t["w_fc1"], t["w_fc2"], buf)
    torch.cuda.synchronize()
    off = P.ptb_fp8_weights_layout(dims)
    host = buf.cpu().numpy()
    f = I.bf16_bits_to_f64
    w1 = np.concatenate([f(lay["w_qkv"]), f(lay["w_fc1"])], axis=1)
    w2 = np.concatenate([f(lay["w_o"]), f(lay["w_fc2"])], axis=0)
    amax = host[off["amax"]:off["amax"] + 8].view(np.float32)
    assert amax[0] == np.abs(w1).max() and amax[1] == np.abs(w2).max()
    pad = lambda v: (v + 127) // 128 * 128
    for name, mat, tname in (("w1", w1, "w1t"), ("w2", w2, "w2t")):
        codes, _ = F8.quantize(mat, F8.current_scale(mat, F8.E4M3), F8.E4M3)
        R, C = mat.shape
        rowwise = host[off[name]:off[name] + R * pad(C)].reshape(R, pad(C))
        np.testing.assert_array_equal(rowwise[:, :C], codes)
        assert not rowwise[:, C:].any()
        trans = host[off[tname]:off[tname] + C * pad(R)].reshape(C, pad(R))
        np.testing.assert_array_equal(trans[:, :R], codes.T)
        assert not trans[:, R:].any()


CASES = [
    ("tiny_workload", I.WORKLOADS["tiny_h256_s256_w64"], True),
    ("ragged_h192_s200_w37", W("f8r", 1, 200, 192, 3, 64, 768, 37, seed=910), True),
    ("d128_b3_s97_w33", W("f8d", 3, 97, 256, 2, 128, 512, 33, seed=911), True),
    ("rmsnorm", W("f8rms", 2, 160, 256, 2, 128, 256, 40, seed=912, norm="rmsnorm"), True),
    ("single_token", W("f8s1", 1, 1, 128, 1, 128, 128, 1, seed=913), True),
    ("window1_d64_s77", W("f8w1", 2, 77, 192, 3, 64, 384, 1, seed=914), True),
    ("h2048_s2048_w512", I.WORKLOADS["h2048_s2048_w512"], False),
    ("gpt175b_tp8_share_s2048", I.WORKLOADS["gpt175b_tp8_share_s2048"], False),
    ("long_h4096_s8192_w1024", I.WORKLOADS["long_h4096_s8192_w1024"], False),
]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("recipe", ["current", "mx"])
@pytest.mark.parametrize("name,w,random_ln", CASES, ids=[c[0] for c in CASES])
def test_fp8_layer_parity(name, w, random_ln, recipe):
    log(f"fp8 case {name} ({recipe}): {w}")
    inp = I.make_inputs(w, random_ln=random_ln)
    lyr = Fp8Layer(w, inp, "cuda", recipe)
    lyr.step()
    torch.cuda.synchronize()
    log(f"[fp8 {name}] gpu step done; running the oracle")
    f = I.bf16_bits_to_f64
    x, dy = f(inp["x"]), f(inp["dy"])
    p = {k: f(v) for k, v in inp["layers"][0].items()}
    y, cache = F8.fp8_ptb_forward(x, p, w.batch, w.seq, w.heads, w.head_dim, w.window,
                                  w.ln_eps, norm=w.norm, recipe=recipe)
    log(f"[fp8 {name}] oracle forward done")
    g = F8.fp8_ptb_backward(dy, cache, p, w.window)
    errs = {}
    for key, got, ref, res in (("y-x", _np(lyr.y), y, x), ("dx-dy", _np(lyr.dx), g["dx"], dy)):
        branch = ref - res
        floor = 2.0 ** -8 * np.linalg.norm(ref) / max(np.linalg.norm(branch), 1e-300)
        errs[key] = rel_fro(got - res, branch) / (1.0 + floor / FP8_TOL)
    for k in ("d_ln_gamma", "d_ln_beta", "dw_qkv", "dw_o", "dw_fc1", "dw_fc2"):
        ref = g[k]
        if w.norm == "rmsnorm" and k == "d_ln_beta":
            assert not _np(lyr.grads[k]).any()
            continue
        errs[k] = rel_fro(_np(lyr.grads[k]), ref)
    for k in ("a", "qkv", "u", "g", "c"):
        errs[f"saved.{k}"] = rel_fro(_np(lyr.saved_tensor(k)), cache[k])
    log(f"[fp8 {name}] " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not np.isfinite(v) or v > FP8_TOL}
    assert not bad, f"parity failures (tol {FP8_TOL:.3f}): {bad}"


@pytest.mark.parametrize("recipe", ["current", "mx"])
def test_fp8_repeat_runs_are_bitwise_identical(recipe):
    w = W("f8det", 2, 200, 256, 2, 128, 512, 80, seed=920)
    lyr = Fp8Layer(w, I.make_inputs(w, random_ln=True), "cuda", recipe)
    lyr.step()
    torch.cuda.synchronize()
    first = [lyr.y.clone(), lyr.dx.clone()] + [t.clone() for t in lyr.grads.values()]
    lyr.step()
    torch.cuda.synchronize()
    again = [lyr.y, lyr.dx] + list(lyr.grads.values())
    for a, b in zip(first, again):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("recipe", ["current", "mx"])
def test_fp8_zero_output_weights_give_the_identity(recipe):
    """W_o = W_fc2 = 0: the operand [W_o ; W_fc2] has amax 0 (every block
    too), so its scale is 1 and its codes are all zero; the layer is then
    exactly y = x and dx = dy (da = 0), while dW_o and dW_fc2 still match the
    oracle."""
    w = W("f8zero", 2, 96, 256, 2, 128, 512, 40, seed=930)
    inp = I.make_inputs(w, random_ln=True)
    lay = inp["layers"][0]
    lay["w_o"] = np.zeros_like(lay["w_o"])
    lay["w_fc2"] = np.zeros_like(lay["w_fc2"])
    lyr = Fp8Layer(w, inp, "cuda", recipe)
    lyr.step()
    torch.cuda.synchronize()
    assert torch.equal(lyr.y.view(torch.int16), lyr.x.view(torch.int16))
    assert torch.equal(lyr.dx.view(torch.int16), lyr.dy.view(torch.int16))
    for k in ("d_ln_gamma", "d_ln_beta", "dw_qkv", "dw_fc1"):
        assert not _np(lyr.grads[k]).any(), k
    f = I.bf16_bits_to_f64
    x, dy = f(inp["x"]), f(inp["dy"])
    p = {k: f(v) for k, v in lay.items()}
    y, cache = F8.fp8_ptb_forward(x, p, w.batch, w.seq, w.heads, w.head_dim, w.window,
                                  w.ln_eps, recipe=recipe)
    g = F8.fp8_ptb_backward(dy, cache, p, w.window)
    assert np.array_equal(y, x) and np.array_equal(g["dx"], dy)
    for k in ("dw_o", "dw_fc2"):
        e = rel_fro(_np(lyr.grads[k]), g[k])
        log(f"[fp8 zero] {k}={e:.2e}")
        assert e < FP8_TOL, (k, e)
