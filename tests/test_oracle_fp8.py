"""Pins of the FP8 oracle (Megatron-LM tuning post, mixed-precision section:
E4M3 forward operands and weights, E5M2 gradients, current scaling, only the
matrix products in FP8).

* the two formats' value tables against published code values and torch's
  float8 dtypes;
* bf16 rounding against torch's bfloat16 on fp32-exact inputs and on ties;
* the quantizer against torch's float8 casts (bit-exact codes), including
  grid points, midpoints and their fp32 neighbours, and against a brute-force
  nearest search;
* current scaling: the largest element lands on the largest code;
* the FP8 product: exact when every operand is on the grid with a power-of-two
  scale, and within the formats' rounding bounds otherwise;
* the whole layer against the fp64 layer (FP8-level differences, nothing
  structural) and the format of each of the six products.  CPU only."""
import math

import numpy as np
import pytest
import torch

from oracle import fp8_oracle as F8
from oracle import ptb_oracle as O

TORCH_FMT = {F8.E4M3: torch.float8_e4m3fn, F8.E5M2: torch.float8_e5m2}


def test_decode_table_published_values():
    t = F8.decode_table(F8.E4M3)
    assert t[0x00] == 0.0 and t[0x01] == 2.0 ** -9 and t[0x07] == 7 * 2.0 ** -9
    assert t[0x08] == 2.0 ** -6 and t[0x38] == 1.0 and t[0x3C] == 1.5
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert math.isnan(t[0x7F]) and math.isnan(t[0xFF])
    assert np.isnan(t).sum() == 2 and not np.isinf(t).any()
    t = F8.decode_table(F8.E5M2)
    assert t[0x01] == 2.0 ** -16 and t[0x04] == 2.0 ** -14 and t[0x3C] == 1.0
    assert t[0x7B] == 57344.0 and t[0x7C] == math.inf and t[0xFC] == -math.inf
    assert np.isnan(t).sum() == 6
    assert F8.fmax(F8.E4M3) == 448.0 and F8.fmax(F8.E5M2) == 57344.0


@pytest.mark.parametrize("fmt", [F8.E4M3, F8.E5M2])
def test_decode_table_matches_torch(fmt):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(TORCH_FMT[fmt]).to(torch.float64).numpy()
    got = F8.decode_table(fmt)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])
    pos = got[:128][np.isfinite(got[:128])]
    assert np.all(np.diff(pos) > 0)


def test_round_bf16_against_torch():
    rng = np.random.default_rng(800)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    ref = torch.tensor(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(F8.round_bf16(x.astype(np.float64)), ref)
    # ties go to the even significand
    assert F8.round_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert F8.round_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    assert F8.round_bf16(np.array([-(1 + 3 * 2.0 ** -8)]))[0] == -(1 + 2.0 ** -6)


def _probe_values(fmt, rng):
    """Grid points, midpoints, their fp32 neighbours and random values over
    every binade, all within +-FMAX."""
    grid = F8.decode_table(fmt)[:128]
    grid = grid[np.isfinite(grid)]
    mids = (grid[1:] + grid[:-1]) / 2
    m32 = mids.astype(np.float32)
    vals = [grid, mids, np.nextafter(m32, np.float32(np.inf)),
            np.nextafter(m32, np.float32(-np.inf))]
    top = grid[-1]
    vals.append(np.exp(rng.uniform(np.log(grid[1] / 4), np.log(top), 50000)))
    v = np.concatenate(vals).astype(np.float32)
    v = v[np.abs(v) <= top]
    return np.concatenate([v, -v])


@pytest.mark.parametrize("fmt", [F8.E4M3, F8.E5M2])
def test_quantize_matches_torch_cast(fmt):
    rng = np.random.default_rng(801)
    y = _probe_values(fmt, rng)
    codes, vals = F8.quantize(y.astype(np.float64), np.float32(1.0), fmt)
    ref = torch.tensor(y).to(TORCH_FMT[fmt])
    np.testing.assert_array_equal(codes, ref.view(torch.uint8).numpy())
    np.testing.assert_array_equal(vals, ref.to(torch.float64).numpy())
    # beyond the range: clamped to the largest finite value
    c, v = F8.quantize(np.array([1e6, -1e6, F8.fmax(fmt) * 1.01]), np.float32(1.0), fmt)
    np.testing.assert_array_equal(v, [F8.fmax(fmt), -F8.fmax(fmt), F8.fmax(fmt)])


@pytest.mark.parametrize("fmt", [F8.E4M3, F8.E5M2])
def test_quantize_brute_force(fmt):
    rng = np.random.default_rng(802)
    table = F8.decode_table(fmt)
    fin = np.where(np.isfinite(table))[0]
    y = (rng.standard_normal(3000) * 3).astype(np.float32)
    scale = np.float32(1.7)
    codes, vals = F8.quantize(y.astype(np.float64), scale, fmt)
    ys = np.clip(y * scale, -F8.fmax(fmt), F8.fmax(fmt)).astype(np.float64)
    for i in range(y.size):
        half = fin[fin < 128] if ys[i] >= 0 else fin[fin >= 128]  # same sign
        d = np.abs(table[half] - ys[i])
        best = half[d == d.min()]
        if best.size > 1:  # a tie between neighbours: the even code
            best = best[best % 2 == 0]
        assert best.size == 1
        assert codes[i] == best[0], (i, ys[i])
        assert vals[i] == table[best[0]]


@pytest.mark.parametrize("fmt", [F8.E4M3, F8.E5M2])
def test_current_scale(fmt):
    rng = np.random.default_rng(803)
    x = F8.round_bf16(rng.standard_normal((64, 48)) * 0.37)
    s = F8.current_scale(x, fmt)
    assert s.dtype == np.float32
    amax = np.abs(x).max()
    assert abs(amax * float(s) / F8.fmax(fmt) - 1) < 2.0 ** -22
    codes, vals = F8.quantize(x, s, fmt)
    assert np.abs(vals).max() == F8.fmax(fmt)
    assert F8.current_scale(np.zeros((3, 4)), fmt) == 1.0


def test_fp8_matmul_exact_on_the_grid():
    """Operands already on the FP8 grid with amax = FMAX 2^-k: the scale is
    2^k, quantization loses nothing, the product is the exact one."""
    rng = np.random.default_rng(804)
    g4 = F8.decode_table(F8.E4M3)
    g5 = F8.decode_table(F8.E5M2)
    pos4 = np.where(np.isfinite(g4))[0]
    pos5 = np.where(np.isfinite(g5))[0]
    a = g4[rng.choice(pos4, (40, 96))] * 2.0 ** -5
    b = g5[rng.choice(pos5, (96, 24))] * 2.0 ** -12
    a[3, 7] = 448.0 * 2.0 ** -5
    b[5, 2] = -57344.0 * 2.0 ** -12
    assert F8.current_scale(a, F8.E4M3) == 2.0 ** 5
    assert F8.current_scale(b, F8.E5M2) == 2.0 ** 12
    np.testing.assert_allclose(F8.fp8_matmul(a, b, F8.E4M3, F8.E5M2), a @ b, rtol=1e-12,
                               atol=1e-12 * np.abs(a @ b).max())


@pytest.mark.parametrize("fa,fb,hi", [(F8.E4M3, F8.E4M3, 2.0 ** -4 * math.sqrt(2)),
                                      (F8.E5M2, F8.E4M3, 2.0 ** -3 * math.sqrt(2))])
def test_fp8_matmul_error_bound(fa, fb, hi):
    """Each element is rounded with relative error at most half a step (2^-4
    E4M3, 2^-3 E5M2, for values in the normal range); independent errors
    keep the product's relative Frobenius error below the square-root sum of
    those, and quantization does happen (error well above bf16's)."""
    rng = np.random.default_rng(805)
    a = F8.round_bf16(rng.standard_normal((128, 512)))
    b = F8.round_bf16(rng.standard_normal((512, 96)) * 0.02)
    got = F8.fp8_matmul(a, b, fa, fb)
    ref = a @ b
    err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert 2.0 ** -9 < err < hi


def _layer(rng, b=2, s=16, n=2, d=16, h=32, f=128):
    hl = n * d
    p = dict(ln_gamma=F8.round_bf16(1 + 0.1 * rng.standard_normal(h)),
             ln_beta=F8.round_bf16(0.1 * rng.standard_normal(h)),
             w_qkv=F8.round_bf16(rng.standard_normal((h, 3 * hl)) * 0.2),
             w_o=F8.round_bf16(rng.standard_normal((hl, h)) * 0.2),
             w_fc1=F8.round_bf16(rng.standard_normal((h, f)) * 0.2),
             w_fc2=F8.round_bf16(rng.standard_normal((f, h)) * 0.1))
    x = F8.round_bf16(rng.standard_normal((b * s, h)))
    dy = F8.round_bf16(rng.standard_normal((b * s, h)))
    return x, dy, p, dict(batch=b, seq=s, heads=n, head_dim=d)


def test_layer_is_the_fp64_layer_up_to_fp8_rounding():
    rng = np.random.default_rng(806)
    x, dy, p, dm = _layer(rng)
    args = (dm["batch"], dm["seq"], dm["heads"], dm["head_dim"], 8, 1e-5)
    y8, c8 = F8.fp8_ptb_forward(x, p, *args)
    g8 = F8.fp8_ptb_backward(dy, c8, p, 8)
    y, c = O.ptb_forward(x, p, *args)
    g = O.ptb_backward(dy, c, p, 8)

    def rel(u, v):
        return np.linalg.norm(u - v) / np.linalg.norm(v)

    errs = {"y": rel(y8 - x, y - x), "dx": rel(g8["dx"] - dy, g["dx"] - dy)}
    for k in ("d_ln_gamma", "d_ln_beta", "dw_qkv", "dw_o", "dw_fc1", "dw_fc2"):
        errs[k] = rel(g8[k], g[k])
    for k, e in errs.items():
        # E4M3/E5M2 rounding of every product operand: a few percent, never
        # the O(1) of a missing or mis-signed term, and never zero
        assert 1e-3 < e < 0.15, (k, e)
    assert c8["formats"] == [(F8.E4M3, F8.E4M3), (F8.E4M3, F8.E4M3),
                             (F8.E5M2, F8.E4M3), (F8.E4M3, F8.E5M2),
                             (F8.E5M2, F8.E4M3), (F8.E4M3, F8.E5M2)]


# ---------------------------------------------------------------------------
# Block (MX) scaling: blocks of 32 along the contraction axis, E8M0 scales
# 2^(floor(log2 amax) - emax) (OCP Microscaling Formats v1.0, mxfp8 as the
# tuning post names it)
# ---------------------------------------------------------------------------
def _floor_log2(v: float) -> int:
    """floor(log2 v) by repeated halving/doubling (exact for floats)."""
    k = 0
    while v >= 2.0:
        v /= 2.0
        k += 1
    while v < 1.0:
        v *= 2.0
        k -= 1
    return k


@pytest.mark.parametrize("fmt,em", [(F8.E4M3, 8), (F8.E5M2, 15)])
def test_mx_scale_code(fmt, em):
    assert F8.emax(fmt) == em
    rng = np.random.default_rng(810)
    # powers of two, values just below and above them, random values; bf16
    k = rng.integers(-60, 60, 400)
    vals = np.concatenate([np.ldexp(1.0, k), np.ldexp(1.0 - 2.0 ** -8, k),
                           np.ldexp(1.0 + 2.0 ** -7, k), F8.round_bf16(np.exp(rng.uniform(-40, 40, 400)))])
    got = F8.mx_scale_code(vals, fmt)
    want = np.array([127 + _floor_log2(float(v)) - em for v in vals])
    np.testing.assert_array_equal(got, want)
    # all-zero block: scale 1; tiny and huge blocks: the code range 0..254
    assert F8.mx_scale_code(np.array([0.0]), fmt)[0] == 127
    assert F8.mx_scale_code(np.array([2.0 ** -133]), fmt)[0] == 0
    assert F8.mx_scale_code(np.array([float(np.finfo(np.float32).max)]), fmt)[0] == 127 + 127 - em


@pytest.mark.parametrize("fmt", [F8.E4M3, F8.E5M2])
def test_mx_quantize_matches_torch_cast(fmt):
    """Codes are torch's float8 cast of x 2^-X clamped to +-FMAX, with X from
    the block's amax by the rule above; blocks run along the requested axis
    and the last one may be short."""
    rng = np.random.default_rng(811)
    R, C = 37, 100  # 100 = 3 whole blocks + a short one of 4
    x = F8.round_bf16(rng.standard_normal((R, C)) * np.exp2(rng.integers(-20, 20, (R, 1))))
    x[5, 40:64] = 0.0
    x[6, 64:96] = 0.0   # an all-zero block
    for axis in (1, 0):
        codes, sc, vals = F8.mx_quantize(x, fmt, axis)
        xt = x if axis == 1 else x.T
        ct = codes if axis == 1 else codes.T
        st = sc if axis == 1 else sc.T
        vt = vals if axis == 1 else vals.T
        assert st.shape == (xt.shape[0], -(-xt.shape[1] // 32))
        for r in range(xt.shape[0]):
            for b in range(st.shape[1]):
                blk = xt[r, 32 * b:32 * b + 32]
                amax = np.abs(blk).max()
                X = _floor_log2(float(amax)) - F8.emax(fmt) if amax > 0 else 0
                assert st[r, b] == X + 127
                y = np.clip(blk.astype(np.float32) * np.float32(2.0 ** -X), -F8.fmax(fmt), F8.fmax(fmt))
                ref = torch.tensor(y).to(TORCH_FMT[fmt])
                np.testing.assert_array_equal(ct[r, 32 * b:32 * b + 32], ref.view(torch.uint8).numpy())
                np.testing.assert_array_equal(vt[r, 32 * b:32 * b + 32],
                                              ref.to(torch.float64).numpy() * 2.0 ** X)


def test_mx_matmul_exact_on_the_grid():
    """Every block of A (rows) and B (columns) holds grid values times its own
    power of two 2^X_b, X_b spread over 40 binades, with one value in the
    top binade: the block scales are exactly 2^X_b, nothing is rounded, and
    the product is the exact one.  A wrong block axis or block boundary would
    mix binades and round."""
    rng = np.random.default_rng(812)
    M, K, N = 12, 160, 9
    g4 = F8.decode_table(F8.E4M3)[:127]
    g5 = F8.decode_table(F8.E5M2)[:124]
    sign = lambda shape: np.where(rng.random(shape) < 0.5, -1.0, 1.0)
    a = g4[rng.integers(0, 127, (M, K))] * sign((M, K))
    b = g5[rng.integers(0, 124, (K, N))] * sign((K, N))
    xa = rng.integers(-20, 20, (M, K // 32))
    xb = rng.integers(-20, 20, (K // 32, N))
    for blk in range(K // 32):
        a[:, 32 * blk + 3] = 448.0
        b[32 * blk + 7, :] = -57344.0
        a[:, 32 * blk:32 * blk + 32] *= np.exp2(xa[:, blk:blk + 1])
        b[32 * blk:32 * blk + 32, :] *= np.exp2(xb[blk:blk + 1, :])
    _, sa, _ = F8.mx_quantize(a, F8.E4M3, 1)
    _, sb, _ = F8.mx_quantize(b, F8.E5M2, 0)
    np.testing.assert_array_equal(sa, xa + 127)
    np.testing.assert_array_equal(sb, xb + 127)
    ref = a @ b
    np.testing.assert_allclose(F8.mx_matmul(a, b, F8.E4M3, F8.E5M2), ref, rtol=1e-12,
                               atol=1e-12 * np.abs(ref).max())


def test_mx_blocks_are_local():
    """A large value in one block changes that block's scale and codes only."""
    rng = np.random.default_rng(813)
    x = F8.round_bf16(rng.standard_normal((4, 128)))
    c0, s0, _ = F8.mx_quantize(x, F8.E4M3, 1)
    y = x.copy()
    y[2, 70] = 1000.0
    c1, s1, _ = F8.mx_quantize(y, F8.E4M3, 1)
    changed = (c0 != c1)
    assert changed[2, 64:96].any() and s1[2, 2] != s0[2, 2]
    changed[2, 64:96] = False
    assert not changed.any()
    s1[2, 2] = s0[2, 2]
    np.testing.assert_array_equal(s0, s1)


def test_mx_keeps_small_rows_that_current_scaling_loses():
    """Rows of very different magnitude (2^-24 .. 2^24): one tensor-wide scale
    flushes the small rows to zero, block scales keep every row to a few
    percent (E4M3 half-step 2^-4, plus the saturation of the top binade's
    last step)."""
    rng = np.random.default_rng(814)
    a = F8.round_bf16(rng.standard_normal((64, 256)) * np.exp2(rng.integers(-24, 24, (64, 1))))
    b = F8.round_bf16(rng.standard_normal((256, 32)))
    ref = a @ b
    row_err = lambda c: (np.linalg.norm(c - ref, axis=1) / np.linalg.norm(ref, axis=1))
    cur = row_err(F8.fp8_matmul(a, b, F8.E4M3, F8.E4M3))
    mx = row_err(F8.mx_matmul(a, b, F8.E4M3, F8.E4M3))
    assert cur.max() > 0.5          # some rows lost
    assert mx.max() < 0.1 and mx.min() > 2.0 ** -9


def test_mx_layer_is_the_fp64_layer_up_to_fp8_rounding():
    rng = np.random.default_rng(815)
    x, dy, p, dm = _layer(rng, s=40, h=64, f=96)   # axes not all multiples of 32
    args = (dm["batch"], dm["seq"], dm["heads"], dm["head_dim"], 8, 1e-5)
    y8, c8 = F8.fp8_ptb_forward(x, p, *args, recipe="mx")
    g8 = F8.fp8_ptb_backward(dy, c8, p, 8)
    y, c = O.ptb_forward(x, p, *args)
    g = O.ptb_backward(dy, c, p, 8)
    rel = lambda u, v: np.linalg.norm(u - v) / np.linalg.norm(v)
    errs = {"y": rel(y8 - x, y - x), "dx": rel(g8["dx"] - dy, g["dx"] - dy)}
    for k in ("d_ln_gamma", "d_ln_beta", "dw_qkv", "dw_o", "dw_fc1", "dw_fc2"):
        errs[k] = rel(g8[k], g[k])
    for k, e in errs.items():
        assert 1e-3 < e < 0.15, (k, e)
    assert c8["formats"] == [(F8.E4M3, F8.E4M3), (F8.E4M3, F8.E4M3),
                             (F8.E5M2, F8.E4M3), (F8.E4M3, F8.E5M2),
                             (F8.E5M2, F8.E4M3), (F8.E4M3, F8.E5M2)]
    # the recipe matters: the two FP8 layers differ
    yc, _ = F8.fp8_ptb_forward(x, p, *args)
    assert rel(y8 - x, yc - x) > 1e-4
