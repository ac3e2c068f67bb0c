"""fp64 CPU oracle of the FP8-GEMM variant of one Parallel Transformer Block
layer (forward and backward).

TEST INFRASTRUCTURE. Only the test-suite, the package's smoke entry and the
benchmark's CPU-baseline leg may import or run this module; the HIP library
never calls it and shares no code with it.

Pages followed (cited by title and section):
  [MT]  "Megatron-LM 分布式训练（七）：显存与性能调优", mixed-precision section
        (BF16 vs FP16, then FP8): two 8-bit formats, E4M3 (more mantissa, used
        for forward operands and weights) and E5M2 (more range, used for
        backward gradients); scaling recipes delayed, current and block-wise
        (mxfp8); only the matrix products run in FP8, while LayerNorm,
        softmax, residual sums and the optimizer stay in BF16/FP32.
  [MS]  MegaScale reading notes, section 1.1 eq (4): the layer itself (taken
        from ptb_oracle).

Readings where the pages leave a step open (each is also the library's):
  * Formats: the two named formats as commonly defined (OCP 8-bit floating
    point): E4M3 with exponent bias 7, no infinities, S.1111.111 the only NaN,
    largest finite 448; E5M2 with bias 15 and IEEE-style infinities and NaNs,
    largest finite 57344.  Both have subnormals.
  * Recipes: current scaling (below) and block scaling (mxfp8, further
    below); a layer call uses one of them for all six products.
  * Current scaling: one scale per GEMM operand.  An operand that is a
    concatenation of tensors ([W_qkv | W_fc1], [c | g], [W_o ; W_fc2],
    [dqkv | du]) is one tensor for scaling.  s = fp32(FMAX / amax) with amax
    the largest magnitude of the bf16 operand (s = 1 when amax = 0).
  * Quantization: code = round-to-nearest-even(clamp(fp32(x * s), -FMAX, FMAX))
    on the format's grid, x the bf16 operand; the product x * s is one fp32
    multiply.  Dequantized product: C = (sum_k qa qb) / (sa sb).
  * Which operands: forward a, [W_qkv | W_fc1], [c | g], [W_o ; W_fc2] in
    E4M3; backward dy and [dqkv | du] in E5M2 against E4M3 weights and E4M3
    saved activations (the weight gradients take E4M3 a^T, [c | g]^T).
  * Block scaling: the pages name mxfp8 and nothing more; its published
    definition (OCP Microscaling Formats v1.0) is taken as is.  Blocks of 32
    consecutive values along the product's contraction axis (a short last
    block where the axis is not a multiple of 32), one E8M0 scale per block
    (a power of two, code e meaning 2^(e - 127), e in 0..254),
    X = floor(log2 amax_block) - emax with emax the exponent of the format's
    largest power of two (8 for E4M3, 15 for E5M2), an all-zero block taking
    X = 0; element codes = RNE(clamp(fp32(x * 2^-X), -FMAX, FMAX)) (the
    multiply is exact).  Dequantized product: sum over k of
    qa 2^Xa qb 2^Xb, the block scales of the two operands at the same k.
    Each product quantizes its operands along its own contraction axis, so
    a tensor that feeds two products (dy, dZ, the weights) is quantized
    twice, once per orientation.
  * BF16 points: the tensors the pages keep in BF16 and that feed a product
    (a, c, g, dqkv, du) are rounded to bf16 (round to nearest even) before
    they are quantized; dy and the weights are bf16 already.  Everything else
    (LayerNorm, attention, GeLU, residual, the LayerNorm backward) is fp64 as
    in ptb_oracle.
"""
from __future__ import annotations

import math
from typing import Dict, Tuple

import numpy as np

from oracle.ptb_oracle import (attention_backward, attention_forward, gelu, gelu_grad,
                               merge_heads, norm_backward, norm_forward, split_heads)

E4M3 = "e4m3"
E5M2 = "e5m2"

# (exponent bits, mantissa bits, bias)
_LAYOUT = {E4M3: (4, 3, 7), E5M2: (5, 2, 15)}


def decode_table(fmt: str) -> np.ndarray:
    """Value of every one of the 256 codes, from the bit fields: sign, then
    exponent, then mantissa; exponent field 0 is subnormal (no implicit one,
    exponent 1 - bias).  E4M3: only S.1111.111 is NaN, the rest of the top
    binade is finite.  E5M2: exponent field 31 is infinity (mantissa 0) or NaN."""
    eb, mb, bias = _LAYOUT[fmt]
    out = np.empty(256)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> mb) & ((1 << eb) - 1)
        m = code & ((1 << mb) - 1)
        top = (1 << eb) - 1
        if fmt == E4M3 and e == top and m == (1 << mb) - 1:
            out[code] = math.nan
        elif fmt == E5M2 and e == top:
            out[code] = sign * math.inf if m == 0 else math.nan
        elif e == 0:
            out[code] = sign * m * 2.0 ** (1 - bias - mb)
        else:
            out[code] = sign * (1.0 + m / (1 << mb)) * 2.0 ** (e - bias)
    return out


def fmax(fmt: str) -> float:
    """Largest finite value of the format."""
    t = decode_table(fmt)[:128]
    return float(np.max(t[np.isfinite(t)]))


def _positive_grid(fmt: str) -> np.ndarray:
    """Finite non-negative values in code order 0, 1, ... (increasing)."""
    t = decode_table(fmt)[:128]
    return t[np.isfinite(t)]


def round_bf16(x: np.ndarray) -> np.ndarray:
    """x rounded to bfloat16 (8 significant bits), nearest, ties to even;
    for the normal range of bf16, which is all this layer produces."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def current_scale(x: np.ndarray, fmt: str) -> np.float32:
    """s = fp32(FMAX / amax) over the whole operand, 1 when it is all zero."""
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(np.float32(fmax(fmt)) / amax)


def quantize(x: np.ndarray, scale: np.float32, fmt: str) -> Tuple[np.ndarray, np.ndarray]:
    """(codes uint8, values float64) of x (bf16-valued) scaled by `scale`.

    y = fp32(x * scale), clamped to +-FMAX, goes to the nearer of the two grid
    values around |y|; a tie goes to the even code (even last mantissa bit).
    The sign bit is copied, so -0 gives the negative zero code."""
    y = np.asarray(x, dtype=np.float32) * np.float32(scale)
    top = np.float32(fmax(fmt))
    y = np.clip(y, -top, top).astype(np.float64)
    grid = _positive_grid(fmt)
    mag = np.abs(y)
    hi = np.clip(np.searchsorted(grid, mag, side="left"), 0, grid.size - 1)
    lo = np.clip(hi - 1, 0, grid.size - 1)
    dlo, dhi = mag - grid[lo], grid[hi] - mag
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(mag == grid[hi], hi, idx)
    neg = np.signbit(y)  # the sign bit is kept, -0 included
    codes = idx.astype(np.uint8) | np.where(neg, 0x80, 0).astype(np.uint8)
    vals = np.where(neg, -grid[idx], grid[idx])
    return codes, vals


def fp8_matmul(a: np.ndarray, b: np.ndarray, fmt_a: str, fmt_b: str,
               record: list | None = None) -> np.ndarray:
    """C = A B with each operand quantized on its own current scale."""
    sa, sb = current_scale(a, fmt_a), current_scale(b, fmt_b)
    _, qa = quantize(a, sa, fmt_a)
    _, qb = quantize(b, sb, fmt_b)
    if record is not None:
        record.append((fmt_a, fmt_b))
    return (qa @ qb) / (float(sa) * float(sb))


# ---------------------------------------------------------------------------
# Block (MX) scaling
# ---------------------------------------------------------------------------
MX_BLOCK = 32


def emax(fmt: str) -> int:
    """Exponent of the format's largest power of two: 8 (E4M3), 15 (E5M2)."""
    return math.frexp(fmax(fmt))[1] - 1


def mx_scale_code(amax: np.ndarray, fmt: str) -> np.ndarray:
    """E8M0 code of each block: 127 + floor(log2 amax) - emax, within
    0..254; 127 (scale 1) for an all-zero block."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)               # amax = m 2^e, 0.5 <= m < 1
    x = np.where(amax > 0, e - 1 - emax(fmt), 0)
    return np.clip(x + 127, 0, 254).astype(np.int64)


def mx_quantize(x: np.ndarray, fmt: str, axis: int):
    """(codes uint8, scale codes int64, values float64) of a 2-D x with blocks
    of 32 along `axis`.  Scale codes have the blocks' shape: [R, ceil(C/32)]
    for axis 1, [ceil(R/32), C] for axis 0."""
    x = np.asarray(x, dtype=np.float64)
    xt = x if axis == 1 else x.T
    rows, n = xt.shape
    nb = -(-n // MX_BLOCK)
    padded = np.zeros((rows, nb * MX_BLOCK))
    padded[:, :n] = xt
    blocks = padded.reshape(rows, nb, MX_BLOCK)
    sc = mx_scale_code(np.abs(blocks).max(axis=2), fmt)
    mult = np.ldexp(np.float32(1.0), 127 - sc).astype(np.float32)   # 2^-X, exact
    codes, vals = quantize(blocks, mult[:, :, None], fmt)
    vals = vals * np.ldexp(1.0, sc - 127)[:, :, None]
    codes = codes.reshape(rows, -1)[:, :n]
    vals = vals.reshape(rows, -1)[:, :n]
    if axis == 0:
        return codes.T, sc.T, vals.T
    return codes, sc, vals


def mx_matmul(a: np.ndarray, b: np.ndarray, fmt_a: str, fmt_b: str,
              record: list | None = None) -> np.ndarray:
    """C = A B with both operands block-scaled along the contraction axis."""
    _, _, qa = mx_quantize(a, fmt_a, axis=1)
    _, _, qb = mx_quantize(b, fmt_b, axis=0)
    if record is not None:
        record.append((fmt_a, fmt_b))
    return qa @ qb


_RECIPES = {"current": fp8_matmul, "mx": mx_matmul}


# ---------------------------------------------------------------------------
# The layer ([MS] 1.1 eq (4)) with its four GEMM parts in FP8 ([MT]).
# ---------------------------------------------------------------------------
def fp8_ptb_forward(x: np.ndarray, p: Dict[str, np.ndarray], batch: int, seq: int,
                    heads: int, head_dim: int, window: int, eps: float,
                    norm: str = "layernorm", recipe: str = "current"):
    """y = x + Attn(LN(x)) + MLP(LN(x)) with [QKV | FC1] and [O ; FC2] as FP8
    products, scaled by `recipe` ("current" or "mx").  p as in
    ptb_oracle.ptb_forward (GeLU MLP)."""
    hl = heads * head_dim
    rec: list = []
    fp8_mm = _RECIPES[recipe]
    a_full, mu, rstd = norm_forward(norm, x, p["ln_gamma"], p["ln_beta"], eps)
    a = round_bf16(a_full)
    w1 = np.concatenate([p["w_qkv"], p["w_fc1"]], axis=1)
    z = fp8_mm(a, w1, E4M3, E4M3, rec)
    qkv, u = z[:, :3 * hl], z[:, 3 * hl:]
    g = gelu(u)
    q = split_heads(qkv[:, :hl], batch, seq, heads, head_dim)
    k = split_heads(qkv[:, hl:2 * hl], batch, seq, heads, head_dim)
    v = split_heads(qkv[:, 2 * hl:], batch, seq, heads, head_dim)
    c = merge_heads(attention_forward(q, k, v, window))
    cg = round_bf16(np.concatenate([c, g], axis=1))
    w2 = np.concatenate([p["w_o"], p["w_fc2"]], axis=0)
    y = x + fp8_mm(cg, w2, E4M3, E4M3, rec)
    cache = dict(x=x, a=a, mu=mu, rstd=rstd, q=q, k=k, v=v, c=c, u=u, g=g, qkv=qkv, cg=cg,
                 norm=norm, formats=rec, recipe=recipe)
    return y, cache


def fp8_ptb_backward(dy: np.ndarray, cache: dict, p: Dict[str, np.ndarray],
                     window: int) -> Dict[str, np.ndarray]:
    """Gradients of fp8_ptb_forward: the same four GEMM parts in FP8 (gradient
    operands E5M2), quantization passed straight through."""
    rec = cache["formats"]
    fp8_matmul = _RECIPES[cache["recipe"]]
    x, a, u, cg = cache["x"], cache["a"], cache["u"], cache["cg"]
    q, k, v = cache["q"], cache["k"], cache["v"]
    hl = cache["c"].shape[1]
    w1 = np.concatenate([p["w_qkv"], p["w_fc1"]], axis=1)
    w2 = np.concatenate([p["w_o"], p["w_fc2"]], axis=0)
    # [O ; FC2]: dgrad and wgrad
    dcg = fp8_matmul(dy, w2.T, E5M2, E4M3, rec)
    dc, dg = dcg[:, :hl], dcg[:, hl:]
    du = dg * gelu_grad(u)
    dw2 = fp8_matmul(cg.T, dy, E4M3, E5M2, rec)
    # attention
    b, n, s, d = q.shape
    dq, dk, dv = attention_backward(q, k, v, split_heads(dc, b, s, n, d), window)
    dz = round_bf16(np.concatenate([merge_heads(dq), merge_heads(dk), merge_heads(dv), du],
                                   axis=1))
    # [QKV | FC1]: dgrad and wgrad
    da = fp8_matmul(dz, w1.T, E5M2, E4M3, rec)
    dw1 = fp8_matmul(a.T, dz, E4M3, E5M2, rec)
    dx_ln, dgamma, dbeta = norm_backward(cache["norm"], da, x, p["ln_gamma"], cache["mu"],
                                         cache["rstd"])
    nqkv = p["w_qkv"].shape[1]
    return dict(dx=dy + dx_ln, d_ln_gamma=dgamma, d_ln_beta=dbeta,
                dw_qkv=dw1[:, :nqkv], dw_fc1=dw1[:, nqkv:], dw_o=dw2[:hl], dw_fc2=dw2[hl:],
                da=da, dz=dz, dc=dc)
