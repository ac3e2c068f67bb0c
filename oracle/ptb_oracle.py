"""fp64 CPU oracle of one Parallel Transformer Block (PTB) layer, forward and
backward, with sliding-window causal attention and a GeLU MLP.

TEST INFRASTRUCTURE. Only the test-suite, the package's smoke entry and the
benchmark's CPU-baseline leg may import or run this module.  The HIP library
never calls it, and it shares no code with the HIP path: inputs arrive as plain
numpy arrays (bf16 values widened to float64 by the caller) and everything here
is computed in float64 with plain numpy.

Pages followed (cited by title and section):
  [MS]  Zhongzhu Zhou, "MegaScale: ByteDance 如何在 12,288 块 GPU 上实现 55% MFU
        的大规模 LLM 训练" (reading notes on MegaScale, NSDI'24):
        section 1.1 eq (4) parallel block, eq (3) serial block (for
        comparison), eq (5)-(6) sliding-window attention;
        section 1.3 flash attention as an exact re-tiling, selective recompute.
  [TP]  "Megatron-LM：张量并行与大规模训练": section 2.1 MLP ``Y = GeLU(XA)B``
        with ``A: [h,4h]``, ``B: [4h,h]``; section 2.2 fused QKV ``[b,s,3h]``
        split by heads; section 5.5 bf16.
  [MT]  "Megatron-LM 分布式训练（七）：显存与性能调优": section on recompute
        (selective ``core_attn``), section on MFU (6ND + attention s^2 term,
        recompute excluded from model FLOPs, included in HFU).

Readings taken where the pages are silent (each is also a documented choice of
the library): window = the w most recent keys including the query itself
(0 <= i - j < w); causal; softmax scale 1/sqrt(d); LayerNorm (not RMSNorm) with
biased variance and eps inside the square root; exact-erf GeLU; no biases;
dropout (optional, [MS] 1.3) on the block's branch output before the residual
add, given as a multiplier matrix (0 or 1/(1-p) per element, drawn by
oracle/dropout_oracle.py); QKV columns ordered [Q heads | K heads | V heads], each head's d
columns contiguous, and the attention output ``c`` uses the same head order for
the rows of ``W_o``.

Layout: every activation is token-major ``[T, .]`` with ``T = b*s`` and token
index ``t = batch_index*s + position``.

Variants ([MS] 1.3 names MegaScale's own fused RMSNorm and SwiGLU kernels):
``norm="rmsnorm"`` replaces each LayerNorm by a = gamma * x / sqrt(mean(x^2) +
eps) (no beta); ``mlp="swiglu"`` replaces GeLU(a W_fc1) by silu(a W1) * (a W3),
silu(u) = u sigmoid(u), with W1 and W3 carried in one w_fc1 [h, 2f] whose
32-column blocks alternate W1 and W3 (the library's layout; split_w13 and
merge_w13 below are that permutation and nothing else).
"""
from __future__ import annotations

import math
from typing import Dict, List, Tuple

import numpy as np
from scipy.special import erf


# ---------------------------------------------------------------------------
# FLOP bookkeeping.  Counts are taken from the work actually done below:
# 2*M*N*K per matrix product and 2*d per *unmasked* (query, key) pair per
# attention contraction, the pairs being counted from the boolean mask itself.
# Model FLOPs exclude the recomputed QK^T of the backward pass; hardware FLOPs
# include it ([MT] MFU section: MFU vs HFU).
# ---------------------------------------------------------------------------
class FlopCounter:
    def __init__(self) -> None:
        self.model = 0
        self.recompute = 0

    def gemm(self, m: int, n: int, k: int) -> None:
        self.model += 2 * m * n * k

    def attn(self, unmasked_pairs: int, d: int, recompute: bool = False) -> None:
        f = 2 * unmasked_pairs * d
        if recompute:
            self.recompute += f
        else:
            self.model += f


def _mm(a: np.ndarray, b: np.ndarray, fc: FlopCounter | None) -> np.ndarray:
    if fc is not None:
        fc.gemm(a.shape[0], b.shape[1], a.shape[1])
    return a @ b


# ---------------------------------------------------------------------------
# LayerNorm ([MS] 1.1 eq (4): both branches read LN(x)).
# ---------------------------------------------------------------------------
def layernorm_forward(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray,
                      eps: float) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """a = gamma * (x - mean) / sqrt(var + eps) + beta, per row of x [T, h]."""
    mu = x.mean(axis=1)
    var = ((x - mu[:, None]) ** 2).mean(axis=1)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (x - mu[:, None]) * rstd[:, None]
    return xhat * gamma[None, :] + beta[None, :], mu, rstd


def layernorm_backward(da: np.ndarray, x: np.ndarray, gamma: np.ndarray,
                       mu: np.ndarray, rstd: np.ndarray):
    """Gradient of the LayerNorm above: returns (dx, dgamma, dbeta).

    With xhat = (x - mean) * rstd and g = da * gamma, the row-wise chain rule
    through the mean and the variance gives
        dx = rstd * (g - mean_k(g) - xhat * mean_k(g * xhat)).
    """
    xhat = (x - mu[:, None]) * rstd[:, None]
    g = da * gamma[None, :]
    dx = rstd[:, None] * (g - g.mean(axis=1, keepdims=True)
                          - xhat * (g * xhat).mean(axis=1, keepdims=True))
    return dx, (da * xhat).sum(axis=0), da.sum(axis=0)


def rmsnorm_forward(x: np.ndarray, gamma: np.ndarray,
                    eps: float) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """a = gamma * x / sqrt(mean(x^2) + eps) per row; returns (a, 0, rstd)
    (a zero row mean, so that xhat = (x - mean) * rstd holds as for LN)."""
    rstd = 1.0 / np.sqrt((x * x).mean(axis=1) + eps)
    return x * rstd[:, None] * gamma[None, :], np.zeros(x.shape[0]), rstd


def rmsnorm_backward(da: np.ndarray, x: np.ndarray, gamma: np.ndarray, rstd: np.ndarray):
    """Gradient of rmsnorm_forward: (dx, dgamma, dbeta = 0).  With
    xhat = x * rstd and g = da * gamma, dx = rstd * (g - xhat * mean_k(g * xhat))."""
    xhat = x * rstd[:, None]
    g = da * gamma[None, :]
    dx = rstd[:, None] * (g - xhat * (g * xhat).mean(axis=1, keepdims=True))
    return dx, (da * xhat).sum(axis=0), np.zeros(x.shape[1])


def norm_forward(kind: str, x, gamma, beta, eps):
    if kind == "rmsnorm":
        return rmsnorm_forward(x, gamma, eps)
    return layernorm_forward(x, gamma, beta, eps)


def norm_backward(kind: str, da, x, gamma, mu, rstd):
    if kind == "rmsnorm":
        return rmsnorm_backward(da, x, gamma, rstd)
    return layernorm_backward(da, x, gamma, mu, rstd)


# ---------------------------------------------------------------------------
# GeLU ([TP] 2.1): exact form u * Phi(u), Phi the standard normal CDF.
# ---------------------------------------------------------------------------
def normal_cdf(u: np.ndarray) -> np.ndarray:
    return 0.5 * (1.0 + erf(u / math.sqrt(2.0)))


def normal_pdf(u: np.ndarray) -> np.ndarray:
    return np.exp(-0.5 * u * u) / math.sqrt(2.0 * math.pi)


def gelu(u: np.ndarray) -> np.ndarray:
    return u * normal_cdf(u)


def gelu_grad(u: np.ndarray) -> np.ndarray:
    """d/du [u Phi(u)] = Phi(u) + u phi(u)."""
    return normal_cdf(u) + u * normal_pdf(u)


# ---------------------------------------------------------------------------
# SwiGLU ([MS] 1.3): silu(a W1) * (a W3), silu(u) = u * sigmoid(u).
# ---------------------------------------------------------------------------
def sigmoid(u: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-u))


def silu(u: np.ndarray) -> np.ndarray:
    return u * sigmoid(u)


def silu_grad(u: np.ndarray) -> np.ndarray:
    """d/du [u sigmoid(u)] = sigmoid(u) + u sigmoid(u) (1 - sigmoid(u))."""
    s = sigmoid(u)
    return s + u * s * (1.0 - s)


def split_w13(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """[rows, 2f] with 32-column blocks alternating W1, W3 -> (W1, W3) [rows, f]."""
    rows, two_f = w.shape
    blocks = w.reshape(rows, two_f // 64, 2, 32)
    return blocks[:, :, 0, :].reshape(rows, two_f // 2), blocks[:, :, 1, :].reshape(rows, two_f // 2)


def merge_w13(w1: np.ndarray, w3: np.ndarray) -> np.ndarray:
    """Inverse of split_w13."""
    rows, f = w1.shape
    return np.stack([w1.reshape(rows, f // 32, 32), w3.reshape(rows, f // 32, 32)],
                    axis=2).reshape(rows, 2 * f)


def mlp_forward(kind: str, a: np.ndarray, w_fc1: np.ndarray, fc):
    """(u, g): u the pre-activation in w_fc1's column layout, g the activation."""
    if kind == "swiglu":
        w1, w3 = split_w13(w_fc1)
        u1, u3 = _mm(a, w1, fc), _mm(a, w3, fc)
        return merge_w13(u1, u3), silu(u1) * u3
    u = _mm(a, w_fc1, fc)
    return u, gelu(u)


def mlp_backward(kind: str, dg: np.ndarray, u: np.ndarray, a: np.ndarray, w_fc1: np.ndarray,
                 fc):
    """(dw_fc1, da) of mlp_forward for upstream gradient dg of g."""
    if kind == "swiglu":
        u1, u3 = split_w13(u)
        w1, w3 = split_w13(w_fc1)
        du1 = dg * u3 * silu_grad(u1)
        du3 = dg * silu(u1)
        dw = merge_w13(_mm(a.T, du1, fc), _mm(a.T, du3, fc))
        return dw, _mm(du1, w1.T, fc) + _mm(du3, w3.T, fc)
    du = dg * gelu_grad(u)
    return _mm(a.T, du, fc), _mm(du, w_fc1.T, fc)


# ---------------------------------------------------------------------------
# Sliding-window causal attention ([MS] 1.1 eq (5)-(6), 1.3).  Computed densely
# per (batch, head): the s x s logits are formed, keys outside the window are
# masked, and each row is soft-maxed.  Flash tiling and selective recompute
# change memory traffic, not these values ([MS] 1.3).
# ---------------------------------------------------------------------------
def window_mask(s: int, window: int) -> np.ndarray:
    """mask[i, j] is True iff key j is one of the `window` most recent tokens
    seen by query i, the query itself included: 0 <= i - j < window."""
    i = np.arange(s)[:, None]
    j = np.arange(s)[None, :]
    diff = i - j
    return (diff >= 0) & (diff < window)


def attention_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, window: int,
                      fc: FlopCounter | None = None) -> np.ndarray:
    """q, k, v: [b, n, s, d] -> o: [b, n, s, d].

    o_i = sum_j P_ij v_j with P_i = softmax over the window of q_i . k_j / sqrt(d).
    """
    b, n, s, d = q.shape
    scale = 1.0 / math.sqrt(d)
    mask = window_mask(s, window)
    o = np.empty_like(q)
    for bi in range(b):
        for hi in range(n):
            logits = (q[bi, hi] @ k[bi, hi].T) * scale
            logits = np.where(mask, logits, -np.inf)
            p = np.exp(logits - logits.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            o[bi, hi] = p @ v[bi, hi]
            if fc is not None:
                pairs = int(mask.sum())
                fc.attn(pairs, d)          # q k^T
                fc.attn(pairs, d)          # P v
    return o


def attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                       do: np.ndarray, window: int,
                       fc: FlopCounter | None = None):
    """Gradients of attention_forward w.r.t. q, k, v given do = dL/do.

    The probabilities are recomputed from q and k (selective recompute of the
    core attention, [MS] 1.3 and [MT] recompute section); only the values of
    P, not its storage, enter the result:
      dV = P^T dO,  dP = dO V^T,
      dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)   (softmax Jacobian, row-wise),
      dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d).
    """
    b, n, s, d = q.shape
    scale = 1.0 / math.sqrt(d)
    mask = window_mask(s, window)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    for bi in range(b):
        for hi in range(n):
            logits = (q[bi, hi] @ k[bi, hi].T) * scale
            logits = np.where(mask, logits, -np.inf)
            p = np.exp(logits - logits.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            dov = do[bi, hi]
            dv[bi, hi] = p.T @ dov
            dp = dov @ v[bi, hi].T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[bi, hi] = (ds @ k[bi, hi]) * scale
            dk[bi, hi] = (ds.T @ q[bi, hi]) * scale
            if fc is not None:
                pairs = int(mask.sum())
                fc.attn(pairs, d, recompute=True)  # q k^T again
                for _ in range(4):                 # dV, dP, dQ, dK
                    fc.attn(pairs, d)
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Head split/merge for the QKV layout [Q heads | K heads | V heads] ([TP] 2.2).
# ---------------------------------------------------------------------------
def split_heads(t: np.ndarray, b: int, s: int, n: int, d: int) -> np.ndarray:
    """[T, n*d] -> [b, n, s, d]."""
    return t.reshape(b, s, n, d).transpose(0, 2, 1, 3)


def merge_heads(t: np.ndarray) -> np.ndarray:
    """[b, n, s, d] -> [T, n*d]."""
    b, n, s, d = t.shape
    return t.transpose(0, 2, 1, 3).reshape(b * s, n * d)


# ---------------------------------------------------------------------------
# One PTB layer: y = x + Attention(LN(x)) + MLP(LN(x))   ([MS] 1.1 eq (4)).
# ---------------------------------------------------------------------------
def ptb_forward(x: np.ndarray, p: Dict[str, np.ndarray], batch: int, seq: int,
                heads: int, head_dim: int, window: int, eps: float,
                fc: FlopCounter | None = None, norm: str = "layernorm", mlp: str = "gelu",
                drop: np.ndarray | None = None):
    """x: [T, h]; p holds ln_gamma, ln_beta, w_qkv [h,3hl], w_o [hl,h],
    w_fc1 [h,f] ([h,2f] for SwiGLU), w_fc2 [f,h] (float64).  drop: None, or the
    dropout multiplier [T, h] of the branch output (0 dropped, 1/(1-p) kept):
    y = x + drop * (Attn + MLP).  Returns (y, cache)."""
    hl = heads * head_dim
    a, mu, rstd = norm_forward(norm, x, p["ln_gamma"], p["ln_beta"], eps)
    # attention branch
    qkv = _mm(a, p["w_qkv"], fc)
    q = split_heads(qkv[:, :hl], batch, seq, heads, head_dim)
    k = split_heads(qkv[:, hl:2 * hl], batch, seq, heads, head_dim)
    v = split_heads(qkv[:, 2 * hl:], batch, seq, heads, head_dim)
    o = attention_forward(q, k, v, window, fc)
    c = merge_heads(o)
    attn_out = _mm(c, p["w_o"], fc)
    # MLP branch on the same LN output
    u, g = mlp_forward(mlp, a, p["w_fc1"], fc)
    mlp_out = _mm(g, p["w_fc2"], fc)
    branch = attn_out + mlp_out
    y = x + (branch if drop is None else drop * branch)
    cache = dict(x=x, a=a, mu=mu, rstd=rstd, q=q, k=k, v=v, c=c, u=u, g=g,
                 qkv=qkv, norm=norm, mlp=mlp, drop=drop)
    return y, cache


def ptb_backward(dy: np.ndarray, cache: dict, p: Dict[str, np.ndarray],
                 window: int, fc: FlopCounter | None = None) -> Dict[str, np.ndarray]:
    """Gradients of ptb_forward for upstream gradient dy [T, h]."""
    x, a, c, u, g = cache["x"], cache["a"], cache["c"], cache["u"], cache["g"]
    q, k, v = cache["q"], cache["k"], cache["v"]
    # the branch output's gradient passes the dropout mask; the residual's does not
    drop = cache.get("drop")
    db = dy if drop is None else drop * dy
    # output projections of both branches
    dc = _mm(db, p["w_o"].T, fc)
    dg = _mm(db, p["w_fc2"].T, fc)
    dw_o = _mm(c.T, db, fc)
    dw_fc2 = _mm(g.T, db, fc)
    # MLP branch
    dw_fc1, da_mlp = mlp_backward(cache["mlp"], dg, u, a, p["w_fc1"], fc)
    # attention branch
    b, n, s, d = q.shape
    dq, dk, dv = attention_backward(q, k, v, split_heads(dc, b, s, n, d),
                                    window, fc)
    dqkv = np.concatenate([merge_heads(dq), merge_heads(dk), merge_heads(dv)],
                          axis=1)
    dw_qkv = _mm(a.T, dqkv, fc)
    da_attn = _mm(dqkv, p["w_qkv"].T, fc)
    # shared LayerNorm and the residual
    dx_ln, dgamma, dbeta = norm_backward(cache["norm"], da_attn + da_mlp, x,
                                         p["ln_gamma"], cache["mu"], cache["rstd"])
    return dict(dx=dy + dx_ln, d_ln_gamma=dgamma, d_ln_beta=dbeta,
                dw_qkv=dw_qkv, dw_o=dw_o, dw_fc1=dw_fc1, dw_fc2=dw_fc2)


def ptb_stack_forward(x: np.ndarray, params: List[Dict[str, np.ndarray]],
                      batch: int, seq: int, heads: int, head_dim: int,
                      window: int, eps: float, fc: FlopCounter | None = None,
                      norm: str = "layernorm", mlp: str = "gelu", drops=None):
    """L stacked layers: x_{l+1} = PTB(x_l; theta_l); drops: None or one
    dropout multiplier (or None) per layer.  Returns (y, caches)."""
    caches = []
    for li, p in enumerate(params):
        x, cache = ptb_forward(x, p, batch, seq, heads, head_dim, window, eps, fc, norm, mlp,
                               drop=None if drops is None else drops[li])
        caches.append(cache)
    return x, caches


def ptb_stack_backward(dy: np.ndarray, caches: list,
                       params: List[Dict[str, np.ndarray]], window: int,
                       fc: FlopCounter | None = None):
    """Backward through the stack, last layer first; dx of layer l+1 is the
    upstream gradient of layer l.  Returns (dx, per-layer gradient dicts)."""
    grads = [None] * len(params)
    for li in range(len(params) - 1, -1, -1):
        grads[li] = ptb_backward(dy, caches[li], params[li], window, fc)
        dy = grads[li]["dx"]
    return dy, grads


# ---------------------------------------------------------------------------
# Serial (standard) block, [MS] 1.1 eq (3), the block the parallel one
# replaces.  Reading: the notes print eq (3) with x alone in the outer sum,
# y = x + MLP(LN(x + Attn(LN(x)))), but describe the parallel block (eq (4))
# as the standard one with LN(x) in place of LN(x + h2), h2 = Attn(LN(x)), as
# the MLP's input and nothing else changed; eq (4) keeps h2 in the outer sum,
# so the standard block is read with it there as well:
#     a1 = LN1(x),  h2 = Attn(a1) W_o,  x1 = x + h2,
#     y  = x1 + MLP(LN2(x1)),
# the two LayerNorms with their own gamma and beta (p["ln_gamma"],
# p["ln_beta"] for LN1 as in the parallel block, p["ln2_gamma"],
# p["ln2_beta"] for LN2).
# ---------------------------------------------------------------------------
def serial_forward(x: np.ndarray, p: Dict[str, np.ndarray], batch: int, seq: int,
                   heads: int, head_dim: int, window: int, eps: float,
                   fc: FlopCounter | None = None, norm: str = "layernorm", mlp: str = "gelu",
                   drop1: np.ndarray | None = None, drop2: np.ndarray | None = None):
    """x: [T, h] -> (y, cache) for the serial block above; drop1, drop2: the
    dropout multipliers of the attention and MLP branch outputs (or None):
    x1 = x + drop1 * Attn(a1) W_o, y = x1 + drop2 * MLP(a2)."""
    hl = heads * head_dim
    a1, mu1, rstd1 = norm_forward(norm, x, p["ln_gamma"], p["ln_beta"], eps)
    qkv = _mm(a1, p["w_qkv"], fc)
    q = split_heads(qkv[:, :hl], batch, seq, heads, head_dim)
    k = split_heads(qkv[:, hl:2 * hl], batch, seq, heads, head_dim)
    v = split_heads(qkv[:, 2 * hl:], batch, seq, heads, head_dim)
    c = merge_heads(attention_forward(q, k, v, window, fc))
    h2 = _mm(c, p["w_o"], fc)
    x1 = x + (h2 if drop1 is None else drop1 * h2)
    a2, mu2, rstd2 = norm_forward(norm, x1, p["ln2_gamma"], p["ln2_beta"], eps)
    u, g = mlp_forward(mlp, a2, p["w_fc1"], fc)
    m = _mm(g, p["w_fc2"], fc)
    y = x1 + (m if drop2 is None else drop2 * m)
    cache = dict(x=x, a1=a1, mu1=mu1, rstd1=rstd1, qkv=qkv, q=q, k=k, v=v, c=c,
                 x1=x1, a2=a2, mu2=mu2, rstd2=rstd2, u=u, g=g, norm=norm, mlp=mlp,
                 drop1=drop1, drop2=drop2)
    return y, cache


def serial_backward(dy: np.ndarray, cache: dict, p: Dict[str, np.ndarray],
                    window: int, fc: FlopCounter | None = None) -> Dict[str, np.ndarray]:
    """Gradients of serial_forward for upstream gradient dy [T, h]: the MLP
    sub-block first, then the attention sub-block, each with its residual."""
    # MLP sub-block: y = x1 + drop2 * GeLU(LN2(x1) W_fc1) W_fc2
    d2 = cache.get("drop2")
    dm = dy if d2 is None else d2 * dy
    dg = _mm(dm, p["w_fc2"].T, fc)
    dw_fc2 = _mm(cache["g"].T, dm, fc)
    dw_fc1, da2 = mlp_backward(cache["mlp"], dg, cache["u"], cache["a2"], p["w_fc1"], fc)
    dx1_ln, dgamma2, dbeta2 = norm_backward(cache["norm"], da2, cache["x1"], p["ln2_gamma"],
                                            cache["mu2"], cache["rstd2"])
    dx1 = dy + dx1_ln
    # attention sub-block: x1 = x + drop1 * Attn(LN1(x)) W_o
    d1 = cache.get("drop1")
    dh = dx1 if d1 is None else d1 * dx1
    dc = _mm(dh, p["w_o"].T, fc)
    dw_o = _mm(cache["c"].T, dh, fc)
    q, k, v = cache["q"], cache["k"], cache["v"]
    b, n, s, d = q.shape
    dq, dk, dv = attention_backward(q, k, v, split_heads(dc, b, s, n, d), window, fc)
    dqkv = np.concatenate([merge_heads(dq), merge_heads(dk), merge_heads(dv)], axis=1)
    dw_qkv = _mm(cache["a1"].T, dqkv, fc)
    da1 = _mm(dqkv, p["w_qkv"].T, fc)
    dx_ln, dgamma1, dbeta1 = norm_backward(cache["norm"], da1, cache["x"], p["ln_gamma"],
                                           cache["mu1"], cache["rstd1"])
    return dict(dx=dx1 + dx_ln, d_ln_gamma=dgamma1, d_ln_beta=dbeta1,
                d_ln2_gamma=dgamma2, d_ln2_beta=dbeta2, dw_qkv=dw_qkv, dw_o=dw_o,
                dw_fc1=dw_fc1, dw_fc2=dw_fc2)
