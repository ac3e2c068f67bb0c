"""Shared test plumbing: run the oracle and the HIP path on the same seeded
inputs and compare them.  The oracle and the HIP path never see each other's
values: both start from the generator's bf16 bits."""
from __future__ import annotations

import math
import os
import sys

import numpy as np

from oracle import ptb_oracle as O
from transformer_block_amd import inputs as I

# Parity bar: relative Frobenius error per output tensor (bf16 operands, fp32
# accumulation, compared with the fp64 oracle).
REL_TOL = 1e-2


def rel_fro(got: np.ndarray, ref: np.ndarray) -> float:
    den = float(np.linalg.norm(ref))
    num = float(np.linalg.norm(got - ref))
    if den == 0.0:
        return num
    return num / den


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def dropout_multipliers(w: I.Workload):
    """Per-layer dropout multipliers of the parallel block (None without
    dropout): layer l draws stream 2 l."""
    if w.dropout_p == 0.0:
        return None
    from oracle import dropout_oracle as D
    return [D.dropout_multiplier((w.tokens, w.hidden), w.dropout_seed, D.layer_stream(li),
                                 w.dropout_p) for li in range(w.layers)]


def oracle_run(w: I.Workload, inp: dict) -> dict:
    f = I.bf16_bits_to_f64
    x = f(inp["x"])
    dy = f(inp["dy"])
    params = [{k: f(v) for k, v in lay.items()} for lay in inp["layers"]]
    y, caches = O.ptb_stack_forward(x, params, w.batch, w.seq, w.heads, w.head_dim,
                                    w.window, w.ln_eps, norm=w.norm, mlp=w.mlp,
                                    drops=dropout_multipliers(w))
    dx, grads = O.ptb_stack_backward(dy, caches, params, w.window)
    return dict(x=x, dy=dy, y=y, dx=dx, grads=grads, caches=caches)


def oracle_lse2(cache: dict, w: I.Workload) -> np.ndarray:
    """Base-2 log-sum-exp of the logits scaled by log2(e)/sqrt(d), from the
    oracle's q and k (fp64), shape [b, n, s]."""
    q, k = cache["q"], cache["k"]
    mask = O.window_mask(w.seq, w.window)
    out = np.empty((w.batch, w.heads, w.seq))
    for bi in range(w.batch):
        for hi in range(w.heads):
            z = (q[bi, hi] @ k[bi, hi].T) / math.sqrt(w.head_dim)
            z = np.where(mask, z, -np.inf)
            m = z.max(axis=1, keepdims=True)
            out[bi, hi] = (m[:, 0] + np.log(np.exp(z - m).sum(axis=1))) / math.log(2.0)
    return out


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False
