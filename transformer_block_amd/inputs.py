"""Workload registry and seeded synthetic input generator for one Parallel
Transformer Block (PTB) layer.

This module is shared by the fp64 oracle tests and the HIP path. It holds no
arithmetic of the layer itself: it only names workload shapes and draws seeded
random tensors, rounded once to bfloat16.

Shapes follow the pages:
  * activations are token-major ``[b, s, h]`` and the MLP weights use the
    ``Y = GeLU(X A) B`` orientation with ``A: [h, 4h]``, ``B: [4h, h]``
    (Megatron-LM tensor-parallel explainer, section 2.1);
  * the 175B-shape workload takes h = 12288, 96 heads and context 2048 from the
    GPT-3 table (same explainer, section 5.6) and one tensor-parallel share of
    it with TP = 8 (same explainer, section 5 on 3D parallelism): 12 local
    heads and an FFN shard of 4h/8 = 6144.

Distributions: x ~ N(0,1), every weight ~ N(0, 0.02^2), LayerNorm gamma = 1 and
beta = 0, dy ~ N(0,1); all drawn in fp32 with ``numpy.random.default_rng(seed)``
and rounded to bf16 with round-to-nearest-even.  Draw order: x, then per layer
(W_qkv, W_o, W_fc1, W_fc2), then dy.  An optional non-trivial gamma/beta
(gamma ~ 1 + N(0, 0.1^2), beta ~ N(0, 0.1^2)) is drawn after dy, so it never
changes the default streams; the second LayerNorm of the serial block
(``ln2_gamma``, ``ln2_beta``, unused by the parallel block) is drawn after
that, layer by layer, so it changes nothing drawn before it either.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seq: int
    hidden: int
    heads: int
    head_dim: int
    ffn: int
    window: int
    layers: int = 1
    seed: int = 1000
    ln_eps: float = 1e-5
    norm: str = "layernorm"   # or "rmsnorm"
    mlp: str = "gelu"         # or "swiglu" (W1 | W3 in w_fc1, 32-column blocks)
    dropout_p: float = 0.0    # dropout rate of the branch output (0 = none)
    dropout_seed: int = 0     # key of the dropout masks

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    @property
    def h_local(self) -> int:
        return self.heads * self.head_dim

    @property
    def fc1_width(self) -> int:
        """Columns of w_fc1: f, or 2f for SwiGLU's [W1 | W3]."""
        return 2 * self.ffn if self.mlp == "swiglu" else self.ffn

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def as_dict(self) -> dict:
        return dataclasses.asdict(self)


# The five workloads: a small one the oracle finishes in well under a second,
# a mid-size SWA layer, one TP=8 share of a 175B-shape layer, a long-sequence
# SWA layer and a two-layer stack.
WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_h256_s256_w64", batch=2, seq=256, hidden=256, heads=4,
                 head_dim=64, ffn=1024, window=64, seed=1001),
        Workload("h2048_s2048_w512", batch=4, seq=2048, hidden=2048, heads=16,
                 head_dim=128, ffn=8192, window=512, seed=1002),
        Workload("gpt175b_tp8_share_s2048", batch=1, seq=2048, hidden=12288,
                 heads=12, head_dim=128, ffn=6144, window=2048, seed=1003),
        Workload("long_h4096_s8192_w1024", batch=1, seq=8192, hidden=4096,
                 heads=32, head_dim=128, ffn=16384, window=1024, seed=1004),
        Workload("stack2_h5120_s4096", batch=2, seq=4096, hidden=5120,
                 heads=40, head_dim=128, ffn=20480, window=4096, layers=2,
                 seed=1005),
    ]
}
WORKLOAD_ORDER: List[str] = list(WORKLOADS)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round-to-nearest-even) and return the bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    # finite inputs only: the largest finite pattern plus 0x8000 stays < 2^32
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bits to fp32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


def _normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return f32_to_bf16_bits(a)


def make_inputs(w: Workload, seed: int | None = None,
                random_ln: bool = False) -> dict:
    """Draw every input of ``w.layers`` stacked PTB layers as bf16 bits.

    Returns a dict with ``x [T,h]``, ``dy [T,h]`` and a list ``layers`` of dicts
    holding ``ln_gamma [h]``, ``ln_beta [h]``, ``w_qkv [h, 3*h_l]``,
    ``w_o [h_l, h]``, ``w_fc1 [h, f]`` (``[h, 2f]`` for SwiGLU),
    ``w_fc2 [f, h]`` and the serial block's
    ``ln2_gamma [h]``, ``ln2_beta [h]`` (all ``uint16``).
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    T, h, hl, f = w.tokens, w.hidden, w.h_local, w.ffn
    out = {"x": _normal_bf16(rng, (T, h), 1.0)}
    layers = []
    for _ in range(w.layers):
        layers.append({
            "w_qkv": _normal_bf16(rng, (h, 3 * hl), 0.02),
            "w_o": _normal_bf16(rng, (hl, h), 0.02),
            "w_fc1": _normal_bf16(rng, (h, w.fc1_width), 0.02),
            "w_fc2": _normal_bf16(rng, (f, h), 0.02),
        })
    out["dy"] = _normal_bf16(rng, (T, h), 1.0)
    one = f32_to_bf16_bits(np.ones(h, np.float32))
    zero = f32_to_bf16_bits(np.zeros(h, np.float32))
    for pre in ("ln", "ln2"):
        for lay in layers:
            if random_ln:
                g = 1.0 + 0.1 * rng.standard_normal(size=h, dtype=np.float32)
                b = 0.1 * rng.standard_normal(size=h, dtype=np.float32)
                lay[pre + "_gamma"] = f32_to_bf16_bits(g)
                lay[pre + "_beta"] = f32_to_bf16_bits(b)
            else:
                lay[pre + "_gamma"] = one.copy()
                lay[pre + "_beta"] = zero.copy()
    out["layers"] = layers
    return out
