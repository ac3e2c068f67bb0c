"""Model-FLOP accounting for the PTB layer (closed form).

The FLOP model follows the Megatron tuning post ("Megatron-LM 分布式训练（七）：
显存与性能调优", MFU section): 6 FLOPs per parameter per token (2 forward,
4 backward) for the matrix products plus the attention term that grows with the
square of the sequence; the recomputed forward of the core attention is not
model work (it counts toward HFU only).

Made exact for sliding-window attention (MegaScale reading notes, section 1.1,
eq (5)-(6): only pairs inside the window are computed):

    pairs(s, w) = s*w - w*(w-1)/2   if w <= s,   s*(s+1)/2 otherwise
    P           = h * (4*h_l + 2*f)          matmul weights per layer
                  (h * (4*h_l + 3*f) with the SwiGLU MLP)
    F_model     = L * (6*T*P + 12*b*n*d*pairs(s, w))
    F_recompute = L * 2*b*n*d*pairs(s, w)    (QK^T again in backward)
"""
from __future__ import annotations


def window_pairs(s: int, w: int) -> int:
    """(query, key) pairs with 0 <= i - j < w inside one length-s sequence."""
    if w >= s:
        return s * (s + 1) // 2
    return s * w - w * (w - 1) // 2


def matmul_params(hidden: int, heads: int, head_dim: int, ffn: int, mlp: str = "gelu") -> int:
    """Matmul weights of one layer: QKV and O (4 h h_l) plus the MLP, 2 h f
    for GeLU (W_fc1, W_fc2) and 3 h f for SwiGLU (W1, W3, W2)."""
    hl = heads * head_dim
    return hidden * (4 * hl + (3 if mlp == "swiglu" else 2) * ffn)


def model_flops(batch: int, seq: int, hidden: int, heads: int, head_dim: int,
                ffn: int, window: int, layers: int = 1, mlp: str = "gelu") -> int:
    T = batch * seq
    P = matmul_params(hidden, heads, head_dim, ffn, mlp)
    return layers * (6 * T * P
                     + 12 * batch * heads * head_dim * window_pairs(seq, window))


def recompute_flops(batch: int, seq: int, heads: int, head_dim: int,
                    window: int, layers: int = 1) -> int:
    return layers * 2 * batch * heads * head_dim * window_pairs(seq, window)


def workload_model_flops(w) -> int:
    return model_flops(w.batch, w.seq, w.hidden, w.heads, w.head_dim, w.ffn,
                       w.window, w.layers, getattr(w, "mlp", "gelu"))


def workload_recompute_flops(w) -> int:
    return recompute_flops(w.batch, w.seq, w.heads, w.head_dim, w.window,
                           w.layers)
