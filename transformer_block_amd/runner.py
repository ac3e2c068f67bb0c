"""Device buffers for a stack of PTB layers and the calls that run it.

Plumbing only: torch allocates device memory and provides the stream; every
step of the layer runs in libptb through ``transformer_block_amd.ptb``.
"""
from __future__ import annotations

from typing import Dict, List

import numpy as np
import torch

from . import ptb as P
from .inputs import Workload

PARAM_NAMES = ("ln_gamma", "ln_beta", "w_qkv", "w_o", "w_fc1", "w_fc2")
GRAD_NAMES = ("d_ln_gamma", "d_ln_beta", "dw_qkv", "dw_o", "dw_fc1", "dw_fc2")


def to_device_bf16(bits: np.ndarray, device) -> torch.Tensor:
    """uint16 bf16 bits (numpy) -> torch.bfloat16 tensor on `device`."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def bf16_to_numpy_f64(t: torch.Tensor) -> np.ndarray:
    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class LayerStack:
    """`w.layers` PTB layers applied in sequence, forward then backward."""

    def __init__(self, w: Workload, inputs: dict, device: str = "cuda"):
        self.w = w
        self.dims = P.dims_of(w)
        # per-layer dims: the layer index picks the layer's dropout masks
        self.layer_dims = [P.dims_of(w, li) for li in range(w.layers)]
        self.device = torch.device(device)
        dev = self.device
        self.x = to_device_bf16(inputs["x"], dev)
        self.dy = to_device_bf16(inputs["dy"], dev)
        self.params: List[Dict[str, torch.Tensor]] = [
            {k: to_device_bf16(lay[k], dev) for k in PARAM_NAMES} for lay in inputs["layers"]]
        nsaved = P.ptb_saved_bytes(self.dims)
        nwork = P.ptb_workspace_bytes(self.dims)
        self.saved = [torch.empty(nsaved, dtype=torch.uint8, device=dev) for _ in self.params]
        self.workspace = torch.empty(nwork, dtype=torch.uint8, device=dev)
        self.ys = [torch.empty_like(self.x) for _ in self.params]
        self.dxs = [torch.empty_like(self.x) for _ in self.params]
        self.grads: List[Dict[str, torch.Tensor]] = []
        for p in self.params:
            self.grads.append({
                "d_ln_gamma": torch.empty_like(p["ln_gamma"]),
                "d_ln_beta": torch.empty_like(p["ln_beta"]),
                "dw_qkv": torch.empty_like(p["w_qkv"]),
                "dw_o": torch.empty_like(p["w_o"]),
                "dw_fc1": torch.empty_like(p["w_fc1"]),
                "dw_fc2": torch.empty_like(p["w_fc2"]),
            })

    @property
    def y(self) -> torch.Tensor:
        return self.ys[-1]

    @property
    def dx(self) -> torch.Tensor:
        return self.dxs[0]

    def layer_input(self, li: int) -> torch.Tensor:
        return self.x if li == 0 else self.ys[li - 1]

    def forward(self, stream=None, events=None) -> None:
        """events: optional per-layer lists of 2*PTB_FWD_STAGES hipEvent_t handles."""
        for li, p in enumerate(self.params):
            P.ptb_forward_timed(self.layer_dims[li], self.layer_input(li), p["ln_gamma"], p["ln_beta"],
                                p["w_qkv"], p["w_o"], p["w_fc1"], p["w_fc2"], self.ys[li],
                                self.saved[li], self.workspace, stream,
                                events[li] if events else None)

    def backward(self, stream=None, events=None) -> None:
        """events: optional per-layer lists of 2*PTB_BWD_STAGES hipEvent_t handles."""
        g = self.dy
        for li in range(len(self.params) - 1, -1, -1):
            p, gr = self.params[li], self.grads[li]
            P.ptb_backward_timed(self.layer_dims[li], g, self.layer_input(li), p["ln_gamma"],
                                 p["w_qkv"],
                                 p["w_o"], p["w_fc1"], p["w_fc2"], self.saved[li], self.dxs[li],
                                 gr["d_ln_gamma"], gr["d_ln_beta"], gr["dw_qkv"], gr["dw_o"],
                                 gr["dw_fc1"], gr["dw_fc2"], self.workspace, stream,
                                 events[li] if events else None)
            g = self.dxs[li]

    def step(self, stream=None, fwd_events=None, bwd_events=None) -> None:
        self.forward(stream, fwd_events)
        self.backward(stream, bwd_events)

    def saved_tensor(self, li: int, name: str) -> torch.Tensor:
        """A view of one stashed tensor of layer `li` (see ptb_saved_layout)."""
        w = self.w
        T, h, hl, f = w.tokens, w.hidden, w.h_local, w.ffn
        shapes = {"a": ((T, h), torch.bfloat16), "mu": ((T,), torch.float32),
                  "rstd": ((T,), torch.float32), "qkv": ((T, 3 * hl), torch.bfloat16),
                  "u": ((T, w.fc1_width), torch.bfloat16), "g": ((T, f), torch.bfloat16),
                  "c": ((T, hl), torch.bfloat16),
                  "lse": ((w.batch, w.heads, w.seq), torch.float32),
                  "a16": ((T, h), torch.float16), "qk16": ((T, 2 * hl), torch.float16)}
        off = P.ptb_saved_layout(self.dims)[name]
        shape, dt = shapes[name]
        nbytes = int(np.prod(shape)) * (4 if dt == torch.float32 else 2)
        return self.saved[li][off:off + nbytes].view(dt).view(shape)


class SerialBlock:
    """One serial (standard) block, the comparison point of the parallel one
    (include/ptb.h, ptb_serial_*): LN1 and LN2 take `ln_*` and `ln2_*` of the
    inputs' first layer."""

    def __init__(self, w: Workload, inputs: dict, device: str = "cuda"):
        if w.layers != 1:
            raise ValueError("SerialBlock runs one block")
        self.w = w
        self.dims = P.dims_of(w)
        dev = torch.device(device)
        self.x = to_device_bf16(inputs["x"], dev)
        self.dy = to_device_bf16(inputs["dy"], dev)
        lay = inputs["layers"][0]
        self.p = {k: to_device_bf16(lay[k], dev) for k in PARAM_NAMES + ("ln2_gamma", "ln2_beta")}
        self.saved = torch.empty(P.ptb_serial_saved_bytes(self.dims), dtype=torch.uint8, device=dev)
        self.workspace = torch.empty(P.ptb_serial_workspace_bytes(self.dims), dtype=torch.uint8,
                                     device=dev)
        self.y = torch.empty_like(self.x)
        self.dx = torch.empty_like(self.x)
        p = self.p
        self.grads = {"d_ln_gamma": torch.empty_like(p["ln_gamma"]),
                      "d_ln_beta": torch.empty_like(p["ln_beta"]),
                      "d_ln2_gamma": torch.empty_like(p["ln2_gamma"]),
                      "d_ln2_beta": torch.empty_like(p["ln2_beta"]),
                      "dw_qkv": torch.empty_like(p["w_qkv"]), "dw_o": torch.empty_like(p["w_o"]),
                      "dw_fc1": torch.empty_like(p["w_fc1"]),
                      "dw_fc2": torch.empty_like(p["w_fc2"])}

    def forward(self, stream=None, events=None) -> None:
        p = self.p
        P.ptb_serial_forward_timed(self.dims, self.x, p["ln_gamma"], p["ln_beta"], p["ln2_gamma"],
                                   p["ln2_beta"], p["w_qkv"], p["w_o"], p["w_fc1"], p["w_fc2"],
                                   self.y, self.saved, self.workspace, stream, events)

    def backward(self, stream=None, events=None) -> None:
        p, g = self.p, self.grads
        P.ptb_serial_backward_timed(self.dims, self.dy, self.x, p["ln_gamma"], p["ln2_gamma"],
                                    p["w_qkv"], p["w_o"], p["w_fc1"], p["w_fc2"], self.saved,
                                    self.dx, g["d_ln_gamma"], g["d_ln_beta"], g["d_ln2_gamma"],
                                    g["d_ln2_beta"], g["dw_qkv"], g["dw_o"], g["dw_fc1"],
                                    g["dw_fc2"], self.workspace, stream, events)

    def step(self, stream=None, fwd_events=None, bwd_events=None) -> None:
        self.forward(stream, fwd_events)
        self.backward(stream, bwd_events)

    def saved_tensor(self, name: str) -> torch.Tensor:
        """A view of one stashed tensor (see ptb_serial_saved_layout)."""
        w = self.w
        T, h, hl, f = w.tokens, w.hidden, w.h_local, w.ffn
        bf, f32 = torch.bfloat16, torch.float32
        shapes = {"a1": ((T, h), bf), "mu1": ((T,), f32), "rstd1": ((T,), f32),
                  "a1_16": ((T, h), torch.float16), "qkv": ((T, 3 * hl), bf),
                  "qk16": ((T, 2 * hl), torch.float16),
                  "c": ((T, hl), bf), "lse": ((w.batch, w.heads, w.seq), f32),
                  "x1": ((T, h), bf), "a2": ((T, h), bf), "mu2": ((T,), f32),
                  "rstd2": ((T,), f32), "u": ((T, w.fc1_width), bf), "g": ((T, f), bf)}
        off = P.ptb_serial_saved_layout(self.dims)[name]
        shape, dt = shapes[name]
        nbytes = int(np.prod(shape)) * (4 if dt == f32 else 2)
        return self.saved[off:off + nbytes].view(dt).view(shape)


class Fp8Layer:
    """One parallel block with its four GEMM parts in FP8 (include/ptb.h,
    ptb_fp8_*), scaled by `recipe`: "current" (one scale per operand) or "mx"
    (block scales).  A step is the weight cast, the forward and the backward:
    the weights change at every optimizer step, so their FP8 copies do too."""

    def __init__(self, w: Workload, inputs: dict, device: str = "cuda", recipe: str = "current"):
        if w.layers != 1:
            raise ValueError("Fp8Layer runs one layer")
        self.w = w
        self.recipe = recipe
        self.dims = P.dims_of(w)
        dev = torch.device(device)
        self.x = to_device_bf16(inputs["x"], dev)
        self.dy = to_device_bf16(inputs["dy"], dev)
        lay = inputs["layers"][0]
        self.p = {k: to_device_bf16(lay[k], dev) for k in PARAM_NAMES}
        self.fp8_weights = torch.empty(P.ptb_fp8_weights_bytes(self.dims, recipe),
                                       dtype=torch.uint8, device=dev)
        self.saved = torch.empty(P.ptb_fp8_saved_bytes(self.dims, recipe), dtype=torch.uint8,
                                 device=dev)
        self.workspace = torch.empty(P.ptb_fp8_workspace_bytes(self.dims, recipe),
                                     dtype=torch.uint8, device=dev)
        self.y = torch.empty_like(self.x)
        self.dx = torch.empty_like(self.x)
        p = self.p
        self.grads = {"d_ln_gamma": torch.empty_like(p["ln_gamma"]),
                      "d_ln_beta": torch.empty_like(p["ln_beta"]),
                      "dw_qkv": torch.empty_like(p["w_qkv"]), "dw_o": torch.empty_like(p["w_o"]),
                      "dw_fc1": torch.empty_like(p["w_fc1"]),
                      "dw_fc2": torch.empty_like(p["w_fc2"])}

    def cast_weights(self, stream=None) -> None:
        p = self.p
        P.ptb_fp8_cast_weights(self.dims, p["w_qkv"], p["w_o"], p["w_fc1"], p["w_fc2"],
                               self.fp8_weights, stream, recipe=self.recipe)

    def forward(self, stream=None, events=None) -> None:
        p = self.p
        P.ptb_fp8_forward(self.dims, self.x, p["ln_gamma"], p["ln_beta"], self.fp8_weights,
                          self.y, self.saved, self.workspace, stream, events,
                          recipe=self.recipe)

    def backward(self, stream=None, events=None) -> None:
        p, g = self.p, self.grads
        P.ptb_fp8_backward(self.dims, self.dy, self.x, p["ln_gamma"], self.fp8_weights,
                           self.saved, self.dx, g["d_ln_gamma"], g["d_ln_beta"], g["dw_qkv"],
                           g["dw_o"], g["dw_fc1"], g["dw_fc2"], self.workspace, stream, events,
                           recipe=self.recipe)

    def step(self, stream=None, fwd_events=None, bwd_events=None) -> None:
        self.cast_weights(stream)
        self.forward(stream, fwd_events)
        self.backward(stream, bwd_events)

    def saved_tensor(self, name: str) -> torch.Tensor:
        """A view of one stashed tensor (the parallel block's slots)."""
        w = self.w
        T, h, hl, f = w.tokens, w.hidden, w.h_local, w.ffn
        bf, f32 = torch.bfloat16, torch.float32
        shapes = {"a": ((T, h), bf), "mu": ((T,), f32), "rstd": ((T,), f32),
                  "qkv": ((T, 3 * hl), bf), "qk16": ((T, 2 * hl), torch.float16),
                  "c": ((T, hl), bf),
                  "lse": ((w.batch, w.heads, w.seq), f32), "u": ((T, f), bf), "g": ((T, f), bf)}
        off = P.ptb_saved_layout(self.dims)[name]
        shape, dt = shapes[name]
        nbytes = int(np.prod(shape)) * (4 if dt == f32 else 2)
        return self.saved[off:off + nbytes].view(dt).view(shape)
