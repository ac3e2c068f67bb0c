"""Thin ctypes binding of libptb (C ABI in include/ptb.h).

Argument marshalling only: tensors are passed as raw device pointers
(``tensor.data_ptr()``), the stream as the HIP stream handle of a
``torch.cuda.Stream`` (torch's current stream by default).  Every step of the
layer runs inside libptb's HIP kernels; nothing here computes, and there is no
fallback: if the library is missing, loading fails loudly.

The functions carry the C names.  A non-zero status raises ``PtbError`` unless
``check=False`` is passed, in which case the status code is returned.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libptb.so")

PTB_OK = 0
PTB_ERR_NULL = -1
PTB_ERR_DIMS = -2
PTB_ERR_HEAD_DIM = -3
PTB_ERR_ALIGN = -4
PTB_ERR_WINDOW = -5
PTB_ERR_EPS = -6
PTB_ERR_HIP = -7
PTB_ERR_ARG = -8
PTB_ERR_SCRATCH = -9
PTB_LAMB_MAX_TENSORS = 32
PTB_LAMB_NOALLOC_SCRATCH_BYTES = 4 << 20

SAVED_SLOTS = ("a", "mu", "rstd", "qkv", "u", "g", "c", "lse", "a16", "qk16")
SERIAL_SAVED_SLOTS = ("a1", "mu1", "rstd1", "a1_16", "qkv", "qk16", "c", "lse", "x1", "a2",
                      "mu2", "rstd2", "u", "g")


class PtbError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where} failed: status {status} ({ptb_status_string(status)})")
        self.status = status


class ptb_dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("window", ctypes.c_int32), ("ln_eps", ctypes.c_float),
                ("norm", ctypes.c_int32), ("mlp", ctypes.c_int32),
                ("dropout_p", ctypes.c_float), ("dropout_layer", ctypes.c_uint32),
                ("dropout_seed", ctypes.c_uint64)]


PTB_NORM_LAYERNORM, PTB_NORM_RMSNORM = 0, 1
PTB_MLP_GELU, PTB_MLP_SWIGLU = 0, 1
NORM_KINDS = {"layernorm": PTB_NORM_LAYERNORM, "rmsnorm": PTB_NORM_RMSNORM}
MLP_KINDS = {"gelu": PTB_MLP_GELU, "swiglu": PTB_MLP_SWIGLU}


def dims_of(w, layer: int = 0) -> ptb_dims:
    """ptb_dims of a Workload (transformer_block_amd.inputs) for layer `layer`
    (which picks the layer's dropout masks)."""
    return ptb_dims(w.batch, w.seq, w.hidden, w.heads, w.head_dim, w.ffn, w.window,
                    w.ln_eps, NORM_KINDS[w.norm], MLP_KINDS[w.mlp], w.dropout_p, layer,
                    w.dropout_seed)


class ptb_lamb_hyper(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("step", ctypes.c_int32)]


class ptb_lamb_tensor(ctypes.Structure):
    _fields_ = [("theta", ctypes.c_void_p), ("m", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("grad", ctypes.c_void_p), ("weight", ctypes.c_void_p),
                ("numel", ctypes.c_int64)]


_lib: Optional[ctypes.CDLL] = None
_P = ctypes.c_void_p
_D = ctypes.POINTER(ptb_dims)
_I = ctypes.c_int32


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libptb.so (built by transformer_block_amd.build) once."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"libptb.so not found at {path}: build it first with "
            "`python -m transformer_block_amd.build` (or __graft_entry__.build())")
    # torch ships its own HIP runtime with the same soname; loading torch first
    # makes libptb bind to that one copy, so torch's streams and memory are
    # valid handles inside libptb (two runtimes in one process would not share
    # them).
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    sig = {
        "ptb_abi_version": (ctypes.c_int32, []),
        "ptb_status_string": (ctypes.c_char_p, [ctypes.c_int32]),
        "ptb_validate_dims": (ctypes.c_int32, [_D]),
        "ptb_saved_bytes": (ctypes.c_int32, [_D, ctypes.POINTER(ctypes.c_size_t)]),
        "ptb_workspace_bytes": (ctypes.c_int32, [_D, ctypes.POINTER(ctypes.c_size_t)]),
        "ptb_saved_layout": (ctypes.c_int32, [_D, ctypes.POINTER(ctypes.c_size_t)]),
        "ptb_forward": (ctypes.c_int32, [_D] + [_P] * 11),
        "ptb_backward": (ctypes.c_int32, [_D] + [_P] * 17),
        "ptb_forward_timed": (ctypes.c_int32, [_D] + [_P] * 12),
        "ptb_backward_timed": (ctypes.c_int32, [_D] + [_P] * 18),
        "ptb_serial_saved_bytes": (ctypes.c_int32, [_D, ctypes.POINTER(ctypes.c_size_t)]),
        "ptb_serial_workspace_bytes": (ctypes.c_int32, [_D, ctypes.POINTER(ctypes.c_size_t)]),
        "ptb_serial_saved_layout": (ctypes.c_int32, [_D, ctypes.POINTER(ctypes.c_size_t)]),
        "ptb_serial_forward": (ctypes.c_int32, [_D] + [_P] * 13),
        "ptb_serial_backward": (ctypes.c_int32, [_D] + [_P] * 20),
        "ptb_serial_forward_timed": (ctypes.c_int32, [_D] + [_P] * 14),
        "ptb_serial_backward_timed": (ctypes.c_int32, [_D] + [_P] * 21),
        "ptb_lamb_workspace_bytes": (ctypes.c_int32, [ctypes.POINTER(ptb_lamb_tensor),
                                                      ctypes.c_int32,
                                                      ctypes.POINTER(ctypes.c_size_t)]),
        "ptb_lamb_step": (ctypes.c_int32, [ctypes.POINTER(ptb_lamb_hyper),
                                           ctypes.POINTER(ptb_lamb_tensor), ctypes.c_int32,
                                           _P, _P, _P]),
        "ptb_lamb_step_noalloc": (ctypes.c_int32, [ctypes.POINTER(ptb_lamb_hyper),
                                                   ctypes.POINTER(ptb_lamb_tensor),
                                                   ctypes.c_int32, _P, _P]),
        "ptb_dropout_mask": (ctypes.c_int32, [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_float,
                                              ctypes.c_int64, _P, _P]),
        "ptb_fp8_weights_bytes": (ctypes.c_int32, [_D, _I, ctypes.POINTER(ctypes.c_size_t)]),
        "ptb_fp8_weights_layout": (ctypes.c_int32, [_D, _I, ctypes.POINTER(ctypes.c_size_t)]),
        "ptb_fp8_quantize": (ctypes.c_int32, [_P, _I, _I, _I, _P, _P, _P, _P]),
        "ptb_fp8_quantize_mx": (ctypes.c_int32, [_P, _I, _I, _I, _P, _P, _P, _P, _P]),
        "ptb_fp8_workspace_bytes": (ctypes.c_int32, [_D, _I, ctypes.POINTER(ctypes.c_size_t)]),
        "ptb_fp8_saved_bytes": (ctypes.c_int32, [_D, _I, ctypes.POINTER(ctypes.c_size_t)]),
        "ptb_fp8_cast_weights": (ctypes.c_int32, [_D, _I] + [_P] * 6),
        "ptb_fp8_forward": (ctypes.c_int32, [_D, _I] + [_P] * 9),
        "ptb_fp8_backward": (ctypes.c_int32, [_D, _I] + [_P] * 15),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _done(status: int, where: str, check: bool) -> int:
    if check and status != PTB_OK:
        raise PtbError(status, where)
    return status


def ptb_abi_version() -> int:
    return load_library().ptb_abi_version()


def ptb_status_string(status: int) -> str:
    return load_library().ptb_status_string(status).decode()


def ptb_validate_dims(dims: ptb_dims) -> int:
    return load_library().ptb_validate_dims(ctypes.byref(dims) if dims is not None else None)


def ptb_saved_bytes(dims: ptb_dims) -> int:
    n = ctypes.c_size_t(0)
    _done(load_library().ptb_saved_bytes(ctypes.byref(dims), ctypes.byref(n)),
          "ptb_saved_bytes", True)
    return n.value


def ptb_workspace_bytes(dims: ptb_dims) -> int:
    n = ctypes.c_size_t(0)
    _done(load_library().ptb_workspace_bytes(ctypes.byref(dims), ctypes.byref(n)),
          "ptb_workspace_bytes", True)
    return n.value


def ptb_saved_layout(dims: ptb_dims) -> dict:
    arr = (ctypes.c_size_t * len(SAVED_SLOTS))()
    _done(load_library().ptb_saved_layout(ctypes.byref(dims), arr), "ptb_saved_layout", True)
    return dict(zip(SAVED_SLOTS, list(arr)))


def ptb_forward(dims: ptb_dims, x, ln_gamma, ln_beta, w_qkv, w_o, w_fc1, w_fc2, y,
                saved, workspace, stream=None, check: bool = True) -> int:
    st = load_library().ptb_forward(
        ctypes.byref(dims), _ptr(x), _ptr(ln_gamma), _ptr(ln_beta), _ptr(w_qkv), _ptr(w_o),
        _ptr(w_fc1), _ptr(w_fc2), _ptr(y), _ptr(saved), _ptr(workspace), _stream(stream))
    return _done(st, "ptb_forward", check)


def ptb_backward(dims: ptb_dims, dy, x, ln_gamma, w_qkv, w_o, w_fc1, w_fc2, saved, dx,
                 d_ln_gamma, d_ln_beta, dw_qkv, dw_o, dw_fc1, dw_fc2, workspace,
                 stream=None, check: bool = True) -> int:
    st = load_library().ptb_backward(
        ctypes.byref(dims), _ptr(dy), _ptr(x), _ptr(ln_gamma), _ptr(w_qkv), _ptr(w_o),
        _ptr(w_fc1), _ptr(w_fc2), _ptr(saved), _ptr(dx), _ptr(d_ln_gamma), _ptr(d_ln_beta),
        _ptr(dw_qkv), _ptr(dw_o), _ptr(dw_fc1), _ptr(dw_fc2), _ptr(workspace),
        _stream(stream))
    return _done(st, "ptb_backward", check)


PTB_FWD_STAGES = 5
PTB_BWD_STAGES = 6
FWD_STAGE_NAMES = ("layernorm_fwd", "cast_wqk_f16", "gemm_qkv_fc1", "attention_fwd",
                   "gemm_o_fc2_residual")
BWD_STAGE_NAMES = ("gemm_dgrad_o_fc2", "attention_bwd", "gemm_wgrad_o_fc2",
                   "gemm_dgrad_qkv_fc1", "gemm_wgrad_qkv_fc1", "layernorm_bwd")


def _events(stage_events) -> Optional[ctypes.Array]:
    if stage_events is None:
        return None
    arr = (ctypes.c_void_p * len(stage_events))()
    for i, e in enumerate(stage_events):
        arr[i] = e
    return arr


def ptb_forward_timed(dims: ptb_dims, x, ln_gamma, ln_beta, w_qkv, w_o, w_fc1, w_fc2, y,
                      saved, workspace, stream, stage_events, check: bool = True) -> int:
    """ptb_forward plus raw hipEvent_t handles (2 per stage) recorded around
    each stage on `stream`."""
    st = load_library().ptb_forward_timed(
        ctypes.byref(dims), _ptr(x), _ptr(ln_gamma), _ptr(ln_beta), _ptr(w_qkv), _ptr(w_o),
        _ptr(w_fc1), _ptr(w_fc2), _ptr(y), _ptr(saved), _ptr(workspace), _stream(stream),
        _events(stage_events))
    return _done(st, "ptb_forward_timed", check)


def ptb_backward_timed(dims: ptb_dims, dy, x, ln_gamma, w_qkv, w_o, w_fc1, w_fc2, saved, dx,
                       d_ln_gamma, d_ln_beta, dw_qkv, dw_o, dw_fc1, dw_fc2, workspace,
                       stream, stage_events, check: bool = True) -> int:
    st = load_library().ptb_backward_timed(
        ctypes.byref(dims), _ptr(dy), _ptr(x), _ptr(ln_gamma), _ptr(w_qkv), _ptr(w_o),
        _ptr(w_fc1), _ptr(w_fc2), _ptr(saved), _ptr(dx), _ptr(d_ln_gamma), _ptr(d_ln_beta),
        _ptr(dw_qkv), _ptr(dw_o), _ptr(dw_fc1), _ptr(dw_fc2), _ptr(workspace),
        _stream(stream), _events(stage_events))
    return _done(st, "ptb_backward_timed", check)


# ---- serial (standard) block, for comparison: see include/ptb.h
PTB_SERIAL_FWD_STAGES = 8
PTB_SERIAL_BWD_STAGES = 11
SERIAL_FWD_STAGE_NAMES = ("layernorm1_fwd", "cast_wqk_f16", "gemm_qkv", "attention_fwd",
                          "gemm_o_residual",
                          "layernorm2_fwd", "gemm_fc1_gelu", "gemm_fc2_residual")
SERIAL_BWD_STAGE_NAMES = ("gemm_dgrad_fc2", "gemm_wgrad_fc2", "gemm_dgrad_fc1",
                          "gemm_wgrad_fc1", "layernorm2_bwd", "gemm_dgrad_o", "gemm_wgrad_o",
                          "attention_bwd", "gemm_dgrad_qkv", "gemm_wgrad_qkv",
                          "layernorm1_bwd")


def ptb_serial_saved_bytes(dims: ptb_dims) -> int:
    n = ctypes.c_size_t(0)
    _done(load_library().ptb_serial_saved_bytes(ctypes.byref(dims), ctypes.byref(n)),
          "ptb_serial_saved_bytes", True)
    return n.value


def ptb_serial_workspace_bytes(dims: ptb_dims) -> int:
    n = ctypes.c_size_t(0)
    _done(load_library().ptb_serial_workspace_bytes(ctypes.byref(dims), ctypes.byref(n)),
          "ptb_serial_workspace_bytes", True)
    return n.value


def ptb_serial_saved_layout(dims: ptb_dims) -> dict:
    arr = (ctypes.c_size_t * len(SERIAL_SAVED_SLOTS))()
    _done(load_library().ptb_serial_saved_layout(ctypes.byref(dims), arr),
          "ptb_serial_saved_layout", True)
    return dict(zip(SERIAL_SAVED_SLOTS, list(arr)))


def ptb_serial_forward(dims: ptb_dims, x, ln1_gamma, ln1_beta, ln2_gamma, ln2_beta, w_qkv,
                       w_o, w_fc1, w_fc2, y, saved, workspace, stream=None,
                       check: bool = True) -> int:
    st = load_library().ptb_serial_forward(
        ctypes.byref(dims), _ptr(x), _ptr(ln1_gamma), _ptr(ln1_beta), _ptr(ln2_gamma),
        _ptr(ln2_beta), _ptr(w_qkv), _ptr(w_o), _ptr(w_fc1), _ptr(w_fc2), _ptr(y), _ptr(saved),
        _ptr(workspace), _stream(stream))
    return _done(st, "ptb_serial_forward", check)


def ptb_serial_backward(dims: ptb_dims, dy, x, ln1_gamma, ln2_gamma, w_qkv, w_o, w_fc1, w_fc2,
                        saved, dx, d_ln1_gamma, d_ln1_beta, d_ln2_gamma, d_ln2_beta, dw_qkv,
                        dw_o, dw_fc1, dw_fc2, workspace, stream=None,
                        check: bool = True) -> int:
    st = load_library().ptb_serial_backward(
        ctypes.byref(dims), _ptr(dy), _ptr(x), _ptr(ln1_gamma), _ptr(ln2_gamma), _ptr(w_qkv),
        _ptr(w_o), _ptr(w_fc1), _ptr(w_fc2), _ptr(saved), _ptr(dx), _ptr(d_ln1_gamma),
        _ptr(d_ln1_beta), _ptr(d_ln2_gamma), _ptr(d_ln2_beta), _ptr(dw_qkv), _ptr(dw_o),
        _ptr(dw_fc1), _ptr(dw_fc2), _ptr(workspace), _stream(stream))
    return _done(st, "ptb_serial_backward", check)


def ptb_serial_forward_timed(dims: ptb_dims, x, ln1_gamma, ln1_beta, ln2_gamma, ln2_beta,
                             w_qkv, w_o, w_fc1, w_fc2, y, saved, workspace, stream,
                             stage_events, check: bool = True) -> int:
    st = load_library().ptb_serial_forward_timed(
        ctypes.byref(dims), _ptr(x), _ptr(ln1_gamma), _ptr(ln1_beta), _ptr(ln2_gamma),
        _ptr(ln2_beta), _ptr(w_qkv), _ptr(w_o), _ptr(w_fc1), _ptr(w_fc2), _ptr(y), _ptr(saved),
        _ptr(workspace), _stream(stream), _events(stage_events))
    return _done(st, "ptb_serial_forward_timed", check)


def ptb_serial_backward_timed(dims: ptb_dims, dy, x, ln1_gamma, ln2_gamma, w_qkv, w_o, w_fc1,
                              w_fc2, saved, dx, d_ln1_gamma, d_ln1_beta, d_ln2_gamma,
                              d_ln2_beta, dw_qkv, dw_o, dw_fc1, dw_fc2, workspace, stream,
                              stage_events, check: bool = True) -> int:
    st = load_library().ptb_serial_backward_timed(
        ctypes.byref(dims), _ptr(dy), _ptr(x), _ptr(ln1_gamma), _ptr(ln2_gamma), _ptr(w_qkv),
        _ptr(w_o), _ptr(w_fc1), _ptr(w_fc2), _ptr(saved), _ptr(dx), _ptr(d_ln1_gamma),
        _ptr(d_ln1_beta), _ptr(d_ln2_gamma), _ptr(d_ln2_beta), _ptr(dw_qkv), _ptr(dw_o),
        _ptr(dw_fc1), _ptr(dw_fc2), _ptr(workspace), _stream(stream), _events(stage_events))
    return _done(st, "ptb_serial_backward_timed", check)


# ---- LAMB optimizer step: see include/ptb.h
def lamb_tensor_list(tensors) -> ctypes.Array:
    """ptb_lamb_tensor array from (theta, m, v, grad, weight) tuples of
    tensors (or raw addresses plus a numel: (theta, m, v, grad, weight, numel))."""
    arr = (ptb_lamb_tensor * len(tensors))()
    for i, t in enumerate(tensors):
        numel = t[5] if len(t) > 5 else t[0].numel()
        arr[i] = ptb_lamb_tensor(*(_ptr(x) for x in t[:5]), numel)
    return arr


def ptb_lamb_workspace_bytes(tensors) -> int:
    arr = lamb_tensor_list(tensors)
    n = ctypes.c_size_t(0)
    _done(load_library().ptb_lamb_workspace_bytes(arr, len(arr), ctypes.byref(n)),
          "ptb_lamb_workspace_bytes", True)
    return n.value


def ptb_lamb_step(hyper: ptb_lamb_hyper, tensors, norms, workspace, stream=None,
                  check: bool = True) -> int:
    """tensors: (theta, m, v, grad, weight) per parameter tensor."""
    arr = lamb_tensor_list(tensors)
    st = load_library().ptb_lamb_step(ctypes.byref(hyper), arr, len(arr), _ptr(norms),
                                      _ptr(workspace), _stream(stream))
    return _done(st, "ptb_lamb_step", check)


def ptb_lamb_step_noalloc(hyper: ptb_lamb_hyper, tensors, norms, stream=None,
                          check: bool = True) -> int:
    """ptb_lamb_step with the library's static scratch instead of a workspace."""
    arr = lamb_tensor_list(tensors)
    st = load_library().ptb_lamb_step_noalloc(ctypes.byref(hyper), arr, len(arr), _ptr(norms),
                                              _stream(stream))
    return _done(st, "ptb_lamb_step_noalloc", check)


# ---- dropout masks: see include/ptb.h
def ptb_dropout_mask(seed: int, stream_id: int, p: float, n: int, mask, stream=None,
                     check: bool = True) -> int:
    """mask: a device uint8 tensor of >= n elements (1 kept, 0 dropped)."""
    st = load_library().ptb_dropout_mask(seed, stream_id, p, n, _ptr(mask), _stream(stream))
    return _done(st, "ptb_dropout_mask", check)


# ---- FP8 GEMM variant: see include/ptb.h
PTB_FP8_FWD_STAGES = 6
PTB_FP8_BWD_STAGES = 8
FP8_FWD_STAGE_NAMES = ("layernorm_fwd", "cast_a", "gemm_qkv_fc1_fp8", "attention_fwd",
                       "cast_cg", "gemm_o_fc2_residual_fp8")
FP8_BWD_STAGE_NAMES = ("cast_dy", "gemm_dgrad_o_fc2_fp8", "attention_bwd",
                       "gemm_wgrad_o_fc2_fp8", "cast_dz", "gemm_dgrad_qkv_fc1_fp8",
                       "gemm_wgrad_qkv_fc1_fp8", "layernorm_bwd")


FP8_RECIPES = {"current": 0, "mx": 1}
FP8_WEIGHT_PARTS = ("amax", "w1t", "w1", "w2t", "w2", "w1t_s", "w1_s", "w2t_s", "w2_s")
FP8_FORMATS = {"e4m3": 0, "e5m2": 1}
FP8_ABSENT = ctypes.c_size_t(-1).value  # offset of a part the recipe does not use


def _size_query(name: str, dims: ptb_dims, recipe: str) -> int:
    n = ctypes.c_size_t(0)
    _done(getattr(load_library(), name)(ctypes.byref(dims), FP8_RECIPES[recipe], ctypes.byref(n)),
          name, True)
    return n.value


def ptb_fp8_weights_bytes(dims: ptb_dims, recipe: str = "current") -> int:
    return _size_query("ptb_fp8_weights_bytes", dims, recipe)


def ptb_fp8_saved_bytes(dims: ptb_dims, recipe: str = "current") -> int:
    return _size_query("ptb_fp8_saved_bytes", dims, recipe)


def ptb_fp8_workspace_bytes(dims: ptb_dims, recipe: str = "current") -> int:
    return _size_query("ptb_fp8_workspace_bytes", dims, recipe)


def ptb_fp8_weights_layout(dims: ptb_dims, recipe: str = "current") -> dict:
    arr = (ctypes.c_size_t * len(FP8_WEIGHT_PARTS))()
    _done(load_library().ptb_fp8_weights_layout(ctypes.byref(dims), FP8_RECIPES[recipe], arr),
          "ptb_fp8_weights_layout", True)
    return dict(zip(FP8_WEIGHT_PARTS, list(arr)))


def ptb_fp8_quantize(x, rows: int, cols: int, fmt: str, amax, q, qt, stream=None,
                     check: bool = True) -> int:
    st = load_library().ptb_fp8_quantize(_ptr(x), rows, cols, FP8_FORMATS[fmt], _ptr(amax),
                                         _ptr(q), _ptr(qt), _stream(stream))
    return _done(st, "ptb_fp8_quantize", check)


def ptb_fp8_quantize_mx(x, rows: int, cols: int, fmt: str, q, q_scales, qt, qt_scales,
                        stream=None, check: bool = True) -> int:
    st = load_library().ptb_fp8_quantize_mx(_ptr(x), rows, cols, FP8_FORMATS[fmt], _ptr(q),
                                            _ptr(q_scales), _ptr(qt), _ptr(qt_scales),
                                            _stream(stream))
    return _done(st, "ptb_fp8_quantize_mx", check)


def ptb_fp8_cast_weights(dims: ptb_dims, w_qkv, w_o, w_fc1, w_fc2, fp8_weights, stream=None,
                         check: bool = True, recipe: str = "current") -> int:
    st = load_library().ptb_fp8_cast_weights(
        ctypes.byref(dims), FP8_RECIPES[recipe], _ptr(w_qkv), _ptr(w_o), _ptr(w_fc1),
        _ptr(w_fc2), _ptr(fp8_weights), _stream(stream))
    return _done(st, "ptb_fp8_cast_weights", check)


def ptb_fp8_forward(dims: ptb_dims, x, ln_gamma, ln_beta, fp8_weights, y, saved, workspace,
                    stream=None, stage_events=None, check: bool = True,
                    recipe: str = "current") -> int:
    st = load_library().ptb_fp8_forward(
        ctypes.byref(dims), FP8_RECIPES[recipe], _ptr(x), _ptr(ln_gamma), _ptr(ln_beta),
        _ptr(fp8_weights), _ptr(y), _ptr(saved), _ptr(workspace), _stream(stream),
        _events(stage_events))
    return _done(st, "ptb_fp8_forward", check)


def ptb_fp8_backward(dims: ptb_dims, dy, x, ln_gamma, fp8_weights, saved, dx, d_ln_gamma,
                     d_ln_beta, dw_qkv, dw_o, dw_fc1, dw_fc2, workspace, stream=None,
                     stage_events=None, check: bool = True, recipe: str = "current") -> int:
    st = load_library().ptb_fp8_backward(
        ctypes.byref(dims), FP8_RECIPES[recipe], _ptr(dy), _ptr(x), _ptr(ln_gamma),
        _ptr(fp8_weights), _ptr(saved), _ptr(dx), _ptr(d_ln_gamma), _ptr(d_ln_beta),
        _ptr(dw_qkv), _ptr(dw_o), _ptr(dw_fc1), _ptr(dw_fc2), _ptr(workspace), _stream(stream),
        _events(stage_events))
    return _done(st, "ptb_fp8_backward", check)


def exported_symbols() -> Sequence[str]:
    return ("ptb_abi_version", "ptb_status_string", "ptb_validate_dims", "ptb_saved_bytes",
            "ptb_workspace_bytes", "ptb_saved_layout", "ptb_forward", "ptb_backward",
            "ptb_forward_timed", "ptb_backward_timed", "ptb_serial_saved_bytes",
            "ptb_serial_workspace_bytes", "ptb_serial_saved_layout", "ptb_serial_forward",
            "ptb_serial_backward", "ptb_serial_forward_timed", "ptb_serial_backward_timed",
            "ptb_lamb_workspace_bytes", "ptb_lamb_step", "ptb_lamb_step_noalloc",
            "ptb_dropout_mask",
            "ptb_fp8_weights_bytes",
            "ptb_fp8_weights_layout", "ptb_fp8_quantize", "ptb_fp8_quantize_mx",
            "ptb_fp8_saved_bytes",
            "ptb_fp8_workspace_bytes", "ptb_fp8_cast_weights", "ptb_fp8_forward",
            "ptb_fp8_backward")
