"""The C-ABI library: it loads, exports every function include/ptb.h declares,
and rejects invalid arguments with the documented status codes before any HIP
call (so these run on a machine without a GPU)."""
import ctypes
import os
import re

import pytest

from transformer_block_amd import ptb as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ptb.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ptb_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(P.LIB_PATH):
        pytest.fail("libptb.so is not built (run __graft_entry__.build())")
    return P.load_library()


def test_library_exports_every_declared_function(lib):
    declared = _declared_functions()
    assert declared, "no declarations parsed from include/ptb.h"
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in ptb.h but not exported"
    assert set(declared) == set(P.exported_symbols())


def test_version_and_status_strings(lib):
    assert P.ptb_abi_version() == 11
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -8, -9):
        assert P.ptb_status_string(code) and P.ptb_status_string(code) != "unknown status"
    assert P.ptb_status_string(12345) == "unknown status"


def good_dims(**kw):
    base = dict(batch=2, seq=256, hidden=256, heads=4, head_dim=64, ffn=1024, window=64,
                ln_eps=1e-5)
    base.update(kw)
    return P.ptb_dims(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(), P.PTB_OK),
    (dict(batch=0), P.PTB_ERR_DIMS),
    (dict(seq=0), P.PTB_ERR_DIMS),
    (dict(heads=0), P.PTB_ERR_DIMS),
    (dict(hidden=100), P.PTB_ERR_DIMS),
    (dict(hidden=32768), P.PTB_ERR_DIMS),
    (dict(ffn=96), P.PTB_ERR_DIMS),
    (dict(head_dim=96), P.PTB_ERR_HEAD_DIM),
    (dict(head_dim=256), P.PTB_ERR_HEAD_DIM),
    (dict(window=0), P.PTB_ERR_WINDOW),
    (dict(window=-3), P.PTB_ERR_WINDOW),
    (dict(ln_eps=0.0), P.PTB_ERR_EPS),
    (dict(ln_eps=float("nan")), P.PTB_ERR_EPS),
    (dict(ln_eps=float("inf")), P.PTB_ERR_EPS),
    (dict(batch=65536, seq=65536), P.PTB_ERR_DIMS),   # T*(3*h_l+f) >= 2^30
    (dict(batch=1024, seq=1024, hidden=1024, ffn=4096), P.PTB_ERR_DIMS),
    (dict(window=1), P.PTB_OK),
    (dict(seq=1, window=10 ** 9), P.PTB_OK),
    (dict(norm=1), P.PTB_OK),
    (dict(mlp=1), P.PTB_OK),
    (dict(norm=1, mlp=1), P.PTB_OK),
    (dict(dropout_p=-0.1), P.PTB_ERR_ARG),
    (dict(dropout_p=1.0), P.PTB_ERR_ARG),
    (dict(dropout_p=float("nan")), P.PTB_ERR_ARG),
    (dict(dropout_layer=2 ** 31), P.PTB_ERR_ARG),
    (dict(dropout_p=0.5, dropout_layer=7, dropout_seed=2 ** 63 + 5), P.PTB_OK),
    (dict(norm=2), P.PTB_ERR_ARG),
    (dict(norm=-1), P.PTB_ERR_ARG),
    (dict(mlp=2), P.PTB_ERR_ARG),
])
def test_validate_dims(lib, kw, code):
    assert P.ptb_validate_dims(good_dims(**kw)) == code


def test_null_dims_pointer(lib):
    assert lib.ptb_validate_dims(None) == P.PTB_ERR_NULL
    n = ctypes.c_size_t(0)
    assert lib.ptb_saved_bytes(None, ctypes.byref(n)) == P.PTB_ERR_NULL
    assert lib.ptb_saved_bytes(ctypes.byref(good_dims()), None) == P.PTB_ERR_NULL


def test_saved_layout_is_ordered_aligned_and_sized(lib):
    d = good_dims()
    lay = P.ptb_saved_layout(d)
    offs = [lay[k] for k in P.SAVED_SLOTS]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    T, h, hl, f = 512, 256, 256, 1024
    sizes = dict(a=T * h * 2, mu=T * 4, rstd=T * 4, qkv=T * 3 * hl * 2, u=T * f * 2,
                 g=T * f * 2, c=T * hl * 2, lse=2 * 4 * 256 * 4, a16=T * h * 2,
                 qk16=T * 2 * hl * 2)
    for a_, b_ in zip(P.SAVED_SLOTS, P.SAVED_SLOTS[1:]):
        assert lay[b_] - lay[a_] >= sizes[a_]
    assert P.ptb_saved_bytes(d) >= lay["qk16"] + sizes["qk16"]
    # split-tile partials (2 fp32 256x256 tiles per workgroup, 256 workgroups)
    # come first, then the backward's dc, dZ and da
    assert P.ptb_workspace_bytes(d) >= 2 * 256 * 256 * 256 * 4 + T * (3 * hl + f) * 2 + T * h * 2
    # the forward's fp16 copy of W_qkv's q, k columns fits in the workspace too
    assert P.ptb_workspace_bytes(d) >= 2 * 256 * 256 * 256 * 4 + h * 2 * hl * 2
    wide = good_dims(batch=1, seq=64, hidden=4096, heads=32, head_dim=128, ffn=64)
    assert P.ptb_workspace_bytes(wide) >= 4096 * 2 * 4096 * 2
    assert P.ptb_serial_workspace_bytes(wide) >= 4096 * 2 * 4096 * 2


def test_forward_backward_reject_null_and_misaligned_before_any_hip_call(lib):
    d = good_dims()
    A = 0x10000  # never dereferenced: the checks fail first
    assert P.ptb_forward(d, *([0] * 10), stream=0, check=False) == P.PTB_ERR_NULL
    assert P.ptb_forward(d, *([A] * 9), None, stream=0, check=False) == P.PTB_ERR_NULL
    args = [A] * 10
    args[4] = A + 8
    assert P.ptb_forward(d, *args, stream=0, check=False) == P.PTB_ERR_ALIGN
    args = [A] * 10
    args[9] = A + 4   # workspace
    assert P.ptb_forward(d, *args, stream=0, check=False) == P.PTB_ERR_ALIGN
    assert P.ptb_backward(d, *([A] * 15), None, stream=0, check=False) == P.PTB_ERR_NULL
    bargs = [A] * 16
    bargs[15] = A + 2
    assert P.ptb_backward(d, *bargs, stream=0, check=False) == P.PTB_ERR_ALIGN
    bad = good_dims(head_dim=32)
    assert P.ptb_forward(bad, *([A] * 10), stream=0, check=False) == P.PTB_ERR_HEAD_DIM
    assert P.ptb_backward(good_dims(window=0), *([A] * 16), stream=0,
                          check=False) == P.PTB_ERR_WINDOW


def test_error_raises_in_checked_mode(lib):
    with pytest.raises(P.PtbError) as ei:
        P.ptb_forward(good_dims(batch=0), *([0x10000] * 10), stream=0)
    assert ei.value.status == P.PTB_ERR_DIMS


def test_serial_saved_layout_is_ordered_aligned_and_sized(lib):
    d = good_dims()
    lay = P.ptb_serial_saved_layout(d)
    offs = [lay[k] for k in P.SERIAL_SAVED_SLOTS]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    T, h, hl, f = 512, 256, 256, 1024
    sizes = dict(a1=T * h * 2, mu1=T * 4, rstd1=T * 4, a1_16=T * h * 2, qkv=T * 3 * hl * 2,
                 qk16=T * 2 * hl * 2, c=T * hl * 2, lse=2 * 4 * 256 * 4, x1=T * h * 2,
                 a2=T * h * 2, mu2=T * 4, rstd2=T * 4, u=T * f * 2, g=T * f * 2)
    for a_, b_ in zip(P.SERIAL_SAVED_SLOTS, P.SERIAL_SAVED_SLOTS[1:]):
        assert lay[b_] - lay[a_] >= sizes[a_]
    assert P.ptb_serial_saved_bytes(d) >= lay["g"] + sizes["g"]
    # split-tile partials first, then du, da, dx1, dc and dZ of the backward
    assert P.ptb_serial_workspace_bytes(d) >= (2 * 256 * 256 * 256 * 4 + T * f * 2
                                               + 2 * T * h * 2 + T * hl * 2 + T * 3 * hl * 2)
    n = ctypes.c_size_t(0)
    assert lib.ptb_serial_saved_bytes(ctypes.byref(good_dims(batch=0)),
                                      ctypes.byref(n)) == P.PTB_ERR_DIMS
    assert lib.ptb_serial_workspace_bytes(ctypes.byref(d), None) == P.PTB_ERR_NULL


def test_serial_forward_backward_reject_null_and_misaligned_before_any_hip_call(lib):
    d = good_dims()
    A = 0x10000  # never dereferenced: the checks fail first
    assert P.ptb_serial_forward(d, *([0] * 12), stream=0, check=False) == P.PTB_ERR_NULL
    assert P.ptb_serial_forward(d, *([A] * 11), None, stream=0, check=False) == P.PTB_ERR_NULL
    args = [A] * 12
    args[3] = A + 8   # ln2_gamma
    assert P.ptb_serial_forward(d, *args, stream=0, check=False) == P.PTB_ERR_ALIGN
    assert P.ptb_serial_backward(d, *([A] * 18), None, stream=0, check=False) == P.PTB_ERR_NULL
    bargs = [A] * 19
    bargs[11] = A + 2  # d_ln2_beta
    assert P.ptb_serial_backward(d, *bargs, stream=0, check=False) == P.PTB_ERR_ALIGN
    assert P.ptb_serial_forward(good_dims(head_dim=32), *([A] * 12), stream=0,
                                check=False) == P.PTB_ERR_HEAD_DIM
    assert P.ptb_serial_backward(good_dims(window=0), *([A] * 19), stream=0,
                                 check=False) == P.PTB_ERR_WINDOW


def _lamb_list(n=2, numel=64, **over):
    A = 0x10000  # never dereferenced: the checks fail first
    ts = []
    for i in range(n):
        t = dict(theta=A, m=A, v=A, grad=A, weight=A, numel=numel)
        t.update(over)
        ts.append((t["theta"], t["m"], t["v"], t["grad"], t["weight"], t["numel"]))
    return ts


def test_lamb_workspace_and_argument_checks(lib):
    assert P.ptb_lamb_workspace_bytes(_lamb_list(1, 16384)) >= 16
    assert P.ptb_lamb_workspace_bytes(_lamb_list(3, 16384 * 5 + 8)) >= 3 * 6 * 16
    hp = P.ptb_lamb_hyper(1e-3, 0.9, 0.999, 1e-6, 1)
    A = 0x10000
    ok = _lamb_list()
    # invalid tensor lists
    for bad in (_lamb_list(numel=12), _lamb_list(numel=0), _lamb_list(numel=2 ** 31),
                _lamb_list(n=33)):
        assert P.ptb_lamb_step(hp, bad, A, A, stream=0, check=False) == P.PTB_ERR_ARG
    arr = P.lamb_tensor_list(ok)
    assert lib.ptb_lamb_step(ctypes.byref(hp), arr, 0, A, A, 0) == P.PTB_ERR_ARG
    assert lib.ptb_lamb_step(None, arr, 2, A, A, 0) == P.PTB_ERR_NULL
    # invalid hyper-parameters
    for h in (P.ptb_lamb_hyper(float("nan"), 0.9, 0.999, 1e-6, 1),
              P.ptb_lamb_hyper(1e-3, 1.0, 0.999, 1e-6, 1),
              P.ptb_lamb_hyper(1e-3, 0.9, -0.1, 1e-6, 1),
              P.ptb_lamb_hyper(1e-3, 0.9, 0.999, 0.0, 1),
              P.ptb_lamb_hyper(1e-3, 0.9, 0.999, 1e-6, 0)):
        assert P.ptb_lamb_step(h, ok, A, A, stream=0, check=False) == P.PTB_ERR_ARG
    # null and misaligned pointers
    assert P.ptb_lamb_step(hp, _lamb_list(grad=0), A, A, stream=0, check=False) == P.PTB_ERR_NULL
    assert P.ptb_lamb_step(hp, _lamb_list(v=A + 4), A, A, stream=0, check=False) == P.PTB_ERR_ALIGN
    assert P.ptb_lamb_step(hp, ok, 0, A, stream=0, check=False) == P.PTB_ERR_NULL
    assert P.ptb_lamb_step(hp, ok, A, A + 8, stream=0, check=False) == P.PTB_ERR_ALIGN


def test_lamb_noalloc_argument_checks(lib):
    """The allocation-free step makes the same checks as ptb_lamb_step and
    rejects a list whose scratch exceeds its static buffer, before any HIP
    call."""
    hp = P.ptb_lamb_hyper(1e-3, 0.9, 0.999, 1e-6, 1)
    A = 0x10000
    for bad in (_lamb_list(numel=12), _lamb_list(numel=0), _lamb_list(n=33)):
        assert P.ptb_lamb_step_noalloc(hp, bad, A, stream=0, check=False) == P.PTB_ERR_ARG
    assert P.ptb_lamb_step_noalloc(hp, _lamb_list(grad=0), A, stream=0,
                                   check=False) == P.PTB_ERR_NULL
    assert P.ptb_lamb_step_noalloc(hp, _lamb_list(), 0, stream=0, check=False) == P.PTB_ERR_NULL
    assert P.ptb_lamb_step_noalloc(hp, _lamb_list(m=A + 4), A, stream=0,
                                   check=False) == P.PTB_ERR_ALIGN
    assert P.ptb_lamb_step_noalloc(P.ptb_lamb_hyper(1e-3, 0.9, 0.999, 1e-6, 0), _lamb_list(), A,
                                   stream=0, check=False) == P.PTB_ERR_ARG
    # scratch: 16 bytes per 16384 elements; the static buffer holds 2^18 such blocks
    limit_blocks = P.PTB_LAMB_NOALLOC_SCRATCH_BYTES // 16
    big = _lamb_list(n=3, numel=2 ** 31 - 8)     # 3 * 131072 blocks > 262144
    assert P.ptb_lamb_workspace_bytes(big) > P.PTB_LAMB_NOALLOC_SCRATCH_BYTES
    assert P.ptb_lamb_step_noalloc(hp, big, A, stream=0, check=False) == P.PTB_ERR_SCRATCH
    assert 3 * 131072 > limit_blocks >= 2 * 131072
    assert "static buffer" in P.ptb_status_string(P.PTB_ERR_SCRATCH)


def test_swiglu_widens_the_fc1_stash_and_workspace(lib):
    T, h, hl, f = 512, 256, 256, 1024
    g_lay = P.ptb_saved_layout(good_dims())
    s_lay = P.ptb_saved_layout(good_dims(mlp=1))
    assert s_lay["g"] - s_lay["u"] >= T * 2 * f * 2 > g_lay["g"] - g_lay["u"] - 256
    assert P.ptb_saved_bytes(good_dims(mlp=1)) >= P.ptb_saved_bytes(good_dims()) + T * f * 2
    # dZ = [dq | dk | dv | du1 du3] is T x (3 h_l + 2 f)
    assert P.ptb_workspace_bytes(good_dims(mlp=1)) >= P.ptb_workspace_bytes(good_dims()) + T * f * 2
    assert P.ptb_serial_saved_bytes(good_dims(mlp=1)) >= P.ptb_serial_saved_bytes(good_dims()) + T * f * 2
    # RMSNorm changes no size
    assert P.ptb_saved_bytes(good_dims(norm=1)) == P.ptb_saved_bytes(good_dims())


def test_fp8_weight_layout_and_sizes(lib):
    """FP8 weight buffer: amax, then W1^T [N1, pad128(h)], W1 [h, pad128(N1)],
    W2^T [h, pad128(K2)], W2 [K2, pad128(h)], 1 byte per element."""
    d = good_dims()  # h 256, 4 x 64 heads, f 1024
    h, hl, f = 256, 256, 1024
    N1, K2 = 3 * hl + f, hl + f
    pad = lambda v: (v + 127) // 128 * 128
    lay = P.ptb_fp8_weights_layout(d)
    sizes = dict(amax=8, w1t=N1 * pad(h), w1=h * pad(N1), w2t=h * pad(K2), w2=K2 * pad(h))
    parts = ("amax", "w1t", "w1", "w2t", "w2")
    offs = [lay[k] for k in parts]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    for a_, b_ in zip(parts, parts[1:]):
        assert lay[b_] - lay[a_] >= sizes[a_]
    # current scaling has no block scales
    assert all(lay[k] == P.FP8_ABSENT for k in ("w1t_s", "w1_s", "w2t_s", "w2_s"))
    assert P.ptb_fp8_weights_bytes(d) >= lay["w2"] + sizes["w2"]
    # a ragged hidden size pads the contiguous dimension to 128
    r = good_dims(hidden=192, heads=3, ffn=768)
    lr = P.ptb_fp8_weights_layout(r)
    assert lr["w1"] - lr["w1t"] >= (3 * 192 + 768) * 256
    # the workspace holds the bf16 layer's plus the FP8 copies that live
    # within one call; the stash adds the transposed copies of a and [c | g]
    T = 512
    assert P.ptb_fp8_workspace_bytes(d) >= P.ptb_workspace_bytes(d) + T * (
        pad(h) * 2 + pad(K2) + pad(N1)) + pad(T) * (h + N1)
    assert P.ptb_fp8_saved_bytes(d) >= P.ptb_saved_bytes(d) + 8 + pad(T) * (h + K2)


def test_fp8_mx_weight_layout_and_sizes(lib):
    """Block scaling: no amax; each copy followed by its scales,
    pad128(k)/128 x pad128(rows) x 4 bytes; the workspace and the stash grow
    by the scales of their copies."""
    d = good_dims()
    h, hl, f, T = 256, 256, 1024, 512
    N1, K2 = 3 * hl + f, hl + f
    pad = lambda v: (v + 127) // 128 * 128
    words = lambda rows, k: pad(k) // 128 * pad(rows) * 4
    lay = P.ptb_fp8_weights_layout(d, "mx")
    assert lay["amax"] == P.FP8_ABSENT
    order = ("w1t", "w1t_s", "w1", "w1_s", "w2t", "w2t_s", "w2", "w2_s")
    sizes = dict(w1t=N1 * pad(h), w1t_s=words(N1, h), w1=h * pad(N1), w1_s=words(h, N1),
                 w2t=h * pad(K2), w2t_s=words(h, K2), w2=K2 * pad(h), w2_s=words(K2, h))
    offs = [lay[k] for k in order]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    for a_, b_ in zip(order, order[1:]):
        assert lay[b_] - lay[a_] >= sizes[a_]
    assert P.ptb_fp8_weights_bytes(d, "mx") >= lay["w2_s"] + sizes["w2_s"]
    extra_ws = (words(T, h) * 2 + words(T, K2) + words(T, N1) + words(h, T) + words(N1, T))
    assert (P.ptb_fp8_workspace_bytes(d, "mx") >=
            P.ptb_fp8_workspace_bytes(d) + extra_ws - 256)
    assert (P.ptb_fp8_saved_bytes(d, "mx") >=
            P.ptb_fp8_saved_bytes(d) + words(h, T) + words(K2, T))

def test_fp8_calls_reject_bad_arguments_before_any_hip_call(lib):
    A = 0x10000
    d = good_dims()
    # SwiGLU has no FP8 variant
    for fn in (P.ptb_fp8_weights_bytes, P.ptb_fp8_workspace_bytes, P.ptb_fp8_saved_bytes):
        with pytest.raises(P.PtbError) as ei:
            fn(good_dims(mlp=1))
        assert ei.value.status == P.PTB_ERR_ARG
    assert P.ptb_fp8_forward(good_dims(mlp=1), *([A] * 7), stream=0,
                             check=False) == P.PTB_ERR_ARG
    assert P.ptb_fp8_forward(d, *([A] * 6), 0, stream=0, check=False) == P.PTB_ERR_NULL
    args = [A] * 7
    args[3] = A + 8
    assert P.ptb_fp8_forward(d, *args, stream=0, check=False) == P.PTB_ERR_ALIGN
    assert P.ptb_fp8_backward(d, *([A] * 12), 0, stream=0, check=False) == P.PTB_ERR_NULL
    assert P.ptb_fp8_backward(good_dims(window=0), *([A] * 13), stream=0,
                              check=False) == P.PTB_ERR_WINDOW
    assert P.ptb_fp8_cast_weights(d, A, A, 0, A, A, stream=0, check=False) == P.PTB_ERR_NULL
    # the stand-alone cast
    assert P.ptb_fp8_quantize(A, 64, 64, "e4m3", A, 0, 0, stream=0,
                              check=False) == P.PTB_ERR_NULL
    assert P.ptb_fp8_quantize(A, 64, 60, "e4m3", A, A, 0, stream=0,
                              check=False) == P.PTB_ERR_DIMS
    assert P.ptb_fp8_quantize(A, 0, 64, "e5m2", A, A, 0, stream=0,
                              check=False) == P.PTB_ERR_DIMS
    assert P.ptb_fp8_quantize(A + 4, 64, 64, "e5m2", A, A, 0, stream=0,
                              check=False) == P.PTB_ERR_ALIGN
    assert load_fmt_error(lib) == P.PTB_ERR_ARG
    # an unknown recipe
    n = ctypes.c_size_t(0)
    assert lib.ptb_fp8_weights_bytes(ctypes.byref(d), 2, ctypes.byref(n)) == P.PTB_ERR_ARG
    assert lib.ptb_fp8_forward(ctypes.byref(d), -1, *([A] * 7), None, None) == P.PTB_ERR_ARG
    # the block-scaled stand-alone cast: a copy needs both its pointers
    assert P.ptb_fp8_quantize_mx(A, 64, 64, "e4m3", A, 0, 0, A, stream=0,
                                 check=False) == P.PTB_ERR_NULL
    assert P.ptb_fp8_quantize_mx(A, 64, 60, "e4m3", A, A, 0, 0, stream=0,
                                 check=False) == P.PTB_ERR_DIMS
    assert P.ptb_fp8_quantize_mx(A, 64, 64, "e4m3", A, A + 4, 0, 0, stream=0,
                                 check=False) == P.PTB_ERR_ALIGN
    assert lib.ptb_fp8_quantize_mx(A, 64, 64, 3, A, A, None, None, None) == P.PTB_ERR_ARG


def load_fmt_error(lib):
    """An unknown format code is rejected."""
    return lib.ptb_fp8_quantize(0x10000, 64, 64, 7, 0x10000, 0x10000, None, None)


def test_dropout_mask_and_fp8_dropout_checks(lib):
    A = 0x10000
    for p in (-0.5, 1.0, float("nan")):
        assert P.ptb_dropout_mask(1, 0, p, 16, A, stream=0, check=False) == P.PTB_ERR_ARG
    assert P.ptb_dropout_mask(1, 0, 0.1, -1, A, stream=0, check=False) == P.PTB_ERR_ARG
    assert P.ptb_dropout_mask(1, 0, 0.1, 2 ** 32, A, stream=0, check=False) == P.PTB_ERR_ARG
    assert P.ptb_dropout_mask(1, 0, 0.1, 16, None, stream=0, check=False) == P.PTB_ERR_NULL
    # the FP8 calls take no dropout
    d = good_dims(dropout_p=0.1)
    n = ctypes.c_size_t(0)
    assert lib.ptb_fp8_weights_bytes(ctypes.byref(d), 0, ctypes.byref(n)) == P.PTB_ERR_ARG
    assert lib.ptb_fp8_weights_bytes(ctypes.byref(good_dims()), 0, ctypes.byref(n)) == P.PTB_OK
