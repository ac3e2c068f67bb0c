"""Parity of the serial (standard) block's HIP path (ptb_serial_forward /
ptb_serial_backward through the C ABI) with the fp64 oracle's serial block,
on the same seeded bf16 inputs, by relative Frobenius error per output tensor
against REL_TOL.  The residual paths dominate y and dx, so y - x and dx - dy
are compared as well, against a bar that adds the bf16 rounding floor of the
output to REL_TOL (as for the parallel block).  The stashed intermediates
(both LayerNorm outputs, x1, qkv, c, u, g) localise a failure to one stage."""
import numpy as np
import pytest
import torch

from oracle import ptb_oracle as O
from transformer_block_amd import inputs as I
from transformer_block_amd.runner import SerialBlock, bf16_to_numpy_f64

from .helpers import REL_TOL, log, rel_fro

pytestmark = pytest.mark.gpu

W = I.Workload
CASES = [
    ("tiny_workload", I.WORKLOADS["tiny_h256_s256_w64"], False),
    ("tiny_workload_random_ln", I.WORKLOADS["tiny_h256_s256_w64"], True),
    ("ragged_s200_w37_d128", W("sr1", 1, 200, 256, 2, 128, 320, 37, seed=111), True),
    ("window1_d128", W("sw1", 2, 160, 256, 2, 128, 256, 1, seed=112), False),
    ("window_gt_seq", W("swbig", 1, 131, 256, 3, 64, 320, 100000, seed=120), True),
    ("d64_ragged", W("sd64", 3, 97, 320, 5, 64, 448, 33, seed=121), True),
    ("single_token", W("ss1", 1, 1, 128, 1, 128, 128, 1, seed=122), True),
    ("rmsnorm_swiglu", W("ssw", 2, 160, 256, 2, 128, 256, 40, seed=140, norm="rmsnorm",
                         mlp="swiglu"), True),
    ("h2048_s2048_w512", I.WORKLOADS["h2048_s2048_w512"], False),
    ("gpt175b_tp8_share_s2048", I.WORKLOADS["gpt175b_tp8_share_s2048"], False),
    ("long_h4096_s8192_w1024", I.WORKLOADS["long_h4096_s8192_w1024"], False),
]


def _np(t):
    if t.dtype == torch.bfloat16:
        return bf16_to_numpy_f64(t)
    return t.detach().cpu().numpy().astype(np.float64)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,w,random_ln", CASES, ids=[c[0] for c in CASES])
def test_serial_block_parity(name, w, random_ln):
    log(f"serial case {name}: {w}")
    inp = I.make_inputs(w, random_ln=random_ln)
    blk = SerialBlock(w, inp, "cuda")
    blk.step()
    torch.cuda.synchronize()
    log(f"[serial {name}] gpu step done; running the oracle")
    f = I.bf16_bits_to_f64
    x, dy = f(inp["x"]), f(inp["dy"])
    p = {k: f(v) for k, v in inp["layers"][0].items()}
    y, cache = O.serial_forward(x, p, w.batch, w.seq, w.heads, w.head_dim, w.window, w.ln_eps,
                                norm=w.norm, mlp=w.mlp)
    g = O.serial_backward(dy, cache, p, w.window)
    errs = {"y": rel_fro(_np(blk.y), y), "dx": rel_fro(_np(blk.dx), g["dx"])}
    for key, got, ref, res in (("y-x", _np(blk.y), y, x), ("dx-dy", _np(blk.dx), g["dx"], dy)):
        branch = ref - res
        floor = 2.0 ** -8 * np.linalg.norm(ref) / max(np.linalg.norm(branch), 1e-300)
        errs[key] = rel_fro(got - res, branch) / (1.0 + floor / REL_TOL)
    for k in ("d_ln_gamma", "d_ln_beta", "d_ln2_gamma", "d_ln2_beta", "dw_qkv", "dw_o",
              "dw_fc1", "dw_fc2"):
        errs[k] = rel_fro(_np(blk.grads[k]), g[k])
    for name_, key in (("a1", "a1"), ("x1", "x1"), ("a2", "a2"), ("qkv", "qkv"), ("c", "c"),
                       ("u", "u"), ("g", "g"), ("mu2", "mu2"), ("rstd2", "rstd2")):
        errs[f"saved.{name_}"] = rel_fro(_np(blk.saved_tensor(name_)), cache[key])
    hl = w.h_local
    errs["saved.a1_16"] = rel_fro(_np(blk.saved_tensor("a1_16")), cache["a1"])
    errs["saved.qk16"] = rel_fro(_np(blk.saved_tensor("qk16")), cache["qkv"][:, :2 * hl])
    log(f"[serial {name}] " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not np.isfinite(v) or v > REL_TOL}
    assert not bad, f"parity failures (tol {REL_TOL}): {bad}"


def test_serial_repeat_runs_are_bitwise_identical():
    w = W("sdet", 2, 200, 256, 2, 128, 512, 80, seed=130)
    blk = SerialBlock(w, I.make_inputs(w, random_ln=True), "cuda")
    blk.step()
    torch.cuda.synchronize()
    first = [blk.y.clone(), blk.dx.clone()] + [t.clone() for t in blk.grads.values()]
    blk.step()
    torch.cuda.synchronize()
    second = [blk.y, blk.dx] + list(blk.grads.values())
    for a, b in zip(first, second):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
