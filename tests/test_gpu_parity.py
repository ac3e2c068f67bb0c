"""Parity of the HIP path (called through the C ABI) with the fp64 oracle.

Each case draws seeded bf16 inputs, runs the layer (or the stack) forward and
backward on the GPU and in the oracle, and compares every output by relative
Frobenius error against the bar REL_TOL = 1e-2 (bf16 operands, fp32
accumulation).  The residual paths dominate y and dx, so y - x and dx - dy are
compared as well, against a bar that adds the bf16 rounding floor of the
output to the 1e-2 relative error of the branch.  The layer-0 intermediates the forward stashes (LayerNorm
output and its fp16 copy, QKV and the fp16 q and k, u, GeLU(u), attention
output, log-sum-exp) are checked too, which localises a failure to one kernel.
"""
import numpy as np
import pytest
import torch

from transformer_block_amd import inputs as I
from transformer_block_amd.runner import Fp8Layer, LayerStack, SerialBlock, bf16_to_numpy_f64

from .helpers import REL_TOL, log, oracle_lse2, oracle_run, rel_fro

pytestmark = pytest.mark.gpu

W = I.Workload
EDGE_CASES = [
    # name, workload, random LayerNorm parameters
    ("tiny_workload", I.WORKLOADS["tiny_h256_s256_w64"], False),
    ("tiny_workload_random_ln", I.WORKLOADS["tiny_h256_s256_w64"], True),
    ("ragged_s200_w37_d128", W("r1", 1, 200, 256, 2, 128, 320, 37, seed=11), True),
    ("window1_d128", W("w1", 2, 160, 256, 2, 128, 256, 1, seed=12), False),
    ("window63", W("w63", 1, 300, 192, 2, 128, 192, 63, seed=13), False),
    ("window64", W("w64", 1, 300, 192, 2, 128, 192, 64, seed=14), False),
    ("window65", W("w65", 1, 300, 192, 2, 128, 192, 65, seed=15), False),
    ("window127", W("w127", 1, 300, 192, 2, 128, 192, 127, seed=16), False),
    ("window128", W("w128", 1, 300, 192, 2, 128, 192, 128, seed=17), False),
    ("window129", W("w129", 1, 300, 192, 2, 128, 192, 129, seed=18), False),
    ("window_eq_seq", W("wseq", 2, 257, 256, 2, 128, 256, 257, seed=19), False),
    ("window_gt_seq", W("wbig", 1, 131, 256, 3, 64, 320, 100000, seed=20), True),
    ("d64_ragged", W("d64", 3, 97, 320, 5, 64, 448, 33, seed=21), True),
    ("single_token", W("s1", 1, 1, 128, 1, 128, 128, 1, seed=22), True),
    ("two_tokens_batch3", W("s2", 3, 2, 128, 2, 64, 128, 5, seed=23), False),
    ("stack2_small", W("st2", 2, 130, 256, 2, 128, 512, 48, layers=2, seed=24), True),
    # the RMSNorm / SwiGLU variants (include/ptb.h, ptb_dims.norm and .mlp)
    ("rmsnorm_tiny", W("rms", 2, 256, 256, 4, 64, 1024, 64, seed=25, norm="rmsnorm"), True),
    ("swiglu_ragged_s200_w37", W("swi", 1, 200, 256, 2, 128, 320, 37, seed=26, mlp="swiglu"),
     True),
    ("rmsnorm_swiglu_d64_ragged", W("rsw", 3, 97, 320, 5, 64, 448, 33, seed=27, norm="rmsnorm",
                                    mlp="swiglu"), True),
    ("rmsnorm_swiglu_stack2", W("rsw2", 2, 130, 256, 2, 128, 512, 48, layers=2, seed=28,
                                norm="rmsnorm", mlp="swiglu"), True),
    # the widest rows (h = 16384) and the 175B share's row width at 300 tokens:
    # the LayerNorm backward's workgroups then hold one or two rows each
    ("widest_rows_h16384", W("h16k", 1, 300, 16384, 1, 128, 256, 64, seed=29), True),
    ("widest_rows_h16384_rmsnorm", W("h16kr", 1, 300, 16384, 1, 128, 256, 64, seed=31,
                                     norm="rmsnorm"), True),
    ("rows_h12288_s300", W("h12k", 1, 300, 12288, 1, 128, 256, 64, seed=32), True),
    # attention's dispatch: more (batch, head) pairs (576) than workgroup places,
    # and one head whose 32 long causal rows are cut into many chunks
    ("many_heads_b9_n64_d64", W("mh", 9, 130, 4096, 64, 64, 256, 1000, seed=33), False),
    ("long_rows_s4096_one_head", W("lr", 1, 4096, 128, 1, 128, 256, 4096, seed=34), False),
    # 2304 rows of 128 queries at d = 128, each with a ragged last row: enough
    # rows for the dispatch model to launch the three-per-CU forward build
    ("many_rows_b96_s1000_d128", W("mr", 96, 1000, 384, 3, 128, 256, 200, seed=35), False),
]


def _to_np(t):
    if t.dtype == torch.bfloat16:
        return bf16_to_numpy_f64(t)
    return t.detach().cpu().numpy().astype(np.float64)


def run_gpu(w, inp):
    st = LayerStack(w, inp, "cuda")
    st.step()
    torch.cuda.synchronize()
    return st


def compare(w, inp, ref, st, tol=REL_TOL, check_intermediates=True):
    errs = {}
    y = _to_np(st.y)
    dx = _to_np(st.dx)
    errs["y"] = rel_fro(y, ref["y"])
    errs["dx"] = rel_fro(dx, ref["dx"])
    # The branch outputs y - x and dx - dy: y and dx are bf16 outputs, so their
    # own rounding (at most 2^-8 relative per element) is an error floor that
    # the subtraction of the residual does not remove.  The bar for these two
    # is tol * ||branch|| + 2^-8 * ||output||, expressed relative to ||branch||.
    for key, got, out_ref, res in (("y-x", y, ref["y"], ref["x"]),
                                   ("dx-dy", dx, ref["dx"], ref["dy"])):
        branch = out_ref - res
        floor = 2.0 ** -8 * np.linalg.norm(out_ref) / max(np.linalg.norm(branch), 1e-300)
        errs[key] = rel_fro(got - res, branch) / (1.0 + floor / tol)
    for li, g in enumerate(ref["grads"]):
        for k in ("d_ln_gamma", "d_ln_beta", "dw_qkv", "dw_o", "dw_fc1", "dw_fc2"):
            errs[f"L{li}.{k}"] = rel_fro(_to_np(st.grads[li][k]), g[k])
    if check_intermediates:
        c0 = ref["caches"][0]
        for name, key in (("a", "a"), ("qkv", "qkv"), ("u", "u"), ("g", "g"), ("c", "c"),
                          ("mu", "mu"), ("rstd", "rstd")):
            errs[f"L0.{name}"] = rel_fro(_to_np(st.saved_tensor(0, name)), c0[key])
        # the fp16 copies the logit path runs on: LN(x) and the q, k columns
        hl = w.h_local
        errs["L0.a16"] = rel_fro(_to_np(st.saved_tensor(0, "a16")), c0["a"])
        errs["L0.qk16"] = rel_fro(_to_np(st.saved_tensor(0, "qk16")), c0["qkv"][:, :2 * hl])
        # lse is the base-2 log of each row's softmax normaliser Z: it is
        # judged like every other tensor, by the relative error of what it
        # encodes, 2^dlse - 1 per row, RMS over the rows (the relative
        # Frobenius error of Z measured row by row); the largest |dlse| is
        # logged beside it.
        lse = _to_np(st.saved_tensor(0, "lse"))
        dl = lse - oracle_lse2(c0, w)
        errs["L0.lse"] = float(np.sqrt(np.mean(np.expm1(dl * np.log(2.0)) ** 2)))
        log(f"[{w.name}] max |dlse| (log2 units) = {float(np.max(np.abs(dl))):.2e}")
    log(f"[{w.name}] " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not np.isfinite(v) or v > tol}
    assert not bad, f"parity failures (tol {tol}): {bad}"
    return errs


@pytest.mark.parametrize("name,w,random_ln", EDGE_CASES, ids=[c[0] for c in EDGE_CASES])
def test_layer_parity_edge_cases(name, w, random_ln):
    log(f"case {name}: {w}")
    inp = I.make_inputs(w, random_ln=random_ln)
    ref = oracle_run(w, inp)
    st = run_gpu(w, inp)
    compare(w, inp, ref, st)


def test_repeat_runs_are_bitwise_identical():
    """A second run reproduces the first bit for bit: split GEMM tiles are
    summed in a fixed order whatever order their parts finish in."""
    w = W("det", 2, 200, 256, 2, 128, 512, 80, seed=30)
    inp = I.make_inputs(w, random_ln=True)
    st = run_gpu(w, inp)
    first = [st.y.clone(), st.dx.clone()] + [t.clone() for t in st.grads[0].values()]
    st.step()
    torch.cuda.synchronize()
    second = [st.y, st.dx] + list(st.grads[0].values())
    for a, b in zip(first, second):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("shape", ["split", "ragged"])
@pytest.mark.parametrize("kind", ["parallel", "serial", "fp8_current", "fp8_mx"])
def test_a_dirty_workspace_gives_the_same_bits(kind, shape):
    """Every call clears the arrival counters it finds in `workspace` (the
    forward inside its LayerNorm launch, the backward with a kernel of its
    own) and writes every other scratch, stash and FP8-copy value, padding
    included, before it is read: a step on `workspace`, `saved` and the FP8
    weight copies filled with 0xFF bytes reproduces a step on what the
    previous step left, bit for bit.  Uncleared counters would leave split
    GEMM tiles and attention rows unmerged (nothing waits on them, so the
    outcome would be wrong values, not a hang)."""
    if shape == "split":
        # K = 2048 in the weight gradients: their tail tiles are split (and
        # the attention rows too), so the counters are in use
        w = W("dirty", 1, 2048, 256, 2, 128, 512, 300, seed=36)
    else:
        # 400 tokens: the FP8 copies pad their token dimension to 512
        w = W("dirtyr", 2, 200, 256, 2, 128, 512, 80, seed=37)
    inp = I.make_inputs(w, random_ln=True)
    st = (LayerStack(w, inp, "cuda") if kind == "parallel" else
          SerialBlock(w, inp, "cuda") if kind == "serial" else
          Fp8Layer(w, inp, "cuda", recipe=kind[4:]))
    grads = st.grads[0] if kind == "parallel" else st.grads
    dirty = [st.workspace] + (list(st.saved) if kind == "parallel" else [st.saved])
    if kind.startswith("fp8"):
        dirty.append(st.fp8_weights)
    log(f"dirty workspace: {kind}, {shape}, {sum(t.numel() for t in dirty)} bytes")
    st.step()
    torch.cuda.synchronize()
    first = [st.y.clone(), st.dx.clone()] + [t.clone() for t in grads.values()]
    for t in dirty:
        t.fill_(255)
    torch.cuda.synchronize()
    st.step()
    torch.cuda.synchronize()
    second = [st.y, st.dx] + list(grads.values())
    for a, b in zip(first, second):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.timeout(900)
def test_rmsnorm_swiglu_variant_at_the_175b_share():
    """The RMSNorm + SwiGLU variant at the 175B share's full size (FFN shard
    6144, so w_fc1 is [12288, 12288])."""
    w = I.WORKLOADS["gpt175b_tp8_share_s2048"].replace(name="gpt175b_share_rms_swiglu",
                                                       norm="rmsnorm", mlp="swiglu")
    log(f"full variant workload: {w}")
    inp = I.make_inputs(w)
    st = run_gpu(w, inp)
    log("[variant] gpu step done; running the oracle")
    ref = oracle_run(w, inp)
    compare(w, inp, ref, st)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", I.WORKLOAD_ORDER)
def test_full_workload_parity(name):
    """Every workload at its full size, run exactly as bench.py runs it (the
    whole stack forward then backward through the C ABI), against the full
    fp64 oracle."""
    w = I.WORKLOADS[name]
    log(f"full workload {name}: {w}")
    inp = I.make_inputs(w)
    st = run_gpu(w, inp)
    log(f"[{name}] gpu step done; running the oracle")
    ref = oracle_run(w, inp)
    compare(w, inp, ref, st)
