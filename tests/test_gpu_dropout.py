"""Dropout on the GPU (MegaScale reading notes, section 1.3: dropout fused
into the layer, its activations kept for backward) through the C ABI, against
the oracle.

* The mask: ptb_dropout_mask must equal the oracle's Philox-4x32-10 mask bit
  for bit (integer work), for ragged lengths, several seeds and streams, and
  the 175B share's full [T, h].
* The layer: the outputs and every gradient within the 1e-2 bar of the fp64
  oracle run with the same masks (parallel block, serial block, a two-layer
  stack whose layers draw different streams, the RMSNorm + SwiGLU variant),
  and the mask the [O ; FC2] epilogue applied bit-exact as well: wherever the
  oracle drops an element, y equals x bit for bit (the branch is multiplied
  by zero before the residual add).
"""
import numpy as np
import pytest
import torch

from oracle import dropout_oracle as D
from oracle import ptb_oracle as O
from transformer_block_amd import inputs as I
from transformer_block_amd import ptb as P
from transformer_block_amd.runner import LayerStack, SerialBlock, bf16_to_numpy_f64

from .helpers import REL_TOL, log, oracle_run, rel_fro

pytestmark = pytest.mark.gpu

W = I.Workload


@pytest.mark.parametrize("seed,stream,p,n", [
    (1, 0, 0.1, 1001), (2 ** 40 + 7, 3, 0.5, 65536 + 3), (12345, 0, 0.0, 100),
    (99, 1, 0.9, 4096), (2024, 0, 0.1, 2048 * 12288)])
def test_mask_is_bit_exact(seed, stream, p, n):
    mask = torch.full((n,), 7, dtype=torch.uint8, device="cuda")
    P.ptb_dropout_mask(seed, stream, p, n, mask)
    torch.cuda.synchronize()
    got = mask.cpu().numpy()
    ref = D.dropout_keep(n, seed, stream, p).astype(np.uint8)
    log(f"[mask seed {seed} stream {stream} p {p} n {n}] kept {got.mean():.4f}")
    assert np.array_equal(got, ref)


def _bits(t):
    return t.detach().contiguous().view(torch.int16).cpu().numpy()


def _check_layer(w, inp, st, tol=REL_TOL):
    ref = oracle_run(w, inp)
    y, dx = bf16_to_numpy_f64(st.y), bf16_to_numpy_f64(st.dx)
    errs = {"y": rel_fro(y, ref["y"]), "dx": rel_fro(dx, ref["dx"])}
    for key, got, out_ref, res in (("y-x", y, ref["y"], ref["x"]), ("dx-dy", dx, ref["dx"], ref["dy"])):
        branch = out_ref - res
        floor = 2.0 ** -8 * np.linalg.norm(out_ref) / max(np.linalg.norm(branch), 1e-300)
        errs[key] = rel_fro(got - res, branch) / (1.0 + floor / tol)
    for li, g in enumerate(ref["grads"]):
        for k in ("d_ln_gamma", "d_ln_beta", "dw_qkv", "dw_o", "dw_fc1", "dw_fc2"):
            errs[f"L{li}.{k}"] = rel_fro(bf16_to_numpy_f64(st.grads[li][k]), g[k])
    # the epilogue's mask: y == x bit for bit where the last layer drops
    last = w.layers - 1
    keep = D.dropout_keep(w.tokens * w.hidden, w.dropout_seed, D.layer_stream(last),
                          w.dropout_p).reshape(w.tokens, w.hidden)
    y_in = _bits(st.layer_input(last))
    y_out = _bits(st.y)
    dropped_equal = np.array_equal(y_out[~keep], y_in[~keep])
    log(f"[dropout {w.name}] dropped {(~keep).mean():.4f} " +
        " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert dropped_equal, "y differs from x where the oracle's mask drops"
    # kept elements rarely equal x (only where the branch rounds away against
    # x); a mask that dropped extra elements would push this towards p
    assert (y_out[keep] == y_in[keep]).mean() < 0.5 * w.dropout_p + 0.03
    bad = {k: v for k, v in errs.items() if not np.isfinite(v) or v > tol}
    assert not bad, f"parity failures (tol {tol}): {bad}"


CASES = [
    ("tiny_p0.1", I.WORKLOADS["tiny_h256_s256_w64"].replace(dropout_p=0.1, dropout_seed=7), False),
    ("ragged_p0.3", W("r1", 1, 200, 256, 2, 128, 320, 37, seed=11, dropout_p=0.3,
                      dropout_seed=2 ** 33 + 1), True),
    ("stack2_p0.2", W("st2", 2, 130, 256, 2, 128, 512, 48, layers=2, seed=24, dropout_p=0.2,
                      dropout_seed=5), True),
    ("rmsnorm_swiglu_p0.1", W("rsw", 2, 96, 320, 5, 64, 448, 33, seed=27, norm="rmsnorm",
                              mlp="swiglu", dropout_p=0.1, dropout_seed=3), True),
]


@pytest.mark.parametrize("name,w,random_ln", CASES, ids=[c[0] for c in CASES])
def test_layer_with_dropout(name, w, random_ln):
    log(f"dropout case {name}: {w}")
    inp = I.make_inputs(w, random_ln=random_ln)
    st = LayerStack(w, inp, "cuda")
    st.step()
    torch.cuda.synchronize()
    _check_layer(w, inp, st)


@pytest.mark.timeout(600)
def test_layer_with_dropout_at_the_175b_share():
    w = I.WORKLOADS["gpt175b_tp8_share_s2048"].replace(dropout_p=0.1, dropout_seed=2024)
    log(f"dropout case 175b share: {w}")
    inp = I.make_inputs(w)
    st = LayerStack(w, inp, "cuda")
    st.step()
    torch.cuda.synchronize()
    _check_layer(w, inp, st)


def _serial_case(w, random_ln):
    inp = I.make_inputs(w, random_ln=random_ln)
    blk = SerialBlock(w, inp, "cuda")
    blk.step()
    torch.cuda.synchronize()
    f = I.bf16_bits_to_f64
    x, dy = f(inp["x"]), f(inp["dy"])
    p = {k: f(v) for k, v in inp["layers"][0].items()}
    shape = (w.tokens, w.hidden)
    m1 = D.dropout_multiplier(shape, w.dropout_seed, D.layer_stream(0, 0), w.dropout_p)
    m2 = D.dropout_multiplier(shape, w.dropout_seed, D.layer_stream(0, 1), w.dropout_p)
    y, cache = O.serial_forward(x, p, w.batch, w.seq, w.heads, w.head_dim, w.window, w.ln_eps,
                                norm=w.norm, mlp=w.mlp, drop1=m1, drop2=m2)
    g = O.serial_backward(dy, cache, p, w.window)
    errs = {"y": rel_fro(bf16_to_numpy_f64(blk.y), y), "dx": rel_fro(bf16_to_numpy_f64(blk.dx), g["dx"])}
    for k in ("d_ln_gamma", "d_ln_beta", "d_ln2_gamma", "d_ln2_beta", "dw_qkv", "dw_o", "dw_fc1",
              "dw_fc2"):
        errs[k] = rel_fro(bf16_to_numpy_f64(blk.grads[k]), g[k])
    errs["x1"] = rel_fro(bf16_to_numpy_f64(blk.saved_tensor("x1")), cache["x1"])
    # both epilogues' masks: x1 == x where D1 drops, y == x1 where D2 drops
    x_b, x1_b, y_b = _bits(blk.x), _bits(blk.saved_tensor("x1")), _bits(blk.y)
    assert np.array_equal(x1_b[m1 == 0], x_b[m1 == 0])
    assert np.array_equal(y_b[m2 == 0], x1_b[m2 == 0])
    log(f"[serial dropout {w.name}] " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not np.isfinite(v) or v > REL_TOL}
    assert not bad, f"parity failures (tol {REL_TOL}): {bad}"


def test_serial_block_with_dropout_small():
    _serial_case(W("sr", 1, 200, 256, 2, 128, 320, 37, seed=31, dropout_p=0.25, dropout_seed=9),
                 True)


@pytest.mark.timeout(600)
def test_serial_block_with_dropout_at_the_175b_share():
    _serial_case(I.WORKLOADS["gpt175b_tp8_share_s2048"].replace(dropout_p=0.1, dropout_seed=77),
                 False)


def test_dropout_repeat_runs_are_bitwise_identical():
    w = W("rep", 2, 130, 256, 2, 128, 512, 48, layers=2, seed=24, dropout_p=0.2, dropout_seed=5)
    inp = I.make_inputs(w)
    outs = []
    for _ in range(2):
        st = LayerStack(w, inp, "cuda")
        st.step()
        torch.cuda.synchronize()
        outs.append([_bits(st.y), _bits(st.dx)] + [_bits(st.grads[l][k]) for l in range(2)
                                                   for k in ("dw_qkv", "dw_o", "dw_fc1", "dw_fc2")])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
