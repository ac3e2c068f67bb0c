"""Parity of the LAMB step's HIP path (ptb_lamb_step through the C ABI) with
the fp64 oracle (MegaScale reading notes, section 1.1, eq (7)).

Tolerances, derived from the arithmetic: the kernels compute in fp32, so the
new moments carry a few fp32 roundings (relative Frobenius error <= 1e-6) and
the norms a sum of fp32 squares accumulated in fp64 across threads (<= 1e-5).
The update theta_new - theta is compared as such (<= 1e-4): besides its fp32
arithmetic it carries the fp32 rounding of theta itself, about ulp(|theta|)
against a step of lr * trust * |r| per element.  The bf16 weight copy is
integer work: it must equal round-to-nearest-even of the kernel's own fp32
theta bit for bit.  The hyper-parameters cross the ABI as fp32 (0.999 becomes
0.99900001287...), so the oracle is given those same fp32 values."""
import numpy as np
import pytest
import torch

from oracle import lamb_oracle as L
from transformer_block_amd import inputs as I
from transformer_block_amd import ptb as P

from .helpers import log, rel_fro

pytestmark = pytest.mark.gpu


def _rne_bits(t32: torch.Tensor) -> np.ndarray:
    return I.f32_to_bf16_bits(t32.detach().cpu().numpy())


class Lamb:
    """Device state of a list of tensors: fp32 theta, m, v; bf16 grad, weight."""

    def __init__(self, thetas, ms=None, vs=None):
        dev = "cuda"
        self.theta = [torch.tensor(t, dtype=torch.float32, device=dev) for t in thetas]
        self.m = [torch.tensor(x, dtype=torch.float32, device=dev) if ms else
                  torch.zeros_like(t) for x, t in zip(ms or thetas, self.theta)]
        self.v = [torch.tensor(x, dtype=torch.float32, device=dev) if vs else
                  torch.zeros_like(t) for x, t in zip(vs or thetas, self.theta)]
        self.grad = [torch.empty(t.shape, dtype=torch.bfloat16, device=dev) for t in self.theta]
        self.weight = [torch.empty(t.shape, dtype=torch.bfloat16, device=dev) for t in self.theta]
        self.norms = torch.empty((len(self.theta), 2), dtype=torch.float32, device=dev)
        lst = self.tensors()
        self.workspace = torch.empty(P.ptb_lamb_workspace_bytes(lst), dtype=torch.uint8,
                                     device=dev)

    def tensors(self):
        return [(t, m, v, g, w) for t, m, v, g, w in
                zip(self.theta, self.m, self.v, self.grad, self.weight)]

    def step(self, grads_bits, step, lr, b1, b2, eps):
        for dst, gb in zip(self.grad, grads_bits):
            dst.copy_(torch.from_numpy(gb.view(np.int16)).view(torch.bfloat16).reshape(dst.shape))
        P.ptb_lamb_step(P.ptb_lamb_hyper(lr, b1, b2, eps, step), self.tensors(), self.norms,
                        self.workspace)
        torch.cuda.synchronize()


def _f64(t):
    return t.detach().cpu().numpy().astype(np.float64)


def _check_step(st, ref_state, grads_bits, step, lr, b1, b2, eps, tag):
    """One step on the GPU and in the oracle from the same fp32 state."""
    before = [_f64(t) for t in st.theta]
    m0 = [_f64(t) for t in st.m]
    v0 = [_f64(t) for t in st.v]
    st.step(grads_bits, step, lr, b1, b2, eps)
    norms = st.norms.cpu().numpy().astype(np.float64)
    # the library takes fp32 hyper-parameters: the oracle gets the same values
    lr, b1, b2, eps = (float(np.float32(x)) for x in (lr, b1, b2, eps))
    worst = {}
    for i, gb in enumerate(grads_bits):
        g = I.bf16_bits_to_f64(gb).reshape(before[i].shape)
        new, m, v, nt, nr = L.lamb_step(before[i], m0[i], v0[i], g, step, lr, b1, b2, eps)
        errs = {
            "dtheta": rel_fro(_f64(st.theta[i]) - before[i], new - before[i]),
            "m": rel_fro(_f64(st.m[i]), m),
            "v": rel_fro(_f64(st.v[i]), v),
            "norm_theta": abs(norms[i, 0] - nt) / max(nt, 1e-300),
            "norm_r": abs(norms[i, 1] - nr) / max(nr, 1e-300),
        }
        bits_gpu = st.weight[i].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(bits_gpu.reshape(-1), _rne_bits(st.theta[i]).reshape(-1)), \
            f"{tag} tensor {i}: bf16 copy is not RNE of theta"
        for k, e in errs.items():
            worst[k] = max(worst.get(k, 0.0), e)
    log(f"[lamb {tag} step {step}] " + " ".join(f"{k}={v:.2e}" for k, v in worst.items()))
    bars = {"dtheta": 1e-4, "m": 1e-6, "v": 1e-6, "norm_theta": 1e-5, "norm_r": 1e-5}
    bad = {k: v for k, v in worst.items() if not np.isfinite(v) or v > bars[k]}
    assert not bad, f"{tag} step {step}: {bad}"


def _bits(rng, shape, std):
    return I.f32_to_bf16_bits(rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std))


def test_lamb_three_steps_ragged_sizes_and_a_zero_tensor():
    rng = np.random.default_rng(500)
    sizes = [64, 16384, 16384 * 3 + 8, 100000, 40000]
    thetas = [rng.standard_normal(n).astype(np.float32) * 0.02 for n in sizes]
    thetas.append(np.zeros(8192, np.float32))       # trust ratio 1
    st = Lamb(thetas)
    for step in (1, 2, 3):
        grads = [_bits(rng, t.shape, 1e-3) for t in thetas]
        _check_step(st, None, grads, step, 1e-2, 0.9, 0.999, 1e-6, "ragged")


def test_lamb_late_step_with_running_moments_and_2d_tensors():
    rng = np.random.default_rng(501)
    shapes = [(256, 768), (768, 256), (256,), (1024, 40)]
    thetas = [rng.standard_normal(s).astype(np.float32) * 0.05 for s in shapes]
    ms = [rng.standard_normal(s).astype(np.float32) * 1e-3 for s in shapes]
    vs = [(np.abs(rng.standard_normal(s)) * 1e-6).astype(np.float32) for s in shapes]
    st = Lamb(thetas, ms, vs)
    grads = [_bits(rng, s, 3e-3) for s in shapes]
    _check_step(st, None, grads, 1000, 5e-3, 0.85, 0.99, 1e-8, "late")


def test_lamb_repeat_is_bitwise_identical():
    rng = np.random.default_rng(502)
    thetas = [rng.standard_normal(n).astype(np.float32) for n in (50000, 16384 * 2)]
    grads = [_bits(rng, t.shape, 1.0) for t in thetas]
    a, b = Lamb(thetas), Lamb(thetas)
    a.step(grads, 1, 1e-3, 0.9, 0.999, 1e-6)
    b.step(grads, 1, 1e-3, 0.9, 0.999, 1e-6)
    for x, y in zip(a.theta + a.m + a.v + a.weight, b.theta + b.m + b.v + b.weight):
        assert torch.equal(x.view(torch.int32 if x.dtype == torch.float32 else torch.int16),
                           y.view(torch.int32 if y.dtype == torch.float32 else torch.int16))
    assert torch.equal(a.norms, b.norms)


@pytest.mark.timeout(600)
def test_lamb_175b_share_parameters_full_size():
    """The six parameter tensors of the 175B-shape TP=8 share (226.5 M
    parameters), as the bench times them: fp32 masters widened from the
    seeded bf16 weights, zero moments, a seeded N(0, 1e-3^2) bf16 gradient."""
    w = I.WORKLOADS["gpt175b_tp8_share_s2048"]
    inp = I.make_inputs(w)
    lay = inp["layers"][0]
    names = ("ln_gamma", "ln_beta", "w_qkv", "w_o", "w_fc1", "w_fc2")
    thetas = [I.bf16_bits_to_f32(lay[k]) for k in names]
    rng = np.random.default_rng(503)
    grads = [_bits(rng, t.shape, 1e-3) for t in thetas]
    st = Lamb(thetas)
    log("lamb full size: state on the GPU; stepping")
    _check_step(st, None, grads, 1, 1e-3, 0.9, 0.999, 1e-6, "gpt175b_tp8_share")
