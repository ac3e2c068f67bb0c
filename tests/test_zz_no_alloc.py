"""The allocation-free LAMB step (ptb_lamb_step_noalloc, the library's static
scratch in place of a workspace) through the C ABI, against ptb_lamb_step on
identical copies of the same state: two calls in a row, the second over a
smaller list of smaller tensors (so stale partial sums left in the static
array by the first call would show).  Both run the same kernels in the same
order, so the results must agree bit for bit; the first call is also checked
against the fp64 oracle of eq (7) (MegaScale reading notes, section 1.1)."""
import numpy as np
import pytest
import torch

from oracle import lamb_oracle as L
from transformer_block_amd import inputs as I
from transformer_block_amd import ptb as P

from .helpers import log, rel_fro

pytestmark = pytest.mark.gpu


def _state(rng, sizes):
    dev = "cuda"
    theta = [torch.tensor(rng.standard_normal(n, dtype=np.float32) * np.float32(0.02), device=dev)
             for n in sizes]
    m = [torch.tensor(rng.standard_normal(n, dtype=np.float32) * np.float32(1e-3), device=dev)
         for n in sizes]
    v = [torch.tensor(np.abs(rng.standard_normal(n, dtype=np.float32)) * np.float32(1e-6),
                      device=dev) for n in sizes]
    g = [torch.from_numpy(I.f32_to_bf16_bits(rng.standard_normal(n, dtype=np.float32))
                          .view(np.int16)).view(torch.bfloat16).to(dev) for n in sizes]
    return theta, m, v, g


def _copy(state):
    theta, m, v, g = state
    return ([t.clone() for t in theta], [t.clone() for t in m], [t.clone() for t in v], g)


def _tensors(state, weights):
    theta, m, v, g = state
    return [(t, mm, vv, gg, w) for t, mm, vv, gg, w in zip(theta, m, v, g, weights)]


def _bits(t):
    return t.detach().contiguous().view(torch.int32 if t.dtype == torch.float32 else torch.int16) \
        .cpu().numpy()


def test_noalloc_step_matches_the_workspace_step_twice():
    rng = np.random.default_rng(701)
    hp = P.ptb_lamb_hyper(1e-3, 0.9, 0.999, 1e-6, 3)
    for call, sizes in enumerate(([16384 * 40 + 8, 64, 100000, 16384 * 3], [4096, 16384 + 8])):
        log(f"[noalloc call {call}] sizes {sizes}")
        ref_state = _state(rng, sizes)
        na_state = _copy(ref_state)
        theta0 = [t.double().cpu().numpy() for t in ref_state[0]]
        m0 = [t.double().cpu().numpy() for t in ref_state[1]]
        v0 = [t.double().cpu().numpy() for t in ref_state[2]]
        w_ref = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for n in sizes]
        w_na = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for n in sizes]
        n_ref = torch.empty((len(sizes), 2), dtype=torch.float32, device="cuda")
        n_na = torch.full((len(sizes), 2), float("nan"), dtype=torch.float32, device="cuda")
        ws = torch.empty(P.ptb_lamb_workspace_bytes(_tensors(ref_state, w_ref)), dtype=torch.uint8,
                         device="cuda")
        P.ptb_lamb_step(hp, _tensors(ref_state, w_ref), n_ref, ws)
        P.ptb_lamb_step_noalloc(hp, _tensors(na_state, w_na), n_na)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(n_ref), _bits(n_na)), f"call {call}: norms differ"
        for i in range(len(sizes)):
            for a, b, what in ((ref_state[0][i], na_state[0][i], "theta"),
                               (ref_state[1][i], na_state[1][i], "m"),
                               (ref_state[2][i], na_state[2][i], "v"),
                               (w_ref[i], w_na[i], "weight")):
                assert np.array_equal(_bits(a), _bits(b)), f"call {call} tensor {i}: {what} differs"
        # and the step itself against the oracle, from the same fp32 state
        lr, b1, b2, eps = (float(np.float32(x)) for x in (1e-3, 0.9, 0.999, 1e-6))
        norms = n_na.cpu().numpy().astype(np.float64)
        for i in range(len(sizes)):
            g = I.bf16_bits_to_f64(ref_state[3][i].view(torch.int16).cpu().numpy().view(np.uint16))
            new, _, _, nt, nr = L.lamb_step(theta0[i], m0[i], v0[i], g, 3, lr, b1, b2, eps)
            d = rel_fro(na_state[0][i].double().cpu().numpy() - theta0[i], new - theta0[i])
            assert d <= 1e-4, f"call {call} tensor {i}: update error {d:.2e}"
            assert abs(norms[i, 0] - nt) <= 1e-5 * nt and abs(norms[i, 1] - nr) <= 1e-5 * nr
