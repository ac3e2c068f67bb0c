#!/usr/bin/env python3
"""Throughput of one Parallel Transformer Block layer, forward + backward, on
one MI355X, in model TFLOP/s and as a fraction of the dense bf16 MFMA peak.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one forward and one backward of the whole layer stack of the
workload (every kernel of the hot path) on resident, seeded synthetic bf16
inputs.  W untimed warm-up steps, then exactly K steps between two
device-synchronised HIP events, with one more event at each step boundary
(the median step is reported beside the mean); per-stage times come from a
separate pass of K steps with events around every stage.  Model FLOPs follow the Megatron tuning post's
MFU section (6 per weight per token plus the attention term, recompute
excluded) made exact for the sliding window (transformer_block_amd/flops.py).

Prints one JSON line.  Besides the throughput it carries:
  roofline:     the dominant kernel (largest device time per step), its
                algorithmic FLOPs per launch over its mean launch time measured
                with HIP events recorded around it on the library's stream;
  cpu_baseline: the fp64 oracle timed on host cores on a bounded sample of the
                same workload (a reported baseline, not a target);
  stages:       mean device time per kernel stage;
  serial_block: the same workload through the serial (standard) block of the
                MegaScale notes' eq (3), timed the same way: what the parallel
                block buys on one GPU (--no-serial skips it);
  variant:      the same workload with RMSNorm, the SwiGLU MLP and dropout
                (p = 0.1) on the branch output (MegaScale's own fused kernels,
                notes section 1.3; --no-variant skips it), model FLOPs
                counting the SwiGLU MLP's 3 h f weights;
  optimizer:    one LAMB step (the notes' eq (7)) over every parameter tensor
                of the workload, fp32 masters and moments, against the HBM
                roofline (40 algorithmic bytes per parameter); --no-optimizer
                skips it;
  fp8:          the same layer with its four GEMM parts on FP8 operands (E4M3
                forward, E5M2 gradients, current scaling: Megatron tuning
                post, mixed-precision section), the weight cast included in
                the step, model FLOPs as for `value`, with its own roofline
                (dominant FP8 product against the 5.0 PFLOP/s dense FP8
                peak);
  fp8_mx:       the same with block (MX) scaling (E8M0 scale per 32
                values, applied by the matrix cores); --no-fp8 skips both.
                None of these legs is part of `value`.

roofline.traffic is the HBM bytes per launch of the dominant kernel as read
by rocprofv3 counters (FETCH_SIZE, WRITE_SIZE), each scaled by what the same
counter reads for a plain copy of known size.  It is taken from the committed
summary profiles/traffic_<stage>_<workload>.md, and only while the kernel
source it was measured on is unchanged (SHA-256 recorded there); otherwise it
is null.  --copy-probe-mib N runs that calibration copy (N MiB read, N MiB
written, outside the timed region) for the counter runs.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X dense peaks: 256 CUs x 2.4 GHz x 4096 bf16 FLOP per clock per CU
# (published as 2.5 PFLOP/s), twice that for FP8; HBM3E 8 TB/s.
PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5033.2
METRIC = "model TFLOP/s + MFU vs bf16 MFMA peak, PTB layer fwd+bwd, 1 MI355X"
DEFAULT_WORKLOAD = "gpt175b_tp8_share_s2048"


def stage_work(w):
    """Algorithmic work per launch of each stage: (kind, amount)."""
    from transformer_block_amd.flops import window_pairs
    T, h, hl, f = w.tokens, w.hidden, w.h_local, w.ffn
    N1, K2 = 3 * hl + f, hl + f
    attn_pairs = w.batch * w.heads * window_pairs(w.seq, w.window)
    fwd = {
        # x read; a (bf16) and its fp16 copy (the q, k product's operand)
        # written; the row statistics
        "layernorm_fwd": ("bytes", T * h * 2 * 3 + T * 8),
        # read the q, k columns of W_qkv (bf16), write their fp16 copy
        "cast_wqk_f16": ("bytes", h * 2 * hl * (2 + 2)),
        "gemm_qkv_fc1": ("flops", 2 * T * h * N1),
        "attention_fwd": ("flops", 2 * 2 * attn_pairs * w.head_dim),
        "gemm_o_fc2_residual": ("flops", 2 * T * K2 * h),
    }
    bwd = {
        "gemm_dgrad_o_fc2": ("flops", 2 * T * h * K2),
        "attention_bwd": ("flops", 4 * 2 * attn_pairs * w.head_dim),
        "gemm_wgrad_o_fc2": ("flops", 2 * K2 * T * h),
        "gemm_dgrad_qkv_fc1": ("flops", 2 * T * N1 * h),
        "gemm_wgrad_qkv_fc1": ("flops", 2 * h * T * N1),
        # da + x + dy read, dx written (bf16)
        "layernorm_bwd": ("bytes", T * h * (2 + 2 + 2 + 2) + T * 8),
    }
    return fwd, bwd


STAGE_SOURCE = {"gemm": "gemm.hip", "attention": "attention.hip", "layernorm": "layernorm.hip",
                "cast": "layernorm.hip"}


def source_sha256(stage: str) -> str:
    import hashlib
    name = STAGE_SOURCE[stage.split("_")[0]]
    path = os.path.join(ROOT, "transformer_block_amd", "csrc", name)
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()


def recorded_traffic(stage: str, workload: str):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{stage}_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            item = line.strip().lstrip("-* ")
            if item.startswith(("traffic_bytes_per_launch:", "source_sha256:")):
                k, v = item.split(":", 1)
                fields[k] = v.strip(" `")
    if fields.get("source_sha256") != source_sha256(stage):
        return None
    try:
        return int(float(fields["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def copy_probe(mib: int) -> None:
    """A plain elementwise copy of `mib` MiB (fp32), the calibration kernel of
    the HBM byte counters."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = []

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        self.events.extend(out)
        return out

    def ms(self, a, b) -> float:
        t = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(t), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return t.value

    def close(self):
        for e in self.events:
            self.hip.hipEventDestroy(e)
        self.events = []


def cpu_baseline(w, budget_s: float):
    """Time the fp64 oracle (as it stands) on a bounded sample of `w`."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import ptb_oracle as O
    from transformer_block_amd import inputs as I
    from transformer_block_amd.flops import model_flops

    # One layer; trim the batch, then the sequence, until the estimated fp64
    # work fits the budget at ~0.25 TFLOP/s.
    b, s = w.batch, w.seq
    est = lambda bb, ss: model_flops(bb, ss, w.hidden, w.heads, w.head_dim, w.ffn,
                                     min(w.window, ss)) / 0.25e12
    while b > 1 and est(b, s) > budget_s:
        b -= 1
    while s > 128 and est(b, s) > budget_s:
        s //= 2
    sw = w.replace(batch=b, seq=s, layers=1)
    inp = I.make_inputs(sw)
    f = I.bf16_bits_to_f64
    x, dy = f(inp["x"]), f(inp["dy"])
    p = {k: f(v) for k, v in inp["layers"][0].items()}
    t0 = time.perf_counter()
    y, cache = O.ptb_forward(x, p, sw.batch, sw.seq, sw.heads, sw.head_dim, sw.window,
                             sw.ln_eps)
    O.ptb_backward(dy, cache, p, sw.window)
    dt = time.perf_counter() - t0
    fl = model_flops(sw.batch, sw.seq, sw.hidden, sw.heads, sw.head_dim, sw.ffn, sw.window)
    threads = max([d.get("num_threads", 1) for d in threadpool_info()
                   if d.get("user_api") == "blas"] or [1])
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"one layer fwd+bwd at batch {sw.batch}, seq {sw.seq}, window "
                      f"{min(sw.window, sw.seq)} (hidden {sw.hidden}, heads {sw.heads}x"
                      f"{sw.head_dim}, ffn {sw.ffn}); fp64 numpy; {dt:.1f} s wall",
            "seconds": dt, "nproc": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": cpu_model(), "blas_threads": int(threads)}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def time_serial(w, inp, warmup: int, steps: int, ptb_ms: float) -> dict:
    """The serial block (MegaScale notes, eq (3)) on the same inputs: mean
    ms per forward+backward step and per stage, HIP events on one stream."""
    import torch

    from transformer_block_amd import ptb as P
    from transformer_block_amd.flops import workload_model_flops
    from transformer_block_amd.runner import SerialBlock

    print("bench: timing the serial block", file=sys.stderr, flush=True)
    blk = SerialBlock(w, inp, "cuda")
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        blk.step(stream)
    torch.cuda.synchronize()
    ev = HipEvents()
    fwd_ev = [ev.create(2 * P.PTB_SERIAL_FWD_STAGES) for _ in range(steps)]
    bwd_ev = [ev.create(2 * P.PTB_SERIAL_BWD_STAGES) for _ in range(steps)]
    t0, t1 = ev.create(2)
    ev.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    torch.cuda.synchronize()
    ev.hip.hipEventRecord(t0, stream.cuda_stream)
    for k in range(steps):
        blk.step(stream, fwd_ev[k], bwd_ev[k])
    ev.hip.hipEventRecord(t1, stream.cuda_stream)
    torch.cuda.synchronize()
    ms = ev.ms(t0, t1) / steps
    stages = {}
    for names, evs in ((P.SERIAL_FWD_STAGE_NAMES, fwd_ev), (P.SERIAL_BWD_STAGE_NAMES, bwd_ev)):
        for i, name in enumerate(names):
            stages[name] = round(sum(ev.ms(evs[k][2 * i], evs[k][2 * i + 1])
                                     for k in range(steps)) / steps, 4)
    ev.close()
    tflops = workload_model_flops(w) / (ms * 1e-3) / 1e12
    del blk
    return {"ms_per_step": round(ms, 4), "value": round(tflops, 2), "unit": "TFLOP/s",
            "mfu": round(tflops / PEAK_BF16_TFLOPS, 4),
            "parallel_speedup": round(ms / ptb_ms, 4), "stages_ms": stages}


VARIANT_DROPOUT = 0.1  # dropout rate of the variant leg's branch output


def time_variant(w, warmup: int, steps: int, base_ms: float) -> dict:
    """The layer stack with RMSNorm and the SwiGLU MLP on the same shape:
    mean ms per fwd+bwd step and per stage (HIP events, one stream)."""
    import torch

    from transformer_block_amd import inputs as I
    from transformer_block_amd import ptb as P
    from transformer_block_amd.flops import workload_model_flops
    from transformer_block_amd.runner import LayerStack

    print("bench: timing the RMSNorm + SwiGLU + dropout variant", file=sys.stderr, flush=True)
    wv = w.replace(name=w.name + "_rmsnorm_swiglu_dropout", norm="rmsnorm", mlp="swiglu",
                   dropout_p=VARIANT_DROPOUT, dropout_seed=2024)
    st = LayerStack(wv, I.make_inputs(wv), "cuda")
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        st.step(stream)
    torch.cuda.synchronize()
    ev = HipEvents()
    L = wv.layers
    fwd_ev = [[ev.create(2 * P.PTB_FWD_STAGES) for _ in range(L)] for _ in range(steps)]
    bwd_ev = [[ev.create(2 * P.PTB_BWD_STAGES) for _ in range(L)] for _ in range(steps)]
    t0, t1 = ev.create(2)
    ev.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    torch.cuda.synchronize()
    ev.hip.hipEventRecord(t0, stream.cuda_stream)
    for k in range(steps):
        st.step(stream, fwd_ev[k], bwd_ev[k])
    ev.hip.hipEventRecord(t1, stream.cuda_stream)
    torch.cuda.synchronize()
    ms = ev.ms(t0, t1) / steps
    stages = {}
    for names, evs in ((P.FWD_STAGE_NAMES, fwd_ev), (P.BWD_STAGE_NAMES, bwd_ev)):
        for i, name in enumerate(names):
            stages[name] = round(sum(ev.ms(evs[k][l][2 * i], evs[k][l][2 * i + 1])
                                     for k in range(steps) for l in range(L)) / (steps * L), 4)
    ev.close()
    F = workload_model_flops(wv)
    tflops = F / (ms * 1e-3) / 1e12
    del st
    return {"norm": "rmsnorm", "mlp": "swiglu", "dropout_p": VARIANT_DROPOUT,
            "ms_per_step": round(ms, 4),
            "value": round(tflops, 2), "unit": "TFLOP/s", "mfu": round(tflops / PEAK_BF16_TFLOPS, 4),
            "model_flops_per_step": F, "stages_ms": stages}


def time_fp8(w, inp, warmup: int, steps: int, base_ms: float, recipe: str = "current") -> dict:
    """The FP8-GEMM layer on the same inputs, scaled by `recipe`: mean ms per
    step (weight cast, forward, backward) and per stage, HIP events on one
    stream."""
    import torch

    from transformer_block_amd import ptb as P
    from transformer_block_amd.flops import workload_model_flops
    from transformer_block_amd.runner import Fp8Layer

    print(f"bench: timing the FP8 GEMM variant ({recipe} scaling)", file=sys.stderr, flush=True)
    lyr = Fp8Layer(w, inp, "cuda", recipe)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        lyr.step(stream)
    torch.cuda.synchronize()
    ev = HipEvents()
    fwd_ev = [ev.create(2 * P.PTB_FP8_FWD_STAGES) for _ in range(steps)]
    bwd_ev = [ev.create(2 * P.PTB_FP8_BWD_STAGES) for _ in range(steps)]
    cast_ev = [ev.create(2) for _ in range(steps)]
    t0, t1 = ev.create(2)
    ev.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    torch.cuda.synchronize()
    ev.hip.hipEventRecord(t0, stream.cuda_stream)
    for k in range(steps):
        ev.hip.hipEventRecord(cast_ev[k][0], stream.cuda_stream)
        lyr.cast_weights(stream)
        ev.hip.hipEventRecord(cast_ev[k][1], stream.cuda_stream)
        lyr.forward(stream, fwd_ev[k])
        lyr.backward(stream, bwd_ev[k])
    ev.hip.hipEventRecord(t1, stream.cuda_stream)
    torch.cuda.synchronize()
    ms = ev.ms(t0, t1) / steps
    stages = {"cast_weights": round(sum(ev.ms(c[0], c[1]) for c in cast_ev) / steps, 4)}
    for names, evs in ((P.FP8_FWD_STAGE_NAMES, fwd_ev), (P.FP8_BWD_STAGE_NAMES, bwd_ev)):
        for i, name in enumerate(names):
            stages[name] = round(sum(ev.ms(evs[k][2 * i], evs[k][2 * i + 1])
                                     for k in range(steps)) / steps, 4)
    ev.close()
    F = workload_model_flops(w)
    tflops = F / (ms * 1e-3) / 1e12
    gemm_ms = sum(v for k, v in stages.items() if k.startswith("gemm_"))
    # the leg's dominant kernel against the dense FP8 peak: the six products
    # have the bf16 layer's model FLOPs (stage_work), named with an _fp8 suffix
    fwd_work, bwd_work = stage_work(w)
    work = dict(fwd_work)
    work.update(bwd_work)
    dom = max((k for k in stages if k.startswith("gemm_")), key=lambda k: stages[k])
    flops = work[dom[:-len("_fp8")]][1]
    ach = flops / (stages[dom] * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / PEAK_FP8_TFLOPS, 4), "traffic": None, "kernel": dom,
            "per_launch": flops, "ms_per_launch": stages[dom]}
    del lyr
    scaling = {"current": "per-operand current scaling",
               "mx": "block (MX) scaling, E8M0 per 32 values"}[recipe]
    return {"formats": f"E4M3 fwd / E5M2 grad, {scaling}",
            "ms_per_step": round(ms, 4), "value": round(tflops, 2), "unit": "TFLOP/s",
            "mfu_vs_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
            "frac_of_fp8_peak": round(tflops / PEAK_FP8_TFLOPS, 4),
            "speedup_vs_bf16": round(base_ms / ms, 4),
            "gemm_ms": round(gemm_ms, 4), "roofline": roof, "stages_ms": stages}


LAMB_BYTES_PER_PARAM = 40  # moments pass: g 2 + theta, m, v 12 read, m, v 8 written;
                           # update pass: theta, m, v 12 read, theta 4 + bf16 copy 2 written


def time_lamb(st, warmup: int, steps: int) -> dict:
    """One LAMB step over every parameter tensor of the stack (fp32 masters
    widened from the bf16 weights, zero moments, the stack's own gradients):
    mean device time per step between HIP events, and its HBM roofline."""
    import torch

    from transformer_block_amd import ptb as P

    print("bench: timing the LAMB step", file=sys.stderr, flush=True)
    names = ("ln_gamma", "ln_beta", "w_qkv", "w_o", "w_fc1", "w_fc2")
    grad_of = {"ln_gamma": "d_ln_gamma", "ln_beta": "d_ln_beta", "w_qkv": "dw_qkv",
               "w_o": "dw_o", "w_fc1": "dw_fc1", "w_fc2": "dw_fc2"}
    tensors = []
    for p, g in zip(st.params, st.grads):
        for k in names:
            theta = p[k].float()
            # a separate bf16 output: the bench's own weights stay as they are
            tensors.append((theta, torch.zeros_like(theta), torch.zeros_like(theta),
                            g[grad_of[k]], torch.empty_like(p[k])))
    nparam = sum(t[0].numel() for t in tensors)
    norms = torch.empty((len(tensors), 2), dtype=torch.float32, device="cuda")
    work = torch.empty(P.ptb_lamb_workspace_bytes(tensors), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        P.ptb_lamb_step(P.ptb_lamb_hyper(1e-3, 0.9, 0.999, 1e-6, i + 1), tensors, norms, work,
                        stream)
    torch.cuda.synchronize()
    ev = HipEvents()
    t0, t1 = ev.create(2)
    ev.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    ev.hip.hipEventRecord(t0, stream.cuda_stream)
    for i in range(steps):
        P.ptb_lamb_step(P.ptb_lamb_hyper(1e-3, 0.9, 0.999, 1e-6, warmup + i + 1), tensors,
                        norms, work, stream)
    ev.hip.hipEventRecord(t1, stream.cuda_stream)
    torch.cuda.synchronize()
    ms = ev.ms(t0, t1) / steps
    ev.close()
    gbs = nparam * LAMB_BYTES_PER_PARAM / (ms * 1e-3) / 1e9
    return {"kernel": "lamb", "tensors": len(tensors), "params": nparam, "ms": round(ms, 4),
            "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes_per_param": LAMB_BYTES_PER_PARAM}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--no-serial", action="store_true",
                    help="skip timing the serial-block comparison")
    ap.add_argument("--no-variant", action="store_true",
                    help="skip timing the RMSNorm + SwiGLU variant")
    ap.add_argument("--no-optimizer", action="store_true",
                    help="skip timing the LAMB optimizer step")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip timing the FP8 GEMM variant")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run a plain copy of this many MiB first (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer is benchmarked on one GPU's share of the work)", file=sys.stderr)
        return 2

    import torch

    from transformer_block_amd import inputs as I
    from transformer_block_amd import ptb as P
    from transformer_block_amd.flops import workload_model_flops, workload_recompute_flops
    from transformer_block_amd.runner import LayerStack

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    P.load_library()
    w = I.WORKLOADS[args.workload]
    print(f"bench: workload {w.name} steps {args.steps} warmup {args.warmup}",
          file=sys.stderr, flush=True)
    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib)
    inp = I.make_inputs(w)
    st = LayerStack(w, inp, "cuda")
    stream = torch.cuda.current_stream()
    ev = HipEvents()

    for _ in range(args.warmup):
        st.step(stream)
    torch.cuda.synchronize()

    L = w.layers
    K = args.steps
    hip = ev.hip
    hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    # The timed region: K steps with one HIP event at each step boundary and
    # nothing else inside it.
    bounds = ev.create(K + 1)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    hip.hipEventRecord(bounds[0], stream.cuda_stream)
    for k in range(K):
        st.step(stream)
        hip.hipEventRecord(bounds[k + 1], stream.cuda_stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = ev.ms(bounds[0], bounds[K]) / K
    per_step = sorted(ev.ms(bounds[k], bounds[k + 1]) for k in range(K))
    ms_median = per_step[K // 2] if K % 2 else 0.5 * (per_step[K // 2 - 1] + per_step[K // 2])

    # Per-kernel times come from a separate pass of K steps with HIP events
    # around every stage (each GEMM stage is one launch).
    print("bench: stage pass", file=sys.stderr, flush=True)
    fwd_ev = [[ev.create(2 * P.PTB_FWD_STAGES) for _ in range(L)] for _ in range(K)]
    bwd_ev = [[ev.create(2 * P.PTB_BWD_STAGES) for _ in range(L)] for _ in range(K)]
    torch.cuda.synchronize()
    for k in range(K):
        st.step(stream, fwd_ev[k], bwd_ev[k])
    torch.cuda.synchronize()
    fwd_work, bwd_work = stage_work(w)
    stages = {}
    for names, evs in ((P.FWD_STAGE_NAMES, fwd_ev), (P.BWD_STAGE_NAMES, bwd_ev)):
        for i, name in enumerate(names):
            tot = sum(ev.ms(evs[k][l][2 * i], evs[k][l][2 * i + 1])
                      for k in range(K) for l in range(L))
            stages[name] = tot / (K * L)            # mean ms per launch
    ev.close()

    F = workload_model_flops(w)
    R = workload_recompute_flops(w)
    tflops = F / (ms_step * 1e-3) / 1e12
    work = dict(fwd_work)
    work.update(bwd_work)
    dom = max(stages, key=lambda n: stages[n])
    kind, amount = work[dom]
    if kind == "flops":
        ach = amount / (stages[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": recorded_traffic(dom, w.name),
                "kernel": dom, "per_launch": amount, "ms_per_launch": round(stages[dom], 4)}
    else:
        ach = amount / (stages[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                "traffic": recorded_traffic(dom, w.name),
                "kernel": dom, "per_launch": amount, "ms_per_launch": round(stages[dom], 4)}

    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02^2) weights, bf16)",
        "config": {"workload": w.name, "batch": w.batch, "seq": w.seq, "hidden": w.hidden,
                   "heads": w.heads, "head_dim": w.head_dim, "ffn": w.ffn,
                   "window": w.window, "layers": w.layers, "model_flops_per_step": F},
        "mfu": round(tflops / PEAK_BF16_TFLOPS, 4),
        "hfu": round((F + R) / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "ms_per_step_median": round(ms_median, 4),
        "mfu_median": round(F / (ms_median * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "wall_s_timed": round(wall, 3),
        "roofline": roof,
        "stages_ms": {k: round(v, 4) for k, v in stages.items()},
        "stages_from": f"a separate pass of {K} steps with HIP events around each stage",
    }
    if not args.no_serial and w.layers == 1:
        out["serial_block"] = time_serial(w, inp, args.warmup, K, ms_step)
    if not args.no_optimizer:
        out["optimizer"] = time_lamb(st, args.warmup, K)
    if not args.no_variant:
        out["variant"] = time_variant(w, args.warmup, K, ms_step)
    if not args.no_fp8 and w.layers == 1:
        out["fp8"] = time_fp8(w, inp, args.warmup, K, ms_step)
        out["fp8_mx"] = time_fp8(w, inp, args.warmup, K, ms_step, "mx")
    if not args.no_cpu_baseline:
        print("bench: timing the fp64 oracle on host cores", file=sys.stderr, flush=True)
        cb = cpu_baseline(w, args.cpu_budget_s)
        cb.pop("seconds", None)
        cb["value"] = round(cb["value"], 5)
        out["cpu_baseline"] = cb
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
