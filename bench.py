"""Benchmark of the TTT-layer forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--no-b2048] [--copy-calibration]

A step is one forward pass of the layer over one batch of synthetic input (all
chunks of every (sequence, head) unit), launched through the C ABI. Inputs are
resident in HBM before the timed region. The default workload is TTT-Linear
with LayerNorm+residual, bf16 Q/K/V, B=8 H=12 N=2048 d=64 b=16 with per-token
step sizes. To keep the 256 MB Infinity Cache from serving repeated reads, the
steps rotate over four distinct device copies of the inputs and outputs.

With the default workload the line also carries a "b2048" object: the same
measurement for the large-chunk workload (plain TTT-Linear, bf16, B=1 H=16
N=32768 d=128 b=2048), whose roofline is the bf16 MFMA peak; and "next_rows":
the block-causal outputs of that workload (chunk outputs with the chunk's
starting or ending weights) and the single-token decode step of B*H = 768
TTT-Linear+LN streams (d=64), each against the HBM roofline (decode steps are
timed as replays of a captured HIP graph, as a serving token loop runs them,
with the eager per-call time beside it), and the whole
layer (projections, key normalisation, inner TTT-Linear+LN, output LayerNorm +
residual + output projection; B=8 N=2048 D=768 H=12 d=64 b=16) against the
bf16 MFMA roofline of its GEMM work, and the backward of the b = 16 workload
(gradients with respect to Q, K, V, eta, W0, gamma, beta) against the fp32
matrix-core peak. "practical_peaks" gives, beside the published peaks the
rooflines use, what a plain copy kernel and a bf16 MFMA loop reach on the
device, with its compute-unit count and clock.

Prints ONE JSON line (stdout). Diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from weights_ttt_layer_amd import workloads as wlm  # noqa: E402
from weights_ttt_layer_amd.profile_summary import COPY_BYTES, source_digest  # noqa: E402

DEFAULT_WORKLOAD = "linear_ln_bf16_B8H12N2048_d64_b16"
LARGE_WORKLOAD = "linear_bf16_B1H16N32768_d128_b2048"
DECODE_WORKLOAD = "decode_ln_bf16_B64H12_d64"
OTHER_CONFIGS = ["linear_f32_B1H1N256_d64_b16", "linear_ln_bf16_B16H12N8192_d64_b16", "mlp_bf16_B4H12N4096_d64_b16"]
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
ROTATE = 4
# Distinct input sets a timed loop walks through: at least ROTATE, and enough
# that their bytes exceed twice the 256 MB Infinity Cache, so repeated steps
# cannot be served from it (capped for the tiny single-unit workload, which is
# latency bound).
MALL_BYTES = 256 * 1024 * 1024
MAX_ROTATE = 64
METRIC = "TTT layer fwd tokens/sec"
# Worker threads of the CPU baseline: the host's CPU share that goes with one GPU.
CPU_THREADS_CAP = 16


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic traffic and work of one launch
# ---------------------------------------------------------------------------

def chunk_rows(N, b):
    full, rem = divmod(N, b)
    return [b] * full + ([rem] if rem else [])


def algorithmic_bytes(wl: wlm.Workload) -> int:
    """Compulsory HBM bytes: read Q,K,V (+eta), write Z (fp32), read and write the state."""
    es = 2 if wl.dtype == "bf16" else 4
    tok = wl.B * wl.H * wl.N
    b = 3 * tok * wl.d * es + tok * wl.d * 4
    if wl.eta == "sigmoid":
        b += tok * 4
    state = wl.d * wl.d if wl.kind != "mlp" else 2 * wl.d * wl.hidden
    b += 2 * wl.B * wl.H * state * 4
    if wl.kind in ("ln", "mlp"):
        b += 2 * wl.H * wl.d * 4
    return b


def algorithmic_flops(wl: wlm.Workload) -> int:
    """Per chunk of n rows: linear 6 n d^2 + 2 d n(n+1); MLP 56 n d^2 + 10 d n(n+1)
    (the tril products counted over their causal half only)."""
    d = wl.d
    f = 0
    for n in chunk_rows(wl.N, wl.b):
        if wl.kind == "mlp":
            f += 56 * n * d * d + 10 * d * n * (n + 1)
        else:
            f += 6 * n * d * d + 2 * d * n * (n + 1)
    return f * wl.B * wl.H


def rotation(set_bytes: int) -> int:
    """Number of distinct input/output sets for a loop whose sets are `set_bytes` each."""
    need = -(-2 * MALL_BYTES // max(1, set_bytes))
    return int(min(MAX_ROTATE, max(ROTATE, need)))


def cpu_threads() -> int:
    return min(len(os.sched_getaffinity(0)), CPU_THREADS_CAP)


def timed(stream, steps: int, step):
    """Launch `steps` steps with a HIP event recorded on `stream` before each and
    after the last. Returns (mean ms over the whole bracket, median ms of the
    per-step intervals)."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record(stream)
    for i in range(steps):
        step(i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    return evs[0].elapsed_time(evs[steps]) / steps, float(np.median(per))


def measured_traffic(wl: wlm.Workload, path_key: str, variant: str = "dual"):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when there is none for this workload or the kernel source changed since."""
    suffix = "" if variant == "dual" else f"_{variant}"
    path = os.path.join(ROOT, "profiles", f"traffic_{wl.name}{suffix}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != source_digest(path_key):
        return None
    return rec.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------

def run_gpu(wl: wlm.Workload, inp: wlm.Inputs, steps: int, warmup: int, variant: str = "dual"):
    """Average time of one launch (ms), from HIP events recorded on the stream the
    launches go to, over `steps` back-to-back launches after `warmup` untimed ones.
    variant: "dual" (ttt_linear_fwd / ttt_mlp_fwd), "block_before", "block_after"
    (ttt_linear_fwd_block) or "decode" (ttt_linear_decode, one token per stream,
    the state updated in place)."""
    import torch
    from weights_ttt_layer_amd import (linear_decode, linear_fwd, linear_fwd_block, linear_workspace_bytes,
                                       mlp_fwd)

    dev = torch.device("cuda:0")
    base = wlm.to_device(inp, dev)
    B, H, N, d = wl.B, wl.H, wl.N, wl.d
    set_bytes = sum(t.numel() * t.element_size() for t in base.values() if t is not None)
    if variant == "decode":      # the set is one token of every stream and the state
        set_bytes = (base["w0"].numel() * 4 + 3 * B * H * d * base["q"].element_size() + B * H * d * 4)
    else:
        set_bytes += B * H * N * d * 4
    nrot = rotation(set_bytes)
    sets = [base] + [{k: (None if t is None else t.clone()) for k, t in base.items()}
                     for _ in range(nrot - 1)]
    outs = []
    for s in sets:
        if variant == "decode":
            for key in ("q", "k", "v"):
                s[key] = s[key][:, :, 0].contiguous()
            if s["eta"] is not None:
                s["eta"] = s["eta"][:, :, 0].contiguous()
            outs.append((torch.empty((B, H, d), dtype=torch.float32, device=dev),))
            continue
        z = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
        if wl.kind == "mlp":
            outs.append((z, torch.empty_like(s["w1"]), torch.empty_like(s["w2"])))
        else:
            ws_bytes = linear_workspace_bytes(wl.kind, s["q"].dtype, B, H, N, d, wl.b)
            ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev) if ws_bytes else None
            outs.append((z, torch.empty_like(s["w0"]), ws))
    stream = torch.cuda.current_stream()

    def step(i, st=None):
        s, o = sets[i % nrot], outs[i % nrot]
        if variant == "decode":
            linear_decode(s["q"], s["k"], s["v"], s["w0"], s["eta"], kind=wl.kind, eta_const=inp.eta_const,
                          ln_gamma=s["gamma"], ln_beta=s["beta"], ln_eps=wl.ln_eps, z=o[0],
                          stream=stream if st is None else st)
        elif wl.kind == "mlp":
            mlp_fwd(s["q"], s["k"], s["v"], s["w1"], s["w2"], s["eta"], b=wl.b,
                    eta_const=inp.eta_const, ln_gamma=s["gamma"], ln_beta=s["beta"],
                    ln_eps=wl.ln_eps, z=o[0], w1_end=o[1], w2_end=o[2], stream=stream)
        elif variant in ("block_before", "block_after"):
            linear_fwd_block(s["q"], s["k"], s["v"], s["w0"], s["eta"], b=wl.b, apply=variant[6:],
                             kind=wl.kind, eta_const=inp.eta_const, ln_gamma=s["gamma"], ln_beta=s["beta"],
                             ln_eps=wl.ln_eps, z=o[0], w_end=o[1], workspace=o[2], stream=stream)
        else:
            linear_fwd(s["q"], s["k"], s["v"], s["w0"], s["eta"], b=wl.b, kind=wl.kind,
                       eta_const=inp.eta_const, ln_gamma=s["gamma"], ln_beta=s["beta"],
                       ln_eps=wl.ln_eps, z=o[0], w_end=o[1], workspace=o[2], stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ms_step, med = timed(stream, steps, step)
    extra = {"median_ms_per_step": med, "input_sets": nrot, "input_set_bytes": set_bytes}
    if variant == "decode":
        # A token loop in serving replays captured decode steps instead of paying
        # a host call per token: one HIP graph of one step per input set (their
        # states together exceed twice the Infinity Cache), replayed; the eager
        # per-call time is reported beside it.
        extra["eager_ms_per_step"] = ms_step
        extra["eager_median_ms_per_step"] = med
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream()
            for i in range(nrot):
                step(i, cap)
        graph.replay()
        torch.cuda.synchronize()
        reps = max(3, (10 * steps) // nrot)
        ms_rep, med_rep = timed(stream, reps, lambda i: graph.replay())
        ms_step, extra["median_ms_per_step"] = ms_rep / nrot, med_rep / nrot
        extra["graph_steps_timed"] = reps * nrot
    z = outs[(steps - 1) % nrot][0]
    finite = bool(torch.isfinite(z).all().item())
    del sets, outs, base
    torch.cuda.empty_cache()
    return ms_step, finite, extra


def copy_calibration(reps: int = 3):
    """Plain device-to-device copies of COPY_BYTES: the known traffic that scales
    the FETCH_SIZE / WRITE_SIZE counters of a profiled run."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def practical_peaks():
    """Beside the published peaks: the HBM rate a plain copy kernel reaches and the
    dense bf16 rate of an MFMA loop (both built here, libttt_peak.so), and the
    device's compute units and clock. The rooflines stay against the published
    peaks."""
    import torch
    from weights_ttt_layer_amd.binding import peak_copy, peak_device_info, peak_mfma

    info = peak_device_info(0)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)

    src = torch.arange(COPY_BYTES // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        peak_copy(src, dst, stream)
    torch.cuda.synchronize()
    reps = 10
    start.record(stream)
    for _ in range(reps):
        peak_copy(src, dst, stream)
    end.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * COPY_BYTES * reps / (start.elapsed_time(end) / 1e3) / 1e9
    copy_ok = bool(torch.equal(src, dst))
    del src, dst

    blocks, iters = 2 * info["compute_units"], 20000     # two waves per SIMD
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    peak_mfma(out, blocks, 100, stream)
    torch.cuda.synchronize()
    start.record(stream)
    flops = peak_mfma(out, blocks, iters, stream)
    end.record(stream)
    torch.cuda.synchronize()
    mfma_tfs = flops / (start.elapsed_time(end) / 1e3) / 1e12
    ok = copy_ok and bool(torch.isfinite(out).all().item())
    del out
    torch.cuda.empty_cache()
    log(f"[bench] practical peaks: copy {copy_gbs:.0f} GB/s, bf16 MFMA loop {mfma_tfs:.0f} TFLOP/s, "
        f"{info['compute_units']} CUs at {info['clock_khz'] / 1e3:.0f} MHz")
    return {"copy_GBps": copy_gbs, "copy_bytes": COPY_BYTES, "mfma_bf16_TFLOPs": mfma_tfs,
            "mfma_flops": flops, "checks_ok": ok, **info,
            "published": {"hbm_GBps": HBM_PEAK_GBS, "mfma_bf16_TFLOPs": MFMA_BF16_PEAK_TFS}}


def algorithmic_flops_variant(wl: wlm.Workload, variant: str) -> int:
    """Block-causal outputs drop the causal term: 6 d^2 per token-head (K W, the
    state step, Q W). A decode step is the same 6 d^2 for its single token."""
    if variant in ("block_before", "block_after", "decode"):
        return 6 * wl.d * wl.d * wl.B * wl.H * wl.N
    return algorithmic_flops(wl)


def measure(wl: wlm.Workload, inp: wlm.Inputs, steps: int, warmup: int, variant: str = "dual"):
    """tokens/s and the roofline object of one workload (and output variant)."""
    ms, finite, extra = run_gpu(wl, inp, steps, warmup, variant)
    if not finite:
        log(f"[bench] WARNING: non-finite output in {wl.name} {variant}")
    sec = ms / 1e3
    tokens = wl.B * wl.N
    nbytes = algorithmic_bytes(wl)
    flops = algorithmic_flops_variant(wl, variant)
    path_key = "large" if wl.b >= 256 else wl.kind
    if variant != "dual":
        path_key = variant
    mfma = {"bound": "mfma", "achieved": flops / sec / 1e12, "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s"}
    hbm = {"bound": "hbm", "achieved": nbytes / sec / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    for r in (mfma, hbm):
        r["frac"] = r["achieved"] / r["peak"]
    # large chunks and the MLP (arithmetic intensity at or above the ridge) are
    # priced against the matrix cores, the rest against HBM; the MLP reports both
    roof = mfma if ((wl.b >= 256 and variant == "dual") or wl.kind == "mlp") else hbm
    roof["traffic"] = measured_traffic(wl, path_key, variant)
    if wl.kind == "mlp":
        extra = dict(extra, roofline_hbm=dict(hbm, traffic=roof["traffic"]))
    log(f"[bench] {wl.name} {variant}: {ms*1e3:.1f} us/step, {tokens/sec:.4g} tokens/s, "
        f"{nbytes/sec/1e9:.1f} GB/s algorithmic, {flops/sec/1e12:.2f} TFLOP/s algorithmic")
    return ms, tokens / sec, nbytes, flops, roof, extra


def side_measurement(name: str, steps: int, warmup: int, variant: str):
    """One object of the JSON line for a workload other than the headline one."""
    idx = [w.name for w in wlm.WORKLOADS].index(name)
    wl = wlm.WORKLOADS[idx]
    ms, val, nbytes, flops, roof, extra = measure(wl, wlm.workload_inputs(idx), steps, warmup, variant)
    return {"workload": wl.name, "variant": variant, "value": val, "unit": "tokens/s", "ms_per_step": ms,
            "token_heads_per_s": val * wl.H, "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
            "roofline": roof, **extra}


MFMA_F32_PEAK_TFS = 157.3     # MI355X dense fp32 matrix, TFLOP/s


def bwd_algorithmic_bytes(wl: wlm.Workload) -> int:
    """Compulsory HBM bytes of one backward call: read Q, K, V, eta, W0, gamma,
    beta and the upstream dZ, dW_end; write dQ, dK, dV, deta, dW0, dgamma, dbeta."""
    es = 2 if wl.dtype == "bf16" else 4
    tok = wl.B * wl.H * wl.N
    state = wl.B * wl.H * wl.d * wl.d * 4
    hv = wl.H * wl.d * 4 if wl.kind == "ln" else 0
    read = 3 * tok * wl.d * es + tok * 4 + state + 2 * hv + tok * wl.d * 4 + state
    write = 3 * tok * wl.d * 4 + tok * 4 + state + 2 * hv
    return read + write


def bwd_algorithmic_flops(wl: wlm.Workload) -> int:
    """FLOPs of one backward call (ttt_linear_bwd), per chunk of n rows: ten
    products of an n x d by a d x d matrix (two to recompute the chunk-start
    state; K W_c, Q W_c, K dW, G dW^T, dHq W^T, dh W^T, Q^T dHq, K^T dh) at
    2 n d^2 each, and six causal n x n x d products (Q K^T, A G, dHq G^T,
    A^T dHq, dA K, dA^T Q) at n (n+1) d each."""
    d = wl.d
    f = sum(20 * n * d * d + 6 * n * (n + 1) * d for n in chunk_rows(wl.N, wl.b))
    return f * wl.B * wl.H


def bwd_measurement(steps: int, warmup: int):
    """Backward calls (ttt_linear_bwd) on the b = 16 benchmark workload with
    seeded upstream gradients; inputs and outputs rotate over ROTATE copies."""
    import torch
    from weights_ttt_layer_amd import linear_bwd

    idx = [w.name for w in wlm.WORKLOADS].index(DEFAULT_WORKLOAD)
    wl = wlm.WORKLOADS[idx]
    inp = wlm.workload_inputs(idx)
    dev = torch.device("cuda:0")
    dz, dw = wlm.upstream_grads(wl, 7)
    base = wlm.to_device(inp, dev)
    base["dz"] = torch.from_numpy(dz).to(dev)
    base["dw"] = torch.from_numpy(dw).to(dev)
    sets = [base] + [{k: (None if t is None else t.clone()) for k, t in base.items()} for _ in range(ROTATE - 1)]
    stream = torch.cuda.current_stream()
    kw = dict(b=wl.b, kind=wl.kind, eta_const=inp.eta_const, ln_eps=wl.ln_eps, stream=stream)

    def step(i):
        s = sets[i % ROTATE]
        return linear_bwd(s["q"], s["k"], s["v"], s["w0"], s["dz"], s["eta"], dw_end=s["dw"],
                          ln_gamma=s["gamma"], ln_beta=s["beta"], **kw)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    last = {}

    def keep(i):
        last["out"] = step(i)

    ms, med = timed(stream, steps, keep)
    out = last["out"]
    finite = bool(torch.isfinite(out["dQ"]).all().item())
    if not finite:
        log(f"[bench] WARNING: non-finite backward output in {wl.name}")
    del sets, base, out
    torch.cuda.empty_cache()
    sec = ms / 1e3
    flops = bwd_algorithmic_flops(wl)
    tokens = wl.B * wl.N
    roof = {"bound": "mfma", "achieved": flops / sec / 1e12, "peak": MFMA_F32_PEAK_TFS, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(wl, "backward", "backward")
    log(f"[bench] {wl.name} backward: {ms*1e3:.1f} us/step, {tokens/sec:.4g} tokens/s, "
        f"{flops/sec/1e12:.2f} TFLOP/s algorithmic (fp32)")
    return {"workload": wl.name, "variant": "backward", "value": tokens / sec, "unit": "tokens/s",
            "ms_per_step": ms, "median_ms_per_step": med, "algorithmic_flops": flops, "dtype": "f32",
            "roofline": roof}


def layer_algorithmic(wl: wlm.LayerWorkload):
    """Compulsory HBM bytes of one whole-layer call (read x, the four projection
    weights, eta, the state and the LayerNorm parameters; write y and the state)
    and its FLOPs (the three input projections, the inner model, the output
    projection; the output projection counted once although it runs on two bf16
    terms)."""
    HD = wl.H * wl.d
    tok = wl.B * wl.N
    nbytes = tok * wl.D * 2 + 4 * HD * wl.D * 2 + wl.B * wl.H * wl.N * 4 + tok * wl.D * 4
    nbytes += 2 * wl.B * wl.H * wl.d * wl.d * 4 + (4 if wl.kind == "ln" else 2) * HD * 4
    inner = wlm.Workload("inner", wl.kind, "f32", wl.B, wl.H, wl.N, wl.d, wl.b, "sigmoid")
    flops = 2 * tok * wl.D * 3 * HD + algorithmic_flops(inner) + 2 * tok * HD * wl.D
    return nbytes, flops


def layer_measurement(steps: int, warmup: int):
    """Whole-layer calls (ttt_layer_fwd) on the named layer workload. Per-call
    inputs (x, eta, the state) and outputs rotate over ROTATE device copies; the
    projection weights are shared, as they are across the calls of a model."""
    import torch
    from weights_ttt_layer_amd import layer_fwd, layer_workspace_bytes

    inp = wlm.layer_workload_inputs(0)
    wl = inp.wl
    dev = torch.device("cuda:0")
    base = wlm.layer_to_device(inp, dev)
    sets = [base] + [dict(base, x=base["x"].clone(), eta=base["eta"].clone(), w0=base["w0"].clone())
                     for _ in range(ROTATE - 1)]
    need = layer_workspace_bytes(wl.B, wl.N, wl.H, wl.d)
    outs = [(torch.empty((wl.B, wl.N, wl.D), dtype=torch.float32, device=dev), torch.empty_like(base["w0"]),
             torch.empty(need, dtype=torch.uint8, device=dev)) for _ in range(ROTATE)]
    stream = torch.cuda.current_stream()

    def step(i):
        s, o = sets[i % ROTATE], outs[i % ROTATE]
        layer_fwd(s["x"], s["wq"], s["wk"], s["wv"], s["wo"], s["w0"], s["gamma_o"], s["beta_o"], s["eta"],
                  H=wl.H, b=wl.b, kind=wl.kind, ln_gamma=s["gamma"], ln_beta=s["beta"], ln_eps=wl.ln_eps,
                  y=o[0], w_end=o[1], workspace=o[2], stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ms, med = timed(stream, steps, step)
    finite = bool(torch.isfinite(outs[(steps - 1) % ROTATE][0]).all().item())
    if not finite:
        log(f"[bench] WARNING: non-finite output in {wl.name}")
    del sets, outs, base
    torch.cuda.empty_cache()
    sec = ms / 1e3
    nbytes, flops = layer_algorithmic(wl)
    tokens = wl.B * wl.N
    roof = {"bound": "mfma", "achieved": flops / sec / 1e12, "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(wl, "layer", "layer")
    log(f"[bench] {wl.name}: {ms*1e3:.1f} us/step, {tokens/sec:.4g} tokens/s, "
        f"{flops/sec/1e12:.2f} TFLOP/s algorithmic")
    return {"workload": wl.name, "variant": "layer", "value": tokens / sec, "unit": "tokens/s",
            "ms_per_step": ms, "median_ms_per_step": med, "algorithmic_bytes": nbytes,
            "algorithmic_flops": flops, "roofline": roof}


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle as it stands
# ---------------------------------------------------------------------------

def cpu_baseline(wl: wlm.Workload, inp: wlm.Inputs, max_units: int, min_wall: float = 1.5):
    """The mini-batch primal fp64 oracle over whole sequences of the same inputs:
    one untimed run, then repeated runs until `min_wall` seconds have passed (at
    least three); the best run gives the rate."""
    import oracle
    threads = cpu_threads()
    nb = max(1, min(wl.B, max_units // wl.H))
    sl = slice(0, nb)
    q, k, v = inp.f64("q")[sl], inp.f64("k")[sl], inp.f64("v")[sl]
    eta = inp.eta_f64()[sl]

    def once():
        t0 = time.perf_counter()
        if wl.kind == "mlp":
            oracle.mlp(oracle.MINIBATCH, q, k, v, eta, inp.f64("w1")[sl], inp.f64("w2")[sl],
                       wl.b, inp.f64("gamma"), inp.f64("beta"), wl.ln_eps, nthreads=threads)
        else:
            kind = oracle.LN if wl.kind == "ln" else oracle.PLAIN
            oracle.linear(oracle.MINIBATCH, kind, q, k, v, eta, inp.f64("w0")[sl], wl.b,
                          None if inp.gamma is None else inp.f64("gamma"),
                          None if inp.beta is None else inp.f64("beta"), wl.ln_eps, nthreads=threads)
        return time.perf_counter() - t0

    once()
    times, total = [], 0.0
    while len(times) < 3 or total < min_wall:
        times.append(once())
        total += times[-1]
    best = min(times)
    return {
        "value": nb * wl.N / best,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"mini-batch primal fp64 oracle over {nb} of {wl.B} sequences x {wl.H} heads x "
                  f"{wl.N} tokens, best of {len(times)} runs ({best:.3f} s each at best, "
                  f"{total:.1f} s wall in all)",
    }


def _oracle_rate(run, tokens: int, sample: str, min_wall: float = 1.0):
    """Best rate of `run` (the oracle on a bounded sample) over at least two runs
    and `min_wall` seconds; `tokens` is what one run processes."""
    threads = cpu_threads()
    times, total = [], 0.0
    while len(times) < 2 or total < min_wall:
        t0 = time.perf_counter()
        run(threads)
        times.append(time.perf_counter() - t0)
        total += times[-1]
    best = min(times)
    return {"value": tokens / best, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{sample}; best of {len(times)} runs ({best:.3f} s at best, {total:.1f} s wall)"}


_LARGE_UNIT0 = None


def _large_unit0():
    """The large-chunk workload's first head, generated once."""
    global _LARGE_UNIT0
    if _LARGE_UNIT0 is None:
        idx = [w.name for w in wlm.WORKLOADS].index(LARGE_WORKLOAD)
        _LARGE_UNIT0 = (wlm.WORKLOADS[idx], wlm.workload_inputs(idx).unit(0, 0))
    return _LARGE_UNIT0


def cpu_baseline_side(kind: str):
    """The oracle timed beside one of the side measurements, on a bounded sample
    of the same workload."""
    import oracle
    if kind in ("b2048", "block_before", "block_after"):
        wl, inp = _large_unit0()
        mode = {"b2048": oracle.MINIBATCH, "block_before": oracle.BLOCK_BEFORE,
                "block_after": oracle.BLOCK_AFTER}[kind]
        args = (inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.eta_f64(), inp.f64("w0"), wl.b)
        return _oracle_rate(lambda th: oracle.linear(mode, oracle.PLAIN, *args, nthreads=th), wl.N,
                            f"fp64 oracle ({'mini-batch primal' if kind == 'b2048' else kind}) over one of "
                            f"{wl.H} heads x {wl.N} tokens")
    if kind == "decode":
        idx = [w.name for w in wlm.WORKLOADS].index(DECODE_WORKLOAD)
        wl = wlm.WORKLOADS[idx]
        inp = wlm.workload_inputs(idx)
        args = (inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.eta_f64(), inp.f64("w0"), 1, inp.f64("gamma"),
                inp.f64("beta"), wl.ln_eps)
        return _oracle_rate(lambda th: oracle.linear(oracle.ONLINE, oracle.LN, *args, nthreads=th), wl.B,
                            f"fp64 oracle, one online step for all {wl.B * wl.H} streams")
    if kind == "layer":
        li = wlm.layer_workload_inputs(0)
        wl = li.wl
        s1 = slice(0, 1)
        args = (li.f64("x")[s1], li.f64("wq"), li.f64("wk"), li.f64("wv"), li.f64("wo"), li.f64("eta")[s1],
                li.f64("w0")[s1], wl.b, wl.H, li.f64("gamma"), li.f64("beta"), li.f64("gamma_o"),
                li.f64("beta_o"), wl.ln_eps)
        return _oracle_rate(lambda th: oracle.layer(oracle.LN, *args, nthreads=th), wl.N,
                            f"fp64 oracle (numpy projections + C inner model) over 1 of {wl.B} sequences "
                            f"x {wl.N} tokens")
    if kind == "backward":
        idx = [w.name for w in wlm.WORKLOADS].index(DEFAULT_WORKLOAD)
        wl = wlm.WORKLOADS[idx]
        inp = wlm.workload_inputs(idx)
        dz, dw = wlm.upstream_grads(wl, 7)
        s1 = slice(0, 1)
        args = (inp.f64("q")[s1], inp.f64("k")[s1], inp.f64("v")[s1], inp.eta_f64()[s1], inp.f64("w0")[s1], wl.b,
                dz[s1].astype(np.float64), dw[s1].astype(np.float64), inp.f64("gamma"), inp.f64("beta"),
                wl.ln_eps)
        return _oracle_rate(lambda th: oracle.linear_bwd(oracle.LN, *args, nthreads=th), wl.N,
                            f"fp64 oracle backward over 1 of {wl.B} sequences x {wl.H} heads x {wl.N} tokens")
    raise ValueError(kind)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(wlm.BY_NAME))
    ap.add_argument("--variant", default=None, choices=["dual", "block_before", "block_after", "decode"],
                    help="outputs to measure (default: decode for the decode workload, else dual)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the fp32 single-unit, long-context and TTT-MLP workloads that accompany "
                         "the default workload")
    ap.add_argument("--no-b2048", action="store_true",
                    help="skip the large-chunk measurement that accompanies the default workload")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run plain device copies of a known size (counter calibration)")
    ap.add_argument("--cpu-units", type=int, default=96,
                    help="cap on (sequence, head) units in the CPU-baseline sample")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the TTT forward shards "
              f"over (sequence, head) units with no communication, so N GPUs run N independent "
              f"copies of this benchmark.", file=sys.stderr)
        sys.exit(2)

    idx = [w.name for w in wlm.WORKLOADS].index(args.workload)
    wl = wlm.WORKLOADS[idx]
    inp = wlm.workload_inputs(idx)
    log(f"[bench] workload {wl.name}: generated inputs")

    variant = args.variant or ("decode" if wl.name == DECODE_WORKLOAD else "dual")
    ms, value, nbytes, flops, roof, extra = measure(wl, inp, args.steps, args.warmup, variant)

    b2048 = None
    next_rows = None
    configs = None
    if wl.name == DEFAULT_WORKLOAD and variant == "dual" and not args.no_configs:
        # the other forward workloads: fp32 single unit, long context, TTT-MLP
        configs = {name: side_measurement(name, args.steps, args.warmup, "dual") for name in OTHER_CONFIGS}
    if wl.name == DEFAULT_WORKLOAD and variant == "dual" and not args.no_b2048:
        b2048 = side_measurement(LARGE_WORKLOAD, args.steps, args.warmup, "dual")
        next_rows = {
            "block_before": side_measurement(LARGE_WORKLOAD, args.steps, args.warmup, "block_before"),
            "block_after": side_measurement(LARGE_WORKLOAD, args.steps, args.warmup, "block_after"),
            "decode": side_measurement(DECODE_WORKLOAD, args.steps, args.warmup, "decode"),
            "layer": layer_measurement(args.steps, args.warmup),
            "backward": bwd_measurement(max(3, args.steps // 5), min(args.warmup, 2)),
        }

    if not args.no_cpu_baseline and next_rows is not None:
        b2048["cpu_baseline"] = cpu_baseline_side("b2048")
        for key in next_rows:
            next_rows[key]["cpu_baseline"] = cpu_baseline_side(key)
        log("[bench] side cpu baselines: " + ", ".join(
            f"{k} {v['cpu_baseline']['value']:.3g}" for k, v in [("b2048", b2048), *next_rows.items()]))

    if not args.no_cpu_baseline and configs is not None:
        for name, obj in configs.items():
            idx = [w.name for w in wlm.WORKLOADS].index(name)
            obj["cpu_baseline"] = cpu_baseline(wlm.WORKLOADS[idx], wlm.workload_inputs(idx), args.cpu_units)
        log("[bench] config cpu baselines: " + ", ".join(
            f"{k} {v['cpu_baseline']['value']:.3g}" for k, v in configs.items()))

    if args.copy_calibration:
        copy_calibration()
        log(f"[bench] calibration copies of {COPY_BYTES} bytes done")

    cpu = None
    if not args.no_cpu_baseline and variant == "dual":
        cpu = cpu_baseline(wl, inp, args.cpu_units)
        log(f"[bench] cpu baseline: {cpu['value']:.4g} tokens/s on {cpu['cores']} threads")

    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "kind": wl.kind, "B": wl.B, "H": wl.H, "N": wl.N,
                   "d": wl.d, "b": wl.b, "qkv_dtype": wl.dtype, "state_dtype": "f32",
                   "eta": wl.eta, "token_heads_per_s": value * wl.H,
                   "algorithmic_bytes": nbytes, "algorithmic_flops": flops},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    rec["config"].update(extra)
    if configs is not None:
        rec["configs"] = configs
    if b2048 is not None:
        rec["b2048"] = b2048
        rec["practical_peaks"] = practical_peaks()
    if next_rows is not None:
        rec["next_rows"] = next_rows
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
