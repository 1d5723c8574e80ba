"""Benchmark of the HAM layer on one MI355X.

Default run (N=1): the layer forward at the 800M-model shape (bf16 I/O, fp32
state: B=8, H=16, d=128, T=4096, threshold per head for KV usage rho=0.5) timed
over K steps with inputs resident in HBM; then the decode workload (batch 32,
H=16, d=128, 32K-token prefix at rho=0.5, 256 decode steps).  Per-kernel times
come from HIP events recorded by the library on the launch stream; the oracle
is timed on a bounded sample on the host cores as a CPU baseline.

Prints ONE JSON line on stdout.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_TFLOPS = 157.3
# (The library is built with packed fp32 instructions disabled.  That does not halve the
# vector rate: a plain fp32 FMA of a 64-lane wave issues about every 2 cycles on a SIMD,
# 32 lanes per clock, so 157.3 TFLOP/s is the fp32 roof of vector and matrix-core work.)
CHUNK = 64
STAGES = ["rnn_prep", "rnn_state", "route", "compact", "attention"]


LEGS = ("small", "sweep", "router", "rope", "packed", "blocks", "kv_heads", "paper", "backward",
        "rnn_backward", "long")


def want(args, leg):
    return leg in getattr(args, "leg_set", set(LEGS))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def copy_calibration(dev):
    """A plain device copy of known size (1 GiB read, 1 GiB written), three times:
    the reference reading for the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = 1 << 30
    x = torch.empty(n, dtype=torch.uint8, device=dev)
    x.fill_(1)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: 3 copies of {n} bytes")


def device_info(dev):
    """Name, architecture, compute units and clock of the GPU, and the host's CPU model
    and core counts (rocminfo for the GPU agent, /proc/cpuinfo for the host)."""
    import subprocess
    import torch
    p = torch.cuda.get_device_properties(dev)
    info = dict(name=p.name, arch=getattr(p, "gcnArchName", ""), cus=p.multi_processor_count,
                mem_gib=round(p.total_memory / 2 ** 30, 1))
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
        for blk in txt.split("*******"):
            if "gfx950" in blk and "Compute Unit" in blk:
                for ln in blk.splitlines():
                    if "Max Clock Freq" in ln:
                        info["max_clock_mhz"] = int(ln.split(":")[1].split()[0])
                    if ln.strip().startswith("Compute Unit:"):
                        info["rocminfo_cus"] = int(ln.split(":")[1])
                break
    except (OSError, subprocess.SubprocessError, ValueError):
        pass
    model = ""
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    info.update(cpu_model=model, nproc=os.cpu_count(), cpu_affinity=avail)
    return info


def stream_copy_gbs(dev, nbytes=1 << 30, reps=5):
    """Achieved bandwidth of a plain device-to-device copy (bytes read + written per
    second): the practical ceiling next to the 8 TB/s published figure."""
    import torch
    x = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    x.fill_(1)
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / reps
    del x, y
    torch.cuda.empty_cache()
    return 2 * nbytes / sec / 1e9


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "traffic_layer_bf16_B8_H16_T4096_d128.md")


def measured_traffic(kernel_prefix):
    """HBM bytes per launch of a kernel from the committed counter summary, or None
    when there is no summary for it or the kernel source changed since (the summary
    records the SHA-256 of the source file it was taken with)."""
    import re
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    text = open(TRAFFIC_SUMMARY).read()
    m = re.search(r"^traffic\s+" + re.escape(kernel_prefix) + r"\s+(\S+)\s+(\d+)\s+(\S+)\s*$", text, re.M)
    if not m:
        return None
    src, nbytes, sha = m.group(1), int(m.group(2)), m.group(3)
    if kernel_source_sha(src) != sha:
        return None
    return nbytes


def kernel_source_sha(src):
    """SHA-256 over a kernel's source file and the two shared device headers."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "attention_sequence_mixing_amd", "csrc")
    for path in (os.path.join(ROOT, src), os.path.join(csrc, "ham_common.h"),
                 os.path.join(csrc, "ham_internal.h")):
        if not os.path.exists(path):
            return None
        h.update(open(path, "rb").read())
    return h.hexdigest()


def rnn_flops_per_token_head(d, C=CHUNK):
    """Chunked gated delta rule per token and head (C = 64) plus the fit-error
    score: Tab. E.11 subtotal per head + the Tab. E.13 selection term."""
    return 1 + 3.5 * C + C * C / 2 + 6 * C * d + 4 * C * d + 6 * d * d + 12 * d


def rnn_prep_flops_per_token_head(d, C=CHUNK):
    """The Tab. E.11 rows done by the chunk-parallel prep kernel: g cumsum,
    compute A (C(2d + 3.5) per token), invert A (C^2/2) and the Q K^T half of the
    output row (2 C d)."""
    return 1 + 3.5 * C + C * C / 2 + 2 * C * d + 2 * C * d


def rnn_state_flops_per_token_head(d, C=CHUNK):
    """The rest of Tab. E.11 (recompute w/u 4Cd, the state recurrence 4d^2, the
    output's 2d^2 + 2Cd) plus the 12d selection term of Tab. E.13: the state kernel."""
    return rnn_flops_per_token_head(d, C) - rnn_prep_flops_per_token_head(d, C)


def attn_flops_per_pair(d):
    """QK^T 2d + softmax 4 + PV 2d per visible (query, key) pair (Tab. E.12)."""
    return 4 * d + 4


def collect_stages(lib, n):
    """Stage times (ms, mean over the recorded calls) from the library's HIP events,
    which it records on the launch stream around each kernel of the armed calls."""
    import ctypes
    S = 5
    buf = (ctypes.c_float * (n * S))()
    ncalls = ctypes.c_int(0)
    kinds = (ctypes.c_int * n)()
    rc = lib.ham_profile_stop(buf, n * S, ctypes.byref(ncalls), kinds)
    if rc != 0:
        raise RuntimeError(lib.ham_last_error().decode())
    arr = np.frombuffer(buf, dtype=np.float32).reshape(n, S)[: ncalls.value]
    return [float(x) for x in arr.astype(np.float64).mean(axis=0)]   # ms per stage


def time_steps(step, steps, warmup):
    """Run warmup untimed steps, then time exactly `steps` steps between two events
    on torch's current stream (the launch stream), with nothing else recorded; then
    run `steps` more with the library recording HIP events on that stream around each
    kernel, for the per-stage times (those events add about 20 us to a step at the
    layer shape, so they stay out of the timed steps).  Returns (ms per step, stage
    times in ms)."""
    import torch
    from attention_sequence_mixing_amd import _lib
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    lib = _lib.lib()
    lib.ham_profile_start(steps)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return ms, collect_stages(lib, steps)


def visible_pairs(routed):
    """Sum over queries of the routed tokens at or before them (the attention's exact
    (query, key) pair count for per-token routing without a continued cache)."""
    import torch
    return float(torch.cumsum(routed.to(torch.int64), dim=1).sum().item())


def stage_report(stages, B, T, H, d, pairs, nroute):
    """Per-kernel achieved rate against the roof of the arithmetic each kernel runs:
    the prep kernel's Gram products are a small share of its HBM traffic (67 FLOP/B);
    the state kernel and attention run bf16 MFMA (the state kernel's fp32-accurate
    products as split bf16 terms; only algorithmic FLOPs are counted)."""
    BTH = B * T * H
    state_flops = BTH * rnn_state_flops_per_token_head(d)
    att_flops = pairs * attn_flops_per_pair(d)
    # algorithmic bytes (inputs read once, outputs written once)
    bytes_ = {"rnn_prep": BTH * (2 * d * 2 + 8),                # q, k bf16; beta, g fp32
              "route": BTH * (16 * (d // 64) + 4 + 1),          # score partials (one float4 per 64
                                                                # state columns) in; e, routed out
              "compact": BTH * (1 + 4) + nroute * (2 * (2 * d * 2) + 4)}
    per = []
    for i, nm in enumerate(STAGES):
        sec = max(stages[i], 1e-9) / 1e3
        if nm in ("rnn_state", "attention"):
            f = state_flops if nm == "rnn_state" else att_flops
            per.append(dict(stage=nm, ms=stages[i], bound="mfma", unit="TFLOP/s",
                            achieved=f / sec / 1e12, peak=PEAK_BF16_TFLOPS))
        else:
            per.append(dict(stage=nm, ms=stages[i], bound="hbm", unit="GB/s",
                            achieved=bytes_[nm] / sec / 1e9, peak=PEAK_HBM_GBS))
        per[-1]["frac"] = per[-1]["achieved"] / per[-1]["peak"]
    return per


def rounded(d):
    return {k: (round(v, 4) if isinstance(v, float) else v) for k, v in d.items()}


def bench_rho_sweep(args, dev, w, t, e_scores, rhos):
    """The layer at the same inputs for each targeted KV fraction rho (tau per head
    from the fit-error scores of the RNN-only pass): rho = 0 routes nothing (pure
    gated DeltaNet plus an empty attention), rho = 1 routes every token (full causal
    attention next to the RNN)."""
    import torch
    import attention_sequence_mixing_amd as ham
    from attention_sequence_mixing_amd.inputs import tau_for_rho
    out = []
    plan = ham.ForwardPlan(w.B, w.T, w.H, w.d, w.d, torch.bfloat16, dev, scale=w.attn_scale)
    for rho in rhos:
        tau = torch.from_numpy(tau_for_rho(e_scores, rho)).to(dev)
        ms, stages = time_steps(lambda: plan(t["q"], t["k"], t["v"], t["beta"], t["g"], tau),
                                args.steps, args.warmup)
        pairs = visible_pairs(plan.routed)
        nroute = float(plan.count.sum().item())
        per = stage_report(stages, w.B, w.T, w.H, w.d, pairs, nroute)
        rho_m = nroute / (w.B * w.T * w.H)
        log(f"[bench] rho sweep {rho}: {ms:.3f} ms/step, rho {rho_m:.4f}, pairs {pairs:.3e}, "
            f"stages {dict(zip(STAGES, [round(x, 4) for x in stages]))}")
        out.append(dict(workload=f"{w.name}_rho{rho}", rho_target=rho, rho_measured=round(rho_m, 6),
                        ms_per_step=round(ms, 4), tokens_per_s=round(w.B * w.T / (ms / 1e3), 1),
                        visible_pairs=pairs, stages=[rounded(x) for x in per]))
    return out


def bench_small(args, dev):
    """The small fp32 workload (B 1, H 2, T 256, d 64, scale 1/8, rho 0.5): launch-latency
    bound; reported as time per forward."""
    import torch
    import attention_sequence_mixing_amd as ham
    from attention_sequence_mixing_amd.inputs import SMALL, make_workload, tau_for_rho
    w = SMALL
    inp = make_workload(w)
    t = {n: torch.from_numpy(a).to(dev) for n, a in inp.items()}
    st = ham.ham_route_stats(t["k"], t["v"], t["beta"], t["g"],
                             torch.full((w.H,), float("inf"), device=dev), want_rho=False)
    tau = torch.from_numpy(tau_for_rho(st["e"].cpu().numpy(), w.rho)).to(dev)
    plan = ham.ForwardPlan(w.B, w.T, w.H, w.d, w.d, torch.float32, dev, scale=w.attn_scale)
    ms, stages = time_steps(lambda: plan(t["q"], t["k"], t["v"], t["beta"], t["g"], tau),
                            max(args.steps, 50), max(args.warmup, 20))
    rho = float(plan.count.sum().item()) / (w.B * w.T * w.H)
    log(f"[bench] {w.name}: {ms * 1e3:.1f} us/step, stages {dict(zip(STAGES, [round(x, 4) for x in stages]))}")
    return dict(workload=w.name, us_per_step=round(ms * 1e3, 2), tokens_per_s=round(w.B * w.T / (ms / 1e3), 1),
                rho_measured=round(rho, 6), stages_ms=dict(zip(STAGES, [round(x, 4) for x in stages])))


def bench_forward(args, dev):
    import torch
    import attention_sequence_mixing_amd as ham
    from attention_sequence_mixing_amd.inputs import LAYER, RHO_SWEEP, make_workload, tau_for_rho

    w = LAYER
    t0 = time.time()
    inp = make_workload(w)
    dt = torch.bfloat16
    t = {n: torch.from_numpy(a).to(dev) for n, a in inp.items()}
    for n in ("q", "k", "v"):
        t[n] = t[n].to(dt)
    log(f"[bench] inputs {w.name} drawn in {time.time() - t0:.1f}s")
    st = ham.ham_route_stats(t["k"], t["v"], t["beta"], t["g"],
                             torch.full((w.H,), float("inf"), device=dev), want_rho=False)
    e_scores = st["e"].cpu().numpy()
    tau_np = tau_for_rho(e_scores, w.rho)
    tau = torch.from_numpy(tau_np).to(dev)
    # The rho sweep runs first: besides its own numbers it brings the GPU clock to its
    # loaded steady state before the headline measurement.
    sweep = bench_rho_sweep(args, dev, w, t, e_scores, [r for r in RHO_SWEEP if r != w.rho]) \
        if want(args, "sweep") else None
    plan = ham.ForwardPlan(w.B, w.T, w.H, w.d, w.d, dt, dev, scale=w.attn_scale)
    t_start = time.perf_counter()
    ms, stages = time_steps(lambda: plan(t["q"], t["k"], t["v"], t["beta"], t["g"], tau),
                            args.steps, args.warmup)
    wall = time.perf_counter() - t_start

    count = plan.count
    rho = float(count.sum().item()) / (w.B * w.T * w.H)
    pairs = visible_pairs(plan.routed)
    nroute = float(count.sum().item())
    BTH = w.B * w.T * w.H
    rnn_flops = BTH * rnn_flops_per_token_head(w.d)
    att_flops = pairs * attn_flops_per_pair(w.d)
    per = stage_report(stages, w.B, w.T, w.H, w.d, pairs, nroute)
    dom = max(per, key=lambda x: x["ms"])
    if sweep is not None:
        sweep.insert([r for r in RHO_SWEEP].index(w.rho),
                     dict(workload=f"{w.name}_rho{w.rho}", rho_target=w.rho, rho_measured=round(rho, 6),
                          ms_per_step=round(ms, 4), tokens_per_s=round(w.B * w.T / (ms / 1e3), 1),
                          visible_pairs=pairs, stages=[rounded(x) for x in per], note="the headline run"))
    router = rope = packed = blocks = kvh = paper = bwd = rbwd = None
    from attention_sequence_mixing_amd.inputs import make_doc_start, make_inputs_torch
    if want(args, "router"):
        router = bench_router(args, dev, w, t)
    if want(args, "rope"):
        rope = bench_variant(args, dev, w, t, tau, "rope500000", rope_base=500000.0)
    if want(args, "packed"):
        packed = bench_variant(args, dev, w, t, tau, "packed_docs_mean1024_rope500000",
                               rope_base=500000.0, doc_start=make_doc_start(w.B, w.T, 1024, w.seed))
    if want(args, "blocks"):
        # block-contiguous routing: 64-token blocks, tau per head for half of the
        # blocks on their mean score
        nb = 64
        means = st["e"].view(w.B, w.T // nb, nb, w.H).mean(dim=2).contiguous()
        tau_b = ham.ham_select_tau(means, w.rho)
        blocks = bench_variant(args, dev, w, t, tau_b, f"block_routing{nb}", route_block=nb)
    if want(args, "kv_heads"):
        # the paper's head layout at the kernels' sizes: twice the RNN heads as KV heads,
        # key size 128, value size half the RNN's (their outputs tile the RNN heads')
        att = make_inputs_torch(w.B, w.T, 2 * w.H, w.d, w.d // 2, dtype="bf16", seed=w.seed + 3,
                                device=dev)
        kvh = bench_variant(args, dev, w, t, tau, f"kv_heads{2 * w.H}_dk{w.d}_dv{w.d // 2}", attn=att)
    if want(args, "paper"):
        paper = bench_paper_heads(args, dev, w)
    if want(args, "backward"):
        bwd = bench_backward(args, dev, w, t, plan, pairs)
    if want(args, "rnn_backward"):
        rbwd = bench_rnn_backward(args, dev, w, t)
    return dict(w=w, ms=ms, wall=wall, tokens_per_s=w.B * w.T / (ms / 1e3), stages=per, dom=dom,
                rho=rho, pairs=pairs, tau=tau_np, inp=inp, rnn_flops=rnn_flops, att_flops=att_flops,
                router=router, rope=rope, packed=packed, blocks=blocks, kvh=kvh, paper=paper, bwd=bwd,
                rbwd=rbwd, sweep=sweep)


def bench_variant(args, dev, w, t, tau, label, rope_base=0.0, doc_start=None, route_block=0,
                  attn=None):
    """The same layer with the fit-error routing, plus RoPE on the attention query and
    key (rope_base > 0), same-document masking of packed sequences (doc_start [B,T]),
    block-contiguous routing (route_block > 1, with its own tau) and/or attention
    heads of their own geometry (attn: dict q, k, v of the attention path)."""
    import torch
    import attention_sequence_mixing_amd as ham
    kv = {} if attn is None else dict(kv_heads=attn["q"].shape[2], dk_kv=attn["q"].shape[3],
                                      dv_kv=attn["v"].shape[3])
    scale = w.attn_scale if attn is None else attn["q"].shape[3] ** -0.5
    plan = ham.ForwardPlan(w.B, w.T, w.H, w.d, w.d, torch.bfloat16, dev, scale=scale,
                           rope_base=rope_base, route_block=route_block, **kv)
    ds = None if doc_start is None else torch.from_numpy(doc_start.astype(np.int32)).to(dev)
    qa, ka, va = (None, None, None) if attn is None else (attn["q"], attn["k"], attn["v"])

    def step():
        plan(t["q"], t["k"], t["v"], t["beta"], t["g"], tau, doc_start=ds, q_attn=qa, k_attn=ka,
             v_attn=va)

    ms, stages = time_steps(step, args.steps, args.warmup)
    names = ["rnn_prep", "rnn_state", "route", "compact", "attention"]
    rho = float(plan.count.sum().item()) / (w.B * w.T * plan.count.shape[1])
    log(f"[bench] {label}: {ms:.3f} ms/step, rho {rho:.4f}, "
        f"stages {dict(zip(names, [round(x, 4) for x in stages]))}")
    return dict(workload=f"{w.name}_{label}", ms_per_step=round(ms, 4),
                tokens_per_s=round(w.B * w.T / (ms / 1e3), 1), rho_measured=round(rho, 6),
                stages_ms=dict(zip(names, [round(x, 4) for x in stages])))


def bench_paper_heads(args, dev, w, steps=5, warmup=5):
    """The 800M model's layer geometry ("Hybrid Associative Memories" §4 and Tab. E.1 at
    hidden size 1792): 5 RNN heads of key/value size 256/384 and 10 KV heads of 128/192,
    B 8, T 4096, bf16, rho 0.5 per RNN head.  The RNN heads run on the token-serial
    kernel (the chunked state kernel takes d_k <= 128), so this measures that path."""
    import torch
    import attention_sequence_mixing_amd as ham
    from attention_sequence_mixing_amd.inputs import make_inputs_torch
    H, dk, dv, HK, dkk, dvk = 5, 256, 384, 10, 128, 192
    t = make_inputs_torch(w.B, w.T, H, dk, dv, dtype="bf16", seed=w.seed + 5, device=dev)
    att = make_inputs_torch(w.B, w.T, HK, dkk, dvk, dtype="bf16", seed=w.seed + 6, device=dev)
    st = ham.ham_route_stats(t["k"], t["v"], t["beta"], t["g"], torch.full((H,), float("inf"), device=dev),
                             want_rho=False)
    tau = ham.ham_select_tau(st["e"], w.rho)
    plan = ham.ForwardPlan(w.B, w.T, H, dk, dv, torch.bfloat16, dev, scale=dkk ** -0.5, kv_heads=HK,
                           dk_kv=dkk, dv_kv=dvk)

    def step():
        plan(t["q"], t["k"], t["v"], t["beta"], t["g"], tau, q_attn=att["q"], k_attn=att["k"],
             v_attn=att["v"])

    ms, stages = time_steps(step, steps, warmup)
    names = ["rnn_prep", "rnn_state", "route", "compact", "attention"]
    rho = float(plan.count.sum().item()) / (w.B * w.T * HK)
    label = f"paper_heads_bf16_B{w.B}_T{w.T}_rnn{H}x{dk}x{dv}_kv{HK}x{dkk}x{dvk}"
    log(f"[bench] {label}: {ms:.3f} ms/step, rho {rho:.4f}, "
        f"stages {dict(zip(names, [round(x, 4) for x in stages]))}")
    return dict(workload=label, ms_per_step=round(ms, 4), tokens_per_s=round(w.B * w.T / (ms / 1e3), 1),
                rho_measured=round(rho, 6), steps=steps, warmup=warmup,
                stages_ms=dict(zip(names, [round(x, 4) for x in stages])))


def bench_backward(args, dev, w, t, plan, pairs, steps=3, warmup=1):
    """Gradients of the attention readout at the layer shape (the cache of the main
    forward plan, dO ~ N(0,1)): bf16 MFMA kernels with the fp32 operands (dO, P, dS) as
    two bf16 terms, priced at 10 d FLOPs per visible pair (the score recompute and the
    four products of the backward) against the bf16 MFMA peak."""
    import torch
    import attention_sequence_mixing_amd as ham
    cache = dict(Kc=plan.Kc, Vc=plan.Vc, pos=plan.pos, count=plan.count)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed + 9)
    dO = torch.randn((w.B, w.T, w.H, w.d), generator=gen, device=dev, dtype=torch.float32)
    for _ in range(warmup):
        ham.ham_attention_backward(t["q"], cache, dO, scale=w.attn_scale)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        ham.ham_attention_backward(t["q"], cache, dO, scale=w.attn_scale)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    tflops = pairs * 10 * w.d / (ms / 1e3) / 1e12
    tq, tkv = measured_traffic("attn_bwd_q"), measured_traffic("attn_bwd_kv")
    traffic = None if tq is None or tkv is None else tq + tkv      # HBM bytes of the two kernels
    log(f"[bench] attention backward: {ms:.3f} ms/step, {tflops:.1f} TFLOP/s algorithmic "
        f"({100 * tflops / PEAK_BF16_TFLOPS:.1f}% of the bf16 MFMA peak)")
    return dict(workload=f"{w.name}_attention_backward", ms_per_step=round(ms, 4), steps=steps,
                warmup=warmup, roofline=dict(bound="mfma", achieved=round(tflops, 3), peak=PEAK_BF16_TFLOPS,
                                             unit="TFLOP/s", frac=round(tflops / PEAK_BF16_TFLOPS, 4),
                                             traffic=traffic))


def bench_rnn_backward(args, dev, w, t, steps=3, warmup=1):
    """Gradients of the gated delta-rule RNN at the layer shape (dO = dL/do_rnn and
    dS_T ~ N(0,1)): the chunked form (chunk prep, the forward and reverse state chains
    over chunks, two chunk-parallel gradient kernels) on the fp32 matrix cores, priced
    at 20 d_k d_v FLOPs per token and head (two forward passes of the recurrence,
    4 d_k d_v each, and the reverse step, 12 d_k d_v) against the fp32 peak.  The
    token-serial reverse (HAM_FORCE_RECURRENT) is timed once beside it."""
    import torch
    import attention_sequence_mixing_amd as ham
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed + 11)
    dO = torch.randn((w.B, w.T, w.H, w.d), generator=gen, device=dev, dtype=torch.float32)
    dST = torch.randn((w.B, w.H, w.d, w.d), generator=gen, device=dev, dtype=torch.float32)

    def run(serial=False):
        ham.ham_rnn_backward(t["q"], t["k"], t["v"], t["beta"], t["g"], dO, dS_T=dST, force_recurrent=serial)

    def timed(n, serial=False):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            run(serial)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    ms = timed(steps)
    run(True)
    torch.cuda.synchronize()
    ms_serial = timed(1, True)
    tflops = w.B * w.T * w.H * 20 * w.d * w.d / (ms / 1e3) / 1e12
    log(f"[bench] rnn backward: {ms:.3f} ms/step (token-serial reverse {ms_serial:.3f} ms), {tflops:.1f} TFLOP/s "
        f"algorithmic ({100 * tflops / PEAK_FP32_TFLOPS:.1f}% of the fp32 peak)")
    parts = [measured_traffic(k) for k in ("cbwd_prep", "cbwd_fwd", "cbwd_rev", "cbwd_cols", "cbwd_final")]
    return dict(workload=f"{w.name}_rnn_backward", ms_per_step=round(ms, 4), steps=steps, warmup=warmup,
                token_serial_ms=round(ms_serial, 3),
                roofline=dict(bound="mfma", achieved=round(tflops, 3), peak=PEAK_FP32_TFLOPS,
                              unit="TFLOP/s", frac=round(tflops / PEAK_FP32_TFLOPS, 4),
                              traffic=None if None in parts else sum(parts)))


def bench_long(args, dev, steps=10, warmup=10):
    """The long-context forward (B=1, H=16, T=32768, planted pairs, rho = 0.25): with 16
    heads the chunked state pass runs in segments side by side."""
    import torch
    import attention_sequence_mixing_amd as ham
    from attention_sequence_mixing_amd.inputs import LONG, make_workload, tau_for_rho
    w = LONG
    inp = make_workload(w)
    t = {n: torch.from_numpy(a).to(dev) for n, a in inp.items()}
    for n in ("q", "k", "v"):
        t[n] = t[n].to(torch.bfloat16)
    st = ham.ham_route_stats(t["k"], t["v"], t["beta"], t["g"],
                             torch.full((w.H,), float("inf"), device=dev), want_rho=False)
    tau = torch.from_numpy(tau_for_rho(st["e"].cpu().numpy(), w.rho)).to(dev)
    plan = ham.ForwardPlan(w.B, w.T, w.H, w.d, w.d, torch.bfloat16, dev, scale=w.attn_scale)

    def step():
        plan(t["q"], t["k"], t["v"], t["beta"], t["g"], tau)

    ms, stages = time_steps(step, steps, warmup)
    names = ["rnn_prep", "rnn_state", "route", "compact", "attention"]
    rho = float(plan.count.sum().item()) / (w.B * w.T * w.H)
    log(f"[bench] long context: {ms:.3f} ms/step, stages {dict(zip(names, [round(x, 4) for x in stages]))}")
    return dict(workload=w.name, ms_per_step=round(ms, 4), tokens_per_s=round(w.B * w.T / (ms / 1e3), 1),
                rho_measured=round(rho, 6), steps=steps, warmup=warmup,
                stages_ms=dict(zip(names, [round(x, 4) for x in stages])))


def bench_router(args, dev, w, t):
    """The same layer routed by learned-router scores (synthetic sigmoid(N(0,1)) per
    token-head, as inputs.make_router_scores draws them): the threshold for the target
    fraction comes from ham_select_tau on the GPU."""
    import torch
    import attention_sequence_mixing_amd as ham
    from attention_sequence_mixing_amd.inputs import make_router_scores
    rs = torch.from_numpy(make_router_scores(w.B, w.T, w.H, w.seed)).to(dev)
    tau = ham.ham_select_tau(rs, w.rho)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    nsel = 20
    e0.record()
    for _ in range(nsel):
        ham.ham_select_tau(rs, w.rho, out=tau)
    e1.record()
    torch.cuda.synchronize()
    sel_us = e0.elapsed_time(e1) / nsel * 1e3
    plan = ham.ForwardPlan(w.B, w.T, w.H, w.d, w.d, torch.bfloat16, dev, scale=w.attn_scale,
                           flags=ham.HAM_EXTERNAL_SCORES)

    def step():
        plan(t["q"], t["k"], t["v"], t["beta"], t["g"], tau, router_scores=rs)

    ms, stages = time_steps(step, args.steps, args.warmup)
    rho = float(plan.count.sum().item()) / (w.B * w.T * w.H)
    names = ["rnn_prep", "rnn_state", "route", "compact", "attention"]
    log(f"[bench] learned router: {ms:.3f} ms/step, select_tau {sel_us:.1f} us, rho {rho:.4f}, "
        f"stages {dict(zip(names, [round(x, 4) for x in stages]))}")
    # the same with the RNN on the library's second stream beside routing and attention
    oplan = ham.ForwardPlan(w.B, w.T, w.H, w.d, w.d, torch.bfloat16, dev, scale=w.attn_scale,
                            flags=ham.HAM_EXTERNAL_SCORES | ham.HAM_OVERLAP)
    oms, ostages = time_steps(lambda: oplan(t["q"], t["k"], t["v"], t["beta"], t["g"], tau, router_scores=rs),
                              args.steps, args.warmup)
    log(f"[bench] learned router, overlapped: {oms:.3f} ms/step, stages (their sum exceeds the step when "
        f"they overlap) {dict(zip(names, [round(x, 4) for x in ostages]))}")
    return dict(workload=f"{w.name}_learned_router", ms_per_step=round(ms, 4),
                tokens_per_s=round(w.B * w.T / (ms / 1e3), 1), rho_measured=round(rho, 6),
                select_tau_us=round(sel_us, 2), stages_ms=dict(zip(names, [round(x, 4) for x in stages])),
                overlapped=dict(ms_per_step=round(oms, 4), tokens_per_s=round(w.B * w.T / (oms / 1e3), 1),
                                stages_ms=dict(zip(names, [round(x, 4) for x in ostages])),
                                note="rnn_prep and rnn_state run on a second stream beside route, compact "
                                     "and attention; the mix pass after the join is inside the step but "
                                     "in no stage"))


def bench_decode(args, dev):
    import torch
    import attention_sequence_mixing_amd as ham
    from attention_sequence_mixing_amd import _lib
    from attention_sequence_mixing_amd.inputs import (DECODE_B, DECODE_D, DECODE_H, DECODE_PREFIX,
                                                      DECODE_STEPS, make_inputs_torch, tau_for_rho)
    B, H, d, T0, steps = DECODE_B, DECODE_H, DECODE_D, args.decode_prefix or DECODE_PREFIX, DECODE_STEPS
    cap = T0 + steps
    dt = torch.bfloat16
    t0 = time.time()
    pre = make_inputs_torch(B, T0, H, d, dtype="bf16", seed=4, device=dev)
    st = ham.ham_route_stats(pre["k"], pre["v"], pre["beta"], pre["g"],
                             torch.full((H,), float("inf"), device=dev), want_rho=False)
    tau = torch.from_numpy(tau_for_rho(st["e"].cpu().numpy(), 0.5)).to(dev)
    del st
    plan = ham.ForwardPlan(B, T0, H, d, d, dt, dev, cap=cap, scale=d ** -0.5)
    plan(pre["q"], pre["k"], pre["v"], pre["beta"], pre["g"], tau)
    torch.cuda.synchronize()
    log(f"[bench] decode prefill B={B} T={T0} done in {time.time() - t0:.1f}s")
    del pre
    S, Kc, Vc, pos, count = plan.S, plan.Kc, plan.Vc, plan.pos, plan.count
    plan.o = None
    plan.ws = None
    torch.cuda.empty_cache()
    S0, count0 = S.clone(), count.clone()
    x = make_inputs_torch(steps, B, H, d, dtype="bf16", seed=5, device=dev)   # [steps, B, H, d]
    dplan = ham.DecodePlan(B, H, d, d, cap, dt, dev, scale=d ** -0.5)
    t_abs = [torch.full((B,), T0 + s, dtype=torch.int32, device=dev) for s in range(steps)]

    # (b, h) heads sampled for the oracle's decode from the GPU prefill
    sample = [(0, 0), (B // 3, H // 2), (2 * B // 3, H - 1), (B - 1, 3 % H)]
    bs = torch.tensor([b for b, _ in sample], device=dev)
    hs = torch.tensor([h for _, h in sample], device=dev)
    pre_host = dict(S=S0[bs, hs].cpu().numpy(), count=count0[bs, hs].cpu().numpy(),
                    Kc=Kc[bs, hs].float().cpu().numpy(), Vc=Vc[bs, hs].float().cpu().numpy(),
                    pos=pos[bs, hs].cpu().numpy(), tau=tau[hs].cpu().numpy(),
                    x={n: x[n][:, bs, hs].float().cpu().numpy() for n in x})
    o_sampled = []

    def run_all(collect=False):
        for s in range(steps):
            dplan(x["q"][s], x["k"][s], x["v"][s], x["beta"][s], x["g"][s], tau, S, Kc, Vc, pos,
                  count, t_abs[s])
            if collect:
                o_sampled.append(dplan.o[bs, hs].float())

    cache_keys0 = float(count0.sum().item())
    run_all(collect=True)                   # warm-up pass over the same steps
    torch.cuda.synchronize()
    pre_host["o_gpu"] = torch.stack(o_sampled, 1).cpu().numpy()      # [4, steps, d]
    S.copy_(S0); count.copy_(count0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    run_all()                               # the timed pass: nothing else recorded
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    cache_keys1 = float(count.sum().item())
    S.copy_(S0); count.copy_(count0)
    lib = _lib.lib()
    lib.ham_profile_start(steps)            # per-kernel HIP events on a second pass over the same steps
    run_all()
    torch.cuda.synchronize()
    stg = collect_stages(lib, steps)
    mean_keys = 0.5 * (cache_keys0 + cache_keys1)
    cache_bytes = mean_keys * 2 * d * 2                     # K and V rows, bf16
    state_bytes = B * H * d * d * 4 * 2                     # S read + write
    attn_sec = stg[3] / 1e3
    roof = dict(stage="decode_attention", ms=float(stg[3]), bound="hbm", unit="GB/s",
                achieved=cache_bytes / attn_sec / 1e9, peak=PEAK_HBM_GBS)
    roof["frac"] = roof["achieved"] / PEAK_HBM_GBS
    roof["traffic"] = measured_traffic("decode_attention")
    return dict(us_per_step=us, tokens_per_s=B / (us / 1e6), steps=steps, prefix=T0, sampled=pre_host,
                sample_heads=sample, B=B, H=H, d=d,
                cache_keys_mean=mean_keys, step_bytes=cache_bytes + state_bytes,
                step_gbs=(cache_bytes + state_bytes) / (us / 1e6) / 1e9,
                stages_ms=dict(zip(["rnn", "route", "append", "attention", "combine"],
                                   [float(v) for v in stg])),
                roofline=roof)


def cpu_baseline(res, nbatch):
    """The fp64 C oracle, as it stands, on the first nbatch sequences of the same
    workload and threshold (all heads, all tokens), threads over heads."""
    import oracle
    w = res["w"]
    inp = res["inp"]
    nb = max(1, min(nbatch, w.B))
    sub = {n: np.ascontiguousarray(a[0:nb]) for n, a in inp.items()}
    tau = res["tau"]
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    # the GPU machine allots 16 host CPUs to each GPU, whatever nproc shows
    threads = max(1, min(16, w.H * nb, avail))
    oracle.forward(**{n: a[:1, :64] for n, a in sub.items()}, tau=tau, scale=w.attn_scale,
                   threads=threads)   # load outside the timing
    t0 = time.perf_counter()
    oracle.forward(**sub, tau=tau, scale=w.attn_scale, threads=threads)
    sec = time.perf_counter() - t0
    tokens = nb * w.T
    return dict(value=tokens / sec, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"sequences 0..{nb - 1} of {w.name} (all {w.H} heads, all {w.T} tokens, "
                       f"same tau), fp64 C oracle, {sec:.1f}s wall on {threads} threads")


def cpu_decode_baseline(dec, threads):
    """The fp64 oracle's decode of the sampled (b, h) heads from the GPU-produced prefill
    (state and cache copied to the host): all decode steps, the same inputs and
    thresholds, as the continuation of a forward (each sampled head as its own
    sequence).  Returns the timing and the largest per-head relative difference of the
    GPU's decode outputs from the oracle's."""
    import oracle
    sp = dec["sampled"]
    n, steps, d = len(dec["sample_heads"]), dec["steps"], dec["d"]
    xs = {k: np.ascontiguousarray(np.swapaxes(v, 0, 1)[:, :, None]) for k, v in sp["x"].items()}  # [n,steps,1,..]
    tau = np.ascontiguousarray(np.broadcast_to(sp["tau"].reshape(n, 1, 1), (n, steps, 1)))
    cap = sp["Kc"].shape[1]
    cache = dict(Kc=sp["Kc"][:, None], Vc=sp["Vc"][:, None], pos=sp["pos"][:, None].astype(np.int64),
                 count=sp["count"].reshape(n, 1).astype(np.int64))
    thr = max(1, min(threads, n))
    t0 = time.perf_counter()
    ref = oracle.forward(xs["q"], xs["k"], xs["v"], xs["beta"], xs["g"], tau, scale=d ** -0.5,
                         S0=sp["S"][:, None], cache=cache, cap=cap, t0=dec["prefix"], threads=thr)
    sec = time.perf_counter() - t0
    err = 0.0
    for i in range(n):
        y = ref["o"][i, :, 0]
        err = max(err, float(np.abs(sp["o_gpu"][i] - y).max() / max(np.abs(y).max(), 1e-30)))
    us_head_step = sec / steps / n * thr * 1e6
    return dict(value=round(us_head_step, 1), unit="us per decode step per (b,h) head, one thread",
                cores=thr, kind="oracle",
                sample=f"{n} (b,h) heads of the decode workload, {steps} steps from the GPU prefill "
                       f"(mean {float(sp['count'].mean()):.0f} cached keys), {sec:.1f}s wall on {thr} threads",
                whole_batch_us_per_step_16_threads=round(us_head_step * dec["B"] * dec["H"] / 16, 1),
                max_rel_err_gpu_vs_oracle=err)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the GPU clock takes some tens of milliseconds of load to settle: fewer than ~20
    # warmup steps of the layer leave the first timed steps at a lower clock
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--main-only", action="store_true",
                    help="only the layer forward (no other leg; same as --legs none)")
    ap.add_argument("--legs", default="all",
                    help="comma-separated legs to run besides the layer forward and decode: "
                         + ",".join(LEGS) + " (or all, none)")
    ap.add_argument("--decode-prefix", type=int, default=0)
    ap.add_argument("--cpu-batch", type=int, default=8,
                    help="sequences of the layer workload the CPU oracle baseline runs")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    legs = set(LEGS) if args.legs == "all" else set() if args.legs == "none" else set(args.legs.split(","))
    unknown = legs - set(LEGS)
    if unknown:
        ap.error("unknown legs: " + ",".join(sorted(unknown)))
    args.leg_set = set() if args.main_only else legs
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build runs the HAM layer on a single MI355X "
              "(heads shard across GPUs without communication; see the design notes).", file=sys.stderr)
        sys.exit(2)
    import torch
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(dev)
        return
    info = device_info(dev)
    info["stream_copy_GBps"] = round(stream_copy_gbs(dev), 1)
    log(f"[bench] device {info}")
    small = bench_small(args, dev) if want(args, "small") else None
    res = bench_forward(args, dev)
    for s in res["stages"]:
        log(f"[bench] stage {s['stage']:10s} {s['ms']:8.3f} ms  {s['achieved']:9.1f} {s['unit']} "
            f"({100 * s['frac']:.1f}% of {s['peak']})")
    long_ctx = bench_long(args, dev) if want(args, "long") else None
    dec = None
    if not args.no_decode:
        dec = bench_decode(args, dev)
        log(f"[bench] decode {dec['us_per_step']:.1f} us/step, stages {dec['stages_ms']}")
    cpu = None if args.no_cpu else cpu_baseline(res, args.cpu_batch)
    if cpu is not None:
        cpu.update(cpu_model=info.get("cpu_model"), nproc=info.get("nproc"), affinity=info.get("cpu_affinity"))
    dec_cpu = None
    if dec is not None and not args.no_cpu:
        dec_cpu = cpu_decode_baseline(dec, 16)
        log(f"[bench] decode oracle: {dec_cpu}")
    w = res["w"]
    dom = res["dom"]
    traffic = measured_traffic(dom["stage"])
    roof = dict(bound=dom["bound"], achieved=round(dom["achieved"], 3), peak=dom["peak"],
                unit=dom["unit"], frac=round(dom["frac"], 4), traffic=traffic, kernel=dom["stage"])
    out = {
        "metric": "HAM layer fwd tokens/sec at T=4096, rho_KV=0.5; decode us/token at 32k",
        "value": round(res["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "d": w.d, "rho_kv": w.rho,
                   "state": "fp32", "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "rho_measured": round(res["rho"], 6),
        "visible_pairs": res["pairs"],
        "stages": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in s.items()}
                   for s in res["stages"]],
        "device": info,
        "rho_sweep": res["sweep"],
        "small_f32": small,
        "learned_router": res["router"],
        "rope": res["rope"],
        "packed_docs": res["packed"],
        "block_routing": res["blocks"],
        "kv_heads": res["kvh"],
        "paper_heads": res["paper"],
        "attention_backward": res["bwd"],
        "rnn_backward": res["rbwd"],
        "long_context": long_ctx,
        "decode": None if dec is None else {
            "workload": f"decode_bf16_B32_H16_d128_prefix{dec['prefix']}_rho0.5",
            "us_per_step": round(dec["us_per_step"], 2), "tokens_per_s": round(dec["tokens_per_s"], 1),
            "steps": dec["steps"], "stages_ms": {k: round(v, 4) for k, v in dec["stages_ms"].items()},
            "step_GBps": round(dec["step_gbs"], 1),
            "roofline": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in dec["roofline"].items()},
            "cpu_baseline": dec_cpu},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
