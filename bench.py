#!/usr/bin/env python3
"""Throughput of the headwise-chunked causal GQA attention layer on one MI355X.

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--workload 2] [--chunk N]

A step is one forward and one backward pass of the whole layer (chunked QKV
projection, RoPE, causal attention forward and backward, output projection and
all gradients) over one batch of synthetic bf16 input already resident in HBM.
The default workload is the Llama-3-8B-shaped layer (hidden 4096, 32 q / 8 KV
heads, head_dim 128, L 32768, head chunk 8).  Prints ONE JSON line.

value = model FLOPs per step / time per step, with
  model FLOPs = 14 d Hq L(L+1)/2            (causal attention fwd 4 + bwd 10)
              + 6 L hidden (Hq+2Hkv) d      (QKV projection fwd + dx + dW)
              + 6 L Hq d hidden             (output projection fwd + dO + dW)
Recomputation inside the backward is executed but not counted.

roofline: the kernel class with the largest GPU time (found on the last
warm-up step, which times every class; that step also gives
kernel_breakdown and the attn_*_tflops figures), timed live over the timed
steps with HIP events the library records around each of its launches on the
launch stream, and around no other launch (events around every launch
cost about 1% of a step); achieved = its algorithmic FLOPs per launch / its
average launch duration.  traffic comes from profiles/traffic_*.json (rocprofv3 PMC
counters scaled by a copy-kernel calibration) when that file's kernel source
hash matches the current source, else null.

cpu_baseline: the fp64 oracle timed on this host on a bounded sample (the same
layer shape at a short sequence), reported in the same unit.

workloads: every other layer shape the metric is quoted on, each timed the
same way for a few steps on inputs drawn on the device (same distributions as
the seeded host recipe): the small GQA layer (also as a HIP
graph replay of its recorded step, where it is launch-bound), the two one-GPU shares of the
Llama-3-8B model (q/k/v given, L 524288 and 1048576), the 32B-class share
at every head chunk of its sweep (with and without the two-slot pipeline),
and the benchmarked layer with the full-recompute backward and with the
pipeline.  Each entry gives ms per step, TFLOP/s, the
dominant kernel's fraction of the bf16 peak, the planner's workspace and the
allocator's peak, and the HBM rate of the RoPE / layout pass, the dO
preparation and the dx accumulate (an epilogue of the dx GEMMs).

mlp_workloads: the sequence-tiled SwiGLU MLP of the same training stack at
the Llama-3-8B shape (hidden 4096, intermediate 14336) over L 32768, forward
+ backward at tiles of 2048, 8192 and 32768 rows.

loss_workloads: the sequence-tiled cross-entropy loss of the same stack at
the Llama-3-8B output projection (hidden 4096, vocabulary 128256) over
L 32768, forward + backward at tiles of 2048, 4096 and 8192 rows, as two
passes and as the fused forward-backward.

mfma_probe: the bf16 MFMA rate this chip sustains in the same run (after
the timed steps), from a probe kernel of four independent
v_mfma_f32_32x32x16_bf16 chains per wave at two waves per SIMD, on N(0, 1)
operands (the layer's data) and on constant operands, with the clock the
waves ran at (shader over constant clock ticks).  Under MFMA load the chip is
power-limited and the clock depends on the data; the roofline fraction stays
against the published 2.5 PFLOP/s.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
CPU_SAMPLE_L = 8192

KERNEL_SOURCES = {
    "attn_fwd": "headwise_chunked_context_amd/csrc/flash_fwd.hip",
    "attn_bwd_dkdv": "headwise_chunked_context_amd/csrc/flash_bwd.hip",
    "attn_bwd_dq": "headwise_chunked_context_amd/csrc/flash_bwd_dq.hip",
    "gemm": "headwise_chunked_context_amd/csrc/gemm.hip",
    "prep": "headwise_chunked_context_amd/csrc/prep.hip",
}


def model_flops(w, L=None) -> float:
    L = w.L if L is None else L
    d = w.head_dim
    attn = 14.0 * d * w.n_q * L * (L + 1) / 2
    proj = 0.0
    if w.projection:
        proj = 6.0 * L * w.hidden * (w.n_q + 2 * w.n_kv) * d + 6.0 * L * w.n_q * d * w.hidden
    return attn + proj


def gemm_flops_per_step(w) -> float:
    """Algorithmic GEMM FLOPs per step (forward, dO, dx, dW; not the recompute)."""
    if not w.projection:
        return 0.0
    d = w.head_dim
    return 6.0 * w.L * w.hidden * (w.n_q + 2 * w.n_kv) * d + 6.0 * w.L * w.n_q * d * w.hidden


def gemm_accum_flops_per_step(w) -> float:
    """FLOPs of the dx GEMMs after the first chunk (the accumulating ones):
    2 L hidden K each, K = the chunk's dq columns, plus its dk and dv
    columns when the chunk completes its KV groups."""
    if not w.projection:
        return 0.0
    d, hc, G = w.head_dim, w.head_chunk, w.n_q // w.n_kv
    kc = hc // G if hc >= G else 1
    total = 0.0
    for c in range(1, w.n_q // hc):
        kv_last = ((c + 1) * hc) % G == 0
        total += 2.0 * w.L * w.hidden * ((hc + 2 * kc) * d if kv_last else hc * d)
    return total


def source_hash(rel: str) -> str:
    with open(os.path.join(ROOT, rel), "rb") as f:
        h = hashlib.sha256(f.read())
    with open(os.path.join(ROOT, "headwise_chunked_context_amd/csrc/common.h"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kind: str, workload: str):
    path = os.path.join(ROOT, "profiles", f"traffic_{kind}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_hash") != source_hash(KERNEL_SOURCES[kind]):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w) -> dict:
    """Time the fp64 oracle (as it stands) on the same layer shape at a short L."""
    import numpy as np  # noqa: F401

    import oracle
    import synthetic

    ws = w.with_(L=CPU_SAMPLE_L)
    inp = synthetic.make_inputs(ws)
    f = {k: (None if inp[k] is None else synthetic.bf16_bits_to_f64(inp[k]))
         for k in ("x", "w_qkv", "w_o", "dy")}
    t0 = time.perf_counter()
    oracle.layer_fwd(f["x"], f["w_qkv"], f["w_o"], ws.n_q, ws.n_kv, ws.head_dim, ws.theta,
                     ws.head_chunk)
    oracle.layer_bwd(f["x"], f["w_qkv"], f["w_o"], f["dy"], ws.n_q, ws.n_kv, ws.head_dim,
                     ws.theta, ws.head_chunk)
    dt = time.perf_counter() - t0
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return {
        "value": round(model_flops(ws) / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"one forward + backward of the same layer shape at L={CPU_SAMPLE_L} "
                   f"({model_flops(ws):.3e} model FLOPs, {dt:.1f} s, fp64 NumPy)"),
    }


def copy_calibration() -> None:
    """A plain 1 GiB device copy, for scaling rocprofv3 FETCH/WRITE_SIZE counters."""
    import torch

    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}), flush=True)


def executed_mfma_flops_per_step(w) -> dict:
    """MFMA FLOPs each kernel class executes per step (recomputation included):
    the attention forward 4 d P Hq, dK/dV 8 d P Hq, dQ 6 d P Hq (its S and dP
    again), the GEMMs the model's projection FLOPs plus the backward's
    recompute of the QKV projection, 2 L hidden (Hq + 2 Hkv) d."""
    d = w.head_dim
    P = w.L * (w.L + 1) / 2
    out = {"attn_fwd": 4.0 * d * P * w.n_q, "attn_bwd_dkdv": 8.0 * d * P * w.n_q,
           "attn_bwd_dq": 6.0 * d * P * w.n_q}
    if w.projection:
        acc = gemm_accum_flops_per_step(w)
        out["gemm"] = gemm_flops_per_step(w) - acc + 2.0 * w.L * w.hidden * (w.n_q + 2 * w.n_kv) * d
        out["gemm_accum"] = acc
    return out


def hbm_bytes_per_step(w) -> dict:
    """Algorithmic HBM bytes per step of the passes that move data rather than
    contract it, for the classes the library times separately:
      prep        the RoPE / layout pass, 2 B read + 2 B written per element of
                  every head it prepares, in the forward and again in the
                  backward (q/k/v given: every q, k and v head; projection
                  mode: only v, the GEMM epilogue rotates q and k)
      prep_dout   dO and O read, dO written (2 B each per element) and per row
                  LSE read, base-2 LSE and D written (12 B), for every q head
      gemm_accum  dx read and written (2 B each per element) by the epilogue of
                  every dx GEMM after the first chunk's; the accumulate is that
                  GEMM's epilogue, so its rate is these bytes over the whole
                  (MFMA-bound) GEMM's time, a lower bound of what the epilogue
                  sustains"""
    d, L = w.head_dim, w.L
    heads = (w.n_q + 2 * w.n_kv) if not w.projection else w.n_kv
    out = {
        "prep": 2 * heads * L * d * 4.0,
        "prep_dout": w.n_q * L * (6.0 * d + 12.0),
    }
    if w.projection:
        out["gemm_accum"] = (w.n_q // w.head_chunk - 1) * L * w.hidden * 4.0
    return out


CLASSES = ("attn_fwd", "attn_bwd_dkdv", "attn_bwd_dq", "gemm", "gemm_accum")


def algo_flops_per_launch(w, kind):
    """Algorithmic FLOPs per launch (one launch = one head chunk of hc query
    heads, P = L(L+1)/2 causal pairs):
      attn_fwd       4 d P hc   (S = Q K^T and O = P V)
      attn_bwd_dkdv  8 d P hc   (S, dP = dO V^T, dV = P^T dO, dK = dS^T Q)
      attn_bwd_dq    2 d P hc   (dQ = dS K; its recomputed S and dP, 4 d P hc
                                 more, are executed, not counted)"""
    d, hc = w.head_dim, w.head_chunk
    P = w.L * (w.L + 1) / 2
    return {"attn_fwd": 4.0 * d * P * hc, "attn_bwd_dkdv": 8.0 * d * P * hc,
            "attn_bwd_dq": 2.0 * d * P * hc}[kind]


def device_inputs(w, seed):
    """N(0, sigma^2) draws on the device, rounded to bf16: the host recipe's
    distributions without generating gigabytes on the host."""
    import torch

    g = torch.Generator(device="cuda:0").manual_seed(seed)

    def draw(shape, sigma):
        t = torch.randn(*shape, generator=g, device="cuda:0", dtype=torch.float32)
        if sigma != 1.0:
            t.mul_(sigma)
        return t.to(torch.bfloat16)

    d = w.head_dim
    if w.projection:
        return (draw((w.L, w.hidden), w.x_sigma), draw((w.qkv_width, w.hidden), w.w_sigma),
                draw((w.hidden, w.n_q * d), w.w_sigma), draw((w.L, w.hidden), 1.0))
    return draw((w.L, w.qkv_width), w.x_sigma), None, None, draw((w.L, w.n_q * d), 1.0)


def time_layer(lib, w, x, wq, wo, dy, steps, warmup, recompute=False):
    """Warm-up steps (the last one times every kernel class), then `steps`
    timed steps with only the dominant class bracketed.  Returns the
    measurements of one workload."""
    import torch

    dev = torch.device("cuda:0")
    hc = w.head_chunk
    ws_f = lib.workspace_bytes(w.L, w.hidden, w.n_q, w.n_kv, w.head_dim, hc, lib.fwd_pass())
    bwd_pass = lib.bwd_pass(recompute)
    ws_b = lib.workspace_bytes(w.L, w.hidden, w.n_q, w.n_kv, w.head_dim, hc, bwd_pass)
    # one workspace, sized for the larger pass, reused by every call
    ws = torch.empty(max(ws_f, ws_b), dtype=torch.uint8, device=dev)

    def step():
        _, o, lse = lib.attn_fwd(x, wq, wo, w.n_q, w.n_kv, hc, w.theta, workspace=ws)
        lib.attn_bwd(x, wq, wo, None if recompute else o, lse, dy, w.n_q, w.n_kv, hc, w.theta,
                     workspace=ws)

    prof_all = None
    for i in range(warmup):
        if i == warmup - 1:
            torch.cuda.synchronize()
            lib.profile_enable(True)
        step()
    torch.cuda.synchronize()
    if warmup > 0:
        prof_all = lib.profile_read()
        lib.profile_enable(False)
    # with the two-slot pipeline the preparation classes run on a second
    # stream beside the attention kernels, and their event brackets measure
    # that shared time; the roofline class is then taken among the
    # attention kernels, which stay on the caller's stream
    classes = CLASSES if not lib.pipeline_enabled() else CLASSES[:3]
    dom = None
    if prof_all is not None:
        dom = max((k for k in classes if prof_all[k][1] > 0), key=lambda k: prof_all[k][0])
    lib.profile_enable(True, kinds=None if dom is None else [dom])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    prof = lib.profile_read()
    lib.profile_enable(False)
    prof_steps = 1
    if prof_all is None:
        prof_all, prof_steps = prof, steps
        dom = max((k for k in classes if prof[k][1] > 0), key=lambda k: prof[k][0])
    ms = (t1 - t0) * 1e3 / steps
    tot_ms, launches = prof[dom]
    avg_ms = tot_ms / launches
    if dom == "gemm_accum":
        per_launch = gemm_accum_flops_per_step(w) * steps / launches
    elif dom == "gemm":
        per_launch = (gemm_flops_per_step(w) - gemm_accum_flops_per_step(w)) * steps / launches
    else:
        per_launch = algo_flops_per_launch(w, dom)
    achieved = per_launch / (avg_ms * 1e-3) / 1e12
    hbm = {}
    for k, nbytes in hbm_bytes_per_step(w).items():
        t = prof_all[k][0] / prof_steps
        if prof_all[k][1] and t > 0:
            hbm[k] = {"gbs": round(nbytes / (t * 1e-3) / 1e9, 1), "ms_per_step": round(t, 3),
                      "bytes_per_step": nbytes}
    return dict(ms=ms, dom=dom, achieved=achieved, avg_ms=avg_ms, launches=launches,
                prof_all=prof_all, prof_steps=prof_steps, ws_f=ws_f, ws_b=ws_b, hbm=hbm,
                bwd_pass=bwd_pass)


def time_layer_graph(lib, w, x, wq, wo, dy, steps, warmup):
    """The step of time_layer recorded once into a HIP graph (torch's
    CUDAGraph on its capture stream; every entry point enqueues kernel
    launches only), then replayed: `warmup` untimed replays, then `steps`
    timed ones.  Returns the workspace sizes and ms per step."""
    import torch

    dev = torch.device("cuda:0")
    hc = w.head_chunk
    ws_f = lib.workspace_bytes(w.L, w.hidden, w.n_q, w.n_kv, w.head_dim, hc, lib.PASS_FWD)
    ws_b = lib.workspace_bytes(w.L, w.hidden, w.n_q, w.n_kv, w.head_dim, hc, lib.PASS_BWD)
    ws = torch.empty(max(ws_f, ws_b), dtype=torch.uint8, device=dev)

    def step():
        _, o, lse = lib.attn_fwd(x, wq, wo, w.n_q, w.n_kv, hc, w.theta, workspace=ws)
        lib.attn_bwd(x, wq, wo, o, lse, dy, w.n_q, w.n_kv, hc, w.theta, workspace=ws)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return dict(ms=(t1 - t0) * 1e3 / steps, ws_f=ws_f, ws_b=ws_b)


def sweep(lib) -> dict:
    """Every other workload, a few steps each (inputs drawn on the device)."""
    import torch

    import synthetic

    W = synthetic.WORKLOADS
    plan = [(W[1], 3, 10, False), (W[1], 3, 10, "graph"), (W[3], 1, 2, False), (W[5], 1, 1, False)]
    # the benchmarked layer in its optional modes: full recompute (o_saved
    # NULL) and the two-slot pipeline
    plan += [(W[2], 1, 3, "recompute"), (W[2], 1, 3, True)]
    # the 32B-class share at every chunk of its sweep, on one stream and with
    # the two-slot pipeline (next chunk's preparation on a second stream)
    plan += [(W[4].with_(head_chunk=c), 1, 2, pipe) for pipe in (False, True) for c in (1, 2, 4, 8)]
    out = {}
    for w, warmup, steps, mode in plan:
        pipe, recompute, graph = mode is True, mode == "recompute", mode == "graph"
        key = w.name if w.wid != 4 else f"{w.name}_chunk{w.head_chunk}"
        if pipe:
            key += "_pipelined"
        if recompute:
            key += "_recompute"
        if graph:
            key += "_graph"
        torch.cuda.empty_cache()
        x, wq, wo, dy = device_inputs(w, seed=1000 * w.wid)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()   # the layer's own peak, not the draw's
        lib.pipeline_enable(pipe)
        try:
            if graph:
                r = time_layer_graph(lib, w, x, wq, wo, dy, steps, warmup)
            else:
                r = time_layer(lib, w, x, wq, wo, dy, steps, warmup, recompute=recompute)
        finally:
            lib.pipeline_enable(False)
        peak = torch.cuda.max_memory_allocated()
        io = sum(t.numel() * t.element_size() for t in (x, wq, wo, dy) if t is not None)
        del x, wq, wo, dy
        flops = model_flops(w)
        out[key] = {
            "seq_len": w.L, "hidden": w.hidden, "n_q_heads": w.n_q, "n_kv_heads": w.n_kv,
            "head_chunk": w.head_chunk, "pipeline": pipe,
            "backward": "recompute attention output" if recompute else "saved attention output",
            "launch": "hip graph replay" if graph else "eager",
            "steps": steps, "warmup": warmup,
            "ms_per_step": round(r["ms"], 3),
            "tflops": round(flops / (r["ms"] * 1e-3) / 1e12, 2),
            "roofline_kernel": r.get("dom"),
            "roofline_frac": round(r["achieved"] / PEAK_BF16_TFLOPS, 4) if "achieved" in r else None,
            "workspace_gib": {"fwd": round(r["ws_f"] / 2**30, 4), "bwd": round(r["ws_b"] / 2**30, 4)},
            "peak_allocated_gib": round(peak / 2**30, 3),
            "peak_allocated_minus_inputs_gib": round((peak - io) / 2**30, 3),
            "hbm_passes": r.get("hbm"),
        }
        print(f"bench: {key}: {out[key]['ms_per_step']} ms/step, {out[key]['tflops']} TFLOP/s",
              file=sys.stderr, flush=True)
    return out


def mlp_sweep(lib) -> dict:
    """The sequence-tiled SwiGLU MLP at the Llama-3-8B shape (hidden 4096,
    intermediate 14336) over L 32768, forward + backward, at several tile
    sizes: ms per step, TFLOP/s of model work (18 L hidden ffn: forward 6,
    backward 12; the backward's recompute of the gate/up projection, 4 more,
    is executed, not counted), workspace and allocator peak."""
    import torch

    import synthetic

    base = synthetic.MLP_WORKLOADS[12]
    out = {}
    g = torch.Generator(device="cuda:0").manual_seed(1000 * base.wid)

    def draw(shape, sigma):
        t = torch.randn(*shape, generator=g, device="cuda:0", dtype=torch.float32)
        if sigma != 1.0:
            t.mul_(sigma)
        return t.to(torch.bfloat16)

    L, D, F = base.L, base.hidden, base.ffn
    x, wgu, wd, dy = draw((L, D), 1.0), draw((2 * F, D), 0.02), draw((D, F), 0.02), draw((L, D), 1.0)
    io = sum(t.numel() * t.element_size() for t in (x, wgu, wd, dy))
    for tile in (2048, 8192, 32768):
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        ws_f = lib.mlp_workspace_bytes(L, D, F, tile, lib.PASS_FWD)
        ws_b = lib.mlp_workspace_bytes(L, D, F, tile, lib.PASS_BWD)
        ws = torch.empty(max(ws_f, ws_b), dtype=torch.uint8, device="cuda:0")

        def step():
            lib.mlp_fwd(x, wgu, wd, tile, workspace=ws)
            lib.mlp_bwd(x, wgu, wd, dy, tile, workspace=ws)

        step()
        torch.cuda.synchronize()
        steps = 5
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        peak = torch.cuda.max_memory_allocated()
        del ws
        key = f"llama3_8b_mlp_hidden4096_ffn14336_L32768_tile{tile}"
        out[key] = {
            "seq_len": L, "hidden": D, "ffn": F, "tile_rows": tile, "steps": steps, "warmup": 1,
            "ms_per_step": round(ms, 3),
            "tflops": round(18.0 * L * D * F / (ms * 1e-3) / 1e12, 2),
            "workspace_gib": {"fwd": round(ws_f / 2**30, 4), "bwd": round(ws_b / 2**30, 4)},
            "peak_allocated_gib": round(peak / 2**30, 3),
            "peak_allocated_minus_inputs_gib": round((peak - io) / 2**30, 3),
        }
        print(f"bench: {key}: {out[key]['ms_per_step']} ms/step, {out[key]['tflops']} TFLOP/s",
              file=sys.stderr, flush=True)
    return out


def loss_sweep(lib) -> dict:
    """The sequence-tiled cross-entropy loss at the Llama-3-8B output
    projection (hidden 4096, vocabulary 128256) over L 32768, forward +
    backward, at several tile sizes, as two passes and fused: ms per step,
    TFLOP/s of model work (6 L hidden vocab: forward 2, backward 4; the
    separate backward's recompute of the logits, 2 more, is executed, not
    counted), workspace and allocator peak."""
    import torch

    import synthetic

    base = synthetic.LOSS_WORKLOADS[22]
    out = {}
    L, D, V = base.L, base.hidden, base.vocab
    dev = synthetic.make_loss_inputs_device(base)
    h, w, t = dev["h"], dev["w"], dev["targets"]
    io = sum(x.numel() * x.element_size() for x in (h, w, t))
    for tile, fused in ((2048, False), (4096, False), (8192, False), (2048, True), (4096, True),
                        (8192, True)):
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        if fused:
            ws_f = ws_b = lib.loss_workspace_bytes(L, D, V, tile, lib.PASS_FWD_BWD)
        else:
            ws_f = lib.loss_workspace_bytes(L, D, V, tile, lib.PASS_FWD)
            ws_b = lib.loss_workspace_bytes(L, D, V, tile, lib.PASS_BWD)
        ws = torch.empty(max(ws_f, ws_b), dtype=torch.uint8, device="cuda:0")

        def step():
            if fused:
                lib.loss_fwd_bwd(h, w, t, 1.0, tile, synthetic.IGNORE_INDEX, workspace=ws)
                return
            _, lse = lib.loss_fwd(h, w, t, tile, synthetic.IGNORE_INDEX, workspace=ws)
            lib.loss_bwd(h, w, t, lse, 1.0, tile, synthetic.IGNORE_INDEX, workspace=ws)

        step()
        torch.cuda.synchronize()
        steps = 3
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        peak = torch.cuda.max_memory_allocated()
        del ws
        key = f"llama3_8b_loss_hidden4096_vocab128256_L32768_tile{tile}" + ("_fused" if fused else "")
        out[key] = {
            "seq_len": L, "hidden": D, "vocab": V, "tile_rows": tile, "steps": steps, "warmup": 1,
            "mode": "fused forward-backward" if fused else "forward, then backward",
            "ms_per_step": round(ms, 3),
            "tflops": round(6.0 * L * D * V / (ms * 1e-3) / 1e12, 2),
            "workspace_gib": {"fwd": round(ws_f / 2**30, 4), "bwd": round(ws_b / 2**30, 4)},
            "peak_allocated_gib": round(peak / 2**30, 3),
            "peak_allocated_minus_inputs_gib": round((peak - io) / 2**30, 3),
            "full_sequence_fp32_logits_gib": round(L * V * 4 / 2**30, 3),
        }
        print(f"bench: {key}: {out[key]['ms_per_step']} ms/step, {out[key]['tflops']} TFLOP/s",
              file=sys.stderr, flush=True)
    return out


def mfma_probe(lib) -> dict:
    """Sustained bf16 MFMA rate and clock on N(0, 1) and on constant
    operands (about 80 ms each)."""
    import torch

    from headwise_chunked_context_amd.binding import PROBE_FLOP_PER_ROUND

    g = torch.Generator(device="cuda:0").manual_seed(11)
    out = {"kernel": "v_mfma_f32_32x32x16_bf16, 4 independent accumulator chains per wave over 8 "
                     "operand pairs, 512 workgroups x 4 waves (2 waves per SIMD)"}
    wg, iters = 512, 60000
    for kind in ("normal_operands", "constant_operands"):
        if kind == "normal_operands":
            ops = torch.randn(8 << 20, generator=g, device="cuda:0").to(torch.bfloat16)
        else:
            ops = torch.full((8 << 20,), 1.0, device="cuda:0", dtype=torch.bfloat16)
        lib.probe_mfma(ops, 200, wg)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        _, clocks = lib.probe_mfma(ops, iters, wg)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1)
        tflops = wg * 4 * iters * PROBE_FLOP_PER_ROUND / (ms * 1e-3) / 1e12
        ck = clocks.view(-1, 2).double()
        ghz = float((ck[:, 0] / ck[:, 1]).mean()) * 0.1   # constant clock: 100 MHz
        out[kind] = {"tflops": round(tflops, 1), "clock_ghz": round(ghz, 3),
                     "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4), "ms": round(ms, 2)}
        print(f"bench: mfma probe, {kind}: {tflops:.0f} TFLOP/s at {ghz:.2f} GHz", file=sys.stderr,
              flush=True)
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=2, help="workload id in synthetic.WORKLOADS")
    ap.add_argument("--chunk", type=int, default=0, help="override the head chunk")
    ap.add_argument("--seq-len", type=int, default=0, help="override L (not a metric run)")
    ap.add_argument("--recompute", action="store_true",
                    help="backward without the saved attention output (recomputed per chunk)")
    ap.add_argument("--pipeline", action="store_true",
                    help="overlap the forward's next-chunk projection on a second stream")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="time only the main workload, not the other layer shapes")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this layer is measured on one GPU only; --gpus {args.gpus} is not "
              "supported (the multi-GPU exchange is out of scope).", file=sys.stderr)
        return 2
    if args.copy_calibration:
        copy_calibration()
        return 0

    import numpy as np
    import torch

    import headwise_chunked_context_amd as lib
    import synthetic

    lib.pipeline_enable(args.pipeline)
    w = synthetic.WORKLOADS[args.workload]
    if args.chunk:
        w = w.with_(head_chunk=args.chunk)
    if args.seq_len:
        w = w.with_(L=args.seq_len)
    hc = w.head_chunk
    dev = torch.device("cuda:0")

    inp = synthetic.make_inputs(w)

    def to_dev(bits):
        if bits is None:
            return None
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).to(dev)

    x, wq, wo, dy = (to_dev(inp[k]) for k in ("x", "w_qkv", "w_o", "dy"))
    del inp
    hidden = w.hidden
    r = time_layer(lib, w, x, wq, wo, dy, args.steps, args.warmup, recompute=args.recompute)
    mem0 = torch.cuda.max_memory_allocated(dev)
    ms, dom, prof_all, prof_steps = r["ms"], r["dom"], r["prof_all"], r["prof_steps"]
    ws_f, ws_b, bwd_pass = r["ws_f"], r["ws_b"], r["bwd_pass"]
    flops = model_flops(w)
    value = flops / (ms * 1e-3) / 1e12
    d = w.head_dim
    P = w.L * (w.L + 1) / 2
    roofline = {
        "bound": "mfma",
        "kernel": dom,
        "achieved": round(r["achieved"], 2),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(r["achieved"] / PEAK_BF16_TFLOPS, 4),
        "traffic": traffic_for(dom, w.name) if dom in KERNEL_SOURCES else None,
        "avg_launch_ms": round(r["avg_ms"], 4),
        "launches": r["launches"],
    }
    # the whole attention backward (both kernels) against its 10 d P hc, and
    # the forward, from the step that timed every class
    nb = prof_all["attn_bwd_dkdv"][1]
    if nb:
        bwd_ms = (prof_all["attn_bwd_dkdv"][0] + prof_all["attn_bwd_dq"][0]) / nb
        roofline["attn_bwd_tflops"] = round(10.0 * d * P * hc / (bwd_ms * 1e-3) / 1e12, 2)
    nf = prof_all["attn_fwd"][1]
    if nf:
        roofline["attn_fwd_tflops"] = round(
            algo_flops_per_launch(w, "attn_fwd") / (prof_all["attn_fwd"][0] / nf * 1e-3) / 1e12, 2)
    breakdown = {k: {"ms_per_step": round(v[0] / prof_steps, 3), "launches_per_step": v[1] // prof_steps}
                 for k, v in prof_all.items()}
    # MFMA utilisation per class: executed MFMA FLOPs over the class's
    # event-timed time at the bf16 peak (the rocprofv3 ratio
    # SQ_VALU_MFMA_BUSY_CYCLES / SIMD-cycles at 2.4 GHz, from the timing)
    mfma_util = {k: round(f / (prof_all[k][0] / prof_steps * 1e-3) / (PEAK_BF16_TFLOPS * 1e12), 4)
                 for k, f in executed_mfma_flops_per_step(w).items() if prof_all[k][0] > 0}

    chunks = [c for c in range(1, w.n_q + 1)
              if w.n_q % c == 0 and (c % (w.n_q // w.n_kv) == 0 or (w.n_q // w.n_kv) % c == 0)]
    ws_vs_chunk = {str(c): round(lib.workspace_bytes(w.L, hidden, w.n_q, w.n_kv, d, c,
                                                     bwd_pass) / 2**30, 4) for c in chunks}

    out = {
        "metric": "chunked causal attn fwd+bwd TFLOP/s at 1 GPU; peak workspace GiB vs chunk",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 (P V product fp16)",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights, rounded to bf16)",
        "config": {
            "workload": w.name,
            "seq_len": w.L,
            "hidden": w.hidden,
            "n_q_heads": w.n_q,
            "n_kv_heads": w.n_kv,
            "head_dim": w.head_dim,
            "head_chunk": hc,
            "rope_theta": w.theta,
            "batch": 1,
            "causal": True,
            "parallelism": "single GPU (one GPU's share; no collectives)",
            "backward": "recompute attention output" if args.recompute else "saved attention output",
            "pipeline": args.pipeline,
        },
        "model_flops_per_step": flops,
        "roofline": roofline,
        "kernel_breakdown": breakdown,
        "mfma_util": mfma_util,
        "kernel_breakdown_from": ("the last warm-up step, every kernel class timed" if prof_steps == 1
                                  else "the timed steps, every kernel class timed"),
        "workspace_gib": {"fwd": round(ws_f / 2**30, 4), "bwd": round(ws_b / 2**30, 4),
                          "bwd_vs_chunk": ws_vs_chunk},
        "peak_allocated_gib": round(mem0 / 2**30, 3),
        "hbm_passes": r["hbm"],
    }
    out["mfma_probe"] = mfma_probe(lib)
    if not args.no_sweep and not args.seq_len and args.workload == 2 and not args.chunk:
        del x, wq, wo, dy
        out["workloads"] = sweep(lib)
        out["mlp_workloads"] = mlp_sweep(lib)
        out["loss_workloads"] = loss_sweep(lib)
    if not args.no_cpu_baseline and not args.seq_len:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
