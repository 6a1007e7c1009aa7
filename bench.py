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
    ws_f = lib.workspace_bytes(w.L, hidden, w.n_q, w.n_kv, w.head_dim, hc, lib.fwd_pass())
    bwd_pass = lib.PASS_BWD_RECOMPUTE if args.recompute else lib.PASS_BWD
    ws_b = lib.workspace_bytes(w.L, hidden, w.n_q, w.n_kv, w.head_dim, hc, bwd_pass)
    # one workspace, sized for the larger pass, reused by every call
    ws = torch.empty(max(ws_f, ws_b), dtype=torch.uint8, device=dev)

    def step():
        _, o, lse = lib.attn_fwd(x, wq, wo, w.n_q, w.n_kv, hc, w.theta, workspace=ws)
        lib.attn_bwd(x, wq, wo, None if args.recompute else o, lse, dy, w.n_q, w.n_kv, hc, w.theta,
                     workspace=ws)

    # The last warm-up step times every kernel class (the breakdown, and which
    # class dominates); the timed steps bracket only the dominant class's
    # launches with events, since events around every launch cost ~1% of a
    # step.  With no warm-up the timed steps bracket every class.
    prof_all = None
    for i in range(args.warmup):
        if i == args.warmup - 1:
            torch.cuda.synchronize()
            lib.profile_enable(True)
        step()
    torch.cuda.synchronize()
    if args.warmup > 0:
        prof_all = lib.profile_read()
        lib.profile_enable(False)
    mem0 = torch.cuda.max_memory_allocated(dev)

    classes = ("attn_fwd", "attn_bwd_dkdv", "attn_bwd_dq", "gemm")
    dom = None
    if prof_all is not None:
        dom = max((k for k in classes if prof_all[k][1] > 0), key=lambda k: prof_all[k][0])
    lib.profile_enable(True, kinds=None if dom is None else [dom])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    prof = lib.profile_read()
    lib.profile_enable(False)
    prof_steps = 1
    if prof_all is None:
        prof_all, prof_steps = prof, args.steps
        dom = max((k for k in classes if prof[k][1] > 0), key=lambda k: prof[k][0])

    ms = (t1 - t0) * 1e3 / args.steps
    flops = model_flops(w)
    value = flops / (ms * 1e-3) / 1e12

    # dominant kernel class and its roofline.  Algorithmic FLOPs per launch
    # (one launch = one head chunk of hc query heads, P = L(L+1)/2 pairs):
    #   attn_fwd       4 d P hc   (S = Q K^T and O = P V)
    #   attn_bwd_dkdv  8 d P hc   (S, dP = dO V^T, dV = P^T dO, dK = dS^T Q)
    #   attn_bwd_dq    2 d P hc   (dQ = dS K; its recomputed S and dP,
    #                              4 d P hc more, are executed, not counted)
    #   gemm           the projection GEMMs of a step / their launches
    d = w.head_dim
    P = w.L * (w.L + 1) / 2
    algo = {
        "attn_fwd": 4.0 * d * P * hc,
        "attn_bwd_dkdv": 8.0 * d * P * hc,
        "attn_bwd_dq": 2.0 * d * P * hc,
    }
    tot_ms, launches = prof[dom]
    avg_ms = tot_ms / launches
    if dom == "gemm":
        per_launch = gemm_flops_per_step(w) * args.steps / launches
    else:
        per_launch = algo[dom]
    achieved = per_launch / (avg_ms * 1e-3) / 1e12
    roofline = {
        "bound": "mfma",
        "kernel": dom,
        "achieved": round(achieved, 2),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": traffic_for(dom, w.name) if dom in KERNEL_SOURCES else None,
        "avg_launch_ms": round(avg_ms, 4),
        "launches": launches,
    }
    # the whole attention backward (both kernels) against its 10 d P hc, and
    # the forward, from the step that timed every class
    nb = prof_all["attn_bwd_dkdv"][1]
    if nb:
        bwd_ms = (prof_all["attn_bwd_dkdv"][0] + prof_all["attn_bwd_dq"][0]) / nb
        roofline["attn_bwd_tflops"] = round(10.0 * d * P * hc / (bwd_ms * 1e-3) / 1e12, 2)
    nf = prof_all["attn_fwd"][1]
    if nf:
        roofline["attn_fwd_tflops"] = round(algo["attn_fwd"] / (prof_all["attn_fwd"][0] / nf * 1e-3) / 1e12, 2)
    breakdown = {k: {"ms_per_step": round(v[0] / prof_steps, 3), "launches_per_step": v[1] // prof_steps}
                 for k, v in prof_all.items()}

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
        "dtype": "bf16",
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
        "kernel_breakdown_from": ("the last warm-up step, every kernel class timed" if prof_steps == 1
                                  else "the timed steps, every kernel class timed"),
        "workspace_gib": {"fwd": round(ws_f / 2**30, 4), "bwd": round(ws_b / 2**30, 4),
                          "bwd_vs_chunk": ws_vs_chunk},
        "peak_allocated_gib": round(mem0 / 2**30, 3),
    }
    if not args.no_cpu_baseline and not args.seq_len:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
