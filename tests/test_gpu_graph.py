"""HIP graph capture of the C ABI's calls (MI355X only).

The one-stream schedule of every entry point enqueues kernel launches only
(no allocation, no memset, no synchronization, no event unless profiling is
on), so a caller can record a whole step of the attention layer, the MLP or
the loss into a HIP graph and replay it: the launch-bound small shapes then
cost one graph launch instead of dozens of kernel launches.  Each test
records the calls once on torch's capture stream, then replays the graph
three times; before every replay it writes fresh inputs into the captured
input buffers, runs the same calls eagerly on them (the program's own work
between replays, on a workspace of its own) and synchronizes, and after it
compares every output of the replay with the eager one bit for bit.  At
these lengths every weight-gradient GEMM sums its reduction in one part (the
split count grows with K / 512 only from K = 1024 on), so the weight
gradients are reproducible bit for bit as well.  The eager results on the
first replay's inputs are checked against the oracle with the gates of the
parity tests.
"""
import numpy as np
import pytest

import synthetic
from _helpers import to_dev

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _torch():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _bits(t):
    import torch

    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _replay_and_compare(torch, fill, eager, static_out, graph, label):
    """Replays `graph` REPLAYS times.  Before each replay fill(rep) writes
    new inputs into the captured buffers and eager() computes the same
    outputs eagerly; every replayed output must equal the eager one bit for
    bit.  Returns the eager outputs of replay 0."""
    first = None
    for rep in range(REPLAYS):
        fill(rep)
        ref = eager()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a in static_out.items():
            if a is None:
                continue
            same = torch.equal(_bits(a), _bits(ref[name]))
            print(f"graph {label} replay {rep}: {name} bitwise equal to eager = {same}", flush=True)
            assert same, (label, rep, name)
        if rep == 0:
            first = {k: (v.clone() if v is not None else None) for k, v in ref.items()}
    return first


def _seed(rep):
    return 70000 + 100 * rep


@pytest.mark.parametrize("L,hidden,nq,nkv,hc,mode", [
    (1000, 1024, 8, 2, 2, "saved"),     # the launch-bound small layer: four chunks
    (777, 256, 8, 2, 1, "saved"),       # groups span four chunks, ragged tail
    (513, 384, 8, 2, 4, "recompute"),   # o_saved NULL: O recomputed from the lse
    (1000, 0, 8, 2, 2, "saved"),        # q/k/v given
])
def test_layer_step_replays_from_graph(L, hidden, nq, nkv, hc, mode):
    import headwise_chunked_context_amd as lib
    from _helpers import from_dev_bf16, from_dev_f32
    from test_gpu_parity import check, run_oracle

    torch = _torch()
    w = synthetic.WORKLOADS[1].with_(L=L, hidden=hidden, n_q=nq, n_kv=nkv, head_chunk=hc)
    draws = [synthetic.make_inputs(w, seed_base=_seed(r)) for r in range(REPLAYS)]
    names = ("x", "w_qkv", "w_o", "dy")
    x, wq, wo, dy = (to_dev(draws[0][k]) for k in names)
    recompute = mode == "recompute"
    nf = lib.workspace_bytes(L, hidden, nq, nkv, 128, hc, lib.PASS_FWD)
    nb = lib.workspace_bytes(L, hidden, nq, nkv, 128, hc,
                             lib.PASS_BWD_RECOMPUTE if recompute else lib.PASS_BWD)
    ws = torch.empty(max(nf, nb), dtype=torch.uint8, device="cuda:0")
    ws_eager = torch.empty_like(ws)

    def step(workspace):
        y, o, lse = lib.attn_fwd(x, wq, wo, nq, nkv, hc, w.theta, workspace=workspace)
        dx, dwq, dwo = lib.attn_bwd(x, wq, wo, None if recompute else o, lse, dy, nq, nkv, hc,
                                    w.theta, workspace=workspace)
        return dict(y=y, o=o, lse=lse, dx=dx, dwq=dwq, dwo=dwo)

    step(ws)                        # library loaded and first-call set-up done
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step(ws)

    def fill(rep):
        for t, k in zip((x, wq, wo, dy), names):
            if t is not None:
                t.copy_(to_dev(draws[rep][k]))

    ref = _replay_and_compare(torch, fill, lambda: step(ws_eager), out, g,
                              f"layer L={L} hidden={hidden} {nq}q{nkv}kv hc={hc} {mode}")
    gres = dict(o=from_dev_bf16(ref["o"]), lse=from_dev_f32(ref["lse"]), dx=from_dev_bf16(ref["dx"]))
    if hidden:
        gres.update(y=from_dev_bf16(ref["y"]), dwq=from_dev_bf16(ref["dwq"]),
                    dwo=from_dev_bf16(ref["dwo"]))
    check(gres, run_oracle(w, draws[0], hc), f"graph layer L={L} hc={hc} {mode}")


def test_mlp_step_replays_from_graph():
    """hidden 512, intermediate 1536, L 777 in ragged tiles of 300."""
    import headwise_chunked_context_amd as lib
    from test_gpu_mlp import check

    torch = _torch()
    w = synthetic.MLP_WORKLOADS[11].with_(L=777, tile_rows=300)
    draws = [synthetic.make_mlp_inputs(w, seed_base=_seed(r)) for r in range(REPLAYS)]
    names = ("x", "w_gate_up", "w_down", "dy")
    x, wgu, wd, dy = (to_dev(draws[0][k]) for k in names)
    tile = w.tile_rows

    def step():
        y = lib.mlp_fwd(x, wgu, wd, tile)
        dx, dwgu, dwd = lib.mlp_bwd(x, wgu, wd, dy, tile)
        return dict(y=y, dx=dx, dwgu=dwgu, dwd=dwd)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step()

    def fill(rep):
        for t, k in zip((x, wgu, wd, dy), names):
            t.copy_(to_dev(draws[rep][k]))

    ref = _replay_and_compare(torch, fill, step, out, g, f"mlp L={w.L} tile={tile}")
    check(ref, draws[0], tile, f"graph mlp L={w.L} tile={tile}")


@pytest.mark.parametrize("fused", [False, True])
def test_loss_step_replays_from_graph(fused):
    """hidden 256, vocabulary 1024, L 777 in ragged tiles of 300, every
    ignore_every-th row ignored; the separate forward and backward, or the
    fused call."""
    import headwise_chunked_context_amd as lib
    from test_gpu_loss import IGN, check

    torch = _torch()
    w = synthetic.LOSS_WORKLOADS[21].with_(L=777, tile_rows=300)
    draws = [synthetic.make_loss_inputs(w, seed_base=_seed(r)) for r in range(REPLAYS)]

    def targets(rep):
        return torch.from_numpy(np.ascontiguousarray(draws[rep]["targets"], dtype=np.int32))

    h, wt = to_dev(draws[0]["h"]), to_dev(draws[0]["w"])
    tg = targets(0).to("cuda:0")
    tile = w.tile_rows

    def step():
        if fused:
            loss, lse, dh, dw = lib.loss_fwd_bwd(h, wt, tg, 1.0, tile, IGN)
        else:
            loss, lse = lib.loss_fwd(h, wt, tg, tile, IGN)
            dh, dw = lib.loss_bwd(h, wt, tg, lse, 1.0, tile, IGN)
        return dict(loss=loss, lse=lse, dh=dh, dw=dw)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step()

    def fill(rep):
        h.copy_(to_dev(draws[rep]["h"]))
        wt.copy_(to_dev(draws[rep]["w"]))
        tg.copy_(targets(rep))

    label = f"loss L={w.L} tile={tile} {'fused' if fused else 'separate'}"
    ref = _replay_and_compare(torch, fill, step, out, g, label)
    check(ref, draws[0], tile, f"graph {label}")


def test_static_forward_replays_from_graph():
    """The allocation-free forward (static scratch, caller-allocated outputs)
    recorded into a graph: the capture allocates nothing, and each replay on
    fresh inputs equals the workspace forward's bits."""
    import headwise_chunked_context_amd as lib

    torch = _torch()
    L, hidden, nq, nkv, hc = 1000, 512, 8, 2, 2
    w = synthetic.WORKLOADS[1].with_(L=L, hidden=hidden, n_q=nq, n_kv=nkv, head_chunk=hc)
    draws = [synthetic.make_inputs(w, with_grad=False, seed_base=_seed(r)) for r in range(REPLAYS)]
    names = ("x", "w_qkv", "w_o")
    x, wq, wo = (to_dev(draws[0][k]) for k in names)
    out = (torch.empty(L, hidden, dtype=torch.bfloat16, device="cuda:0"),
           torch.empty(L, nq * 128, dtype=torch.bfloat16, device="cuda:0"),
           torch.empty(nq, L, dtype=torch.float32, device="cuda:0"))
    lib.attn_fwd_static(x, wq, wo, nq, nkv, hc, w.theta, out=out)   # scratch looked up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lib.attn_fwd_static(x, wq, wo, nq, nkv, hc, w.theta, out=out)

    def fill(rep):
        for t, k in zip((x, wq, wo), names):
            t.copy_(to_dev(draws[rep][k]))

    def eager():
        y, o, lse = lib.attn_fwd(x, wq, wo, nq, nkv, hc, w.theta)
        return dict(y=y, o=o, lse=lse)

    _replay_and_compare(torch, fill, eager, dict(y=out[0], o=out[1], lse=out[2]), g,
                        f"static forward L={L} hidden={hidden} hc={hc}")
