"""The torch.autograd wrappers (headwise_chunked_context_amd.autograd) on
the GPU: gradients from loss.backward() through them equal, bit for bit,
the outputs of the library's backward entry points called directly on the
same inputs (at these lengths every weight-gradient GEMM sums its
reduction in one part, so the weight gradients are reproducible bit for
bit as well)."""
import numpy as np
import pytest

import synthetic
from _helpers import to_dev

pytestmark = pytest.mark.gpu


def _torch():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _bits(t):
    import torch

    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _leaf(t):
    return t.detach().clone().requires_grad_(True)


@pytest.mark.parametrize("L,hidden,nq,nkv,hc,recompute", [
    (777, 256, 8, 2, 2, False),
    (513, 384, 8, 2, 4, True),     # the backward recomputes the attention output
    (1000, 0, 8, 2, 2, False),     # q/k/v given: the output is O, the gradient dqkv
])
def test_attention_function_gradients_equal_direct_calls(L, hidden, nq, nkv, hc, recompute):
    import headwise_chunked_context_amd as lib
    from headwise_chunked_context_amd import autograd as ag

    torch = _torch()
    w = synthetic.WORKLOADS[1].with_(L=L, hidden=hidden, n_q=nq, n_kv=nkv, head_chunk=hc)
    inp = synthetic.make_inputs(w)
    x, wq, wo, dy = (to_dev(inp[k]) for k in ("x", "w_qkv", "w_o", "dy"))
    xl = _leaf(x)
    wql = _leaf(wq) if hidden else None
    wol = _leaf(wo) if hidden else None
    out = ag.attention(xl, wql, wol, nq, nkv, hc, w.theta, recompute=recompute)
    out.backward(dy)
    y, o, lse = lib.attn_fwd(x, wq, wo, nq, nkv, hc, w.theta)
    ref = lib.attn_bwd(x, wq, wo, None if recompute else o, lse, dy, nq, nkv, hc, w.theta)
    torch.cuda.synchronize()
    checks = [("out", out.detach(), y if hidden else o), ("dx", xl.grad, ref[0])]
    if hidden:
        checks += [("dw_qkv", wql.grad, ref[1]), ("dw_o", wol.grad, ref[2])]
    for name, a, b in checks:
        same = torch.equal(_bits(a), _bits(b))
        print(f"autograd attention L={L} hidden={hidden} hc={hc} recompute={recompute}: "
              f"{name} bitwise equal = {same}", flush=True)
        assert same, name


def test_mlp_function_gradients_equal_direct_calls():
    import headwise_chunked_context_amd as lib
    from headwise_chunked_context_amd import autograd as ag

    torch = _torch()
    w = synthetic.MLP_WORKLOADS[11].with_(L=777, tile_rows=300)
    inp = synthetic.make_mlp_inputs(w)
    x, wgu, wd, dy = (to_dev(inp[k]) for k in ("x", "w_gate_up", "w_down", "dy"))
    xl, wgul, wdl = _leaf(x), _leaf(wgu), _leaf(wd)
    y = ag.swiglu_mlp(xl, wgul, wdl, w.tile_rows)
    y.backward(dy)
    ry = lib.mlp_fwd(x, wgu, wd, w.tile_rows)
    rdx, rdgu, rdwd = lib.mlp_bwd(x, wgu, wd, dy, w.tile_rows)
    torch.cuda.synchronize()
    for name, a, b in (("y", y.detach(), ry), ("dx", xl.grad, rdx), ("dw_gate_up", wgul.grad, rdgu),
                       ("dw_down", wdl.grad, rdwd)):
        same = torch.equal(_bits(a), _bits(b))
        print(f"autograd mlp: {name} bitwise equal = {same}", flush=True)
        assert same, name


@pytest.mark.parametrize("scale", [1.0, 0.25])
def test_loss_function_gradients_equal_direct_calls(scale):
    """loss.backward() with upstream gradient 1 and a scaled loss (the
    upstream gradient then reaches the library as dloss)."""
    import headwise_chunked_context_amd as lib
    from headwise_chunked_context_amd import autograd as ag
    from test_gpu_loss import IGN

    torch = _torch()
    w = synthetic.LOSS_WORKLOADS[21].with_(L=777, tile_rows=300)
    inp = synthetic.make_loss_inputs(w)
    h, wt = to_dev(inp["h"]), to_dev(inp["w"])
    tg = torch.from_numpy(np.ascontiguousarray(inp["targets"], dtype=np.int32)).to("cuda:0")
    hl, wl = _leaf(h), _leaf(wt)
    loss = ag.cross_entropy(hl, wl, tg, w.tile_rows, IGN)
    (loss * scale).backward()
    rl, rlse = lib.loss_fwd(h, wt, tg, w.tile_rows, IGN)
    rdh, rdw = lib.loss_bwd(h, wt, tg, rlse, scale, w.tile_rows, IGN)
    torch.cuda.synchronize()
    assert loss.dim() == 0
    for name, a, b in (("loss", loss.detach().reshape(1), rl), ("dh", hl.grad, rdh), ("dw", wl.grad, rdw)):
        same = torch.equal(_bits(a), _bits(b))
        print(f"autograd loss scale={scale}: {name} bitwise equal = {same}", flush=True)
        assert same, name
