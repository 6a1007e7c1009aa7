"""fp64 CPU oracle for headwise-chunked causal GQA attention and the
sequence-tiled SwiGLU MLP and language-model loss.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only the tests, the smoke check of __graft_entry__ and the
cpu_baseline leg of bench.py use it.  It shares no code with the HIP library.
"""
from .attention import (  # noqa: F401
    attention_bwd_head,
    attention_fwd_head,
    attention_rows,
    dq_rows,
    kv_grad_tail,
    layer_bwd,
    layer_fwd,
    layer_rows,
    rope,
    rope_angles,
)
from .mlp import mlp_bwd, mlp_fwd, silu, silu_grad  # noqa: F401
from .loss import logsumexp_rows, loss_bwd, loss_fwd  # noqa: F401
