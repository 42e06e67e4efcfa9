"""The Python binding on a stream other than the current one.

The binding makes temporaries (a host kv_len copied to the device, the split forward's and the
backward's workspaces, outputs it allocates) from torch's caching allocator on the current
stream. When the kernels are queued on another stream, those tensors are marked as used there,
so their memory cannot be handed to a later allocation on the current stream while the kernels
still wait to run. The test keeps the side stream busy with matrix products, calls the split
forward and the backward on it, and at once allocates and fills tensors of the same sizes on the
current stream: without the marking the queued kernels would read those fills (a kv_len of 0
gives an all-zero output). Results must equal the same calls made on the current stream.
"""

import numpy as np
import pytest
import torch

import exact_tiled_attention_23_amd as fa
from exact_tiled_attention_23_amd.workloads import generate, generate_grad_output

from test_parity_gpu import say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def test_side_stream_temporaries():
    B, H, N, D = 4, 4, 1024, 128
    kv = [N, 500, 37, 900]
    x = generate(B, H, N, D, "bf16", causal=True, seed=9100)
    do = generate_grad_output(B, H, N, D, "bf16", seed=9101)
    q, k, v, dO = (t.to(DEV) for t in (x.q, x.k, x.v, do))
    say("side stream: reference calls on the current stream")
    o_ref, l_ref = fa.forward(q, k, v, causal=True, scale=x.scale, kv_len=kv, n_splits=3)
    g_ref = fa.backward(q, k, v, o_ref, l_ref, dO, causal=True, scale=x.scale, kv_len=kv)
    torch.cuda.synchronize()

    ws_fwd = fa.fa_fwd_split_workspace_bytes(B, H, N, D, 3)
    ws_bwd = fa.fa_bwd_workspace_bytes(B, H, N, D)
    side = torch.cuda.Stream(device=DEV)
    a = torch.randn(8192, 8192, device=DEV, dtype=torch.bfloat16)
    side.wait_stream(torch.cuda.current_stream(DEV))
    outs = []
    for call in range(2):
        say(f"side stream: call {call}, with the side stream busy")
        with torch.cuda.stream(side):
            for _ in range(6):
                a = torch.mm(a, a) * 1e-3  # a few milliseconds of work queued ahead
        o, l = fa.forward(q, k, v, causal=True, scale=x.scale, kv_len=kv, n_splits=3, stream=side)
        junk = [torch.zeros(B, dtype=torch.int32, device=DEV), torch.full((ws_fwd,), 255, dtype=torch.uint8, device=DEV)]
        g = fa.backward(q, k, v, o, l, dO, causal=True, scale=x.scale, kv_len=kv, stream=side.cuda_stream)
        junk += [torch.zeros(B, dtype=torch.int32, device=DEV), torch.full((ws_bwd,), 255, dtype=torch.uint8, device=DEV),
                 torch.full_like(q, float("nan"))]
        outs.append((o, l, g, junk))
    torch.cuda.synchronize()
    for o, l, g, _ in outs:
        assert torch.equal(o, o_ref) and torch.equal(l, l_ref), "forward on the side stream differs"
        for name, gg, rr in zip(("dQ", "dK", "dV"), g, g_ref):
            assert torch.equal(gg, rr), f"{name} on the side stream differs"
    assert np.isfinite(o_ref.float().cpu().numpy()).all()
