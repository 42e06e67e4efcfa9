"""The entry points under HIP graph capture: they allocate nothing, synchronise nothing and
record no memset, so a captured forward, split forward and backward replay correctly.

The graph is replayed several times with new inputs written between replays (eager work
between them), and every replay is compared bit for bit with eager calls on the same inputs
(the kernels are deterministic). Parity with the oracle is covered elsewhere; here the eager
path is the reference.
"""

import pytest
import torch

import exact_tiled_attention_23_amd as fa
from exact_tiled_attention_23_amd.workloads import generate, generate_grad_output

from test_parity_gpu import say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.mark.parametrize("D", [64, 128])
def test_forward_split_backward_in_graph(D):
    B, H, N = 1, 4, 1000
    x = generate(B, H, N, D, "bf16", causal=True, seed=301)
    q, k, v = (t.to(DEV) for t in (x.q, x.k, x.v))
    do = generate_grad_output(B, H, N, D, "bf16", seed=302).to(DEV)
    o, o2 = torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    lse2 = torch.empty_like(lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws_split = torch.empty(fa.fa_fwd_split_workspace_bytes(B, H, N, D, 3), dtype=torch.uint8, device=DEV)
    ws_bwd = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, D), dtype=torch.uint8, device=DEV)

    def step():
        fa.forward(q, k, v, causal=True, scale=x.scale, out=o, lse=lse)
        fa.forward(q, k, v, causal=True, scale=x.scale, out=o2, lse=lse2, n_splits=3, workspace=ws_split)
        fa.backward(q, k, v, o, lse, do, causal=True, scale=x.scale, dq=dq, dk=dk, dv=dv, workspace=ws_bwd)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    say(f"capturing forward + split forward + backward, D={D}")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    gen = torch.Generator(device="cpu").manual_seed(303)
    for rep in range(3):
        # new inputs, written eagerly between replays
        q.copy_(torch.randn(q.shape, generator=gen).to(torch.bfloat16))
        do.copy_(torch.randn(do.shape, generator=gen).to(torch.bfloat16))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (o, lse, o2, lse2, dq, dk, dv)]
        step()                      # the same work, eagerly
        torch.cuda.synchronize()
        want = (o, lse, o2, lse2, dq, dk, dv)
        say(f"replay {rep}")
        for name, a, b in zip(("O", "LSE", "O split", "LSE split", "dQ", "dK", "dV"), got, want):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"
