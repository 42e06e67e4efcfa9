"""fa_bwd_noalloc (the backward whose workspace is the library's static scratch array) through
the C ABI, against fa_bwd with a workspace the caller allocates: the same kernels, so every
element of dQ, dK and dV must be bitwise equal. Two calls in a row, the second one smaller, so
the second runs on the scratch contents the first left behind. Outputs are NaN-filled first."""

import numpy as np
import pytest
import torch

import exact_tiled_attention_23_amd as fa
from exact_tiled_attention_23_amd import binding
from exact_tiled_attention_23_amd.workloads import generate, generate_grad_output

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _grads_both_ways(B, H, N, D, dtype, causal, kv, seed):
    print(f"noalloc backward B={B} H={H} N={N} D={D} {dtype} causal={causal} kv_len={kv}", flush=True)
    x = generate(B, H, N, D, dtype, causal=causal, seed=seed)
    do = generate_grad_output(B, H, N, D, dtype, seed=seed + 1)
    q, k, v, dO = (t.to(DEV) for t in (x.q, x.k, x.v, do))
    kvd = None if kv is None else torch.as_tensor(np.asarray(kv, dtype=np.int32)).to(DEV)
    o, lse = fa.forward(q, k, v, causal=causal, scale=x.scale, kv_len=kvd)
    code = {"bf16": fa.FA_BF16, "f16": fa.FA_F16}[dtype]
    stream = torch.cuda.current_stream(DEV).cuda_stream
    kvp = 0 if kvd is None else kvd.data_ptr()
    need = fa.fa_bwd_workspace_bytes(B, H, N, D)
    assert 0 < need <= binding.NOALLOC_SCRATCH_BYTES
    ws = torch.full((need,), 255, dtype=torch.uint8, device=DEV)   # all-ones bytes: NaN floats
    ref = [torch.full_like(q, float("nan")) for _ in range(3)]
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    ins = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dO.data_ptr())
    rc = fa.fa_bwd(*ins, *(t.data_ptr() for t in ref), B, H, N, D, x.scale, int(causal), kvp, code,
                   ws.data_ptr(), need, stream)
    assert rc == 0, fa.fa_strerror(rc)
    rc = fa.fa_bwd_noalloc(*ins, *(t.data_ptr() for t in got), B, H, N, D, x.scale, int(causal), kvp, code, stream)
    assert rc == 0, fa.fa_strerror(rc)
    torch.cuda.synchronize()
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert not torch.isnan(g).any().item(), f"{name}: NaN (an element left unwritten)"
        assert torch.equal(g, r), f"{name} differs from fa_bwd's"


def test_noalloc_backward_two_calls():
    _grads_both_ways(2, 4, 1000, 128, "bf16", True, [1000, 517], seed=9300)
    _grads_both_ways(1, 2, 300, 64, "f16", False, [211], seed=9310)
