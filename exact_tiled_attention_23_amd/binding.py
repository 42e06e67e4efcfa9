"""Python binding of libfa.so: the same names as the C ABI, plus a tensor-level forward().

Argument marshalling only: every step of the attention forward runs in the
HIP kernel behind ``fa_fwd``. PyTorch provides device memory and the stream.
If the library is missing this module raises; there is no fallback path.
"""

import ctypes
import math
import os

import torch

from .build import LIB

FA_F32, FA_BF16, FA_F16 = 0, 1, 2
FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED, FA_ERR_ALIGN, FA_ERR_ARG, FA_ERR_HIP = 0, -1, -2, -3, -4, -5, -6
EXPORTED = ("fa_fwd", "fa_fwd_strided", "fa_strerror", "fa_abi_version")

_TORCH_DTYPE = {torch.float32: FA_F32, torch.bfloat16: FA_BF16, torch.float16: FA_F16}
_lib = None


def load_library():
    """Load libfa.so (once) and declare its signatures. Raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"HIP library not built: {LIB} is missing "
                               "(run `python -m exact_tiled_attention_23_amd.build`)")
        lib = ctypes.CDLL(LIB)
        lib.fa_fwd.restype = ctypes.c_int
        lib.fa_fwd.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                               ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        lib.fa_fwd_strided.restype = ctypes.c_int
        lib.fa_fwd_strided.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        lib.fa_strerror.restype = ctypes.c_char_p
        lib.fa_strerror.argtypes = [ctypes.c_int]
        lib.fa_abi_version.restype = ctypes.c_int
        lib.fa_abi_version.argtypes = []
        _lib = lib
    return _lib


def fa_fwd(Q, K, V, O, LSE, B, H, N, D, scale, causal, kv_len, dtype, stream):
    """Raw C call; pointers are ints (0 for NULL). Returns the C return code."""
    return load_library().fa_fwd(Q, K, V, O, LSE, B, H, N, D, scale, causal, kv_len, dtype, stream)


def fa_fwd_strided(Q, K, V, O, LSE, B, H, N, D, strides, scale, causal, kv_len, dtype, stream):
    """Raw C call with strides: None (contiguous) or 12 ints (q, k, v, o; batch, head, token)."""
    arr = None
    if strides is not None:
        if len(strides) != 12:
            raise ValueError("strides needs 12 values")
        arr = (ctypes.c_int64 * 12)(*[int(x) for x in strides])
    return load_library().fa_fwd_strided(Q, K, V, O, LSE, B, H, N, D, arr, scale, causal, kv_len, dtype, stream)


def fa_strerror(code):
    return load_library().fa_strerror(code).decode()


def fa_abi_version():
    return load_library().fa_abi_version()


def _check(rc):
    if rc != FA_OK:
        raise RuntimeError(f"fa_fwd failed ({rc}): {fa_strerror(rc)}")


def forward(q, k, v, *, causal=True, scale=None, kv_len=None, out=None, lse=None, stream=None):
    """Attention forward on device tensors [B, H, N, D]. Returns (o, lse).

    q, k, v (and out) may be any strided views whose last dimension is contiguous,
    e.g. a [B, N, H, D] tensor transposed to [B, H, N, D]; a zero head stride on k and v
    shares one K/V head among all query heads.

    causal defaults to True and scale to 1/sqrt(D) rounded to float32, as the
    pages' constructor options do. kv_len: None, or int32-convertible values
    per batch (a CPU sequence is range-checked here and copied to the device;
    a device int32 tensor is passed through and clamped to [0, N] by the kernel).
    """
    if q.dtype not in _TORCH_DTYPE or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype among float32, bfloat16, float16")
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must be [B, H, N, D] of one shape")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be device tensors")
    for t in (q, k, v):
        if t.stride(3) != 1 and t.shape[3] > 1:
            raise ValueError("the head dimension of q, k, v must be contiguous (stride 1)")
    B, H, N, D = q.shape
    if scale is None:
        scale = float(torch.tensor(1.0 / math.sqrt(D), dtype=torch.float32))
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    if out.shape != q.shape or out.dtype != q.dtype or (out.stride(3) != 1 and D > 1):
        raise ValueError("out must be shaped and typed like q, with a contiguous head dimension")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor [B, H, N]")
    kv_ptr = 0
    kv_dev = None
    if kv_len is not None:
        if isinstance(kv_len, torch.Tensor) and kv_len.is_cuda:
            if kv_len.dtype != torch.int32 or kv_len.shape != (B,) or not kv_len.is_contiguous():
                raise ValueError("device kv_len must be a contiguous int32 tensor [B]")
            kv_dev = kv_len
        else:
            kv_cpu = torch.as_tensor(kv_len).to(torch.int64).reshape(-1)
            if kv_cpu.shape != (B,):
                raise ValueError("kv_len must have one entry per batch")
            if B and (int(kv_cpu.min()) < 0 or int(kv_cpu.max()) > N):
                raise ValueError("kv_len values must lie in [0, N]")
            kv_dev = kv_cpu.to(torch.int32).to(dev)
        kv_ptr = kv_dev.data_ptr()
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    strides = [x for t in (q, k, v, out) for x in t.stride()[:3]]
    with torch.cuda.device(dev):
        rc = fa_fwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                            B, H, N, D, strides, float(scale), 1 if causal else 0, kv_ptr,
                            _TORCH_DTYPE[q.dtype], handle)
    _check(rc)
    return out, lse
