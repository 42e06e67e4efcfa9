"""Exact tiled attention forward (online softmax) for AMD Instinct MI355X (gfx950).

The work runs in hand-written HIP kernels behind the C ABI in include/fa.h
(libfa.so, built in-tree by ``exact_tiled_attention_23_amd.build``). This
package is its thin binding; the library is loaded on first use and its
absence is an error, never a fallback.
"""

from .binding import (FA_BF16, FA_F16, FA_F32, FlashAttention, attention, backward, fa_abi_version, fa_bwd, fa_bwd_strided,
                      fa_bwd_noalloc, fa_bwd_workspace_bytes, fa_fwd,
                      fa_fwd_split, fa_fwd_split_count,
                      fa_fwd_split_workspace_bytes, fa_fwd_strided, fa_merge_states, fa_strerror, forward,
                      load_library, merge_states)

__all__ = ["forward", "backward", "attention", "FlashAttention", "merge_states", "fa_bwd", "fa_bwd_strided", "fa_bwd_noalloc", "fa_bwd_workspace_bytes", "fa_fwd", "fa_fwd_strided", "fa_fwd_split", "fa_fwd_split_count", "fa_fwd_split_workspace_bytes",
           "fa_merge_states", "fa_strerror", "fa_abi_version", "load_library", "FA_F32", "FA_BF16", "FA_F16"]
