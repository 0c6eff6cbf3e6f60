"""Paged-KV attention for AMD MI355X (gfx950): HIP kernels behind a C ABI (include/pkv*.h).

    from paged_kv_cache_199_amd import kv_cache_write, paged_attn_decode, DecodeStep
    from paged_kv_cache_199_amd import paged_attn_prefill, paged_attn_decode_shared_prefix
    from paged_kv_cache_199_amd.blocks import BlockPool, Sequence, RadixIndex, append_step, copy_blocks
"""
from ._lib import (PATH_AUTO, PATH_MFMA, PATH_VALU, PREFIX_AUTO, PREFIX_PER_SEQUENCE, PREFIX_READ_ONCE, DecodeStep,
                   decode_plan, decode_workspace_bytes, kv_cache_write, kv_cache_write_fp8, load, new_workspace,
                   paged_attn_decode, paged_attn_decode_shared_prefix, paged_attn_prefill,
                   shared_prefix_workspace_bytes)

__all__ = ["kv_cache_write", "kv_cache_write_fp8", "paged_attn_decode", "paged_attn_prefill",
           "paged_attn_decode_shared_prefix", "decode_workspace_bytes", "shared_prefix_workspace_bytes",
           "decode_plan", "load", "new_workspace", "DecodeStep", "PATH_AUTO", "PATH_VALU", "PATH_MFMA",
           "PREFIX_AUTO", "PREFIX_READ_ONCE", "PREFIX_PER_SEQUENCE"]
