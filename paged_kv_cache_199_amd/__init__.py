"""Paged-KV decode attention for AMD MI355X (gfx950): HIP kernels behind a C ABI (include/pkv.h).

    from paged_kv_cache_199_amd import kv_cache_write, paged_attn_decode
"""
from ._lib import (PATH_AUTO, PATH_MFMA, PATH_VALU, DecodeStep, decode_plan, decode_workspace_bytes,
                   kv_cache_write, kv_cache_write_fp8, load, new_workspace, paged_attn_decode)

__all__ = ["kv_cache_write", "kv_cache_write_fp8", "paged_attn_decode", "decode_workspace_bytes", "decode_plan",
           "load", "new_workspace", "DecodeStep", "PATH_AUTO", "PATH_VALU", "PATH_MFMA"]
