"""ctypes binding of libpkv.so (the C ABI in include/pkv.h).

Argument marshalling only: shapes and dtypes are checked, raw device pointers and sizes are passed,
and every step of the computation runs in the library's HIP kernels on the caller's current stream.
There is no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpkv.so")

PKV_F32, PKV_BF16, PKV_BF16_FP8KV = 0, 1, 2
PATH_AUTO, PATH_VALU, PATH_MFMA = 0, 1, 2
SCHEDULE_AUTO, SCHEDULE_GRID, SCHEDULE_PERSISTENT = 0, 1, 2
PREFIX_AUTO, PREFIX_READ_ONCE, PREFIX_PER_SEQUENCE = 0, 1, 2
BLOCK_SIZE = 16

_c_int, _c_i64, _c_sz, _c_f, _vp = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p


class DecodeOptions(ctypes.Structure):
    _fields_ = [("partition_size", _c_int), ("path", _c_int), ("pipeline_depth", _c_int),
                ("schedule", _c_int), ("event_main_begin", _vp), ("event_main_end", _vp),
                ("workgroups_per_cu", _c_int), ("k_scale", _c_f), ("v_scale", _c_f),
                ("shared_prefix_mode", _c_int)]


class DecodePlanInfo(ctypes.Structure):
    _fields_ = [("partition_size", _c_int), ("num_partitions", _c_int), ("path", _c_int),
                ("rows_per_tile", _c_int), ("row_tiles", _c_int), ("pipeline_depth", _c_int),
                ("schedule", _c_int), ("grid_waves", _c_int), ("workspace_bytes", _c_sz),
                ("item_cost", _c_int), ("piece_slots", _c_int), ("min_workspace_bytes", _c_sz)]


_lib: Optional[ctypes.CDLL] = None

EXPORTS = {
    "pkv_kv_cache_write": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_int, _c_int, _c_int, _c_int, _vp]),
    "pkv_decode_workspace_bytes": (_c_sz, [_c_int] * 8 + [ctypes.POINTER(DecodeOptions)]),
    "pkv_decode_plan": (_c_int, [_c_int] * 8 + [ctypes.POINTER(DecodeOptions), ctypes.POINTER(DecodePlanInfo)]),
    "pkv_paged_attn_decode": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       _c_int, _c_int, _c_int, _c_int, _c_int, _c_i64,
                                       _c_int, _c_int, _c_int, _c_int, _c_f, _c_int,
                                       ctypes.POINTER(DecodeOptions), _vp, _c_sz, _vp]),
    "pkv_paged_attn_decode_append": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                              _c_int, _c_int, _c_int, _c_int, _c_int, _c_i64,
                                              _c_int, _c_int, _c_int, _c_int, _c_f, _c_int,
                                              ctypes.POINTER(DecodeOptions), _vp, _c_sz, _vp]),
    "pkv_paged_attn_decode_noalloc": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                               _c_int, _c_int, _c_int, _c_int, _c_int, _c_i64,
                                               _c_int, _c_int, _c_int, _c_int, _c_f, _c_int,
                                               ctypes.POINTER(DecodeOptions), _vp]),
    "pkv_kv_cache_write_fp8": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_int, _c_int, _c_int, _c_f, _c_f,
                                        _vp]),
    "pkv_decode_shared_prefix_workspace_bytes": (_c_sz, [_c_int] * 11 + [ctypes.POINTER(DecodeOptions)]),
    "pkv_paged_attn_decode_shared_prefix": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                     _c_int, _c_int, _c_int, _c_int, _c_int, _c_i64,
                                                     _c_int, _c_int, _c_int, _c_int, _c_f, _c_int,
                                                     _vp, _vp, _vp, _c_int, _c_int, _c_int,
                                                     ctypes.POINTER(DecodeOptions), _vp, _c_sz, _vp]),
    "pkv_paged_attn_prefill": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int,
                                        _c_int, _c_i64, _c_int, _c_int, _c_int, _c_int, _c_f, _c_int,
                                        ctypes.POINTER(DecodeOptions), _vp]),
    "pkv_copy_blocks": (_c_int, [_vp, _vp, _vp, _vp, ctypes.c_int32, _c_i64, _c_int, _c_int, _c_int, _vp]),
    # device-side check of the decode preconditions (include/pkv_check.h)
    "pkv_check_decode_inputs": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_i64, _c_int,
                                         _vp, _vp]),
    # host-side block management (include/pkv_blocks.h); handles are opaque pointers
    "pkv_block_pool_create": (_vp, [ctypes.c_int32]),
    "pkv_block_pool_destroy": (None, [_vp]),
    "pkv_block_pool_free_count": (ctypes.c_int32, [_vp]),
    "pkv_block_refcount": (ctypes.c_int32, [_vp, ctypes.c_int32]),
    "pkv_seq_create": (_vp, [_vp]),
    "pkv_seq_destroy": (None, [_vp]),
    "pkv_seq_length": (_c_i64, [_vp]),
    "pkv_seq_num_blocks": (ctypes.c_int32, [_vp]),
    "pkv_seq_block_table": (ctypes.c_int32, [_vp, _vp, ctypes.c_int32]),
    "pkv_seq_append": (ctypes.c_int32, [_vp, ctypes.c_int32, _vp, _vp, _vp, _vp]),
    "pkv_seqs_append": (_c_i64, [_vp, ctypes.c_int32, _vp, _vp, _vp, _vp, _vp]),
    "pkv_seq_fork": (_vp, [_vp]),
    "pkv_seq_adopt_prefix": (ctypes.c_int32, [_vp, _vp, ctypes.c_int32]),
    "pkv_radix_create": (_vp, [_vp]),
    "pkv_radix_destroy": (None, [_vp]),
    "pkv_radix_match": (ctypes.c_int32, [_vp, _vp, _c_i64, _vp, ctypes.c_int32]),
    "pkv_radix_insert": (ctypes.c_int32, [_vp, _vp, _c_i64, _vp]),
    "pkv_radix_evict": (ctypes.c_int32, [_vp, ctypes.c_int32]),
    "pkv_radix_cached_blocks": (ctypes.c_int32, [_vp]),
    "pkv_status_string": (ctypes.c_char_p, [_c_int]),
    "pkv_version": (_c_int, []),
}


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpkv.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m paged_kv_cache_199_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(rc: int, what: str):
    if rc != 0:
        msg = load().pkv_status_string(rc).decode()
        raise RuntimeError(f"{what} failed: {msg} (status {rc})")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PKV_F32
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _decode_code(q, k_cache, v_cache, out) -> int:
    """dtype code of a decode call: all fp32, all bf16, or bf16 q/out over uint8 E4M3 pools."""
    for t in (q, k_cache, v_cache, out):
        _need(t.is_contiguous(), "q, caches and out: contiguous")
    _need(out.dtype == q.dtype and k_cache.dtype == v_cache.dtype, "out matches q, V pool matches K pool")
    if q.dtype == torch.bfloat16 and k_cache.dtype == torch.uint8:
        return PKV_BF16_FP8KV
    _need(k_cache.dtype == q.dtype, "caches in q's dtype (or uint8 E4M3 codes with bf16 q)")
    return _dtype_code(q)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


# Device type the kernels run on (torch names ROCm devices "cuda").
_GPU_TYPE = "cuda"


def _on_gpu_like(ref: torch.Tensor, what: str, *tensors) -> None:
    """Every given tensor (None skipped) lives on ref's device, and that device is a GPU: a host pointer
    handed to a kernel would fault the GPU, so this is checked before any call."""
    _need(ref.device.type == _GPU_TYPE, f"{what}: tensors must be on the GPU")
    for t in tensors:
        if t is not None:
            _need(t.device == ref.device, f"{what}: every tensor must be on {ref.device} (got {t.device})")


def _check_decode_args(q, k_cache, v_cache, block_tables, context_lens, q_lens, out, lse, num_heads,
                       num_kv_heads, head_dim, block_size):
    """Shape, dtype, layout and device checks shared by the decode, prefill and shared-prefix calls.
    Returns (total_q, num_seqs, num_blocks, dtype code)."""
    _need(q.dim() == 3 and tuple(q.shape[1:]) == (num_heads, head_dim), "q must be [total_q, H, D]")
    total_q = q.shape[0]
    S = context_lens.numel()
    NB = k_cache.shape[0]
    _need(tuple(k_cache.shape) == (NB, num_kv_heads, block_size, head_dim), "k_cache [NB, KVH, 16, D]")
    _need(tuple(v_cache.shape) == (NB, num_kv_heads, head_dim, block_size), "v_cache [NB, KVH, D, 16]")
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and block_tables.shape[0] == S
          and block_tables.is_contiguous(), "block_tables: int32 [S, max_blocks], contiguous")
    _need(context_lens.dtype == torch.int32 and context_lens.is_contiguous(), "context_lens: int32 [S]")
    if q_lens is not None:
        _need(q_lens.dtype == torch.int32 and q_lens.numel() == S and q_lens.is_contiguous(), "q_lens: int32 [S]")
    if lse is not None:
        _need(lse.dtype == torch.float32 and tuple(lse.shape) == (total_q, num_heads) and lse.is_contiguous(),
              "lse: fp32 [total_q, H]")
    _on_gpu_like(q, "decode arguments", k_cache, v_cache, block_tables, context_lens, q_lens, out, lse)
    code = _decode_code(q, k_cache, v_cache, out)
    return total_q, S, NB, code


def _check_workspace(ws, q) -> int:
    """Bytes of a caller-supplied workspace (contiguous, on q's device); 0 when None."""
    if ws is None:
        return 0
    _need(ws.is_contiguous(), "workspace must be contiguous")
    _on_gpu_like(q, "workspace", ws)
    return ws.numel() * ws.element_size()


def _workspace_for(nbytes: int, device, stream):
    """A workspace the call allocates itself.  Allocated from `stream`'s pool when a stream is given, so
    the caching allocator does not hand the block to other work on the current stream while the
    kernels enqueued on `stream` still use it."""
    if stream is None:
        return new_workspace(nbytes, device)
    with torch.cuda.stream(stream):
        return new_workspace(nbytes, device)


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _opts(partition_size: int, path: int, events, depth: int = 0, schedule: int = 0,
          wgs_per_cu: int = 0, k_scale: float = 0.0, v_scale: float = 0.0) -> DecodeOptions:
    o = DecodeOptions(partition_size, path, depth, schedule, None, None, wgs_per_cu, k_scale, v_scale)
    if events is not None:
        b, e = events
        o.event_main_begin = b.cuda_event
        o.event_main_end = e.cuda_event
    return o


def kv_cache_write(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                   k_cache: torch.Tensor, v_cache: torch.Tensor, stream=None) -> None:
    """k/v [T, KVH, D] -> k_cache [NB, KVH, 16, D] / v_cache [NB, KVH, D, 16] at slot_mapping (int64)."""
    lib = load()
    _need(k.dim() == 3 and k.shape == v.shape, "k and v must be [T, KVH, D] of one shape")
    T, KVH, D = k.shape
    _need(k_cache.dim() == 4 and v_cache.dim() == 4, "caches must be 4-d")
    NB = k_cache.shape[0]
    _need(tuple(k_cache.shape) == (NB, KVH, BLOCK_SIZE, D), "k_cache must be [NB, KVH, 16, D]")
    _need(tuple(v_cache.shape) == (NB, KVH, D, BLOCK_SIZE), "v_cache must be [NB, KVH, D, 16]")
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.numel() == T, "slot_mapping: int64 [T]")
    for t in (k, v, k_cache, v_cache):
        _need(t.dtype == k.dtype and t.is_contiguous(), "same dtype, contiguous")
    _need(slot_mapping.is_contiguous(), "slot_mapping must be contiguous")
    _on_gpu_like(k, "kv_cache_write", v, k_cache, v_cache, slot_mapping)
    rc = lib.pkv_kv_cache_write(_ptr(k), _ptr(v), _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache),
                                T, NB, KVH, D, BLOCK_SIZE, _dtype_code(k), _stream(stream))
    _check(rc, "pkv_kv_cache_write")


def kv_cache_write_fp8(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor, k_cache: torch.Tensor,
                       v_cache: torch.Tensor, k_scale: float, v_scale: float, stream=None) -> None:
    """bf16 k/v [T, KVH, D] -> E4M3 codes in uint8 pools k_cache [NB, KVH, 16, D] / v_cache [NB, KVH, D, 16]."""
    lib = load()
    _need(k.dim() == 3 and k.shape == v.shape and k.dtype == torch.bfloat16 and v.dtype == torch.bfloat16,
          "k and v: bf16 [T, KVH, D] of one shape")
    T, KVH, D = k.shape
    NB = k_cache.shape[0]
    _need(k_cache.dtype == torch.uint8 and v_cache.dtype == torch.uint8, "uint8 code pools")
    _need(tuple(k_cache.shape) == (NB, KVH, BLOCK_SIZE, D) and tuple(v_cache.shape) == (NB, KVH, D, BLOCK_SIZE),
          "k_cache [NB, KVH, 16, D], v_cache [NB, KVH, D, 16]")
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.numel() == T, "slot_mapping: int64 [T]")
    for t in (k, v, k_cache, v_cache, slot_mapping):
        _need(t.is_contiguous(), "contiguous")
    _on_gpu_like(k, "kv_cache_write_fp8", v, k_cache, v_cache, slot_mapping)
    rc = lib.pkv_kv_cache_write_fp8(_ptr(k), _ptr(v), _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache), T, NB, KVH,
                                    D, BLOCK_SIZE, float(k_scale), float(v_scale), _stream(stream))
    _check(rc, "pkv_kv_cache_write_fp8")


def decode_workspace_bytes(num_seqs, total_q, max_q_len, max_context_len, num_heads, num_kv_heads,
                           head_dim, dtype_code, partition_size=0, path=PATH_AUTO, depth=0,
                           schedule=0, wgs_per_cu=0) -> int:
    o = DecodeOptions(partition_size, path, depth, schedule, None, None, wgs_per_cu)
    return int(load().pkv_decode_workspace_bytes(num_seqs, total_q, max_q_len, max_context_len, num_heads,
                                                 num_kv_heads, head_dim, dtype_code, ctypes.byref(o)))


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """A decode workspace of nbytes on `device` (contents on entry do not matter)."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def decode_plan(num_seqs, total_q, max_q_len, max_context_len, num_heads, num_kv_heads, head_dim,
                dtype_code, partition_size=0, path=PATH_AUTO, depth=0, schedule=0, wgs_per_cu=0) -> dict:
    """What the library launches for these sizes: partition size, kernel path, row tiling, workspace."""
    o = DecodeOptions(partition_size, path, depth, schedule, None, None, wgs_per_cu)
    info = DecodePlanInfo()
    rc = int(load().pkv_decode_plan(num_seqs, total_q, max_q_len, max_context_len, num_heads, num_kv_heads,
                                    head_dim, dtype_code, ctypes.byref(o), ctypes.byref(info)))
    _check(rc, "pkv_decode_plan")
    return {k: getattr(info, k) for k, _ in DecodePlanInfo._fields_}


def paged_attn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      block_tables: torch.Tensor, context_lens: torch.Tensor,
                      q_lens: Optional[torch.Tensor], out: torch.Tensor, lse: Optional[torch.Tensor],
                      num_heads: int, num_kv_heads: int, head_dim: int, block_size: int, scale: float,
                      max_context_len: int, max_q_len: int = 1, partition_size: int = 0,
                      path: int = PATH_AUTO, workspace: Optional[torch.Tensor] = None,
                      events=None, stream=None, depth: int = 0, schedule: int = 0,
                      wgs_per_cu: int = 0, new_k: Optional[torch.Tensor] = None,
                      new_v: Optional[torch.Tensor] = None, k_scale: float = 0.0, v_scale: float = 0.0) -> None:
    """Decode attention through the C ABI.  q/out [total_q, H, D]; lse fp32 [total_q, H] or None.

    With new_k / new_v ([total_q, KVH, D], packed like q) the step appends them first, at each
    sequence's last q positions through its block table (pkv_paged_attn_decode_append).

    q_lens None means every sequence has max_q_len new tokens.  max_context_len is a host-known upper
    bound of context_lens (the kernels never read device data on the host).  A workspace tensor
    (any dtype, contiguous, on the GPU) of decode_workspace_bytes() bytes is allocated when not given;
    a given one may be smaller, down to decode_plan()["min_workspace_bytes"] (fewer piece slots).  `events` = (begin, end) torch.cuda.Event pair that has been recorded once: the library
    records them around its partition kernel."""
    lib = load()
    total_q, S, NB, code = _check_decode_args(q, k_cache, v_cache, block_tables, context_lens, q_lens, out, lse,
                                              num_heads, num_kv_heads, head_dim, block_size)
    o = _opts(partition_size, path, events, depth, schedule, wgs_per_cu, k_scale, v_scale)
    need = int(lib.pkv_decode_workspace_bytes(S, total_q, max_q_len, max_context_len, num_heads,
                                              num_kv_heads, head_dim, code, ctypes.byref(o)))
    if workspace is None and need > 0:
        workspace = _workspace_for(need, q.device, stream)
    ws_bytes = _check_workspace(workspace, q)
    if new_k is None:
        rc = lib.pkv_paged_attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                       _ptr(context_lens), _ptr(q_lens), _ptr(out), _ptr(lse),
                                       S, block_tables.shape[1], total_q, max_q_len, max_context_len, NB,
                                       num_heads, num_kv_heads, head_dim, block_size, float(scale), code,
                                       ctypes.byref(o), _ptr(workspace), ws_bytes, _stream(stream))
        _check(rc, "pkv_paged_attn_decode")
        return
    _need(new_v is not None and new_k.shape == new_v.shape
          and tuple(new_k.shape) == (total_q, num_kv_heads, head_dim), "new_k / new_v must be [total_q, KVH, D]")
    for t in (new_k, new_v):
        _need(t.dtype == q.dtype and t.is_contiguous(), "new_k / new_v: q's dtype, contiguous")
    _on_gpu_like(q, "new_k / new_v", new_k, new_v)
    rc = lib.pkv_paged_attn_decode_append(_ptr(q), _ptr(new_k), _ptr(new_v), _ptr(k_cache), _ptr(v_cache),
                                          _ptr(block_tables), _ptr(context_lens), _ptr(q_lens), _ptr(out),
                                          _ptr(lse), S, block_tables.shape[1], total_q, max_q_len,
                                          max_context_len, NB, num_heads, num_kv_heads, head_dim, block_size,
                                          float(scale), code, ctypes.byref(o), _ptr(workspace), ws_bytes,
                                          _stream(stream))
    _check(rc, "pkv_paged_attn_decode_append")


NOALLOC_SCRATCH_BYTES = 64 << 20     # PKV_NOALLOC_SCRATCH_BYTES in include/pkv.h


def paged_attn_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                              block_tables: torch.Tensor, context_lens: torch.Tensor,
                              q_lens: Optional[torch.Tensor], out: torch.Tensor, lse: Optional[torch.Tensor],
                              num_heads: int, num_kv_heads: int, head_dim: int, block_size: int, scale: float,
                              max_context_len: int, max_q_len: int = 1, partition_size: int = 0,
                              path: int = PATH_AUTO, stream=None, depth: int = 0, schedule: int = 0,
                              wgs_per_cu: int = 0, k_scale: float = 0.0, v_scale: float = 0.0) -> None:
    """paged_attn_decode for callers that cannot allocate (pkv_paged_attn_decode_noalloc): the library's
    static per-GPU scratch (NOALLOC_SCRATCH_BYTES) replaces the workspace, and nothing is allocated here
    or in the library.  The same bits as paged_attn_decode with a workspace of that size (fewer piece
    slots when the full plan needs more).  Calls that overlap on one GPU share that scratch and race."""
    lib = load()
    total_q, S, NB, code = _check_decode_args(q, k_cache, v_cache, block_tables, context_lens, q_lens, out, lse,
                                              num_heads, num_kv_heads, head_dim, block_size)
    o = _opts(partition_size, path, None, depth, schedule, wgs_per_cu, k_scale, v_scale)
    rc = lib.pkv_paged_attn_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                           _ptr(context_lens), _ptr(q_lens), _ptr(out), _ptr(lse),
                                           S, block_tables.shape[1], total_q, max_q_len, max_context_len, NB,
                                           num_heads, num_kv_heads, head_dim, block_size, float(scale), code,
                                           ctypes.byref(o), _stream(stream))
    _check(rc, "pkv_paged_attn_decode_noalloc")


def paged_attn_decode_shared_prefix(q, k_cache, v_cache, block_tables, context_lens, q_lens, out, lse,
                                    num_heads, num_kv_heads, head_dim, block_size, scale, max_context_len,
                                    group_starts, prefix_lens, prefix_blocks, max_group_size, max_prefix_len,
                                    max_q_len: int = 1, partition_size: int = 0, workspace=None, events=None,
                                    stream=None, depth: int = 0, schedule: int = 0, wgs_per_cu: int = 0,
                                    k_scale: float = 0.0, v_scale: float = 0.0, mode: int = PREFIX_AUTO) -> None:
    """Decode attention reading each group's shared prefix once (include/pkv_prefix.h).

    group_starts int32 [G+1], prefix_lens int32 [G] and prefix_blocks int32 [G, max_prefix_len / 16]
    on the GPU describe the groups; max_group_size / max_prefix_len are host-known bounds.  Other
    arguments as paged_attn_decode (bf16 q/out over bf16 or E4M3 pools)."""
    lib = load()
    total_q, S, NB, code = _check_decode_args(q, k_cache, v_cache, block_tables, context_lens, q_lens, out, lse,
                                              num_heads, num_kv_heads, head_dim, block_size)
    G = 0 if group_starts is None else group_starts.numel() - 1
    if G > 0:
        for t in (group_starts, prefix_lens, prefix_blocks):
            _need(t.dtype == torch.int32 and t.is_contiguous(), "group arrays: int32, contiguous")
        _on_gpu_like(q, "group arrays", group_starts, prefix_lens, prefix_blocks)
        _need(prefix_lens.numel() == G and tuple(prefix_blocks.shape) == (G, max_prefix_len // block_size),
              "prefix_lens [G], prefix_blocks [G, max_prefix_len / 16]")
    o = _opts(partition_size, PATH_AUTO, events, depth, schedule, wgs_per_cu, k_scale, v_scale)
    o.shared_prefix_mode = mode
    need = int(lib.pkv_decode_shared_prefix_workspace_bytes(S, total_q, max_q_len, max_context_len, num_heads,
                                                             num_kv_heads, head_dim, code, max(G, 0),
                                                             max_group_size, max_prefix_len, ctypes.byref(o)))
    if workspace is None:
        workspace = _workspace_for(need, q.device, stream)
    ws_bytes = _check_workspace(workspace, q)
    rc = lib.pkv_paged_attn_decode_shared_prefix(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens), _ptr(q_lens), _ptr(out),
        _ptr(lse), S, block_tables.shape[1], total_q, max_q_len, max_context_len, NB, num_heads, num_kv_heads,
        head_dim, block_size, float(scale), code, _ptr(group_starts if G > 0 else None),
        _ptr(prefix_lens if G > 0 else None), _ptr(prefix_blocks if G > 0 else None), max(G, 0), max_group_size,
        max_prefix_len, ctypes.byref(o), _ptr(workspace), ws_bytes, _stream(stream))
    _check(rc, "pkv_paged_attn_decode_shared_prefix")


def paged_attn_prefill(q, k_cache, v_cache, block_tables, context_lens, q_lens, out, lse, num_heads,
                       num_kv_heads, head_dim, block_size, scale, max_context_len, max_q_len, stream=None,
                       k_scale: float = 0.0, v_scale: float = 0.0) -> None:
    """Prefill / chunked-prefill attention through the C ABI (include/pkv_prefill.h): bf16 q/out
    [total_q, H, D] over bf16 pools or uint8 E4M3 pools (with their scales); the new tokens' K/V
    already written to the cache."""
    lib = load()
    total_q, S, NB, code = _check_decode_args(q, k_cache, v_cache, block_tables, context_lens, q_lens, out, lse,
                                              num_heads, num_kv_heads, head_dim, block_size)
    o = _opts(0, PATH_AUTO, None, k_scale=k_scale, v_scale=v_scale)
    rc = lib.pkv_paged_attn_prefill(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
                                    _ptr(q_lens), _ptr(out), _ptr(lse), S, block_tables.shape[1], total_q, max_q_len,
                                    max_context_len, NB, num_heads, num_kv_heads, head_dim, block_size,
                                    float(scale), code, ctypes.byref(o), _stream(stream))
    _check(rc, "pkv_paged_attn_prefill")


# pkv_check_reason (include/pkv_check.h)
CHECK_REASONS = {0: "ok", 1: "q_len", 2: "q_over_context", 3: "context_len", 4: "context_table", 5: "block_id",
                 6: "q_total"}
CHECK_REPORT_INTS = 8


def check_decode_inputs(block_tables: torch.Tensor, context_lens: torch.Tensor, q_lens: Optional[torch.Tensor],
                        num_blocks: int, total_q: int, max_q_len: int, max_context_len: int, block_size: int = 16,
                        stream=None) -> dict:
    """Check a decode batch's device-side preconditions on the GPU (pkv_check_decode_inputs) and return
    the report: violations, the first bad sequence (-1: none), its reason (a CHECK_REASONS name) and
    offending value, and the q_lens sum.  Synchronizes `stream` to read the report: a debugging aid,
    not a step of the decode."""
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and block_tables.is_contiguous()
          and block_tables.shape[1] >= 1, "block_tables: int32 [S, max_blocks >= 1], contiguous")
    S = block_tables.shape[0]
    _need(context_lens.dtype == torch.int32 and context_lens.numel() == S and context_lens.is_contiguous(),
          "context_lens: int32 [S]")
    if q_lens is not None:
        _need(q_lens.dtype == torch.int32 and q_lens.numel() == S and q_lens.is_contiguous(), "q_lens: int32 [S]")
    _on_gpu_like(block_tables, "check arguments", context_lens, q_lens)
    with torch.cuda.device(block_tables.device):
        s = torch.cuda.current_stream() if stream is None else stream
        with torch.cuda.stream(s):
            report = torch.empty(CHECK_REPORT_INTS, dtype=torch.int32, device=block_tables.device)
        _check(load().pkv_check_decode_inputs(_ptr(block_tables), _ptr(context_lens), _ptr(q_lens), S,
                                              int(block_tables.shape[1]), int(total_q), int(max_q_len),
                                              int(max_context_len), int(num_blocks), int(block_size), _ptr(report),
                                              ctypes.c_void_p(s.cuda_stream)), "pkv_check_decode_inputs")
        s.synchronize()
    r = report.cpu().tolist()
    return {"violations": r[0], "first_seq": r[1], "reason": CHECK_REASONS.get(r[2], r[2]), "value": r[3],
            "q_sum": r[4]}


def shared_prefix_workspace_bytes(num_seqs, total_q, max_q_len, max_context_len, num_heads, num_kv_heads,
                                  head_dim, dtype_code, num_groups, max_group_size, max_prefix_len,
                                  partition_size=0, depth=0, schedule=0, wgs_per_cu=0) -> int:
    o = DecodeOptions(partition_size, PATH_AUTO, depth, schedule, None, None, wgs_per_cu)
    return int(load().pkv_decode_shared_prefix_workspace_bytes(num_seqs, total_q, max_q_len, max_context_len,
                                                               num_heads, num_kv_heads, head_dim, dtype_code,
                                                               num_groups, max_group_size, max_prefix_len,
                                                               ctypes.byref(o)))


class DecodeStep:
    """One decode step bound once: the optional append of the new tokens' K/V (through slot_mapping
    with pkv_kv_cache_write, or, given new_k / new_v without slot_mapping, in the decode call itself
    with pkv_paged_attn_decode_append), then paged decode attention, with the same checks as
    kv_cache_write / paged_attn_decode done at construction.  A call only enqueues the two C calls on the current stream, so a serving loop
    pays little host time per step and the step can be captured in a HIP graph.  A call may swap in
    other cache tensors of the same shape, dtype and device (not checked again)."""

    def __init__(self, q, k_cache, v_cache, block_tables, context_lens, q_lens, out, lse, num_heads,
                 num_kv_heads, head_dim, block_size, scale, max_context_len, max_q_len=1,
                 partition_size=0, path=PATH_AUTO, depth=0, schedule=0, workspace=None,
                 new_k=None, new_v=None, slot_mapping=None, wgs_per_cu=0, k_scale=0.0, v_scale=0.0):
        lib = load()
        self._lib = lib
        # the full checks of the one-shot calls, once
        total_q, S, NB, code = _check_decode_args(q, k_cache, v_cache, block_tables, context_lens, q_lens, out,
                                                  lse, num_heads, num_kv_heads, head_dim, block_size)
        self._opts = DecodeOptions(partition_size, path, depth, schedule, None, None, wgs_per_cu, k_scale, v_scale)
        self._opts_ev = DecodeOptions(partition_size, path, depth, schedule, None, None, wgs_per_cu, k_scale,
                                      v_scale)
        need = int(lib.pkv_decode_workspace_bytes(S, total_q, max_q_len, max_context_len, num_heads,
                                                  num_kv_heads, head_dim, code, ctypes.byref(self._opts)))
        if workspace is None and need > 0:
            workspace = new_workspace(need, q.device)
        ws_bytes = _check_workspace(workspace, q)
        _need(ws_bytes >= need, "workspace too small")
        self._keep = (q, k_cache, v_cache, block_tables, context_lens, q_lens, out, lse, workspace,
                      new_k, new_v, slot_mapping)
        self._head = (_ptr(q),)
        self._mid = (_ptr(block_tables), _ptr(context_lens), _ptr(q_lens), _ptr(out), _ptr(lse),
                     S, block_tables.shape[1], total_q, max_q_len, max_context_len, NB,
                     num_heads, num_kv_heads, head_dim, block_size, float(scale), code)
        self._tail = (_ptr(workspace), ws_bytes)
        self._write = None
        self._fused = None
        if new_k is not None and slot_mapping is None:
            _need(new_v is not None and new_k.shape == new_v.shape
                  and tuple(new_k.shape) == (total_q, num_kv_heads, head_dim),
                  "new_k / new_v must be [total_q, KVH, D] for the fused append")
            for t in (new_k, new_v):
                _need(t.dtype == q.dtype and t.is_contiguous(), "new_k / new_v: q's dtype, contiguous")
            _on_gpu_like(q, "new_k / new_v", new_k, new_v)
            self._fused = (_ptr(new_k), _ptr(new_v))
        if slot_mapping is not None:
            T = new_k.shape[0]
            _need(new_k.dim() == 3 and new_k.shape == new_v.shape and tuple(new_k.shape[1:]) == (num_kv_heads, head_dim),
                  "new_k / new_v must be [T, KVH, D]")
            _need(slot_mapping.dtype == torch.int64 and slot_mapping.numel() == T and slot_mapping.is_contiguous(),
                  "slot_mapping: int64 [T], contiguous")
            for t in (new_k, new_v):
                _need(t.dtype == q.dtype and t.is_contiguous(), "new_k / new_v: q's dtype, contiguous")
            _on_gpu_like(q, "appended rows", new_k, new_v, slot_mapping)
            if code == PKV_BF16_FP8KV:
                _need(k_scale > 0 and v_scale > 0, "E4M3 pools need k_scale / v_scale > 0 for the write")
                self._write = ((_ptr(new_k), _ptr(new_v), _ptr(slot_mapping)),
                               (T, NB, num_kv_heads, head_dim, block_size, float(k_scale), float(v_scale)))
            else:
                self._write = ((_ptr(new_k), _ptr(new_v), _ptr(slot_mapping)),
                               (T, NB, num_kv_heads, head_dim, block_size, code))
            self._write_fp8 = code == PKV_BF16_FP8KV
        self._kc, self._vc = _ptr(k_cache), _ptr(v_cache)

    def __call__(self, k_cache=None, v_cache=None, events=None, stream=None):
        kc = self._kc if k_cache is None else ctypes.c_void_p(k_cache.data_ptr())
        vc = self._vc if v_cache is None else ctypes.c_void_p(v_cache.data_ptr())
        st = _stream(stream)
        lib = self._lib
        if self._write is not None:
            ptrs, sizes = self._write
            if self._write_fp8:
                rc = lib.pkv_kv_cache_write_fp8(*ptrs, kc, vc, *sizes, st)
            else:
                rc = lib.pkv_kv_cache_write(*ptrs, kc, vc, *sizes, st)
            if rc != 0:
                _check(rc, "pkv_kv_cache_write")
        o = self._opts
        if events is not None:
            # torch.cuda.Event objects, or raw hipEvent_t handles
            o = self._opts_ev
            o.event_main_begin = getattr(events[0], "cuda_event", events[0])
            o.event_main_end = getattr(events[1], "cuda_event", events[1])
        if self._fused is not None:
            rc = lib.pkv_paged_attn_decode_append(*self._head, *self._fused, kc, vc, *self._mid, ctypes.byref(o),
                                                  *self._tail, st)
            if rc != 0:
                _check(rc, "pkv_paged_attn_decode_append")
            return
        rc = lib.pkv_paged_attn_decode(*self._head, kc, vc, *self._mid, ctypes.byref(o), *self._tail, st)
        if rc != 0:
            _check(rc, "pkv_paged_attn_decode")
