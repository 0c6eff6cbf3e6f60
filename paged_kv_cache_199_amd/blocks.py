"""ctypes binding of the block manager in include/pkv_blocks.h: a block pool, sequences and a radix
prefix index (host-side, in libpkv.so), and the GPU block copy that carries out copy-on-write.

Argument marshalling only: the bookkeeping runs in the library's C++ code, the copies in its HIP
kernel.  The objects are not thread-safe (one scheduler thread owns them).
"""
from __future__ import annotations

import ctypes
from typing import List, Optional, Sequence as Seq, Tuple

import numpy as np
import torch

from ._lib import BLOCK_SIZE, _check, _need, _on_gpu_like, _ptr, _stream, load

ERR_WORKSPACE = -4   # pkv_status: the pool has too few free blocks


def _np_ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _ints(tokens, dtype) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(tokens, dtype=dtype).reshape(-1))


class OutOfBlocks(RuntimeError):
    """The pool cannot supply the blocks a call needs; nothing was changed."""


class BlockPool:
    """num_blocks reference-counted KV blocks of BLOCK_SIZE tokens; ids in [0, num_blocks)."""

    def __init__(self, num_blocks: int):
        self._lib = load()
        self.num_blocks = int(num_blocks)
        self.handle = self._lib.pkv_block_pool_create(self.num_blocks)
        _need(bool(self.handle), "num_blocks >= 0")
        self._owned: List[object] = []   # sequences and indexes that must go before the pool

    def free_count(self) -> int:
        return int(self._lib.pkv_block_pool_free_count(self.handle))

    def refcount(self, block: int) -> int:
        r = int(self._lib.pkv_block_refcount(self.handle, int(block)))
        _check(min(r, 0), "pkv_block_refcount")
        return r

    def close(self) -> None:
        for o in self._owned:
            o.close()
        self._owned.clear()
        if self.handle:
            self._lib.pkv_block_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Sequence:
    """One request's block table; append() hands out the slots of its new tokens."""

    def __init__(self, pool: BlockPool, handle=None):
        self._lib, self.pool = pool._lib, pool
        self.handle = handle if handle is not None else self._lib.pkv_seq_create(pool.handle)
        _need(bool(self.handle), "a live pool")
        pool._owned.append(self)

    def __len__(self) -> int:
        return int(self._lib.pkv_seq_length(self.handle))

    @property
    def num_blocks(self) -> int:
        return int(self._lib.pkv_seq_num_blocks(self.handle))

    def block_table(self) -> np.ndarray:
        row = np.zeros(max(self.num_blocks, 1), dtype=np.int32)
        n = int(self._lib.pkv_seq_block_table(self.handle, _np_ptr(row), row.size))
        _check(min(n, 0), "pkv_seq_block_table")
        return row[:n]

    def append(self, n_tokens: int) -> Tuple[np.ndarray, List[Tuple[int, int]]]:
        """(slots int64 [n_tokens], [(copy_src, copy_dst)]): copy each pair's block before writing."""
        slots = np.zeros(max(int(n_tokens), 1), dtype=np.int64)
        src = np.zeros(1, dtype=np.int32)
        dst = np.zeros(1, dtype=np.int32)
        nc = ctypes.c_int32(0)
        r = int(self._lib.pkv_seq_append(self.handle, int(n_tokens), _np_ptr(slots), _np_ptr(src), _np_ptr(dst),
                                         ctypes.byref(nc)))
        if r == ERR_WORKSPACE:
            raise OutOfBlocks(f"pool has {self.pool.free_count()} free blocks")
        _check(min(r, 0), "pkv_seq_append")
        return slots[:int(n_tokens)], [(int(src[k]), int(dst[k])) for k in range(nc.value)]

    def fork(self) -> "Sequence":
        return Sequence(self.pool, self._lib.pkv_seq_fork(self.handle))

    def adopt_prefix(self, blocks: Seq[int]) -> None:
        b = _ints(blocks, np.int32)
        _check(min(int(self._lib.pkv_seq_adopt_prefix(self.handle, _np_ptr(b), b.size)), 0), "pkv_seq_adopt_prefix")

    def close(self) -> None:
        if self.handle:
            self._lib.pkv_seq_destroy(self.handle)
            self.handle = None


def append_step(seqs: Seq[Sequence], n_tokens) -> Tuple[np.ndarray, List[Tuple[int, int]]]:
    """One step's appends for distinct sequences in one call: (slot_mapping int64 [sum n_tokens],
    copy pairs), all-or-nothing (OutOfBlocks leaves every sequence unchanged)."""
    if not seqs:
        return np.zeros(0, dtype=np.int64), []
    lib = seqs[0]._lib
    handles = (ctypes.c_void_p * len(seqs))(*[s.handle for s in seqs])
    n = _ints(n_tokens, np.int32)
    if n.size == 1 and len(seqs) > 1:
        n = np.full(len(seqs), n[0], dtype=np.int32)
    _need(n.size == len(seqs), "one token count per sequence")
    slots = np.zeros(max(int(n.sum()), 1), dtype=np.int64)
    src = np.zeros(len(seqs), dtype=np.int32)
    dst = np.zeros(len(seqs), dtype=np.int32)
    nc = ctypes.c_int32(0)
    r = int(lib.pkv_seqs_append(handles, len(seqs), _np_ptr(n), _np_ptr(slots), _np_ptr(src), _np_ptr(dst),
                                ctypes.byref(nc)))
    if r == ERR_WORKSPACE:
        raise OutOfBlocks(f"pool has {seqs[0].pool.free_count()} free blocks")
    _check(min(r, 0), "pkv_seqs_append")
    return slots[:int(n.sum())], [(int(src[k]), int(dst[k])) for k in range(nc.value)]


class RadixIndex:
    """Token-id prefixes in whole blocks -> cached blocks (the index holds a reference to each)."""

    def __init__(self, pool: BlockPool):
        self._lib, self.pool = pool._lib, pool
        self.handle = self._lib.pkv_radix_create(pool.handle)
        _need(bool(self.handle), "a live pool")
        pool._owned.append(self)

    def match(self, tokens) -> np.ndarray:
        t = _ints(tokens, np.int32)
        out = np.zeros(max(t.size // BLOCK_SIZE, 1), dtype=np.int32)
        r = int(self._lib.pkv_radix_match(self.handle, _np_ptr(t), t.size, _np_ptr(out), t.size // BLOCK_SIZE))
        _check(min(r, 0), "pkv_radix_match")
        return out[:r]

    def insert(self, tokens, blocks) -> int:
        t = _ints(tokens, np.int32)
        b = _ints(blocks, np.int32)
        _need(b.size >= t.size // BLOCK_SIZE, "one block per whole block of tokens")
        r = int(self._lib.pkv_radix_insert(self.handle, _np_ptr(t), t.size, _np_ptr(b)))
        _check(min(r, 0), "pkv_radix_insert")
        return r

    def evict(self, n_blocks: int) -> int:
        r = int(self._lib.pkv_radix_evict(self.handle, int(n_blocks)))
        _check(min(r, 0), "pkv_radix_evict")
        return r

    def cached_blocks(self) -> int:
        return int(self._lib.pkv_radix_cached_blocks(self.handle))

    def close(self) -> None:
        if self.handle:
            self._lib.pkv_radix_destroy(self.handle)
            self.handle = None


def copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, src: torch.Tensor, dst: torch.Tensor,
                stream=None) -> None:
    """Block dst[k] of both pools (pkv.h layout) becomes a copy of block src[k]; int32 ids on the GPU."""
    lib = load()
    _need(src.dtype == torch.int32 and dst.dtype == torch.int32 and src.numel() == dst.numel(),
          "src and dst: int32 [n]")
    _need(k_cache.dim() == 4 and k_cache.shape[2] == BLOCK_SIZE and v_cache.shape == (
        k_cache.shape[0], k_cache.shape[1], k_cache.shape[3], BLOCK_SIZE) and v_cache.dtype == k_cache.dtype,
        "k_cache [NB, KVH, 16, D], v_cache [NB, KVH, D, 16], one dtype")
    for t in (k_cache, v_cache, src, dst):
        _need(t.is_contiguous(), "contiguous")
    _on_gpu_like(k_cache, "copy_blocks", v_cache, src, dst)
    NB, KVH, _, D = k_cache.shape
    rc = lib.pkv_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(src), _ptr(dst), src.numel(), NB, KVH, D,
                             k_cache.element_size(), _stream(stream))
    _check(rc, "pkv_copy_blocks")
