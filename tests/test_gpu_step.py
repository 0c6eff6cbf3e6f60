"""The bind-once decode step (append + attention) eagerly and replayed from a captured HIP graph.

Eager: the bound step equals the one-shot calls bit for bit, and matches the oracle.  Graph: the
step's kernels are captured once and replayed several times, with eager work of the program and
synchronizations between the replays; every replay must reproduce the eager result bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle import paged_attention as O
from paged_kv_cache_199_amd import _lib
from paged_kv_cache_199_amd import workloads as W
from tests.gpu_helpers import (BF16_TOL, LSE_TOL, compare, host_bits, nan_empty, nan_like, oracle_full)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _step_for(w, out, lse, **kw):
    meta = w.device_meta(DEV)
    return _lib.DecodeStep(w.q, w.k_cache, w.v_cache, meta["block_tables"], meta["context_lens"],
                           None if w.uniform_q else meta["q_lens"], out, lse, w.spec.num_heads,
                           w.spec.num_kv_heads, w.spec.head_dim, w.spec.block_size, w.scale, w.max_context_len,
                           max_q_len=w.max_q_len, new_k=w.new_k, new_v=w.new_v,
                           slot_mapping=meta["slot_mapping"] if w.slot_mapping is not None else None, **kw)


def _small_append_workload():
    spec = W.custom("step_small", [300, 17, 1025, 64, 2000, 5], num_heads=16, num_kv_heads=4, head_dim=128,
                    write_new_token=True)
    return W.build(spec, DEV)


def test_bound_step_matches_one_shot_calls_and_oracle(gpu_lib):
    w = _small_append_workload()
    kc0, vc0 = host_bits(w.k_cache), host_bits(w.v_cache)
    out = nan_like(w.q)
    lse = nan_empty((w.total_q, w.spec.num_heads), DEV)
    _step_for(w, out, lse)()
    torch.cuda.synchronize()
    # the append is in the cache, bit for bit
    want_k, want_v = O.kv_cache_write(kc0, vc0, host_bits(w.new_k), host_bits(w.new_v), w.slot_mapping)
    assert np.array_equal(host_bits(w.k_cache), want_k) and np.array_equal(host_bits(w.v_cache), want_v)
    ref_out, ref_lse, ref_vabs = oracle_full(w)
    d_out, d_lse = compare(w, out, lse, ref_out, ref_lse, ref_vabs)
    print(f"[case] bound step: max|d out| {d_out:.3e} max|d lse| {d_lse:.3e}", flush=True)
    assert d_out <= BF16_TOL and d_lse <= LSE_TOL
    # the one-shot entry point on the same (already appended) cache gives the same bits
    meta = w.device_meta(DEV)
    out2 = nan_like(out)
    lse2 = nan_like(lse)
    _lib.paged_attn_decode(w.q, w.k_cache, w.v_cache, meta["block_tables"], meta["context_lens"], None, out2,
                           lse2, w.spec.num_heads, w.spec.num_kv_heads, w.spec.head_dim, 16, w.scale,
                           w.max_context_len, max_q_len=w.max_q_len)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(out2)) and torch.equal(lse, lse2)


@pytest.mark.parametrize("schedule", [_lib.SCHEDULE_PERSISTENT, _lib.SCHEDULE_GRID])
def test_graph_replays_match_eager(gpu_lib, schedule):
    w = _small_append_workload()
    out = nan_like(w.q)
    lse = nan_empty((w.total_q, w.spec.num_heads), DEV)
    step = _step_for(w, out, lse, schedule=schedule)
    step()
    torch.cuda.synchronize()
    want_out, want_lse = out.clone(), lse.clone()
    want_k, want_v = w.k_cache.clone(), w.v_cache.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    other = W.build(W.custom("step_other", [100, 900], num_heads=8, num_kv_heads=2, head_dim=128), DEV)
    for rep in range(4):
        out.fill_(0)
        lse.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        print(f"[case] graph replay {rep} schedule={schedule}", flush=True)
        assert torch.equal(_bits(out), _bits(want_out)) and torch.equal(lse, want_lse)
        assert torch.equal(_bits(w.k_cache), _bits(want_k)) and torch.equal(_bits(w.v_cache), _bits(want_v))
        # eager work of the program between replays
        o2 = nan_like(other.q)
        m2 = other.device_meta(DEV)
        _lib.paged_attn_decode(other.q, other.k_cache, other.v_cache, m2["block_tables"], m2["context_lens"],
                               None, o2, None, 8, 2, 128, 16, other.scale, other.max_context_len)
        torch.cuda.synchronize()
