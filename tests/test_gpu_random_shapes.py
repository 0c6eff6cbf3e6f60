"""GPU parity on seeded random batch shapes: decode, prefill, the decode step with its append, and the
read-once shared-prefix decode.

Decode: head dims, GQA groups, batch sizes, length mixes (short,
long, page-boundary, one long among short), uniform and ragged new tokens, bf16 and E4M3 pools, each
through a kernel family and schedule drawn at random (balanced persistent split with piece slots,
persistent with fixed partitions, and for bf16 pools the grid schedule and the VALU path), compared
with the oracle on every row.  Prefill: whole prompts and chunks over cached contexts, uniform and
ragged, bf16 and E4M3 pools, over poisoned pools.  The shapes are drawn, not chosen: they reach
combinations the targeted tests do not list."""
import numpy as np
import pytest

from paged_kv_cache_199_amd import _lib
from paged_kv_cache_199_amd import workloads as W
from tests.gpu_helpers import BF16_TOL, LSE_TOL, compare, oracle_full, run_library

pytestmark = pytest.mark.gpu
DEV = "cuda"
B = 16


def _say(*a):
    print(*a, flush=True)


def draw(seed):
    rng = np.random.default_rng(5000 + seed)
    D = int(rng.choice([64, 128]))
    KVH = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8]))
    S = int(rng.choice([1, 3, 8, 17, 40, 100]))
    mix = rng.choice(["short", "long", "edges", "one_long", "wide"])
    if mix == "short":
        ctx = rng.integers(1, 200, S)
    elif mix == "long":
        ctx = rng.integers(1000, 4000 if S <= 17 else 1500, S)
    elif mix == "edges":
        ctx = rng.choice([1, 15, 16, 17, 31, 32, 33, 255, 256, 257, 1023, 1024, 1025], S)
    elif mix == "one_long":
        ctx = rng.integers(8, 120, S)
        ctx[rng.integers(0, S)] = 6000 if S <= 17 else 3000
    else:
        ctx = rng.integers(1, 2500 if S <= 40 else 800, S)
    f8 = bool(rng.random() < 0.3)
    qmax = int(rng.choice([1, 1, 2, 5]))
    ragged = bool(rng.random() < 0.5) and qmax > 1
    ql = np.minimum(rng.integers(1, qmax + 1, S) if ragged else np.full(S, qmax), ctx)
    if not ragged and (ql != qmax).any():       # uniform new tokens need every context to hold them
        ctx = np.maximum(ctx, qmax)
        ql = np.full(S, qmax)
    variant = rng.choice(["persist", "persist", "persist_parts", "grid", "valu"])
    if f8 and variant in ("valu", "grid"):       # E4M3 pools decode with the persistent schedule only
        variant = "persist"
    depth = int(rng.choice([2, 3, 4]))
    return dict(D=D, KVH=KVH, H=KVH * G, ctx=ctx.astype(int).tolist(), ql=ql.astype(int).tolist(), f8=f8,
                variant=str(variant), depth=depth, mix=str(mix))


VARIANTS = {
    "persist": lambda d: dict(path=_lib.PATH_MFMA, schedule=_lib.SCHEDULE_PERSISTENT, depth=d, partition_size=0),
    "persist_parts": lambda d: dict(path=_lib.PATH_MFMA, schedule=_lib.SCHEDULE_PERSISTENT, depth=d,
                                    partition_size=256),
    "grid": lambda d: dict(path=_lib.PATH_MFMA, schedule=_lib.SCHEDULE_GRID, depth=d, partition_size=0),
    "valu": lambda d: dict(path=_lib.PATH_VALU, schedule=_lib.SCHEDULE_AUTO, depth=0, partition_size=0),
}


@pytest.mark.parametrize("seed", range(48))
def test_random_shape(gpu_lib, seed):
    c = draw(seed)
    spec = W.custom(f"rand{seed}", c["ctx"], q_len=c["ql"], num_heads=c["H"], num_kv_heads=c["KVH"],
                    head_dim=c["D"], seed=100 + seed, kv_fp8=c["f8"])
    w = W.build(spec, DEV)
    kw = VARIANTS[c["variant"]](c["depth"])
    _say(f"[case] seed {seed}: S={w.num_seqs} H={c['H']} KVH={c['KVH']} D={c['D']} mix={c['mix']} "
         f"q<={w.max_q_len} {'ragged' if not w.uniform_q else 'uniform'} {'E4M3' if c['f8'] else 'bf16'} "
         f"{c['variant']} {kw}")
    out, lse = run_library(w, DEV, **kw)
    d_out, d_lse = compare(w, out, lse, *oracle_full(w))
    _say(f"   max|d out| = {d_out:.3e}   max|d lse| = {d_lse:.3e}")
    assert np.isfinite(d_out) and d_out <= BF16_TOL
    assert np.isfinite(d_lse) and d_lse <= LSE_TOL


def draw_prefill(seed):
    rng = np.random.default_rng(7000 + seed)
    D = int(rng.choice([64, 128]))
    KVH = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8]))
    S = int(rng.choice([1, 2, 5, 9]))
    prompt = bool(rng.random() < 0.4)
    uniform = bool(rng.random() < 0.3)
    if prompt:
        q = np.full(S, int(rng.integers(1, 700))) if uniform else rng.integers(1, 700, S)
        ctx = q.copy()
    else:
        q = np.full(S, int(rng.integers(1, 600))) if uniform else rng.integers(1, 600, S)
        ctx = q + rng.integers(0, 3000, S)
    # keep the oracle's work (new tokens x context x heads) to a few seconds
    while int((q * ctx).sum()) * KVH * G > 4e7 and S > 1:
        S -= 1
        q, ctx = q[:S], ctx[:S]
    while int((q * ctx).sum()) * KVH * G > 4e7:
        q = np.maximum(q // 2, 1)
        ctx = np.maximum(ctx // 2, q)
    return dict(D=D, KVH=KVH, H=KVH * G, ctx=ctx.astype(int).tolist(), ql=q.astype(int).tolist(),
                f8=bool(rng.random() < 0.3), prompt=prompt, uniform=uniform)


@pytest.mark.parametrize("seed", range(24))
def test_random_prefill_shape(gpu_lib, seed):
    """Prefill and chunked prefill on seeded random shapes over poisoned pools (every slot no sequence
    may read holds NaN), bf16 and E4M3."""
    import torch

    from tests.gpu_helpers import nan_empty, nan_like

    c = draw_prefill(seed)
    spec = W.custom(f"rand_prefill{seed}", c["ctx"], q_len=c["ql"], num_heads=c["H"], num_kv_heads=c["KVH"],
                    head_dim=c["D"], seed=300 + seed, kv_fp8=c["f8"])
    w = W.build(spec, DEV, poison=True)
    _say(f"[case] prefill seed {seed}: S={w.num_seqs} H={c['H']} KVH={c['KVH']} D={c['D']} "
         f"{'prompt' if c['prompt'] else 'chunk'} q<={w.max_q_len} ctx<={w.max_context_len} "
         f"{'uniform' if w.uniform_q else 'ragged'} {'E4M3' if c['f8'] else 'bf16'}")
    meta = w.device_meta(DEV)
    out = nan_like(w.q)
    lse = nan_empty((w.total_q, w.spec.num_heads), DEV)
    scales = dict(k_scale=w.spec.k_scale, v_scale=w.spec.v_scale) if w.kv_fp8 else {}
    _lib.paged_attn_prefill(w.q, w.k_cache, w.v_cache, meta["block_tables"], meta["context_lens"],
                            None if w.uniform_q else meta["q_lens"], out, lse, w.spec.num_heads,
                            w.spec.num_kv_heads, w.spec.head_dim, 16, w.scale, w.max_context_len, w.max_q_len,
                            **scales)
    torch.cuda.synchronize()
    d_out, d_lse = compare(w, out, lse, *oracle_full(w))
    _say(f"   max|d out| = {d_out:.3e}   max|d lse| = {d_lse:.3e}")
    assert np.isfinite(d_out) and d_out <= BF16_TOL
    assert np.isfinite(d_lse) and d_lse <= LSE_TOL


@pytest.mark.parametrize("seed", range(16))
def test_random_append_shape(gpu_lib, seed):
    """The decode step with its append on seeded random bf16 shapes (1..9 new tokens, so also past the
    fused limit of 8), through a drawn schedule: caches equal the oracle's scatter bit for bit, outputs
    match the oracle, and the one call equals write-then-decode bit for bit."""
    from tests.test_gpu_append import _check as check_append

    rng = np.random.default_rng(9000 + seed)
    S = int(rng.choice([1, 4, 13, 32]))
    KVH = int(rng.choice([1, 2, 8]))
    G = int(rng.choice([1, 4, 8]))
    D = int(rng.choice([64, 128]))
    q = int(rng.choice([1, 2, 5, 9]))
    ragged = bool(rng.random() < 0.5) and q > 1
    ctx = rng.integers(q, 1500, S)
    ql = rng.integers(1, q + 1, S) if ragged else np.full(S, q)
    spec = W.custom(f"rand_append{seed}", ctx.astype(int).tolist(), q_len=ql.astype(int).tolist(),
                    num_heads=KVH * G, num_kv_heads=KVH, head_dim=D, seed=500 + seed)
    variant = [dict(path=_lib.PATH_MFMA, schedule=_lib.SCHEDULE_PERSISTENT, depth=int(rng.choice([2, 3, 4]))),
               dict(path=_lib.PATH_MFMA, schedule=_lib.SCHEDULE_PERSISTENT, partition_size=128),
               dict(path=_lib.PATH_MFMA, schedule=_lib.SCHEDULE_GRID),
               dict(path=_lib.PATH_VALU)][int(rng.integers(0, 4))]
    _say(f"[case] append seed {seed}: S={S} H={KVH * G} KVH={KVH} D={D} q<={q} "
         f"{'ragged' if ragged else 'uniform'} {variant}")
    check_append(W.build(spec, DEV), [variant])


@pytest.mark.parametrize("seed", range(16))
def test_random_read_once_shape(gpu_lib, seed):
    """Read-once shared-prefix decode on seeded random batches: one to four groups of consecutive
    sequences sharing drawn prefixes (members shorter than the prefix share what they have), ungrouped
    sequences before and after them, uniform or ragged new tokens, bf16 or E4M3 pools, forced
    read-once; against the oracle and the plain decode."""
    from tests.test_gpu_prefix import _check as check_prefix

    rng = np.random.default_rng(11000 + seed)
    S = int(rng.choice([3, 8, 20, 48]))
    KVH = int(rng.choice([1, 2, 8]))
    G = int(rng.choice([1, 4, 8]))
    D = int(rng.choice([64, 128]))
    f8 = bool(rng.random() < 0.3)
    q = int(rng.choice([1, 1, 3]))
    ragged = bool(rng.random() < 0.5) and q > 1
    ctx = rng.integers(q, 2500, S)
    ql = rng.integers(1, q + 1, S) if ragged else np.full(S, q)
    spec = W.custom(f"rand_prefix{seed}", ctx.astype(int).tolist(), q_len=ql.astype(int).tolist(),
                    num_heads=KVH * G, num_kv_heads=KVH, head_dim=D, seed=700 + seed, kv_fp8=f8)
    w = W.build(spec, DEV)
    # groups are consecutive runs of sequences; the ones before the first and after the last share nothing
    lo = int(rng.integers(0, S // 3 + 1))
    hi = int(rng.integers(max(lo + 1, 2 * S // 3), S + 1))
    n = min(hi - lo, int(rng.integers(1, 5)))
    edges = [lo] + np.sort(rng.choice(np.arange(lo + 1, hi), size=n - 1, replace=False)).tolist() + [hi]
    groups = [(a, b, 16 * int(rng.integers(1, 80))) for a, b in zip(edges[:-1], edges[1:])]
    _say(f"[case] read-once seed {seed}: S={S} H={KVH * G} KVH={KVH} D={D} q<={q} "
         f"{'ragged' if ragged else 'uniform'} {'E4M3' if f8 else 'bf16'} groups {groups}")
    check_prefix(w, W.share_prefixes(w, groups), f"read-once seed {seed}")
