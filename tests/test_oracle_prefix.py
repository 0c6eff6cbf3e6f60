"""Pins for the oracle's read-once shared-prefix decode (CPU only).

oracle.paged_attention.shared_prefix_attention splits every sequence's keys into the group's shared
blocks and its own remainder and merges the two softmaxes by log-sum-exp.  It is pinned to
torch's scaled_dot_product_attention on the unpaged, per-sequence K/V (built first, then laid into a
pool where group members share physical blocks), and planted slips in its splitting must fail that pin.
"""
import numpy as np
import pytest
import torch

from oracle import paged_attention as O


def _grouped_case(rng, ctx, q_lens, groups, H, KVH, D, B=16):
    """Logical K/V per sequence where the members of each group (first, end, prefix tokens) agree on
    their first min(prefix, ctx) rows, laid into a pool: the group's prefix rows in shared blocks,
    everything else in private blocks (random placement)."""
    S = len(ctx)
    Ks = [rng.standard_normal((KVH, n, D)) for n in ctx]
    Vs = [rng.standard_normal((KVH, n, D)) for n in ctx]
    group_of = {}
    for g, (first, end, pre) in enumerate(groups):
        P = rng.standard_normal((2, KVH, pre, D))
        for s in range(first, end):
            k = min(pre, ctx[s])
            Ks[s][:, :k] = P[0, :, :k]
            Vs[s][:, :k] = P[1, :, :k]
            group_of[s] = g
    nblk = [-(-n // B) for n in ctx]
    pool = sum(nblk) + sum(g[2] // B for g in groups) + 3
    perm = rng.permutation(pool)
    kc = np.full((pool, KVH, B, D), np.nan)
    vc = np.full((pool, KVH, D, B), np.nan)
    cur = 0
    pre_ids = []
    for first, end, pre in groups:
        ids = perm[cur:cur + pre // B]
        cur += pre // B
        pre_ids.append(ids)
        donor = max(range(first, end), key=lambda s: ctx[s])
        for t in range(pre):
            kc[ids[t // B], :, t % B, :] = Ks[donor][:, t] if t < ctx[donor] else 0.0
            vc[ids[t // B], :, :, t % B] = Vs[donor][:, t] if t < ctx[donor] else 0.0
    table = np.full((S, max(nblk)), -1, np.int32)
    for s, n in enumerate(ctx):
        g = group_of.get(s)
        shared = min(nblk[s], groups[g][2] // B) if g is not None else 0
        if shared:
            table[s, :shared] = pre_ids[g][:shared]
        for j in range(shared, nblk[s]):
            table[s, j] = perm[cur]
            for t in range(j * B, min(n, (j + 1) * B)):
                kc[perm[cur], :, t % B, :] = Ks[s][:, t]
                vc[perm[cur], :, :, t % B] = Vs[s][:, t]
            cur += 1
    starts = [groups[0][0]] + [g[1] for g in groups]
    lens = [g[2] for g in groups]
    width = max(len(i) for i in pre_ids)
    blocks = np.zeros((len(groups), width), np.int32)
    for g, ids in enumerate(pre_ids):
        blocks[g, :len(ids)] = ids
    q = rng.standard_normal((int(sum(q_lens)), H, D))
    return q, kc, vc, table, np.asarray(ctx, np.int32), np.asarray(q_lens, np.int32), Ks, Vs, \
        np.asarray(starts, np.int32), np.asarray(lens, np.int32), blocks


def _sdpa(q, Ks, Vs, q_lens, H, KVH, scale):
    G = H // KVH
    outs, base = [], 0
    for K, V, qs in zip(Ks, Vs, q_lens):
        qs = int(qs)
        n = K.shape[1]
        Q = torch.from_numpy(q[base:base + qs]).permute(1, 0, 2)[None]
        Kt = torch.from_numpy(K).repeat_interleave(G, dim=0)[None]
        Vt = torch.from_numpy(V).repeat_interleave(G, dim=0)[None]
        mask = torch.arange(n)[None, :] <= (n - qs + torch.arange(qs)[:, None])
        o = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt, attn_mask=mask, scale=scale)
        outs.append(o[0].permute(1, 0, 2).numpy())
        base += qs
    return np.concatenate(outs)


CASES = [
    # ctx, q_lens, groups (first, end, prefix tokens), H, KVH, D
    ([40, 70, 20, 100], [1, 1, 1, 1], [(0, 4, 48)], 4, 2, 8),
    # short members (whole context inside the prefix), ragged q with new tokens right after the
    # prefix, a sequence outside every group, two groups
    ([33, 90, 12, 64, 50, 81, 200], [3, 2, 1, 5, 1, 4, 2], [(0, 3, 32), (3, 6, 48)], 8, 2, 16),
    # one member, prefix longer than every context, G = 1
    ([17, 150], [2, 1], [(0, 1, 64), (1, 2, 96)], 3, 3, 8),
]


def _run(fn, case, seed=5):
    ctx, ql, groups, H, KVH, D = case
    rng = np.random.default_rng(seed)
    q, kc, vc, table, cl, qlens, Ks, Vs, gs, pl, pb = _grouped_case(rng, ctx, ql, groups, H, KVH, D)
    out, lse = fn(q, kc, vc, table, cl, qlens, 0.4, KVH, gs, pl, pb)
    return out, lse, _sdpa(q, Ks, Vs, qlens, H, KVH, 0.4), (q, kc, vc, table, cl, qlens, KVH)


@pytest.mark.parametrize("case", CASES)
def test_read_once_equals_sdpa_on_unpaged_rows(case):
    out, lse, ref, full = _run(O.shared_prefix_attention, case)
    assert np.all(np.isfinite(out)) and np.max(np.abs(out - ref)) <= 1e-12
    # and the oracle's one-pass definition gives the same LSE
    q, kc, vc, table, cl, qlens, KVH = full
    out1, lse1 = O.paged_decode_attention(q, kc, vc, table, cl, qlens, 0.4, KVH, 16)
    assert np.max(np.abs(out1 - ref)) <= 1e-12 and np.max(np.abs(lse - lse1)) <= 1e-12


def test_shared_length_stops_before_the_new_tokens():
    assert O.shared_len(40, 1, 48) == 32       # 39 keys before the new token: two whole pages
    assert O.shared_len(49, 1, 48) == 48
    assert O.shared_len(49, 2, 48) == 32       # new tokens at 47 and 48
    assert O.shared_len(12, 1, 32) == 0        # no whole page before the new token
    assert O.shared_len(200, 2, 0) == 0


MUTATIONS = [
    ("prefix row sees one key too many", "last.append(P[s] - 1)", "last.append(P[s])"),
    ("suffix mask not shifted", "last = n - qs + np.arange(qs) - ps", "last = n - qs + np.arange(qs)"),
    ("new tokens counted as shared", "(int(context_len) - int(q_len)) // block_size", "int(context_len) // block_size"),
    ("suffix reads from the start", "attend(rows, K[ps:], V[ps:]", "attend(rows, K, V"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_slips_in_the_split_are_caught(name, old, new):
    src = open(O.__file__).read()
    assert old in src, f"mutation anchor for {name} missing"
    ns = {"__name__": "oracle_mutant"}
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), ns)
    caught = False
    for case in CASES:
        try:
            out, _, ref, _ = _run(ns["shared_prefix_attention"], case)
            caught |= not (np.all(np.isfinite(out)) and np.max(np.abs(out - ref)) <= 1e-12)
        except Exception:
            caught = True
    assert caught, f"planted slip '{name}' passed the pin"
