"""Pins that tie the CPU oracle to something other than itself (CPU only).

Each test names the property it pins.  Together they are chosen so that a plausible slip in the oracle
(a wrong GQA head map, an off-by-one causal offset, a transposed V block, a dropped scale, a log base
mix-up, a wrong block-table index) fails at least one of them; test_planted_mistakes_are_caught
checks exactly that by planting such slips in a copy of the oracle.
"""
import json
import math
import os
import re
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import paged_attention as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------------------------
# tiny-input construction (test-local; contiguous K/V first, then scattered into pages)


def _contiguous_case(rng, ctx, q_lens, H, KVH, D, B, dtype=np.float32):
    """Random per-sequence contiguous K/V [KVH, n, D] plus the same rows scattered into a paged pool
    with an identity block assignment (sequence after sequence)."""
    S = len(ctx)
    nblk = [-(-n // B) for n in ctx]
    pool = sum(nblk) + 2
    kc = rng.standard_normal((pool, KVH, B, D)).astype(dtype)
    vc = rng.standard_normal((pool, KVH, D, B)).astype(dtype)
    table = np.full((S, max(nblk)), -1, dtype=np.int32)
    Ks, Vs = [], []
    cur = 0
    for s, n in enumerate(ctx):
        K = rng.standard_normal((KVH, n, D)).astype(dtype)
        V = rng.standard_normal((KVH, n, D)).astype(dtype)
        for t in range(n):
            blk, off = cur + t // B, t % B
            kc[blk, :, off, :] = K[:, t, :]
            vc[blk, :, :, off] = V[:, t, :]
        table[s, :nblk[s]] = np.arange(cur, cur + nblk[s])
        cur += nblk[s]
        Ks.append(K)
        Vs.append(V)
    q = rng.standard_normal((int(sum(q_lens)), H, D)).astype(dtype)
    return q, kc, vc, table, np.asarray(ctx, np.int32), np.asarray(q_lens, np.int32), Ks, Vs


def _sdpa_reference(q, Ks, Vs, q_lens, H, KVH, scale):
    """torch.nn.functional.scaled_dot_product_attention in float64 on unpaged K/V.  The LSE comes from
    the same library call with one extra 'sink' key (k = 0, so its score is 0) whose value is a unit
    vector in an extra output dimension: that output equals 1 / (exp(lse) + 1)."""
    G = H // KVH
    outs, lses = [], []
    base = 0
    for s, (K, V) in enumerate(zip(Ks, Vs)):
        qs = int(q_lens[s])
        n = K.shape[1]
        D = K.shape[2]
        Q = torch.from_numpy(q[base:base + qs].astype(np.float64)).permute(1, 0, 2)[None]  # [1,H,qs,D]
        Kt = torch.from_numpy(K.astype(np.float64)).repeat_interleave(G, dim=0)[None]      # [1,H,n,D]
        Vt = torch.from_numpy(V.astype(np.float64)).repeat_interleave(G, dim=0)[None]
        i = torch.arange(qs)[:, None]
        t = torch.arange(n)[None, :]
        mask = t <= (n - qs + i)
        o = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt, attn_mask=mask, scale=scale)
        Ks_ = torch.cat([Kt, torch.zeros(1, H, 1, D, dtype=torch.float64)], dim=2)
        Vs_ = torch.cat([torch.cat([Vt, torch.zeros(1, H, n, 1, dtype=torch.float64)], dim=3),
                         torch.cat([torch.zeros(1, H, 1, D, dtype=torch.float64),
                                    torch.ones(1, H, 1, 1, dtype=torch.float64)], dim=3)], dim=2)
        mask_s = torch.cat([mask, torch.ones(qs, 1, dtype=torch.bool)], dim=1)
        o2 = torch.nn.functional.scaled_dot_product_attention(Q, Ks_, Vs_, attn_mask=mask_s, scale=scale)
        sink = o2[0, :, :, D]                                       # [H, qs]
        lse = torch.log(1.0 / sink - 1.0)
        outs.append(o[0].permute(1, 0, 2).numpy())
        lses.append(lse.T.numpy())
        base += qs
    return np.concatenate(outs), np.concatenate(lses)


CASES = [
    # ctx, q_lens, H, KVH, D, B
    ([5, 17, 40], [1, 3, 2], 6, 2, 8, 4),
    ([1, 16, 33], [1, 1, 1], 4, 2, 16, 16),
    ([48, 9], [5, 4], 8, 8, 4, 16),
    ([70], [5], 8, 1, 8, 16),
]


@pytest.mark.parametrize("case", CASES)
def test_p1_contiguous_equivalence_with_library_sdpa(case):
    ctx, ql, H, KVH, D, B = case
    rng = np.random.default_rng(11)
    q, kc, vc, table, cl, qlens, Ks, Vs = _contiguous_case(rng, ctx, ql, H, KVH, D, B)
    scale = 1.0 / math.sqrt(D)
    out, lse = O.paged_decode_attention(q, kc, vc, table, cl, qlens, scale, KVH, B)
    ref_out, ref_lse = _sdpa_reference(q, Ks, Vs, qlens, H, KVH, scale)
    assert np.max(np.abs(out - ref_out)) <= 1e-12
    assert np.max(np.abs(lse - ref_lse)) <= 1e-10


def test_p2_physical_block_permutation_is_bitwise_invisible():
    rng = np.random.default_rng(12)
    q, kc, vc, table, cl, qlens, _, _ = _contiguous_case(rng, [30, 3, 64], [2, 1, 5], 4, 2, 8, 16)
    out, lse = O.paged_decode_attention(q, kc, vc, table, cl, qlens, 0.3, 2, 16)
    perm = rng.permutation(kc.shape[0])
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    table2 = np.where(table >= 0, perm[np.maximum(table, 0)], -1).astype(np.int32)
    out2, lse2 = O.paged_decode_attention(q, kc2, vc2, table2, cl, qlens, 0.3, 2, 16)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_p3_one_token_context_returns_v_exactly():
    rng = np.random.default_rng(13)
    q, kc, vc, table, cl, qlens, Ks, Vs = _contiguous_case(rng, [1, 1], [1, 1], 4, 2, 8, 16)
    out, lse = O.paged_decode_attention(q, kc, vc, table, cl, qlens, 0.7, 2, 16)
    for s in range(2):
        for h in range(4):
            assert np.array_equal(out[s, h], Vs[s][h // 2, 0].astype(np.float64))
            want = 0.7 * float(np.dot(q[s, h].astype(np.float64), Ks[s][h // 2, 0].astype(np.float64)))
            assert abs(lse[s, h] - want) <= 1e-14 * max(1.0, abs(want))


def test_p4_equal_keys_give_mean_of_visible_values():
    rng = np.random.default_rng(14)
    ctx, ql = [37, 21], [3, 5]
    q, kc, vc, table, cl, qlens, Ks, Vs = _contiguous_case(rng, ctx, ql, 4, 2, 8, 16)
    krow = rng.standard_normal(8).astype(np.float32)
    kc[:] = krow                                           # every key row equal
    out, lse = O.paged_decode_attention(q, kc, vc, table, cl, qlens, 0.25, 2, 16)
    base = 0
    for s, (n, qs) in enumerate(zip(ctx, ql)):
        for i in range(qs):
            nvis = n - qs + i + 1
            for h in range(4):
                mean = Vs[s][h // 2, :nvis].astype(np.float64).mean(axis=0)
                assert np.max(np.abs(out[base + i, h] - mean)) <= 1e-13
                x = 0.25 * float(np.dot(q[base + i, h].astype(np.float64), krow.astype(np.float64)))
                assert abs(lse[base + i, h] - (x + math.log(nvis))) <= 1e-13
        base += qs


def test_p5_causal_row_equals_shorter_single_token_decode():
    rng = np.random.default_rng(15)
    n, qs = 45, 5
    q, kc, vc, table, cl, qlens, _, _ = _contiguous_case(rng, [n], [qs], 4, 2, 8, 16)
    out, lse = O.paged_decode_attention(q, kc, vc, table, cl, qlens, 0.4, 2, 16)
    for i in range(qs):
        o1, l1 = O.paged_decode_attention(q[i:i + 1], kc, vc, table, np.array([n - qs + i + 1], np.int32),
                                          np.array([1], np.int32), 0.4, 2, 16)
        assert np.max(np.abs(out[i] - o1[0])) <= 1e-13
        assert np.max(np.abs(lse[i] - l1[0])) <= 1e-13


def test_p6_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(16)
    H, KVH = 8, 2
    q, kc, vc, table, cl, qlens, _, _ = _contiguous_case(rng, [19, 50], [1, 2], H, KVH, 8, 16)
    out, lse = O.paged_decode_attention(q, kc, vc, table, cl, qlens, 0.35, KVH, 16)
    G = H // KVH
    kc_m = np.repeat(kc, G, axis=1)       # MHA pool: head h holds a copy of kv head h // G
    vc_m = np.repeat(vc, G, axis=1)
    out_m, lse_m = O.paged_decode_attention(q, kc_m, vc_m, table, cl, qlens, 0.35, H, 16)
    assert np.max(np.abs(out - out_m)) <= 1e-15 and np.max(np.abs(lse - lse_m)) <= 1e-15


@pytest.mark.parametrize("P", [16, 32, 48])
def test_p7_partition_then_lse_combine_equals_unsplit(P):
    rng = np.random.default_rng(17)
    # ctx 33 with q 5 and P 32: rows 0..3 see nothing in partition 1 (lse_p = -inf, weight 0)
    ctx, ql = [33, 100, 16, 65], [5, 1, 3, 2]
    q, kc, vc, table, cl, qlens, _, _ = _contiguous_case(rng, ctx, ql, 4, 2, 8, 16)
    out, lse = O.paged_decode_attention(q, kc, vc, table, cl, qlens, 0.3, 2, 16)
    outs, lses = O.partition_attention(q, kc, vc, table, cl, qlens, 0.3, 2, P, 16)
    if P == 32:
        assert np.isneginf(lses[1][0:4]).all() and np.all(outs[1][0:4] == 0)
    out_c, lse_c = O.lse_combine(outs, lses)
    assert np.all(np.isfinite(out_c))
    assert np.max(np.abs(out - out_c)) <= 1e-12 and np.max(np.abs(lse - lse_c)) <= 1e-12


def test_p8_shared_prefix_blocks_equal_private_copies():
    rng = np.random.default_rng(18)
    B, KVH, D, H = 16, 2, 8, 4
    ctx = [40, 70, 20]
    shared = 2
    pool = 20
    kc = rng.standard_normal((pool, KVH, B, D)).astype(np.float32)
    vc = rng.standard_normal((pool, KVH, D, B)).astype(np.float32)
    perm = rng.permutation(pool)
    table = np.full((3, 5), -1, np.int32)
    cur = shared
    for s, n in enumerate(ctx):
        nb = -(-n // B)
        k = min(nb, shared)
        table[s, :k] = perm[:k]
        table[s, k:nb] = perm[cur:cur + nb - k]
        cur += nb - k
    q = rng.standard_normal((3, H, D)).astype(np.float32)
    cl = np.array(ctx, np.int32)
    ql = np.ones(3, np.int32)
    out, lse = O.paged_decode_attention(q, kc, vc, table, cl, ql, 0.3, KVH, B)
    # private copies of the shared blocks for sequences 1 and 2
    kc2 = np.concatenate([kc, kc[perm[:shared]], kc[perm[:shared]]])
    vc2 = np.concatenate([vc, vc[perm[:shared]], vc[perm[:shared]]])
    table2 = table.copy()
    table2[1, :2] = [pool, pool + 1]
    table2[2, :2] = [pool + 2, pool + 3]
    out2, lse2 = O.paged_decode_attention(q, kc2, vc2, table2, cl, ql, 0.3, KVH, B)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_p9_brute_force_scalar_loops_on_tiny_pool():
    """Brute force on a tiny ragged case: every score, softmax weight and output element with Python
    floats and math.exp, indexing the flat pool buffer directly (offset = ((block * KVH + kv head) *
    B + slot) * D + d for K, ((block * KVH + kv head) * D + d) * B + slot for V)."""
    rng = np.random.default_rng(19)
    B, KVH, G, D = 16, 2, 2, 8
    H = KVH * G
    ctx, ql = [1, 7, 16, 33], [1, 2, 1, 3]
    pool = 10
    kc = rng.standard_normal((pool, KVH, B, D)).astype(np.float32)
    vc = rng.standard_normal((pool, KVH, D, B)).astype(np.float32)
    perm = rng.permutation(pool)
    table = np.full((4, 3), -1, dtype=np.int32)
    used = 0
    for s, n in enumerate(ctx):
        for j in range(-(-n // B)):
            table[s, j] = perm[used]
            used += 1
    q = rng.standard_normal((sum(ql), H, D)).astype(np.float32)
    scale = 0.4
    out, lse = O.paged_decode_attention(q, kc, vc, table, np.array(ctx), np.array(ql), scale, KVH, B)
    kf, vf = kc.reshape(-1).tolist(), vc.reshape(-1).tolist()
    row = 0
    for s, n in enumerate(ctx):
        for i in range(ql[s]):
            for h in range(H):
                g = h // G
                xs = []
                for t in range(n - ql[s] + i + 1):
                    blk, slot = int(table[s, t // B]), t % B
                    kbase = ((blk * KVH + g) * B + slot) * D
                    xs.append(scale * sum(float(q[row, h, d]) * kf[kbase + d] for d in range(D)))
                m = max(xs)
                ws = [math.exp(x - m) for x in xs]
                z = sum(ws)
                assert abs(lse[row, h] - (m + math.log(z))) <= 1e-12
                for d in range(D):
                    o = 0.0
                    for t, wt in enumerate(ws):
                        blk, slot = int(table[s, t // B]), t % B
                        o += wt / z * vf[((blk * KVH + g) * D + d) * B + slot]
                    assert abs(out[row, h, d] - o) <= 1e-12
            row += 1



@pytest.mark.parametrize("dtype", [np.float32, np.uint16])
def test_p10_cache_write_moves_bits_to_flat_offsets(dtype):
    rng = np.random.default_rng(19)
    nb, KVH, B, D, T = 6, 3, 16, 8, 7
    if dtype == np.uint16:
        kc = rng.integers(0, 1 << 16, (nb, KVH, B, D)).astype(np.uint16)
        vc = rng.integers(0, 1 << 16, (nb, KVH, D, B)).astype(np.uint16)
        k = rng.integers(0, 1 << 16, (T, KVH, D)).astype(np.uint16)
        v = rng.integers(0, 1 << 16, (T, KVH, D)).astype(np.uint16)
        k[0, 0, 0] = 0x7FC1            # NaN payloads must survive unchanged
    else:
        kc = rng.standard_normal((nb, KVH, B, D)).astype(np.float32)
        vc = rng.standard_normal((nb, KVH, D, B)).astype(np.float32)
        k = rng.standard_normal((T, KVH, D)).astype(np.float32)
        v = rng.standard_normal((T, KVH, D)).astype(np.float32)
    slots = np.array([5, -1, 17, 95, 0, -7, 48], np.int64)
    kc2, vc2 = O.kv_cache_write(kc, vc, k, v, slots, B)
    fk, fv = kc.reshape(-1).copy(), vc.reshape(-1).copy()
    for t, slot in enumerate(slots):
        if slot < 0:
            continue
        blk, off = slot // B, slot % B
        for h in range(KVH):
            for d in range(D):
                fk[((blk * KVH + h) * B + off) * D + d] = k[t, h, d]
                fv[((blk * KVH + h) * D + d) * B + off] = v[t, h, d]
    assert kc2.dtype == kc.dtype and vc2.dtype == vc.dtype
    assert np.array_equal(kc2.reshape(-1).view(np.uint8), fk.view(np.uint8))
    assert np.array_equal(vc2.reshape(-1).view(np.uint8), fv.view(np.uint8))


def test_p11_scale_moves_between_q_and_scale():
    rng = np.random.default_rng(20)
    q, kc, vc, table, cl, qlens, _, _ = _contiguous_case(rng, [29, 3], [2, 1], 4, 2, 8, 16,
                                                         dtype=np.float64)
    out, lse = O.paged_decode_attention(q, kc, vc, table, cl, qlens, 0.5, 2, 16)
    out2, lse2 = O.paged_decode_attention(q * 4.0, kc, vc, table, cl, qlens, 0.125, 2, 16)
    assert np.max(np.abs(out - out2)) <= 1e-12 and np.max(np.abs(lse - lse2)) <= 1e-12


def test_widen_bf16_bit_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3FC0, 0x0001, 0x7F80, 0x4049, 0x8000], np.uint16)
    got = O.widen(bits)
    want = [1.0, -2.0, 1.5, 2.0 ** -133, math.inf, 3.140625, -0.0]
    assert got.dtype == np.float64
    for g, w in zip(got, want):
        assert g == w and math.copysign(1, g) == math.copysign(1, w)


# ----------------------------------------------------------------------------------------------
# golden: the hand-worked example


def _num(x):
    if isinstance(x, (int, float)):
        return float(x)
    m = re.fullmatch(r"ln\((\d+)/(\d+)\)", x)
    if m:
        return math.log(int(m.group(1)) / int(m.group(2)))
    m = re.fullmatch(r"ln(\d+)", x)
    if m:
        return math.log(int(m.group(1)))
    return float(Fraction(x))


def _golden_inputs():
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        g = json.load(f)
    B, KVH = g["block_size"], g["num_kv_heads"]
    table = np.array(g["block_tables"], np.int32)
    D = 2
    kc = np.full((2, KVH, B, D), 100.0)
    vc = np.full((2, KVH, D, B), 100.0)
    for h in range(KVH):
        for t, (krow, vrow) in enumerate(zip(g["k_tokens"][str(h)], g["v_tokens"][str(h)])):
            blk, off = table[0, t // B], t % B
            kc[blk, h, off, :] = [_num(x) for x in krow]
            vc[blk, h, :, off] = [_num(x) for x in vrow]
    qtok = np.array([[_num(x) for x in row] for row in g["q_token"]])
    q = np.stack([qtok, qtok])                     # both new tokens carry the same q per head
    exp_out = np.array([[[_num(x) for x in hrow] for hrow in row] for row in g["expected_out"]])
    exp_lse = np.array([[_num(x) for x in row] for row in g["expected_lse"]])
    args = (q, kc, vc, table, np.array(g["context_lens"], np.int32), np.array(g["q_lens"], np.int32),
            g["scale"], KVH, B)
    return args, exp_out, exp_lse


def _golden_ok(mod):
    args, exp_out, exp_lse = _golden_inputs()
    out, lse = mod.paged_decode_attention(*args)
    return (np.max(np.abs(out - exp_out)) <= 1e-14) and (np.max(np.abs(lse - exp_lse)) <= 1e-14)


def test_golden_hand_example():
    assert _golden_ok(O)


# ----------------------------------------------------------------------------------------------
# planted mistakes: each must break a pin


MUTATIONS = [
    ("gqa head map", "g * G, (g + 1) * G) if head_set", "g, H, KVH) if head_set"),
    ("causal offset", "last = n - qs + np.arange(qs)                     #",
     "last = n - qs + 1 + np.arange(qs)                 #"),
    ("transposed V block", "np.transpose(vb, (0, 2, 1))", "vb"),
    ("dropped scale", "x = scale * (qrows @ K.T)", "x = (qrows @ K.T)"),
    ("log2 lse", "lse = m[:, 0] + np.log(z[:, 0])", "lse = m[:, 0] + np.log2(z[:, 0])"),
    ("block index", "ids = np.asarray(block_table_row[:nblk], dtype=np.int64)",
     "ids = np.arange(nblk)"),
    ("q row base", "base = int(starts[s])", "base = s"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistakes_are_caught(name, old, new):
    src = open(O.__file__).read()
    assert old in src, f"mutation anchor for {name} missing"
    ns = {"__name__": "oracle_mutant"}
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), ns)

    class M:
        pass

    for k in ("paged_decode_attention",):
        setattr(M, k, ns[k])
    try:
        caught = not _golden_ok(M)
    except Exception:
        caught = True
    if not caught:
        # the golden case may not exercise every slip; fall back to the SDPA pin on ragged q
        ctx, ql, H, KVH, D, B = CASES[0]
        rng = np.random.default_rng(11)
        q, kc, vc, table, cl, qlens, Ks, Vs = _contiguous_case(rng, ctx, ql, H, KVH, D, B)
        try:
            out, lse = M.paged_decode_attention(q, kc, vc, table, cl, qlens, 0.3, KVH, B)
            ref_out, ref_lse = _sdpa_reference(q, Ks, Vs, qlens, H, KVH, 0.3)
            caught = not (np.max(np.abs(out - ref_out)) <= 1e-12 and np.max(np.abs(lse - ref_lse)) <= 1e-10)
        except Exception:
            caught = True
    assert caught, f"planted mistake '{name}' passed every pin"
