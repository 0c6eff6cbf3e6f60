"""A CPU model of the balanced persistent decode schedule and of the merge's source search.

The persistent decode kernel (csrc/decode_mfma.hip) lays every work item (kv head, sequence, row tile)
out as one page stream, item_cost virtual pages then the item's real pages, and gives wave `ord` of
NW the share [floor(L ord / NW), floor(L (ord + 1) / NW)), each end moved to the item's start when it
falls on virtual pages and down to a multiple of cut_align real pages otherwise.  A piece that covers
a whole single-partition item writes the final row; a piece that starts a partition writes that
partition's row; any other piece (only a share's first piece can start inside an item) writes the
wave's spill rows.  The merge (csrc/decode_combine.hip) finds a row's sources with no table: the
partitions, plus every share whose rounded start lands inside the item's real pages, off a partition
start, on a non-empty piece.

This model restates those rules in plain Python and checks, on random shapes, that
  * every real page of every item is read by exactly one piece;
  * only a share's first piece starts inside an item;
  * the sources the merge enumerates are exactly the partial pieces the waves write, and a row the
    merge treats as final was written final by one piece.
It checks the rules, not the kernels: the GPU parity tests compare the kernels' outputs with the
oracle on every row, at the sizes and shapes where these rules decide the pieces.
"""
import random

import numpy as np
import pytest

B = 16   # tokens per page


def share_raw(L, NW, o):
    return (L * o) // NW


def first_share_above(L, NW, pos):
    c = 0
    while c < NW and share_raw(L, NW, c) <= pos:
        c += 1
    return c


def first_share_above_f32(L, NW, pos):
    """The decode kernel's form: ceil((pos + 1) NW / L) from a single-precision quotient, settled by
    exact integer products (NW when no share starts above pos)."""
    t = (pos + 1) * NW
    if t >= L * NW:
        return NW
    c = min(max(int(np.float32(t) / np.float32(L)), 0), NW)
    steps = 0
    while c * L < t:
        c += 1
        steps += 1
    down = 0
    while c > 0 and (c - 1) * L >= t:
        c -= 1
        down += 1
    return c, steps, down


def piece_index(L, NW, cost, pos0, o, cap, first_above=first_share_above):
    """Slot of the piece share o starts inside the item at stream pos0 (no fixed partitions)."""
    if L < NW:
        return cap
    return min(o - first_above(L, NW, pos0 + cost) + 1, cap)


def simulate(ctxs, qls, G, ROWS, KVH, cost, NW, N, PP, first_above=first_share_above, max_pieces=0,
             piece=piece_index):
    S = len(ctxs)
    nblk = [(x + B - 1) // B for x in ctxs]
    qs = [max(1, min(q, x)) for q, x in zip(qls, ctxs)]
    rts = [(q * G + ROWS - 1) // ROWS for q in qs]
    span = [(n + cost) if n > 0 else 0 for n in nblk]
    pre = [0]
    for s in range(S):
        pre.append(pre[-1] + span[s] * rts[s])
    I = pre[S]
    L = I * KVH

    def seq_of(r):   # the last sequence s with pre[s] <= r (never an empty one)
        s0, s1 = 0, S
        while s1 - s0 > 1:
            mid = (s0 + s1) // 2
            if pre[mid] <= r:
                s0 = mid
            else:
                s1 = mid
        return s0

    def cut(b):   # a raw share start, moved as the decode kernel moves it
        if b >= L:
            return L
        kvh = b // I
        r = b - kvh * I
        s = seq_of(r)
        off = (r - pre[s]) % span[s]
        ro = off - cost
        if ro <= 0:
            return b - off
        rr = ro - ro % N
        return b - off + (cost + rr if rr > 0 else 0)

    slots = max_pieces > 1 and PP >= 10 ** 6   # piece slots exist only without fixed partitions
    counts = {}   # (kvh, s, rt) -> the piece count the item-ending run stores
    pieces = []   # (kvh, s, rt, first page, end page, ord, destination)
    for o in range(NW):
        k, k_end = cut(share_raw(L, NW, o)), cut(share_raw(L, NW, o + 1))
        first = True
        while k < k_end:
            kvh = k // I
            r = k - kvh * I
            s = seq_of(r)
            local = r - pre[s]
            t = local // span[s]
            off = local - t * span[s]
            j0 = max(off - cost, 0)
            kreal = k - off + cost + j0
            run = min(nblk[s] - j0, k_end - kreal)
            assert run > 0, (o, k, k_end, s, off)
            if j0 > 0:
                assert first, "only the share's first piece starts inside an item"
            nparts = (ctxs[s] + PP * B - 1) // (PP * B)
            kp = 0
            if slots:
                if j0 > 0:
                    kp = piece(L, NW, cost, kvh * I + pre[s] + t * span[s], o, max_pieces)
                if j0 + run == nblk[s]:
                    counts[(kvh, s, t)] = kp + 1 if kp < max_pieces else max_pieces + 1
            j = j0
            while j < j0 + run:   # pieces also end at partition ends
                pend = min(j0 + run, (j // PP + 1) * PP)
                if j == 0 and pend == nblk[s] and nparts == 1:
                    dest = ("final",)
                elif j % PP == 0:
                    dest = ("part", j // PP)
                elif slots and kp < max_pieces:
                    dest = ("part", kp)
                else:
                    dest = ("spill", o)
                pieces.append((kvh, s, t, j, pend, o, dest))
                j = pend
            k = kreal + run
            first = False

    cover = {}
    for kvh, s, t, j0, j1, o, _ in pieces:
        for j in range(j0, j1):
            key = (kvh, s, t, j)
            assert key not in cover, ("page read twice", key)
            cover[key] = o
    for kvh in range(KVH):
        for s in range(S):
            for t in range(rts[s]):
                for j in range(nblk[s]):
                    assert (kvh, s, t, j) in cover, ("page never read", kvh, s, t, j)

    for kvh in range(KVH):
        for s in range(S):
            if nblk[s] == 0:
                continue
            nparts = (ctxs[s] + PP * B - 1) // (PP * B)
            for t in range(rts[s]):
                pos0 = kvh * I + pre[s] + t * span[s]
                pos1 = pos0 + span[s]
                ord0 = first_above(L, NW, pos0)
                ncand = max(0, first_above(L, NW, pos1 - 1) - ord0)

                def real_off(b):
                    ro = b - pos0 - cost
                    return ro & ~(N - 1) if ro > 0 else 0

                sources = {("part", p) for p in range(nparts)}
                any_cut = False
                for o in range(ord0, ord0 + ncand):
                    b = share_raw(L, NW, o)
                    assert pos0 < b < pos1
                    ob = real_off(b)
                    if ob <= 0:
                        continue
                    any_cut = True
                    if ob % PP == 0:
                        continue
                    bn = share_raw(L, NW, o + 1)
                    obn = real_off(bn) if bn < pos1 else nblk[s]
                    if obn <= ob:
                        continue
                    kp = piece(L, NW, cost, pos0, o, max_pieces) if slots else max_pieces
                    sources.add(("part", kp) if kp < max_pieces else ("spill", o))
                mine = sorted((p for p in pieces if p[:3] == (kvh, s, t)), key=lambda p: p[3])
                written = [p[6] for p in mine]
                assert len(set(written)) == len(written), ("two pieces share a row", written)
                written = set(written)
                if nparts <= 1 and not any_cut:
                    assert written == {("final",)}, (written, kvh, s, t)
                else:
                    assert ("final",) not in written
                    assert written == sources, (written, sources, kvh, s, t, cost, N, PP)
                if slots:
                    # the count the item-ending run stores, and the slots the one-round-trip merge
                    # reads when it is at most max_pieces: pieces in stream order fill slots 0, 1, ...
                    # (a stream shorter than the wave count has empty shares: pieces past the first
                    # take spill rows and the count sends the merge to its search)
                    nslot = max_pieces if L >= NW else 1
                    cnt = counts[(kvh, s, t)]
                    assert cnt == (len(mine) if len(mine) <= nslot else max_pieces + 1), (cnt, len(mine))
                    for rank, p in enumerate(mine):
                        if p[6] != ("final",):
                            assert p[6] == (("part", rank) if rank < nslot else ("spill", p[5])), (rank, p)
    return pieces


def random_shape(rng):
    S = rng.choice([1, 2, 3, 5, 8, 32, 64])
    ctxs = [rng.choice([0, 1, 15, 16, 17, rng.randint(1, 700), rng.randint(1, 3000)]) for _ in range(S)]
    if all(x == 0 for x in ctxs):
        ctxs[0] = 5
    maxq = rng.choice([1, 1, 5, 8])
    if rng.random() < 0.5:
        N, PP = 1, 10 ** 6                       # no fixed partitions: cuts on any page
    else:
        N = rng.choice([2, 4])                   # ring depth; partitions of PP pages
        PP = N * rng.choice([1, 2, 8])
    return dict(ctxs=ctxs, qls=[rng.randint(1, maxq) for _ in range(S)], G=rng.choice([1, 4, 8]),
                ROWS=rng.choice([16, 32]), KVH=rng.choice([1, 2, 8]), cost=rng.choice([0, 1, 2, 3, 4]),
                NW=8 * rng.choice([1, 2, 4, 8, 16]), N=N, PP=PP)


@pytest.mark.parametrize("seed", range(4))
def test_every_page_once_and_merge_sources_match_the_pieces(seed):
    rng = random.Random(seed)
    for _ in range(75):
        simulate(**random_shape(rng))


@pytest.mark.parametrize("seed", range(4))
def test_piece_slots_follow_stream_order_and_the_count(seed):
    # no fixed partitions, slots on: the first max_pieces pieces of an item (in stream order) take
    # partition rows 0 .. max_pieces - 1, the rest their waves' spill rows, and the stored count says
    # how many there are (max_pieces + 1 past that); small and large slot counts (down to the 2 a
    # short workspace may leave), streams shorter than the wave count included (their pieces all take
    # spill rows)
    rng = random.Random(100 + seed)
    for _ in range(75):
        shape = random_shape(rng)
        shape.update(N=1, PP=10 ** 6)
        simulate(**shape, max_pieces=rng.choice([2, 3, 4, 6, 18, 32]))


def test_piece_index_catches_an_off_by_one():
    # planted mistake: the slot formula counts one share too few
    def short_by_one(L, NW, cost, pos0, o, cap):
        return cap if L < NW else min(o - first_share_above(L, NW, pos0 + cost), cap)

    rng = random.Random(12)
    with pytest.raises(AssertionError):
        for _ in range(50):
            shape = random_shape(rng)
            shape.update(N=1, PP=10 ** 6)
            simulate(**shape, max_pieces=32, piece=short_by_one)


def test_single_precision_share_search_is_exact():
    # the kernel's share search against the exact one: stream lengths up to 2^31, up to 2^13 waves,
    # positions at share boundaries and off them; the estimate is never above the answer and at most
    # two below it
    rng = random.Random(5)
    for _ in range(20000):
        L = rng.choice([rng.randint(1, 5000), rng.randint(1, 1 << 20), rng.randint(1 << 30, (1 << 31) - 1)])
        NW = rng.choice([8, 64, 1024, 2048, 8192, 8 * rng.randint(1, 1024)])
        if rng.random() < 0.5:
            o = rng.randint(0, NW)
            pos = max(share_raw(L, NW, o) + rng.choice([-1, 0, 1]), 0)
        else:
            pos = rng.randint(0, L + 2)
        want = (-(-(pos + 1) * NW // L)) if (pos + 1) * NW < L * NW else NW
        got = first_share_above_f32(L, NW, pos)
        if isinstance(got, tuple):
            got, up, down = got
            assert up <= 2 and down == 0, (L, NW, pos, up, down)
        assert got == want, (L, NW, pos, got, want)
        if L <= 5000 and NW <= 2048:
            assert got == first_share_above(L, NW, pos), (L, NW, pos)


def test_one_long_sequence_is_cut_across_many_waves():
    # one item per kv head and 1024 waves: every item is cut into many pieces, all found by the merge
    pieces = simulate(ctxs=[32768], qls=[1], G=8, ROWS=16, KVH=8, cost=4, NW=1024, N=1, PP=10 ** 6)
    per_item = {}
    for kvh, s, t, *_ in pieces:
        per_item[(kvh, s, t)] = per_item.get((kvh, s, t), 0) + 1
    assert min(per_item.values()) >= 100


def test_model_catches_a_wrong_source_rule():
    # planted mistake in the merge's search: the first share that starts inside an item is skipped
    def skips_one(L, NW, pos):
        return min(first_share_above(L, NW, pos) + 1, NW)

    rng = random.Random(11)
    with pytest.raises(AssertionError):
        for _ in range(50):
            simulate(**random_shape(rng), first_above=skips_one)
