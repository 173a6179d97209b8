"""CPU replay of the decode kernel's item order (no GPU).

Every workgroup of the persistent decode kernel sorts the batch's sequences
by the size of their last partition, largest first (longest processing time
first), with a stable counting sort that must give the same order in every
workgroup: thread t holds sequences t and t + 256; key counts per 64-sequence
chunk give the equal keys in earlier chunks; a ballot within the wave gives
the rank among equal keys in the wave's own chunk; an exclusive scan over
keys in decreasing order gives each key's first position.  The replay follows
those steps and checks that the result is a permutation, in decreasing key
order with ties by sequence index, for the workloads' length mixes and for
edge cases (one sequence, 512, all equal, zero lengths).
"""

import numpy as np
import pytest

import workloads

NTH, NCH, KEYS = 256, 8, 256


def kernel_order(lens, P, bs):
    S = len(lens)
    assert S <= 2 * NTH
    key = np.full(2 * NTH, -1, np.int64)
    for i in range(S):
        n = int(lens[i])
        last = n - ((n - 1) // P) * P if n > 0 else 0
        key[i] = min((last + bs - 1) // bs, KEYS - 1)
    cnt = np.zeros((NCH, KEYS), np.int64)
    for i in range(S):
        cnt[i >> 6, key[i]] += 1
    run = np.zeros(KEYS, np.int64)
    before = np.zeros((NCH, KEYS), np.int64)
    for k in range(KEYS):
        acc = 0
        for c in range(NCH):
            before[c, k] = acc
            acc += cnt[c, k]
        run[k] = acc
    # thread t owns key KEYS-1-t; exclusive scan over threads
    first = np.zeros(KEYS, np.int64)
    acc = 0
    for t in range(NTH):
        k = KEYS - 1 - t
        first[k] = acc
        acc += run[k]
    order = np.full(S, -1, np.int64)
    for c in range(NCH):                   # one wave per chunk and round
        idx = np.arange(64 * c, 64 * c + 64)
        valid = idx < S
        todo = valid.copy()
        rank = np.zeros(64, np.int64)
        while todo.any():
            leader = int(np.flatnonzero(todo)[0])
            kl = key[idx[leader]]
            m = valid & (key[idx] == kl)
            rank[m] = np.cumsum(m)[m] - 1
            todo &= ~m
        for lane in np.flatnonzero(valid):
            i = idx[lane]
            pos = first[key[i]] + before[c, key[i]] + rank[lane]
            assert 0 <= pos < S
            assert order[pos] == -1, "two sequences at one position"
            order[pos] = i
    return order, key[:S]


def _check(lens, P, bs):
    order, key = kernel_order(lens, P, bs)
    assert sorted(order.tolist()) == list(range(len(lens)))
    ks = key[order]
    assert np.all(np.diff(ks) <= 0)
    for k in np.unique(ks):                 # ties keep sequence order
        same = order[ks == k]
        assert np.all(np.diff(same) > 0)


@pytest.mark.parametrize("cfg,P,bs", [(2, 2032, 16), (2, 512, 16), (4, 1536, 16), (5, 4096, 16),
                                      (5, 1024, 16), (3, 512, 8)])
def test_workload_orders(cfg, P, bs):
    lens = workloads.config_lengths(cfg, np.random.default_rng(1000 + cfg), False)
    _check(np.asarray(lens), P, bs)


@pytest.mark.parametrize("seed", range(6))
def test_random_batches(seed):
    rng = np.random.default_rng(seed)
    S = int(rng.integers(1, 513))
    bs = int(rng.choice([8, 16, 32]))
    P = bs * int(rng.integers(1, 257))
    lens = rng.integers(0, 3 * P, size=S)
    lens[rng.random(S) < 0.1] = 0
    _check(lens, P, bs)


def test_edge_batches():
    _check(np.array([7]), 16, 16)
    _check(np.zeros(512, np.int64), 512, 16)          # every key equal (empty contexts)
    _check(np.full(512, 4096), 4096, 16)               # every key clamped to the top
    _check(np.arange(512) * 8, 4096, 16)



def kernel_items(lens, P, bs, Y):
    """Every item the kernel enumerates, as (sequence, row group, partition):
    the full partitions first, in sequence order (every one holds P tokens,
    so their order does not matter for longest-first; a workgroup can start
    one from a prefix sum over the lengths, before the sort), then the last
    (shorter or only) partitions in the sorted order, decoded the way the
    kernel decodes an item index (item % Y is the row group)."""
    S = len(lens)
    order, _ = kernel_order(lens, P, bs)
    nf = [int(lens[i]) // P for i in range(S)]
    nr = []
    for pos in range(S):
        n = int(lens[int(order[pos])])
        nr.append(1 if (n % P != 0 or n == 0) else 0)
    full = np.concatenate([[0], np.cumsum(nf)])      # by sequence index
    rag = np.concatenate([[0], np.cumsum(nr)])       # by sorted position
    F, R = int(full[-1]), int(rag[-1])
    items = []
    for item in range(Y * (F + R)):
        y, rest = item % Y, item // Y
        if rest < F:
            seq = int(np.searchsorted(full, rest, side="right") - 1)
            part = rest - int(full[seq])
        else:
            pos = int(np.searchsorted(rag, rest - F, side="right") - 1)
            seq = int(order[pos])
            part = int(lens[seq]) // P
        items.append((seq, y, part))
    return items


def _expected_items(lens, P, Y):
    return {(i, y, p) for i in range(len(lens)) for y in range(Y)
            for p in range(max(1, -(-int(lens[i]) // P)))}


@pytest.mark.parametrize("cfg,P,bs,Y", [(2, 1024, 16, 32), (3, 512, 8, 8), (4, 1536, 16, 8),
                                        (5, 4096, 16, 8)])
def test_every_item_exactly_once(cfg, P, bs, Y):
    lens = np.asarray(workloads.config_lengths(cfg, np.random.default_rng(1000 + cfg), False))
    items = kernel_items(lens, P, bs, Y)
    assert len(items) == len(set(items))
    assert set(items) == _expected_items(lens, P, Y)


@pytest.mark.parametrize("seed", range(4))
def test_every_item_exactly_once_random(seed):
    rng = np.random.default_rng(40 + seed)
    S = int(rng.integers(1, 300))
    bs = int(rng.choice([8, 16, 32]))
    P = bs * int(rng.integers(1, 20))
    lens = rng.integers(0, 4 * P, size=S)
    lens[rng.random(S) < 0.2] = 0
    lens[rng.random(S) < 0.2] = P
    Y = int(rng.choice([1, 3, 8, 32]))
    items = kernel_items(lens, P, bs, Y)
    assert len(items) == len(set(items))
    assert set(items) == _expected_items(lens, P, Y)


def queue_items(G, total, one_deep, seed=0, young_from=None):
    """Replay of the decode kernel's work distribution over a grid of G
    persistent workgroups.  Every workgroup starts with item b.  Workgroups
    from young_from on run only that item.  Holding a reserve (as the kernel
    first did), a workgroup also starts with item (queue_wgs + b / nq) * nq +
    queue and claims the item after next at each item's last step; one deep,
    it claims the next item itself.  Claims come from the workgroup's
    per-XCD queue (claim c is item (n_static * queue_wgs + c) * nq + queue)
    until one runs past the local items, then from the shared queue (claim c
    is item n_local + c), interleaved across workgroups in a seeded random
    order.  A workgroup runs items while its current one is below total.
    Returns the items each workgroup processed, in order, and n_local."""
    rng = np.random.default_rng(seed)
    young_from = G if young_from is None else young_from
    nq = min(8, G)
    n_local = total - max(0, min(G, total - 2 * G - 16))
    n_static = 1 if one_deep else 2
    local_ctr = [0] * nq
    shared_ctr = [0]
    state = {}
    for b in range(G):
        queue = b % nq
        queue_wgs = (G - queue + nq - 1) // nq
        nxt = total if one_deep else (queue_wgs + b // nq) * nq + queue
        state[b] = dict(cur=b, nxt=nxt, shared=False, done=[], base=n_static * queue_wgs,
                        stop=b >= young_from and young_from >= nq)
    active = [b for b in range(G) if state[b]["cur"] < total]
    while active:
        b = active[int(rng.integers(len(active)))]
        st = state[b]
        st["done"].append(st["cur"])
        if st["stop"]:
            nn = total
        elif not st["shared"]:
            claim = local_ctr[b % nq]
            local_ctr[b % nq] += 1
            nn = (st["base"] + claim) * nq + b % nq
            if nn >= n_local:
                st["shared"] = True
                nn = n_local + shared_ctr[0]
                shared_ctr[0] += 1
        else:
            nn = n_local + shared_ctr[0]
            shared_ctr[0] += 1
        if one_deep:
            st["cur"] = nn
        else:
            st["cur"], st["nxt"] = st["nxt"], nn
        if st["cur"] >= total:
            assert st["nxt"] >= total, "a claimed item dropped"
            active.remove(b)
    return [st["done"] for st in state.values()], n_local


@pytest.mark.parametrize("one_deep", [True, False])
@pytest.mark.parametrize("G", [768, 1024, 512, 96, 7, 13, 1, 800])
@pytest.mark.parametrize("total", [1, 5, 100, 767, 1536, 1551, 1552, 1553, 1600, 2320, 3090,
                                   4096, 20000])
def test_queue_distribution_covers_every_item_once(one_deep, G, total):
    for seed in range(3):
        done, n_local = queue_items(G, total, one_deep, seed)
        taken = [i for d in done for i in d]
        assert len(taken) == len(set(taken)), "an item taken twice"
        assert set(taken) == set(range(total)), "an item never taken"


@pytest.mark.parametrize("G,young_from", [(768, 512), (1024, 768), (96, 64), (7, 4), (13, 0),
                                          (800, 544)])
@pytest.mark.parametrize("total", [1, 100, 767, 1553, 3090, 20000])
def test_young_workgroups_run_only_their_first_item(G, young_from, total):
    """The youngest workgroups (blockIdx.x >= young_from) take no claims
    when every per-XCD queue keeps a workgroup that claims (young_from at
    least the queue count); the others' claims still cover every item
    exactly once."""
    for seed in range(3):
        done, n_local = queue_items(G, total, True, seed, young_from)
        taken = [i for d in done for i in d]
        assert len(taken) == len(set(taken)), "an item taken twice"
        assert set(taken) == set(range(total)), "an item never taken"
        if young_from >= min(8, G):
            for b in range(young_from, G):
                assert done[b] == ([b] if b < total else [])


def test_claims_follow_the_static_items():
    """The per-XCD queues' claims start right after the static items: item
    G onwards one deep, 2 G onwards with a reserve (whose static second
    items are G .. 2 G - 1)."""
    G, total, nq = 768, 3090, 8
    for one_deep, first_claimed in ((True, G), (False, 2 * G)):
        done, n_local = queue_items(G, total, one_deep, seed=5)
        assert n_local == total - G
        assert sorted(d[0] for d in done) == list(range(G))
        if not one_deep:
            assert sorted(d[1] for d in done) == list(range(G, 2 * G))
        n_static = 1 if one_deep else 2
        claimed = sorted(i for d in done for i in d[n_static:] if i < n_local)
        assert claimed[:nq] == list(range(first_claimed, first_claimed + nq))


def group_major(item, lo, hi, Y):
    """Replay of the decode kernel's group-major item order (FP8 caches):
    in super-rows of 8 Y items, position j becomes row group j // 8 of
    (sequence, partition) group j % 8; a last, shorter super-row keeps the
    plain order."""
    span = 8 * Y
    j = item - lo
    sr = j // span
    if lo + (sr + 1) * span > hi:
        return item
    r = j - sr * span
    return lo + sr * span + (r & 7) * Y + (r >> 3)


def _group_major_order(Y, n_full, total):
    fl = Y * n_full
    return [group_major(i, 0, fl, Y) if i < fl else group_major(i, fl, total, Y)
            for i in range(total)]


@pytest.mark.parametrize("Y", [1, 3, 8, 32, 40])
@pytest.mark.parametrize("n_full,n_rag", [(0, 1), (0, 7), (0, 256), (3, 250), (17, 8), (64, 0),
                                          (9, 13)])
def test_group_major_order_is_a_permutation(Y, n_full, n_rag):
    """Every item index maps to exactly one item, full partitions stay full
    partitions (an early first item is decoded before the last partitions
    are counted) and last partitions stay last partitions."""
    total = Y * (n_full + n_rag)
    order = _group_major_order(Y, n_full, total)
    assert sorted(order) == list(range(total))
    fl = Y * n_full
    assert all((i < fl) == (o < fl) for i, o in enumerate(order))


@pytest.mark.parametrize("Y,n_full,n_rag", [(8, 0, 256), (8, 5, 251), (40, 2, 30), (3, 16, 16)])
def test_group_major_queues_take_whole_groups(Y, n_full, n_rag):
    """Under the per-XCD queues (every eighth item), each queue's items of a
    complete super-row are all Y row groups of one (sequence, partition)
    group, so the KV heads of a block meet on one XCD."""
    total = Y * (n_full + n_rag)
    order = _group_major_order(Y, n_full, total)
    for lo, hi in ((0, Y * n_full), (Y * n_full, total)):
        for sr in range((hi - lo) // (8 * Y)):
            base = lo + sr * 8 * Y
            for q in range(8):
                items = [order[i] for i in range(base, base + 8 * Y) if (i - lo) % 8 == q]
                groups = {i // Y for i in items}
                assert len(groups) == 1 and len(items) == Y
                assert sorted(i % Y for i in items) == list(range(Y))
