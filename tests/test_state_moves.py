"""Host side of the prefix-cache state protocol (no GPU): checkpoint-aligned chunking and slot ownership
under the three state moves, through the C ABI.

The ownership test drives a seeded random walk of requests (open with or without a restore, snapshot,
donate, close, tree eviction) and replays the returned copies, in order, on a model of the pool whose
slots hold version labels (the stream order the moves are enqueued in). It checks the race rules the
protocol exists for: a restore copies the tree's checkpoint as it was donated, no copy ever writes a slot
the tree owns or another request holds, a snapshot holds the working state of its moment, every slot
has one owner, and a failed call (no free slot) changes nothing."""
import random

import pytest

import linear_attention_recurrence_amd as kda


def test_chunk_split_cuts_at_checkpoints():
    # a 1,000-token extend from an empty state with a 300-token budget: three checkpoints, then the rest
    assert kda.kda_chunk_split(0, 1000, 300) == [256, 256, 256, 232]
    # from a restored prefix of 100 tokens the first chunk runs to the next checkpoint
    assert kda.kda_chunk_split(100, 1000, 300) == [156, 256, 256, 256, 76]
    assert kda.kda_chunk_split(0, 200, 300) == [200]          # fits: one chunk, no cut
    assert kda.kda_chunk_split(512, 0, 300) == []
    assert kda.kda_chunk_split(0, 1024, 1024) == [1024]       # the last chunk is never cut
    assert kda.kda_chunk_split(0, 1025, 1024) == [1024, 1]
    # a budget below the checkpoint spacing: full budgets, cut only where a checkpoint falls inside
    assert kda.kda_chunk_split(5, 700, 100) == [100, 100, 51, 100, 100, 56, 100, 93]


@pytest.mark.parametrize("seed", range(3))
def test_chunk_split_rule(seed):
    rng = random.Random(seed)
    for _ in range(400):
        pos0, length = rng.randrange(0, 3000), rng.randrange(0, 5000)
        budget, align = rng.choice([1, 7, 64, 255, 256, 300, 1000, 4096]), rng.choice([1, 32, 256])
        lens = kda.kda_chunk_split(pos0, length, budget, align)
        assert sum(lens) == length and all(1 <= c <= budget for c in lens)
        pos = pos0
        for i, c in enumerate(lens):
            last = i == len(lens) - 1
            if not last:
                boundary = (pos + budget) // align * align  # the last checkpoint within the budget
                assert c == (boundary - pos if boundary > pos else budget)
            else:
                assert pos + c == pos0 + length
            pos += c


def test_chunk_split_rejects():
    for args in [(-1, 10, 4, 1), (0, -1, 4, 1), (0, 10, 0, 1), (0, 10, 4, 0)]:
        with pytest.raises(kda.KdaError) as e:
            kda.kda_chunk_split(*args)
        assert e.value.status == kda.KDA_ERR_INVALID_ARG


@pytest.mark.parametrize("seed", range(6))
def test_slot_ownership_random_walk(seed):
    rng = random.Random(100 + seed)
    n_slots = rng.choice([3, 4, 6, 10])
    pool = kda.SlotPool(n_slots)
    content = {s: ("init", s) for s in range(n_slots)}  # model of the device pool: a version label per slot
    tree = {}            # slot -> the label donated into it
    reqs = []            # open requests: (RequestSlots, [current working label])
    version = [0]

    def fresh():
        version[0] += 1
        return ("v", version[0])

    def owners():
        return [pool.owner(s) for s in range(n_slots)]

    def apply(mv, writable):
        src, dst = mv
        assert dst in writable, "a copy wrote a slot outside the caller's fresh or working slots"
        assert pool.owner(dst) != kda.KDA_SLOT_TREE, "a copy wrote a slot the tree owns"
        content[dst] = content[src]

    for _ in range(300):
        before = owners()
        ev = rng.choice(["open", "open_cached", "snapshot", "snapshot", "forward", "donate", "close", "release"])
        try:
            if ev in ("open", "open_cached"):
                cached = rng.choice(sorted(tree)) if (ev == "open_cached" and tree) else -1
                free_before = {s for s, o in enumerate(before) if o == kda.KDA_SLOT_FREE}
                r, moves = pool.open(cached)
                assert r.working in free_before and r.snap == -1
                if cached != -1:
                    assert moves == [(cached, r.working)]
                    apply(moves[0], {r.working})
                    assert content[r.working] == tree[cached]     # the restore sees the checkpoint as donated
                else:
                    assert moves == []
                    content[r.working] = fresh()                   # a fresh state, written by the first forward
                reqs.append(r)
            elif ev == "forward" and reqs:
                r = rng.choice(reqs)
                content[r.working] = fresh()                       # a forward overwrites the working slot in place
            elif ev == "snapshot" and reqs:
                r = rng.choice(reqs)
                free_before = {s for s, o in enumerate(before) if o == kda.KDA_SLOT_FREE}
                old = r.snap
                mv = pool.snapshot(r)
                assert mv[0] == r.working and mv[1] in free_before and r.snap == mv[1]
                apply(mv, {mv[1]})
                if old != -1:
                    assert pool.owner(old) == kda.KDA_SLOT_FREE    # the superseded snapshot is freed
            elif ev == "donate" and reqs:
                r = rng.choice(reqs)
                if r.snap == -1:
                    with pytest.raises(kda.KdaError):
                        pool.donate(r)
                else:
                    snap = r.snap
                    d = pool.donate(r)
                    assert d == snap and r.snap == -1 and pool.owner(d) == kda.KDA_SLOT_TREE
                    tree[d] = content[d]
            elif ev == "close" and reqs:
                r = reqs.pop(rng.randrange(len(reqs)))
                held = [s for s in (r.working, r.snap) if s != -1]
                pool.close(r)
                assert all(pool.owner(s) == kda.KDA_SLOT_FREE for s in held)
                with pytest.raises(kda.KdaError):
                    pool.close(r)                                   # closed twice
            elif ev == "release" and tree:
                s = rng.choice(sorted(tree))
                pool.release(s)
                del tree[s]
        except kda.KdaError as e:
            assert e.status == kda.KDA_ERR_NO_SLOT, e
            assert owners() == before, "a call that found no free slot changed an owner"
        # invariants after every event
        own = owners()
        assert pool.free_count() == sum(o == kda.KDA_SLOT_FREE for o in own)
        assert {s for s, o in enumerate(own) if o == kda.KDA_SLOT_TREE} == set(tree)
        for s in tree:
            assert content[s] == tree[s], "a tree checkpoint changed while the tree owned it"
        held = {}
        for r in reqs:
            mine = [s for s in (r.working, r.snap) if s != -1]
            assert len(mine) <= 2 and all(own[s] == r.id for s in mine)
            for s in mine:
                assert s not in held
                held[s] = r.id
        assert sum(o >= 0 for o in own) == len(held)
    for r in reqs:
        pool.close(r)
    for s in list(tree):
        pool.release(s)
    assert pool.free_count() == n_slots


def test_slot_rules_reject():
    pool = kda.SlotPool(4)
    with pytest.raises(kda.KdaError):
        pool.open(2)                       # a restore reads only a slot the tree owns
    r, _ = pool.open()
    with pytest.raises(kda.KdaError):
        pool.donate(r)                     # nothing to donate yet
    with pytest.raises(kda.KdaError):
        pool.release(r.working)            # the tree does not own a working slot
    pool.snapshot(r)
    d = pool.donate(r)
    with pytest.raises(kda.KdaError):
        pool.open(r.working)               # not a tree slot
    other = kda.SlotPool(4)
    with pytest.raises(kda.KdaError):
        other.snapshot(r)                  # a request of another pool (ids and slots unknown there)
    r2, mv = pool.open(d)
    assert mv == [(d, r2.working)]
    # fill the pool: the next open finds no slot and changes nothing
    r3, _ = pool.open()
    assert pool.free_count() == 0
    with pytest.raises(kda.KdaError) as e:
        pool.open()
    assert e.value.status == kda.KDA_ERR_NO_SLOT
    with pytest.raises(kda.KdaError) as e:
        pool.snapshot(r3)
    assert e.value.status == kda.KDA_ERR_NO_SLOT and r3.snap == -1
    for q in (r, r2, r3):
        pool.close(q)
    pool.release(d)
    assert pool.free_count() == 4
