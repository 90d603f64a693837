"""Pins the oracle's shared blocks: reference counts, fork, copy-on-write,
the prefix cache, and the sequential meaning of queued copies.

Worked cases come from the pages' own descriptions:
* [KV essay] "Paged attention": two sequences can point at one block, and the
  block is duplicated only when one of them writes;
* [KV management]: beams share the prompt's pages until they diverge, and
  only pages holding positions where they differ are copied;
* [KV essay] "Prefix caching": reuse requires the new request to agree with
  the cached tokens from position 0 on (a value that changes at the very
  start, such as a timestamp, leaves nothing reusable, while the same value
  at the end keeps everything before it reusable); reuse covers the positions
  before the first difference, and an entry survives until its space is
  reallocated.
A brute-force test runs random operation sequences against a shadow model
that tracks what every physical slot holds, so a missing or misplaced copy
shows up as a sequence reading something it never wrote.
"""
import random

import numpy as np
import pytest

from oracle.allocator import AllocatorModel, AllocError, BLOCK_TOKENS
from oracle.inject import copy_blocks
from oracle.layout import PoolSpec


class Shadow:
    """What every physical slot holds (a key per slot) next to what every
    sequence believes it wrote; copies and writes are applied in the order
    the allocator's contract gives (queued copies first, then the write)."""

    def __init__(self, model: AllocatorModel):
        self.m = model
        self.slots = [[None] * model.bt for _ in range(model.num_blocks)]
        self.intended = [[] for _ in range(model.max_seqs)]
        self.copies = 0

    def flush(self):
        for src, dst in self.m.take_pending():
            self.slots[dst] = list(self.slots[src])
            self.copies += 1

    def write(self, seq, pos, key):
        b = self.m.tables[seq][pos // self.m.bt]
        self.slots[b][pos % self.m.bt] = key
        it = self.intended[seq]
        while len(it) <= pos:
            it.append(None)
        it[pos] = key

    def check(self):
        self.m.check_invariants()
        for s in range(self.m.max_seqs):
            n = self.m.lens[s]
            assert n == len(self.intended[s]), (s, n, len(self.intended[s]))
            got = [self.slots[self.m.tables[s][p // self.m.bt]][p % self.m.bt]
                   for p in range(n)]
            assert got == self.intended[s], "sequence %d reads what it did not write" % s

    # operations -------------------------------------------------------------
    def extend(self, seqs, keys_per_seq):
        n = len(keys_per_seq[0])
        first = self.m.extend(seqs, n)
        self.flush()
        for s, f, keys in zip(seqs, first, keys_per_seq):
            for i, k in enumerate(keys):
                self.write(s, f + i, k)

    def inject(self, seq, p0, keys):
        self.m.prepare_inject([(seq, len(keys), p0, 0)])
        self.flush()
        for i, k in enumerate(keys):
            self.write(seq, p0 + i, k)

    def fork(self, src, dst):
        self.m.fork(src, dst)
        self.intended[dst] = list(self.intended[src])

    def free(self, seq):
        self.m.free_seq(seq)
        self.intended[seq] = []

    def match(self, seq, keys):
        n = self.m.prefix_match(seq, keys)
        self.intended[seq] = list(keys[:n])
        return n

    def commit(self, seq, n_keys):
        self.m.prefix_commit(seq, self.intended[seq][:n_keys])


def keys_of(tag, n, start=0):
    return [(tag << 32) | (start + i) for i in range(n)]


def test_fork_shares_until_a_write_duplicates_the_block():
    m = AllocatorModel(16, 4, 8)
    sh = Shadow(m)
    sh.extend([0], [keys_of(1, 40)])                 # 3 blocks, last one half full
    a_blocks = list(m.tables[0])
    free_before = len(m.free)
    sh.fork(0, 1)
    assert m.tables[1] == a_blocks and len(m.free) == free_before
    assert [m.ref[b] for b in a_blocks] == [2, 2, 2]
    sh.extend([1], [keys_of(2, 1)])                  # B writes into the shared last block
    assert m.tables[1][:2] == a_blocks[:2] and m.tables[1][2] != a_blocks[2]
    assert m.tables[0] == a_blocks                   # A keeps its blocks
    assert [m.ref[b] for b in a_blocks] == [2, 2, 1] and m.ref[m.tables[1][2]] == 1
    sh.extend([0], [keys_of(3, 1)])                  # A's last block is private now
    assert m.tables[0] == a_blocks and not m.pending
    sh.check()
    sh.free(0)
    assert [m.ref[b] for b in a_blocks] == [1, 1, 0] and list(m.free)[-1] == a_blocks[2]
    sh.check()


def test_beam_search_copies_only_the_divergent_pages():
    beams, prompt = 4, 40
    m = AllocatorModel(32, beams, 8)
    sh = Shadow(m)
    sh.extend([0], [keys_of(9, prompt)])
    for b in range(1, beams):
        sh.fork(0, b)
    copies = []
    for b in range(1, beams):                        # the first token of each beam differs
        sh.extend([b], [keys_of(100 + b, 1)])
        copies.append(len([1 for _ in m.pending]))
    sh.extend([0], [keys_of(100, 1)])
    sh.check()
    used = {x for t in m.tables for x in t}
    full_prompt_blocks = prompt // BLOCK_TOKENS
    assert len(used) == full_prompt_blocks + beams                  # 2 shared + 4 private
    assert len(used) < beams * -(-prompt // BLOCK_TOKENS)           # vs. 12 unshared
    shared = {x for x in used if m.ref[x] == beams}
    assert shared == set(m.tables[0][:full_prompt_blocks])
    for b in range(beams):                                          # beams grow apart
        sh.extend([b], [keys_of(200 + b, 30)])
    assert not m.pending
    sh.check()


def test_prefix_match_needs_an_exact_match_from_position_zero():
    m = AllocatorModel(64, 8, 16)
    sh = Shadow(m)
    prompt = keys_of(5, 100)                          # 6 full blocks + 4 tokens
    sh.extend([0], [prompt])
    sh.commit(0, 100)
    assert len(m.entries) == 6
    assert sh.match(1, prompt) == 96                  # every full block is reused
    assert m.tables[1] == m.tables[0][:6]
    stamped = [0xDEAD] + prompt[1:]                   # differs at position 0
    assert sh.match(2, stamped) == 0 and m.tables[2] == []
    at_end = prompt[:-1] + [0xDEAD]                   # differs only in the partial block
    assert sh.match(3, at_end) == 96
    mid = list(prompt)
    mid[50] = 0xDEAD                                  # first divergence at position 50
    assert sh.match(4, mid) == 48
    sh.check()
    # a sequence that matched continues privately after the shared blocks
    sh.extend([4], [mid[48:]])
    assert m.tables[4][:3] == m.tables[0][:3] and m.tables[4][3] not in m.tables[0]
    sh.check()


def test_cached_entry_survives_until_its_block_is_reallocated():
    m = AllocatorModel(8, 4, 8)
    sh = Shadow(m)
    prompt = keys_of(7, 48)
    sh.extend([0], [prompt])
    sh.commit(0, 48)
    blocks = list(m.tables[0])
    sh.free(0)
    assert list(m.free)[-3:] == blocks and len(m.entries) == 3
    assert sh.match(1, prompt) == 48                  # revived off the free list
    assert m.tables[1] == blocks and all(b not in m.free for b in blocks)
    sh.check()
    sh.free(1)
    sh.extend([2], [keys_of(8, 16 * 5)])              # the other 5 blocks: no eviction yet
    assert len(m.entries) == 3
    sh.extend([2], [keys_of(8, 16, 80)])              # pops the cached block 0
    assert len(m.entries) == 0                        # and everything registered under it
    assert sh.match(3, prompt) == 0
    sh.check()


def test_eviction_of_a_middle_block_drops_its_descendants():
    m = AllocatorModel(6, 4, 8)
    sh = Shadow(m)
    prompt = keys_of(3, 48)
    sh.extend([0], [prompt])
    sh.commit(0, 48)
    b0, b1, b2 = m.tables[0]
    sh.free(0)
    # put b1 at the head of the free list, then take one block
    m.free.remove(b1)
    m.free.appendleft(b1)
    sh.extend([1], [keys_of(4, 1)])
    assert m.tables[1] == [b1]
    assert list(m.entries.values()) == [b0]
    assert sh.match(2, prompt) == 16
    sh.check()


def test_writing_a_cached_block_in_place_unregisters_it():
    m = AllocatorModel(16, 4, 8)
    sh = Shadow(m)
    prompt = keys_of(2, 48)
    sh.extend([0], [prompt])
    sh.commit(0, 48)
    sh.inject(0, 20, keys_of(6, 4))                   # overwrite inside block 1, private
    assert not m.pending and len(m.entries) == 1      # blocks 1 and 2 no longer cached
    assert sh.match(1, prompt) == 16
    sh.check()


def test_inject_into_shared_blocks_copies_each_touched_block_once():
    m = AllocatorModel(16, 4, 8)
    sh = Shadow(m)
    sh.extend([0], [keys_of(1, 64)])
    sh.fork(0, 1)
    a = list(m.tables[0])
    m.prepare_inject([(1, 20, 10, 0), (1, 3, 12, 0)])  # blocks 0 and 1, block 0 twice
    pend = list(m.pending)
    assert [p[0] for p in pend] == [a[0], a[1]]
    sh.flush()
    for i, k in enumerate(keys_of(5, 20)):
        sh.write(1, 10 + i, k)
    assert m.tables[1][2:] == a[2:] and m.tables[0] == a
    sh.check()


def test_inject_by_all_sharers_needs_one_copy_fewer():
    """Two sequences share a block and both write it in one call: the first
    writer takes a copy, the second then owns the block alone and writes in
    place, so one free block covers the call."""
    m = AllocatorModel(3, 2, 4)
    sh = Shadow(m)
    sh.extend([0], [keys_of(1, 20)])                   # blocks a, b; one block left
    sh.fork(0, 1)
    a = list(m.tables[0])
    m.prepare_inject([(0, 2, 3, 0), (1, 2, 5, 0)])
    assert m.pending == [(a[0], m.tables[0][0])] and m.tables[1][0] == a[0]
    sh.flush()
    for p in (3, 4):
        sh.write(0, p, 0xA0 + p)
    for p in (5, 6):
        sh.write(1, p, 0xB0 + p)
    sh.check()


def test_extend_by_all_sharers_needs_one_copy_fewer():
    m = AllocatorModel(3, 2, 4)
    sh = Shadow(m)
    sh.extend([0], [keys_of(1, 20)])                   # blocks a, b; one block left
    sh.fork(0, 1)
    sh.extend([0, 1], [keys_of(2, 1), keys_of(3, 1)])  # seq 0 copies b, seq 1 keeps it
    assert sh.copies == 1 and not m.free
    sh.check()


@pytest.mark.parametrize("length,n_new", [(32, 1), (30, 5), (48, 20)])
def test_extend_copies_reserved_blocks_a_fork_shares(length, n_new):
    """A fork shares every block of the table, reserved blocks past the
    length included.  When both sharers then extend, every shared block that
    receives new positions is copied for the first of them, so that after
    the extend each sequence writes only blocks it alone names ([KV essay]
    "Paged attention": a shared block is duplicated before a write)."""
    m = AllocatorModel(16, 4, 8)
    m.set_blocks(0, [3, 5, 7, 9], length)
    m.fork(0, 1)
    m.extend([0, 1], n_new)
    touched = range(length // 16, -(-(length + n_new) // 16))
    for i in touched:
        assert m.tables[0][i] != m.tables[1][i], (i, m.tables)
        assert m.ref[m.tables[0][i]] == 1 and m.ref[m.tables[1][i]] == 1, (i, m.ref)
    # only the touched blocks that existed were copied, oldest first, all by seq 0
    existing = [i for i in touched if i < 4]
    assert [src for src, _ in m.pending] == [[3, 5, 7, 9][i] for i in existing]
    for i in range(length // 16):               # untouched blocks stay shared
        assert m.tables[0][i] == m.tables[1][i] and m.ref[m.tables[0][i]] == 2


def test_extend_shared_reserved_block_needs_a_free_block_or_fails_whole():
    """The copies of reserved shared blocks count toward the all-or-nothing
    reservation: with no free block left, the extend fails and changes
    nothing."""
    m = AllocatorModel(4, 2, 4)
    m.set_blocks(0, [0, 1, 2, 3], 32)
    m.fork(0, 1)
    before = ([list(t) for t in m.tables], list(m.lens), list(m.ref))
    with pytest.raises(AllocError) as e:
        m.extend([0], 1)
    assert e.value.code == "OOM"
    assert ([list(t) for t in m.tables], list(m.lens), list(m.ref)) == before


def test_errors_leave_the_state_unchanged():
    m = AllocatorModel(4, 3, 4)
    m.extend([0], 40)
    with pytest.raises(AllocError) as e:
        m.fork(0, 0)
    assert e.value.code == "INVALID"
    m.fork(0, 1)
    with pytest.raises(AllocError) as e:
        m.fork(0, 1)                                   # destination not empty
    assert e.value.code == "INVALID"
    with pytest.raises(AllocError) as e:
        m.prefix_match(0, keys_of(1, 16))              # not an empty sequence
    assert e.value.code == "INVALID"
    snap = (list(m.free), [list(t) for t in m.tables], list(m.lens), list(m.ref))
    # one free block left; two beams each need a copy of the shared partial block
    m.fork(0, 2)
    snap = (list(m.free), [list(t) for t in m.tables], list(m.lens), list(m.ref))
    with pytest.raises(AllocError) as e:
        m.extend([1, 2], 1)
    assert e.value.code == "OOM"
    assert snap == (list(m.free), [list(t) for t in m.tables], list(m.lens), list(m.ref))
    with pytest.raises(AllocError) as e:
        m.prefix_commit(0, keys_of(1, 41))             # more keys than tokens
    assert e.value.code == "RANGE"
    m.check_invariants()


def test_commit_rejects_keys_that_contradict_a_registered_block():
    m = AllocatorModel(8, 3, 4)
    sh = Shadow(m)
    sh.extend([0], [keys_of(1, 32)])
    sh.commit(0, 32)
    assert sh.match(1, keys_of(1, 32)) == 32
    with pytest.raises(AllocError) as e:
        m.prefix_commit(1, keys_of(2, 32))             # these blocks cache other keys
    assert e.value.code == "INVALID"
    sh.check()


def test_duplicate_content_chains_off_the_registered_block():
    m = AllocatorModel(16, 3, 8)
    sh = Shadow(m)
    p = keys_of(1, 48)
    sh.extend([0], [p])
    sh.extend([1], [p])                                # same content, own blocks
    sh.commit(0, 32)
    sh.commit(1, 48)                                   # blocks 0, 1 already cached by seq 0
    assert len(m.entries) == 3
    assert sh.match(2, p) == 48
    assert m.tables[2][:2] == m.tables[0][:2] and m.tables[2][2] == m.tables[1][2]
    sh.check()


def test_queued_copies_act_one_after_another():
    """copy_blocks carries out the queue in order: a chain x->y, y->z leaves
    x's contents in z; a later copy into a block read earlier does not
    disturb the earlier read."""
    spec = PoolSpec(2, 5, 2, 64, "bf16").resolved()
    rng = np.random.default_rng(1)
    k = rng.integers(0, 2 ** 16, size=spec.elements(), dtype=np.uint16)
    v = rng.integers(0, 2 ** 16, size=spec.elements(), dtype=np.uint16)
    plane = BLOCK_TOKENS * 64

    def block(arr, b):
        return np.stack([arr[spec.plane_base(l, b, h):spec.plane_base(l, b, h) + plane]
                         for l in range(2) for h in range(2)])

    k0 = [block(k, b) for b in range(5)]
    v0 = [block(v, b) for b in range(5)]
    copy_blocks(k, v, spec, [(0, 1), (1, 2), (3, 0)])
    assert np.array_equal(block(k, 1), k0[0]) and np.array_equal(block(v, 1), v0[0])
    assert np.array_equal(block(k, 2), k0[0]) and np.array_equal(block(v, 2), v0[0])
    assert np.array_equal(block(k, 0), k0[3]) and np.array_equal(block(v, 0), v0[3])
    assert np.array_equal(block(k, 4), k0[4]) and np.array_equal(block(k, 3), k0[3])


@pytest.mark.parametrize("bt", [16, 32])
def test_brute_force_random_operations_against_slot_contents(bt):
    rng = random.Random(2024 + bt)
    hits = copies = reserved = 0
    for trial in range(600):
        nb, ns = rng.choice([(6, 3), (10, 4), (24, 5)])
        m = AllocatorModel(nb, ns, 6, seed=rng.choice([0, 7, 99]), block_tokens=bt)
        sh = Shadow(m)
        committed = []                                # key lists registered so far
        tag = 0
        for _ in range(30):
            tag += 1
            op = rng.choice(["extend", "extend", "fork", "free", "inject", "match", "match",
                             "commit", "commit", "reserve"])
            s = rng.randrange(ns)
            try:
                if op == "extend":
                    seqs = rng.sample(range(ns), rng.randint(1, 2))
                    n = rng.choice([1, 3, 16, 17, 32, 33])
                    sh.extend(seqs, [keys_of(tag * 8 + i, n) for i in range(len(seqs))])
                elif op == "fork":
                    sh.fork(s, rng.randrange(ns))
                elif op == "reserve":
                    # capacity beyond the length: a later fork shares these
                    # blocks before anything is written to them
                    m.alloc_blocks(s, m.lens[s] + rng.choice([1, 16, 40]))
                    reserved += 1
                elif op == "free":
                    sh.free(s)
                elif op == "inject" and m.lens[s] > 0:
                    p0 = rng.randrange(m.lens[s])
                    sh.inject(s, p0, keys_of(tag, rng.randint(1, m.lens[s] - p0)))
                elif op == "match":
                    pool = committed + [list(sh.intended[rng.randrange(ns)])]
                    keys = list(rng.choice(pool))
                    if keys and rng.random() < 0.3:
                        keys[rng.randrange(len(keys))] = 0xBAD
                    before = len(m.pending)
                    hits += sh.match(s, keys + keys_of(tag, rng.randint(0, 20))) > 0
                    assert len(m.pending) == before
                elif op == "commit" and m.lens[s] > 0:
                    n = rng.randint(bt, max(bt, m.lens[s])) if m.lens[s] >= bt else m.lens[s]
                    sh.commit(s, n)
                    committed.append(list(sh.intended[s][:n]))
            except AllocError:
                pass
            sh.check()
        copies += sh.copies
    assert hits > 60 and copies > 150 and reserved > 500, (hits, copies, reserved)
