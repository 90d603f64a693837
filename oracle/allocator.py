"""Host block allocator model (oracle; test infrastructure only).

[KV essay] "Paged attention" gives the structure: a shared pool of fixed
blocks, a free list, a per-sequence block table, and a new block handed out
only when a sequence reaches it (so only the last block is partly empty).
[Inside engines] "PagedAttention" likewise allocates a further block only
once the sequence has filled the 16 tokens of its last one; "Continuous Batching" returns a finished
sequence's blocks to the pool at once.

The pages print a free list but not the order in which it is consumed.  The
reading taken, which makes the expected table unique:

* the free list is a FIFO: blocks are taken from its head and returned to its
  tail, a freed sequence's blocks in table order;
* its initial order is ascending block ids, or -- for a non-zero seed -- the
  Fisher-Yates shuffle (from the last index down, j = next() mod (i+1)) driven
  by the splitmix64 generator (Vigna's published definition) started at
  that seed;
* a reservation is all-or-nothing: when the pool cannot cover it, nothing
  changes.

Shared blocks ([KV essay] "Paged attention" and "Prefix caching"; [KV
management] on beam search, parallel sampling and prefix caching; [Inside
engines] "Zero-Copy Page Sharing"): a block is an object that several
sequences may name; it is duplicated only when one of them writes into it,
and the engine hashes prefixes to find blocks it can reuse, which requires an
exact match from position 0.  Readings taken:

* every block has a reference count, the number of table entries naming it;
  it is on the free list exactly when the count is 0; freeing a sequence
  decrements its blocks in table order and appends those reaching 0 to the
  free list's tail;
* ``fork(src, dst)`` gives an empty sequence the table and length of another
  (every block's count + 1), as beams and parallel samples share a prompt;
* copy-on-write: before positions of a block whose count exceeds 1 are
  written (by ``extend`` for every block already in the table that holds one
  of the new positions -- reserved blocks past the length included, since a
  fork shares them too -- or by an inject), the writer
  takes a fresh block from the free list's head, the pair (old, new) is
  queued, the writer's table entry is replaced and the old block's count
  drops by one; queued copies take effect, in queue order, before any write;
  within one call the blocks are handled in order of first touch;
* prefix cache: the caller names what each position holds by a 64-bit key
  (a token id for a prompt, the store row for injected memory); a full block
  is registered under (the block registered for the preceding block or -1,
  its keys, one per position), compared exactly; ``prefix_match`` shares, for an empty
  sequence, the longest chain of registered blocks from position 0 (taking a
  block back off the free list when its count was 0); ``prefix_commit``
  registers a sequence's full blocks; an entry lasts until its block is
  handed out again by the free list or written in place, and then goes
  together with every entry registered under it.

Sliding window ([KV essay] "Capping the window instead of shrinking the
rows": attention is limited to a trailing span of W positions, so entries
older than that span can be discarded and the cache's size is bounded by W
rather than by the conversation): ``trim_window``
drops a sequence's references to the blocks that lie wholly before its last
W positions (table order), leaving -1 in their table entries; positions and
capacity keep counting from 0.

Block size ([Inside engines] "PagedAttention": blocks of e.g. 16 or 32
tokens): the model takes 16 or 32 tokens per block.  Reading: a 32-token
block b is the pair of adjacent 16-token planes 2b and 2b+1 of the pool;
allocation, sharing, copy-on-write, prefix entries and trimming work in
32-token blocks, and ``expand_table`` gives the table of 16-token planes that
readers and writers go through.
"""

from collections import deque

BLOCK_TOKENS = 16
_MASK = (1 << 64) - 1


class AllocError(Exception):
    """Raised with ``code`` in {'INVALID', 'OOM', 'RANGE'} and no state change."""

    def __init__(self, code: str, msg: str):
        super().__init__("%s: %s" % (code, msg))
        self.code = code


def splitmix64(seed: int):
    """Yield the splitmix64 sequence for ``seed`` (64-bit unsigned ints)."""
    state = seed & _MASK
    while True:
        state = (state + 0x9E3779B97F4A7C15) & _MASK
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK
        yield z ^ (z >> 31)


def initial_free_order(num_blocks: int, seed: int) -> list:
    """Initial free-list order: ascending, or a seeded Fisher-Yates shuffle."""
    order = list(range(num_blocks))
    if seed == 0:
        return order
    gen = splitmix64(seed)
    for i in range(num_blocks - 1, 0, -1):
        j = next(gen) % (i + 1)
        order[i], order[j] = order[j], order[i]
    return order


def blocks_for(n_tokens: int, block_tokens: int = BLOCK_TOKENS) -> int:
    """Blocks needed to hold ``n_tokens`` positions."""
    return -(-int(n_tokens) // block_tokens)


def expand_table(row, block_tokens: int = BLOCK_TOKENS):
    """A table row of ``block_tokens``-token blocks as the row of 16-token
    planes: block b covers planes b*k .. b*k + k-1, k = block_tokens / 16
    (-1 entries stay -1)."""
    k = block_tokens // BLOCK_TOKENS
    return [int(b) * k + i if b >= 0 else -1 for b in row for i in range(k)]


def expand_pairs(pairs, block_tokens: int = BLOCK_TOKENS):
    """Queued block copies as copies of 16-token planes, in order."""
    k = block_tokens // BLOCK_TOKENS
    return [(s * k + i, d * k + i) for (s, d) in pairs for i in range(k)]


class AllocatorModel:
    """Free list, per-sequence block lists and lengths."""

    def __init__(self, num_blocks: int, max_seqs: int, max_blocks_per_seq: int, seed: int = 0,
                 block_tokens: int = BLOCK_TOKENS):
        if num_blocks <= 0 or max_seqs <= 0 or max_blocks_per_seq <= 0:
            raise AllocError("INVALID", "sizes must be positive")
        if block_tokens not in (16, 32):
            raise AllocError("INVALID", "block size must be 16 or 32 tokens")
        self.bt = block_tokens
        self.num_blocks = num_blocks
        self.max_seqs = max_seqs
        self.max_blocks_per_seq = max_blocks_per_seq
        self.free = deque(initial_free_order(num_blocks, seed))
        self.tables = [[] for _ in range(max_seqs)]
        self.lens = [0] * max_seqs
        self.ref = [0] * num_blocks
        self.pending = []          # queued copies (src, dst), in order
        self.entries = {}          # (parent block or -1, a block's keys) -> block
        self.entry_of = {}         # block -> its (parent, keys)
        self.children = {}         # block -> blocks registered under it

    # -- queries -------------------------------------------------------------
    def _check_seq(self, seq: int):
        if not (0 <= seq < self.max_seqs):
            raise AllocError("INVALID", "sequence %d out of range" % seq)

    def capacity(self, seq: int) -> int:
        self._check_seq(seq)
        return len(self.tables[seq]) * self.bt

    def block_table(self, seqs):
        """Rows padded with -1 to ``max_blocks_per_seq``, and the lengths."""
        rows, lens = [], []
        for s in seqs:
            self._check_seq(s)
            t = self.tables[s]
            rows.append(t + [-1] * (self.max_blocks_per_seq - len(t)))
            lens.append(self.lens[s])
        return rows, lens

    # -- mutations -----------------------------------------------------------
    def alloc_blocks(self, seq: int, n_tokens: int):
        """Grow ``seq`` until it can hold ``n_tokens`` positions."""
        self._check_seq(seq)
        if n_tokens < 0:
            raise AllocError("INVALID", "negative token count")
        want = blocks_for(n_tokens, self.bt)
        if want > self.max_blocks_per_seq:
            raise AllocError("RANGE", "more blocks than a table row holds")
        need = max(0, want - len(self.tables[seq]))
        if need > len(self.free):
            raise AllocError("OOM", "pool exhausted")
        for _ in range(need):
            self.tables[seq].append(self._pop())

    def set_blocks(self, seq: int, ids, length: int):
        """Give an empty sequence an explicit table (ids must all be free)."""
        self._check_seq(seq)
        ids = [int(i) for i in ids]
        if self.tables[seq]:
            raise AllocError("INVALID", "sequence already owns blocks")
        if len(ids) > self.max_blocks_per_seq:
            raise AllocError("RANGE", "more blocks than a table row holds")
        if len(set(ids)) != len(ids):
            raise AllocError("INVALID", "duplicate block id")
        free_set = set(self.free)
        if any(i not in free_set for i in ids):
            raise AllocError("INVALID", "block id not free")
        if not (0 <= length <= len(ids) * self.bt):
            raise AllocError("RANGE", "length exceeds the given blocks")
        taken = set(ids)
        self.free = deque(b for b in self.free if b not in taken)
        for b in ids:
            self._forget(b)
            self.ref[b] = 1
        self.tables[seq] = ids
        self.lens[seq] = int(length)

    def extend(self, seqs, n_new: int):
        """Append ``n_new`` positions to every sequence, all-or-nothing.

        Returns each sequence's first new position (its old length).
        """
        seqs = list(seqs)
        for s in seqs:
            self._check_seq(s)
        if len(set(seqs)) != len(seqs) or n_new < 0:
            raise AllocError("INVALID", "repeated sequence or negative count")
        total, refs = 0, {}
        for s in seqs:
            want = blocks_for(self.lens[s] + n_new, self.bt)
            if want > self.max_blocks_per_seq:
                raise AllocError("RANGE", "more blocks than a table row holds")
            total += max(0, want - len(self.tables[s]))
            for i in self._written_entries(s, n_new):
                b = self.tables[s][i]
                r = refs.get(b, self.ref[b])     # count as it will be when s is reached
                if r > 1:
                    total += 1
                    refs[b] = r - 1
        if total > len(self.free):
            raise AllocError("OOM", "pool exhausted")
        first = []
        for s in seqs:
            for i in self._written_entries(s, n_new):
                if self.ref[self.tables[s][i]] > 1:
                    self._cow(s, i)
            self.alloc_blocks(s, self.lens[s] + n_new)
            first.append(self.lens[s])
            self.lens[s] += n_new
        return first

    def _written_entries(self, s: int, n_new: int):
        """Table indices of the blocks ``s`` already holds that will receive
        some of its next ``n_new`` positions: the block holding position len
        (if the length is inside it) and any reserved blocks beyond it.  A
        fork shares reserved blocks as well, so each of them may need a copy
        before the write."""
        if n_new <= 0:
            return range(0)
        t = self.tables[s]
        lo = self.lens[s] // self.bt
        hi = min(len(t), blocks_for(self.lens[s] + n_new, self.bt))
        return [i for i in range(lo, hi) if t[i] >= 0]

    def set_len(self, seq: int, length: int):
        self._check_seq(seq)
        if not (0 <= length <= self.capacity(seq)):
            raise AllocError("RANGE", "length beyond reserved capacity")
        self.lens[seq] = int(length)

    def free_seq(self, seq: int):
        """Drop a sequence's references; blocks no longer named by any table
        go to the tail of the free list, in table order."""
        self._check_seq(seq)
        for b in self.tables[seq]:
            if b < 0:                  # dropped by a window trim
                continue
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        self.tables[seq] = []
        self.lens[seq] = 0

    def trim_window(self, seqs, window: int):
        """Release, for each sequence, the blocks wholly before its last
        ``window`` positions; returns the number of table entries dropped."""
        seqs = list(seqs)
        for s in seqs:
            self._check_seq(s)
        if window <= 0:
            raise AllocError("INVALID", "window must be positive")
        dropped = 0
        for s in seqs:
            keep_from = max(0, self.lens[s] - window) // self.bt
            t = self.tables[s]
            for i in range(min(keep_from, len(t))):
                b = t[i]
                if b < 0:
                    continue
                self.ref[b] -= 1
                if self.ref[b] == 0:
                    self.free.append(b)
                t[i] = -1
                dropped += 1
        return dropped

    # -- sharing ---------------------------------------------------------------
    def _pop(self) -> int:
        """Hand out the free list's head (forgetting what it cached)."""
        b = self.free.popleft()
        self._forget(b)
        self.ref[b] = 1
        return b

    def _forget(self, b: int):
        """Drop the prefix entry of ``b`` and every entry registered under it."""
        stack = [b]
        while stack:
            x = stack.pop()
            key = self.entry_of.pop(x, None)
            if key is not None:
                del self.entries[key]
                if key[0] >= 0:
                    self.children.get(key[0], set()).discard(x)
            stack.extend(sorted(self.children.pop(x, ())))

    def _cow(self, seq: int, idx: int):
        """Give ``seq`` a private copy of its ``idx``-th block."""
        old = self.tables[seq][idx]
        new = self._pop()
        self.pending.append((old, new))
        self.tables[seq][idx] = new
        self.ref[old] -= 1

    def fork(self, src: int, dst: int):
        """``dst`` (empty) shares every block of ``src``, with its length."""
        self._check_seq(src)
        self._check_seq(dst)
        if src == dst or self.tables[dst] or self.lens[dst]:
            raise AllocError("INVALID", "fork needs a distinct, empty destination")
        for b in self.tables[src]:
            if b >= 0:
                self.ref[b] += 1
        self.tables[dst] = list(self.tables[src])
        self.lens[dst] = self.lens[src]

    def prepare_inject(self, runs):
        """Copy-on-write for the destination blocks of an inject call.

        ``runs`` are (seq, n, dst_pos, src_token); every destination must lie
        inside the sequence's blocks (checked by the inject itself).  Blocks
        are handled in order of first touch (runs in order, positions
        ascending): a shared block is copied, a cached private block loses its
        prefix entry.  All-or-nothing on OOM.
        """
        order, seen = [], set()
        for (seq, n, p0, _) in runs:
            self._check_seq(seq)
            for p in range(int(p0), int(p0) + int(n)):
                key = (int(seq), p // self.bt)
                if key not in seen:
                    seen.add(key)
                    order.append(key)
        for (seq, idx) in order:
            if idx >= len(self.tables[seq]) or self.tables[seq][idx] < 0:
                raise AllocError("RANGE", "destination beyond the reserved blocks")
        need, refs = 0, {}
        for (seq, idx) in order:          # counts as they will be when each block is reached
            b = self.tables[seq][idx]
            r = refs.get(b, self.ref[b])
            if r > 1:
                need += 1
                refs[b] = r - 1
        if need > len(self.free):
            raise AllocError("OOM", "pool exhausted")
        for (seq, idx) in order:
            b = self.tables[seq][idx]
            if self.ref[b] > 1:
                self._cow(seq, idx)
            else:
                self._forget(b)

    def take_pending(self):
        """The queued copies, in order; the queue is emptied."""
        out, self.pending = self.pending, []
        return out

    # -- prefix cache ------------------------------------------------------------
    def _block_keys(self, keys, i):
        return tuple(int(k) & _MASK for k in keys[i * self.bt:(i + 1) * self.bt])

    def prefix_match(self, seq: int, keys) -> int:
        """Share the longest registered chain matching ``keys`` from position 0
        with the empty sequence ``seq``; returns the matched token count."""
        self._check_seq(seq)
        if self.tables[seq] or self.lens[seq]:
            raise AllocError("INVALID", "prefix match needs an empty sequence")
        full = min(len(keys) // self.bt, self.max_blocks_per_seq)
        parent = -1
        for i in range(full):
            b = self.entries.get((parent, self._block_keys(keys, i)))
            if b is None:
                break
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1
            self.tables[seq].append(b)
            parent = b
        self.lens[seq] = len(self.tables[seq]) * self.bt
        return self.lens[seq]

    def prefix_commit(self, seq: int, keys):
        """Register the full blocks of ``seq`` covered by ``keys``."""
        self._check_seq(seq)
        if len(keys) > self.lens[seq]:
            raise AllocError("RANGE", "more keys than the sequence holds")
        full = len(keys) // self.bt
        if any(b < 0 for b in self.tables[seq][:full]):
            raise AllocError("RANGE", "keys cover positions the sequence no longer holds")
        plan, parent = [], -1
        for i in range(full):
            b = self.tables[seq][i]
            key = (parent, self._block_keys(keys, i))
            have = self.entries.get(key)
            if have is not None:
                parent = have
                continue
            if b in self.entry_of:
                raise AllocError("INVALID", "block %d already caches other content" % b)
            plan.append((key, b))
            parent = b
        for key, b in plan:
            self.entries[key] = b
            self.entry_of[b] = key
            if key[0] >= 0:
                self.children.setdefault(key[0], set()).add(b)

    # -- invariants ------------------------------------------------------------
    def check_invariants(self):
        count = [0] * self.num_blocks
        for t in self.tables:
            live = [b for b in t if b >= 0]
            assert len(live) == len(set(live)), "a table names a block twice"
            for b in live:
                count[b] += 1
        assert count == self.ref, "reference counts disagree with the tables"
        free = list(self.free)
        assert len(free) == len(set(free)), "a block is free twice"
        assert set(free) == {b for b in range(self.num_blocks) if self.ref[b] == 0}, \
            "free list differs from the unreferenced blocks"
        for s, t in enumerate(self.tables):
            assert self.lens[s] <= len(t) * self.bt
        assert len(self.entries) == len(self.entry_of)
        for key, b in self.entries.items():
            assert self.entry_of[b] == key
            if key[0] >= 0:
                assert b in self.children.get(key[0], set())
                assert key[0] in self.entry_of, "an entry's parent is not registered"
