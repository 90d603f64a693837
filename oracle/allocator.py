"""Host block allocator model (oracle; test infrastructure only).

[KV essay] "Paged attention" gives the structure: a shared pool of fixed
blocks, a free list, a per-sequence block table, and a new block handed out
only when a sequence reaches it (so only the last block is partly empty).
[Inside engines] "PagedAttention" repeats on-demand allocation when the
current 16-token block fills; "Continuous Batching" returns a finished
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


def blocks_for(n_tokens: int) -> int:
    """Blocks needed to hold ``n_tokens`` positions."""
    return -(-int(n_tokens) // BLOCK_TOKENS)


class AllocatorModel:
    """Free list, per-sequence block lists and lengths."""

    def __init__(self, num_blocks: int, max_seqs: int, max_blocks_per_seq: int, seed: int = 0):
        if num_blocks <= 0 or max_seqs <= 0 or max_blocks_per_seq <= 0:
            raise AllocError("INVALID", "sizes must be positive")
        self.num_blocks = num_blocks
        self.max_seqs = max_seqs
        self.max_blocks_per_seq = max_blocks_per_seq
        self.free = deque(initial_free_order(num_blocks, seed))
        self.tables = [[] for _ in range(max_seqs)]
        self.lens = [0] * max_seqs

    # -- queries -------------------------------------------------------------
    def _check_seq(self, seq: int):
        if not (0 <= seq < self.max_seqs):
            raise AllocError("INVALID", "sequence %d out of range" % seq)

    def capacity(self, seq: int) -> int:
        self._check_seq(seq)
        return len(self.tables[seq]) * BLOCK_TOKENS

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
        want = blocks_for(n_tokens)
        if want > self.max_blocks_per_seq:
            raise AllocError("RANGE", "more blocks than a table row holds")
        need = max(0, want - len(self.tables[seq]))
        if need > len(self.free):
            raise AllocError("OOM", "pool exhausted")
        for _ in range(need):
            self.tables[seq].append(self.free.popleft())

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
        if not (0 <= length <= len(ids) * BLOCK_TOKENS):
            raise AllocError("RANGE", "length exceeds the given blocks")
        taken = set(ids)
        self.free = deque(b for b in self.free if b not in taken)
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
        total = 0
        for s in seqs:
            want = blocks_for(self.lens[s] + n_new)
            if want > self.max_blocks_per_seq:
                raise AllocError("RANGE", "more blocks than a table row holds")
            total += max(0, want - len(self.tables[s]))
        if total > len(self.free):
            raise AllocError("OOM", "pool exhausted")
        first = []
        for s in seqs:
            self.alloc_blocks(s, self.lens[s] + n_new)
            first.append(self.lens[s])
            self.lens[s] += n_new
        return first

    def set_len(self, seq: int, length: int):
        self._check_seq(seq)
        if not (0 <= length <= self.capacity(seq)):
            raise AllocError("RANGE", "length beyond reserved capacity")
        self.lens[seq] = int(length)

    def free_seq(self, seq: int):
        """Return a sequence's blocks to the tail of the free list, in order."""
        self._check_seq(seq)
        self.free.extend(self.tables[seq])
        self.tables[seq] = []
        self.lens[seq] = 0

    # -- invariants ------------------------------------------------------------
    def check_invariants(self):
        owned = [b for t in self.tables for b in t]
        assert len(owned) == len(set(owned)), "a block is owned twice"
        assert not (set(owned) & set(self.free)), "an owned block is also free"
        assert len(owned) + len(self.free) == self.num_blocks, "blocks lost"
        for s, t in enumerate(self.tables):
            assert self.lens[s] <= len(t) * BLOCK_TOKENS
