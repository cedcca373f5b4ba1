"""CPU oracle for the host block manager (the allocator behind block_table
and slot_mapping).

TEST INFRASTRUCTURE, like the rest of ``oracle/``: only the tests, the smoke
check and the benchmark's CPU-baseline leg may use it; the library never
imports it.

What the pages describe, and the readings taken where they are silent:

* A pool of ``num_blocks`` fixed-size blocks is allocated once; sequences
  take blocks from a free list as they grow (vLLM-on-CANN page, its
  ``PagedKVCache`` listing: ``free_blocks`` and ``allocate_slots``; "Paged KV
  infra" page section 2.3 on the pre-allocated page pool and page reuse).
  Which free block comes next: the ATB PagedAttention page's allocator scans
  for the first free page, so the lowest-numbered free block is taken.
* A sequence of n tokens holds ceil(n / block_size) blocks (vLLM-on-CANN
  page: ``(num_tokens + block_size - 1) // block_size``). Token ``pos`` lives
  at slot ``table[pos // bs] * bs + pos % bs`` (skill page, section 3.1).
* Blocks carry a reference count: a new block starts at 1, a sequence that
  shares it (a fork of a common prefix) adds 1, a release subtracts 1 and
  the block returns to the free list at 0 (ATB page, "page reference
  counting": AllocPage / SharePage / ReleasePage).
* Extending a sequence whose last block is shared copies that block first:
  a fresh block is allocated, the old block's contents are copied into it,
  the table's last entry is repointed and the old block released (ATB page,
  copy-on-write ``ExtendKVPage``). The pool lives on the device, so a copy is
  recorded as a (src, dst) pair for ``paged_kv_copy_blocks``. The pairs of
  one ``take_copies`` run concurrently on the device, so until they are taken
  a block named in a pair is not handed out again, and copying from a block
  that is itself the destination of a pending pair is refused (its device
  contents would not be current).
* An append that needs more blocks than are free changes nothing and fails.

Status codes mirror include/pagedkv.h: 0 ok, -2 shape (unknown / duplicate
sequence, bad sizes), -7 out of blocks, -8 pending copy.
"""

from __future__ import annotations

OK, ERR_SHAPE, ERR_NO_BLOCKS, ERR_PENDING_COPY = 0, -2, -7, -8


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.ref = [0] * num_blocks
        self.tables: dict[int, list[int]] = {}
        self.lens: dict[int, int] = {}
        self.pending: list[tuple[int, int]] = []
        self.locked: set[int] = set()   # blocks named by a pending pair

    # -- the free list ---------------------------------------------------
    def num_free(self) -> int:
        return sum(1 for r in self.ref if r == 0)

    def _num_allocatable(self) -> int:
        return sum(1 for b, r in enumerate(self.ref) if r == 0 and b not in self.locked)

    def _take_free(self) -> int:
        for b in range(self.num_blocks):      # first free block (ATB page's scan)
            if self.ref[b] == 0 and b not in self.locked:
                self.ref[b] = 1
                return b
        raise AssertionError("caller checked the free count")

    def _release(self, b: int):
        self.ref[b] -= 1
        assert self.ref[b] >= 0

    # -- sequences -------------------------------------------------------
    def add_sequence(self, seq: int) -> int:
        if seq in self.tables:
            return ERR_SHAPE
        self.tables[seq] = []
        self.lens[seq] = 0
        return OK

    def fork(self, parent: int, child: int) -> int:
        """The child shares every block of the parent (reference count + 1)."""
        if parent not in self.tables or child in self.tables:
            return ERR_SHAPE
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1
        return OK

    def append(self, seq: int, n: int):
        """Extend ``seq`` by n tokens. Returns (status, slots of the new tokens)."""
        if seq not in self.tables or n < 0:
            return ERR_SHAPE, []
        table, length, bs = self.tables[seq], self.lens[seq], self.block_size
        if n == 0:
            return OK, []
        have = len(table)
        need_total = -(-(length + n) // bs)
        new_blocks = need_total - have
        cow = length % bs != 0 and self.ref[table[-1]] > 1   # partial last block, shared
        if cow and any(dst == table[-1] for _, dst in self.pending):
            return ERR_PENDING_COPY, []
        if new_blocks + (1 if cow else 0) > self._num_allocatable():
            return ERR_NO_BLOCKS, []
        if cow:
            old = table[-1]
            new = self._take_free()
            self.pending.append((old, new))
            self.locked.update((old, new))
            table[-1] = new
            self._release(old)
        for _ in range(new_blocks):
            table.append(self._take_free())
        slots = [table[p // bs] * bs + p % bs for p in range(length, length + n)]
        self.lens[seq] = length + n
        return OK, slots

    def free_sequence(self, seq: int) -> int:
        if seq not in self.tables:
            return ERR_SHAPE
        for b in self.tables.pop(seq):
            self._release(b)
        del self.lens[seq]
        return OK

    # -- outputs ---------------------------------------------------------
    def block_table(self, seqs, max_blocks: int):
        """Rows of block ids padded with -1, and the lengths; ERR_SHAPE if a
        sequence is unknown or needs more than max_blocks blocks."""
        rows, lens = [], []
        for s in seqs:
            if s not in self.tables or len(self.tables[s]) > max_blocks:
                return ERR_SHAPE, None, None
            t = self.tables[s]
            rows.append(t + [-1] * (max_blocks - len(t)))
            lens.append(self.lens[s])
        return OK, rows, lens

    def take_copies(self):
        out, self.pending = self.pending, []
        self.locked.clear()
        return out


def copy_blocks(cache, pairs):
    """Apply (src, dst) block copies to a pool [num_blocks, ...] in order."""
    out = cache.copy()
    for src, dst in pairs:
        out[dst] = out[src]
    return out
