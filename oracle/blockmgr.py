"""Reference block manager: pool, block tables, reference counts (oracle, test infrastructure).

This is the host bookkeeping that produces the GPU path's index inputs (block
tables, write slots, copy-on-write pairs).  It follows the pages:

* GPU memory is a pool of equal physical blocks; each request owns a block
  table mapping its logical blocks to physical ids ([PA-notes] §3, §5 ①).
* Allocation is on demand: a prompt of n tokens takes ceil(n / B) blocks
  ([PA-explainer] "动态分配"), and a new token goes to the next free slot after
  the filled ones -- a new block is taken only when the last one is full
  ([PA-notes] §5 ②), so a request wastes less than one block.
* Sharing: parallel samples of one prompt point at the same physical blocks;
  each physical block counts its sharers.  Writing into a block that is still
  shared first copies it (copy-on-write), repoints only the writer's entry and
  adjusts both counts; a finished or pruned sequence decrements its blocks and
  a block whose count reaches zero returns to the pool ([PA-notes] §6.1, §6.2,
  §12 题4).

* Preemption: a suspended request's blocks move to CPU RAM and come back
  later through its block table ([PA-notes] §5 ③).  ``swap_out(seqs)`` moves
  every block the listed sequences reference into a second pool of
  ``num_cpu_blocks`` host blocks and ``swap_in(seqs)`` brings them back into
  fresh GPU blocks; both return the (src, dst) block pairs to copy.

Readings: the free list is a queue whose initial order the caller gives (the
workloads pass a seeded permutation, so placement is random); [PA-explainer]'s
LRU eviction on an empty pool is not modelled -- allocation from an empty pool
raises and leaves every table and count unchanged.  Copy-on-write fires iff the
target block's count is above one at write time, so with k sharers the first
k-1 writers copy and the last writes in place.

Swap readings: the sequences named in one call move together, and a block
they share is moved once, its count carried over (so a sample group swaps as
a group).  A block also held by a sequence outside the call keeps its GPU copy
for that sequence and only loses the leaving sharers.  A swapped-out sequence
can only be swapped in or freed.  Either call raises, changing nothing, when the
target pool has too few free blocks.  The host pool's free list is a queue in
id order.  Blocks freed by a swap-out may be handed out again at once, so the
caller copies the returned pairs before any later write (one stream in order).

Pins (tests/test_oracle_blockmgr.py, tests/test_oracle_swap.py): the 40-token
and 1000-token examples ([PA-notes] §9.2, §12 题1), the four-sharer copy-on-write trace ([PA-notes]
§12 题4), waste < B for every sequence, and no leaked blocks after all frees;
with swaps, every sequence reads back its own token history through its table
from the pool it lives in, after every step of random traces.
"""

from collections import deque


class OutOfBlocks(RuntimeError):
    pass


class BlockManager:
    def __init__(self, num_blocks, block_size, free_order=None, num_cpu_blocks=0):
        self.num_blocks = int(num_blocks)
        self.num_cpu_blocks = int(num_cpu_blocks)
        self.cpu_free = deque(range(self.num_cpu_blocks))
        self.cpu_ref = [0] * self.num_cpu_blocks
        self.swapped = set()
        self.block_size = int(block_size)
        order = range(self.num_blocks) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(self.num_blocks)):
            raise ValueError("free_order must be a permutation of the block ids")
        self.free = deque(order)
        self.ref = [0] * self.num_blocks
        self.tables = {}
        self.lens = {}

    # -- internals ---------------------------------------------------------
    def _take(self):
        b = self.free.popleft()
        self.ref[b] = 1
        return b

    def _need(self, n):
        if len(self.free) < n:
            raise OutOfBlocks(f"need {n} blocks, {len(self.free)} free")

    # -- operations --------------------------------------------------------
    def allocate(self, seq, num_tokens):
        """Prefill: give ``seq`` ceil(num_tokens / B) fresh blocks."""
        if seq in self.tables:
            raise ValueError(f"sequence {seq!r} already allocated")
        n = -(-int(num_tokens) // self.block_size)
        self._need(n)
        self.tables[seq] = [self._take() for _ in range(n)]
        self.lens[seq] = int(num_tokens)
        return list(self.tables[seq])

    def _resident(self, seq):
        if seq in self.swapped:
            raise ValueError(f"sequence {seq!r} is swapped out")

    def append_slot(self, seq):
        """Reserve the slot of ``seq``'s next token.

        Returns ``(slot, cow)`` with ``cow = (src, dst)`` when the write needed a
        private copy of a shared block, else ``None``.
        """
        self._resident(seq)
        B = self.block_size
        table = self.tables[seq]
        pos = self.lens[seq]
        cow = None
        if pos // B == len(table):                 # last block full (or none): new block
            self._need(1)
            table.append(self._take())
        else:
            last = table[pos // B]
            if self.ref[last] > 1:                 # shared: copy before writing
                self._need(1)
                new = self._take()
                self.ref[last] -= 1
                table[pos // B] = new
                cow = (last, new)
        self.lens[seq] = pos + 1
        return table[pos // B] * B + pos % B, cow

    def fork(self, parent, child):
        """``child`` shares every block of ``parent`` (parallel sampling / beam fork)."""
        if child in self.tables:
            raise ValueError(f"sequence {child!r} already exists")
        self._resident(parent)
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1

    def free_seq(self, seq):
        """Drop ``seq``: every block loses one sharer; blocks at zero return to the pool
        (the host pool for a swapped-out sequence)."""
        ref, free = (self.cpu_ref, self.cpu_free) if seq in self.swapped else (self.ref, self.free)
        for b in self.tables.pop(seq):
            ref[b] -= 1
            if ref[b] == 0:
                free.append(b)
        del self.lens[seq]
        self.swapped.discard(seq)

    def _move(self, seqs, to_cpu):
        """Move the listed sequences' blocks to the other pool; returns the (src, dst) pairs."""
        seqs = list(seqs)
        if len(set(seqs)) != len(seqs):
            raise ValueError("a sequence is listed twice")
        for s in seqs:
            if s not in self.tables:
                raise KeyError(s)
            if (s in self.swapped) == to_cpu:
                raise ValueError(f"sequence {s!r} is already {'out' if to_cpu else 'in'}")
        src_ref, src_free = (self.ref, self.free) if to_cpu else (self.cpu_ref, self.cpu_free)
        dst_ref, dst_free = (self.cpu_ref, self.cpu_free) if to_cpu else (self.ref, self.free)
        moving = {}                                # src block -> sharers leaving with it
        for s in seqs:
            for b in self.tables[s]:
                moving[b] = moving.get(b, 0) + 1
        if len(dst_free) < len(moving):
            raise OutOfBlocks(f"need {len(moving)} blocks in the target pool, {len(dst_free)} free")
        new_id, pairs = {}, []
        for b, n in moving.items():                # first-reference order
            d = dst_free.popleft()
            dst_ref[d] = n
            new_id[b] = d
            pairs.append((b, d))
        for b, n in moving.items():
            src_ref[b] -= n
            if src_ref[b] == 0:
                src_free.append(b)
        for s in seqs:
            self.tables[s] = [new_id[b] for b in self.tables[s]]
            if to_cpu:
                self.swapped.add(s)
            else:
                self.swapped.discard(s)
        return pairs

    def swap_out(self, seqs):
        """Preempt ``seqs``: (gpu_block, cpu_block) pairs to copy GPU -> host."""
        return self._move(seqs, True)

    def swap_in(self, seqs):
        """Restore ``seqs``: (cpu_block, gpu_block) pairs to copy host -> GPU."""
        return self._move(seqs, False)

    # -- queries -----------------------------------------------------------
    def slot(self, seq, pos):
        """Flat pool slot of token ``pos`` of ``seq``."""
        B = self.block_size
        return self.tables[seq][pos // B] * B + pos % B

    def waste(self, seq):
        """Slots held by ``seq``'s blocks but not filled."""
        return len(self.tables[seq]) * self.block_size - self.lens[seq]

    def num_free(self):
        return len(self.free)
