"""Reference model of the host block manager, in plain Python.

TEST INFRASTRUCTURE ONLY: the tests may import this module; the product path never does,
and it shares no code with the library's manager.

It follows "Paged KV Cache and Packed Sequence" (hotelren.com source note):
  * 2.1: a pool of num_blocks physical blocks; the free list starts as 0 .. num_blocks-1
    and a block is taken with a pop from its end; a per-block reference count; per
    sequence a list of physical blocks; a request that finds the free list empty fails
    with "kv cache full";
  * 2.1: a sequence of n tokens holds ceil(n / block_size) blocks; 2.2: token position p
    lives at offset p % block_size of logical block p // block_size, and the flat index of
    the row is physical_block * block_size + offset; a decode step takes a new block only
    when its token is the first of a logical block the sequence does not hold yet;
  * 2.2: the table handed to the kernels is fixed-width (max_blocks_per_seq per sequence);
  * 5.2: sequences sharing a prefix share its blocks (count > 1); releasing a sequence
    first lowers the count of each of its blocks and puts a block back on the free list
    only when its count reaches zero.

Readings where the pages are silent:
  * fork(parent, child) is how a prefix comes to be shared (beam search, parallel
    sampling): the child gets the parent's block list and every count goes up by one;
  * copy on write: a sequence about to write into a partly filled last block that is
    shared takes a fresh block for it instead (the writer's count on the old block is
    dropped) and reports (old, new) so that the rows already there are copied first;
  * a failed request changes nothing (the fresh blocks are counted before any is taken);
  * released blocks go back on the free list in the order the sequence holds them.
"""
from __future__ import annotations


class ManagerError(RuntimeError):
    def __init__(self, kind: str, message: str):
        super().__init__(message)
        self.kind = kind          # "shape" (bad id / too long) or "full" (free list short)


class BlockManagerModel:
    def __init__(self, num_blocks: int, block_size: int, max_blocks_per_seq: int):
        if num_blocks <= 0 or block_size <= 0 or max_blocks_per_seq <= 0:
            raise ManagerError("shape", "sizes must be positive")
        self.block_size = block_size
        self.max_blocks_per_seq = max_blocks_per_seq
        self.free_blocks = list(range(num_blocks))
        self.ref_count = [0] * num_blocks
        self.block_table = {}      # seq id -> list of physical blocks
        self.seq_len = {}          # seq id -> tokens held

    def num_free(self) -> int:
        return len(self.free_blocks)

    def add(self, seq: int):
        if seq in self.block_table or (isinstance(seq, int) and seq < 0):
            raise ManagerError("shape", f"sequence {seq} exists or is negative")
        self.block_table[seq] = []
        self.seq_len[seq] = 0

    def fork(self, parent: int, child: int):
        if parent not in self.block_table or child in self.block_table or child < 0:
            raise ManagerError("shape", "bad fork")
        self.block_table[child] = list(self.block_table[parent])
        self.seq_len[child] = self.seq_len[parent]
        for blk in self.block_table[child]:
            self.ref_count[blk] += 1

    def _take(self) -> int:
        blk = self.free_blocks.pop()
        self.ref_count[blk] += 1
        return blk

    def append(self, seq: int, num_tokens: int):
        """Returns (slots of the new tokens, (old, new) block copy or None)."""
        if seq not in self.block_table or num_tokens < 0:
            raise ManagerError("shape", "bad append")
        blocks, n = self.block_table[seq], self.seq_len[seq]
        bs = self.block_size
        if num_tokens == 0:
            return [], None
        held_after = -(-(n + num_tokens) // bs)
        if held_after > self.max_blocks_per_seq:
            raise ManagerError("shape", "sequence longer than max_blocks_per_seq blocks")
        cow = n % bs != 0 and self.ref_count[blocks[-1]] > 1
        fresh = held_after - len(blocks) + (1 if cow else 0)
        if fresh > len(self.free_blocks):
            raise ManagerError("full", "kv cache full")
        copy = None
        if cow:
            old = blocks[-1]
            new = self._take()
            self.ref_count[old] -= 1
            blocks[-1] = new
            copy = (old, new)
        slots = []
        for p in range(n, n + num_tokens):
            if p // bs == len(blocks):          # first token of a block not held yet
                blocks.append(self._take())
            slots.append(blocks[p // bs] * bs + p % bs)
        self.seq_len[seq] = n + num_tokens
        return slots, copy

    def decode_step(self, seqs, pad_block: int = 0):
        """One token for each row's sequence in row order; a negative id is a padding row
        (no sequence: pad_block row, length 0, slot -1).  Returns (rows, lengths, slots,
        copies).  Nothing changes when any row would fail."""
        live = [s for s in seqs if s >= 0]
        if len(set(live)) != len(live) or any(s not in self.block_table for s in live):
            raise ManagerError("shape", "unknown or repeated sequence")
        for s in live:          # a row that would need a block past max_blocks_per_seq
            if self.seq_len[s] % self.block_size == 0 and \
                    len(self.block_table[s]) + 1 > self.max_blocks_per_seq:
                raise ManagerError("shape", "sequence longer than max_blocks_per_seq blocks")
        saved = (list(self.free_blocks), list(self.ref_count),
                 {k: list(v) for k, v in self.block_table.items()}, dict(self.seq_len))
        rows, lens, slots, copies = [], [], [], []
        try:
            for s in seqs:
                if s < 0:
                    rows.append([pad_block] * self.max_blocks_per_seq)
                    lens.append(0)
                    slots.append(-1)
                    continue
                (slot,), copy = self.append(s, 1)
                if copy is not None:
                    copies.append(copy)
                slots.append(slot)
                r, l = self.table([s], pad_block)
                rows.append(r[0])
                lens.append(l[0])
        except ManagerError:
            self.free_blocks, self.ref_count, self.block_table, self.seq_len = saved
            raise
        return rows, lens, slots, copies

    def free(self, seq: int):
        if seq not in self.block_table:
            raise ManagerError("shape", f"no sequence {seq}")
        blocks = self.block_table.pop(seq)
        del self.seq_len[seq]
        for blk in blocks:
            self.ref_count[blk] -= 1
        for blk in blocks:
            if self.ref_count[blk] == 0:
                self.free_blocks.append(blk)

    def table(self, seqs, pad_block: int = 0):
        """Fixed-width rows (blocks, then pad_block) and the lengths."""
        rows, lens = [], []
        for s in seqs:
            if s not in self.block_table:
                raise ManagerError("shape", f"no sequence {s}")
            blocks = self.block_table[s]
            rows.append(blocks + [pad_block] * (self.max_blocks_per_seq - len(blocks)))
            lens.append(self.seq_len[s])
        return rows, lens
