"""Reference model of the host block manager, in plain Python.

TEST INFRASTRUCTURE ONLY: the tests may import this module; the product path never does,
and it shares no code with the library's manager.

Behaviour it follows ("Paged KV Cache and Packed Sequence", hotelren.com source note):
  * 2.1: a pool of num_blocks physical blocks, all spare at the start; a spare block is
    handed out last-in first-out (the spare ids form a stack that starts as 0 at the bottom
    up to num_blocks - 1 on top); each block counts the sequences that hold it; each
    sequence owns an ordered list of physical blocks; a request that needs more spare
    blocks than there are fails (a "full" error);
  * 2.1: a sequence of n tokens holds ceil(n / block_size) blocks; 2.2: token position p
    lives at offset p % block_size of logical block p // block_size, and the flat index of
    its row is physical_block * block_size + offset; a decode step takes a new block only
    when its token is the first of a logical block the sequence does not hold yet;
  * 2.2: the table handed to the kernels is fixed-width (max_blocks_per_seq per sequence);
  * 5.2: sequences that share a prefix share its blocks (a holder count above one);
    releasing a sequence lowers the count of each of its blocks, and a block becomes
    spare again only when no holder remains.

Readings where the pages are silent:
  * fork(parent, child) is how a prefix comes to be shared (beam search, parallel
    sampling): the child gets the parent's block list and every count goes up by one;
  * copy on write: a sequence about to write into a partly filled last block that is
    shared takes a fresh block for it instead (its hold on the old block is dropped) and
    reports (old, new) so that the rows already there are copied first;
  * a failed request changes nothing (the fresh blocks are counted before any is taken);
  * blocks released together become spare in the order the sequence held them (the last
    one ends on top of the stack).
"""
from __future__ import annotations

from dataclasses import dataclass, field


class ManagerError(RuntimeError):
    def __init__(self, kind: str, message: str):
        super().__init__(message)
        self.kind = kind          # "shape" (bad id / too long) or "full" (too few spare)


@dataclass
class SeqRecord:
    blocks: list = field(default_factory=list)   # physical ids in logical order
    length: int = 0                              # tokens held


def blocks_for(tokens: int, block_size: int) -> int:
    """Blocks that hold `tokens` tokens: ceil(tokens / block_size)."""
    return (tokens + block_size - 1) // block_size


class BlockManagerModel:
    def __init__(self, num_blocks: int, block_size: int, max_blocks_per_seq: int):
        if num_blocks <= 0 or block_size <= 0 or max_blocks_per_seq <= 0:
            raise ManagerError("shape", "sizes must be positive")
        self.block_size = block_size
        self.max_blocks_per_seq = max_blocks_per_seq
        self._spare = [i for i in range(num_blocks)]   # stack: the top is the last element
        self._holders = [0 for _ in range(num_blocks)]  # sequences holding each block
        self._seqs: dict = {}                           # seq id -> SeqRecord

    # ------------------------------------------------------------------ read access
    def num_free(self) -> int:
        return len(self._spare)

    def spare_ids(self) -> list:
        """Spare block ids, bottom of the stack first."""
        return list(self._spare)

    def holders(self, blk: int) -> int:
        return self._holders[blk]

    def holder_counts(self) -> list:
        return list(self._holders)

    def sequences(self) -> list:
        return list(self._seqs)

    def blocks_of(self, seq) -> list:
        return list(self._record(seq).blocks)

    def length_of(self, seq) -> int:
        return self._record(seq).length

    def _record(self, seq) -> SeqRecord:
        rec = self._seqs.get(seq)
        if rec is None:
            raise ManagerError("shape", f"no sequence {seq}")
        return rec

    # ------------------------------------------------------------------ ownership
    def _grab(self) -> int:
        """The spare block on top of the stack, now held once."""
        blk = self._spare.pop()
        self._holders[blk] = 1
        return blk

    def _release(self, blocks) -> None:
        """Drop one hold on each block; the ones left with no holder become spare, in the
        order given."""
        emptied = []
        for blk in blocks:
            self._holders[blk] -= 1
            if self._holders[blk] == 0:
                emptied.append(blk)
        self._spare.extend(emptied)

    # ------------------------------------------------------------------ operations
    def add(self, seq):
        if seq in self._seqs or (isinstance(seq, int) and seq < 0):
            raise ManagerError("shape", f"sequence {seq} exists or is negative")
        self._seqs[seq] = SeqRecord()

    def fork(self, parent, child):
        if parent not in self._seqs or child in self._seqs or child < 0:
            raise ManagerError("shape", "bad fork")
        src = self._seqs[parent]
        self._seqs[child] = SeqRecord(list(src.blocks), src.length)
        for blk in src.blocks:
            self._holders[blk] += 1

    def _plan(self, rec: SeqRecord, num_tokens: int):
        """(logical blocks that need a fresh id, whether the first of them replaces a shared
        partly filled last block) for appending num_tokens tokens to rec."""
        bs = self.block_size
        total = blocks_for(rec.length + num_tokens, bs)
        if total > self.max_blocks_per_seq:
            raise ManagerError("shape", "sequence longer than max_blocks_per_seq blocks")
        fresh = list(range(len(rec.blocks), total))
        partial = rec.length % bs != 0
        shared_tail = partial and self._holders[rec.blocks[-1]] > 1
        if shared_tail:
            fresh.insert(0, len(rec.blocks) - 1)
        return fresh, shared_tail

    def append(self, seq, num_tokens: int):
        """Slots of num_tokens new tokens of `seq`, and the (old, new) block copy a copy on
        write needs (or None)."""
        if seq not in self._seqs or num_tokens < 0:
            raise ManagerError("shape", "bad append")
        rec = self._seqs[seq]
        if num_tokens == 0:
            return [], None
        fresh, shared_tail = self._plan(rec, num_tokens)
        if len(fresh) > len(self._spare):
            raise ManagerError("full", f"{len(fresh)} blocks needed, {len(self._spare)} spare")
        copy = None
        for j in fresh:
            blk = self._grab()
            if j < len(rec.blocks):                  # the shared tail: move the writer off it
                old = rec.blocks[j]
                self._holders[old] -= 1
                rec.blocks[j] = blk
                copy = (old, blk)
            else:
                rec.blocks.append(blk)
        assert copy is not None or not shared_tail
        bs = self.block_size
        first = rec.length
        rec.length += num_tokens
        return [rec.blocks[p // bs] * bs + p % bs for p in range(first, rec.length)], copy

    def decode_step(self, seqs, pad_block: int = 0):
        """One token for each row's sequence in row order; a negative id is a padding row
        (no sequence: pad_block row, length 0, slot -1).  Returns (rows, lengths, slots,
        copies).  Nothing changes when any row would fail."""
        live = [s for s in seqs if s >= 0]
        if len(set(live)) != len(live) or any(s not in self._seqs for s in live):
            raise ManagerError("shape", "unknown or repeated sequence")
        for s in live:          # a row that would need a block past max_blocks_per_seq
            rec = self._seqs[s]
            if blocks_for(rec.length + 1, self.block_size) > self.max_blocks_per_seq:
                raise ManagerError("shape", "sequence longer than max_blocks_per_seq blocks")
        snapshot = (list(self._spare), list(self._holders),
                    {k: SeqRecord(list(r.blocks), r.length) for k, r in self._seqs.items()})
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
                r, n = self.table([s], pad_block)
                rows.append(r[0])
                lens.append(n[0])
        except ManagerError:
            self._spare, self._holders, self._seqs = snapshot
            raise
        return rows, lens, slots, copies

    def free(self, seq):
        rec = self._record(seq)
        del self._seqs[seq]
        self._release(rec.blocks)

    def table(self, seqs, pad_block: int = 0):
        """Fixed-width rows (blocks, then pad_block) and the lengths."""
        rows, lens = [], []
        for s in seqs:
            rec = self._record(s)
            rows.append(list(rec.blocks) + [pad_block] * (self.max_blocks_per_seq - len(rec.blocks)))
            lens.append(rec.length)
        return rows, lens
