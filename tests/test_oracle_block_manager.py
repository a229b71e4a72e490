"""Pins of the block-manager model (oracle/block_manager.py) to what the pages fix:
hand traces of the free-list order, the 37-token example, block counts in closed form,
and the pages' dual-track check (a plain per-sequence token history against the paged
store read back through the table; "Paged KV Cache and Packed Sequence", end of 5.4).
The mutants at the bottom plant plausible mistakes in the model and must be caught."""
import random

import pytest

from oracle.block_manager import BlockManagerModel, ManagerError, SeqRecord


def check_invariants(m, live):
    """Counts equal the number of holders; free list and held blocks are disjoint and
    cover the pool; each sequence holds ceil(len / block_size) blocks."""
    holders = {}
    for s in live:
        blocks = m.blocks_of(s)
        assert len(blocks) == len(set(blocks))
        assert len(blocks) == -(-m.length_of(s) // m.block_size)
        for b in blocks:
            holders[b] = holders.get(b, 0) + 1
    assert len(m.spare_ids()) == len(set(m.spare_ids()))
    assert not set(m.spare_ids()) & set(holders)
    assert len(m.spare_ids()) + len(holders) == len(m.holder_counts())
    for b, c in enumerate(m.holder_counts()):
        assert c == holders.get(b, 0), (b, c, holders.get(b, 0))


def pin_pages_37_tokens(cls):
    # 2.1-2.2: 37 tokens at block_size 16 hold 3 blocks, two full and 5 rows in the third;
    # the next token goes to offset 5 of logical block 2 without a new block.
    m = cls(64, 16, 8)
    m.add(0)
    slots, _ = m.append(0, 37)
    blocks = m.blocks_of(0)
    assert len(blocks) == 3 and m.num_free() == 61
    assert slots[:16] == [blocks[0] * 16 + i for i in range(16)]
    assert slots[36] == blocks[2] * 16 + 4
    (s,), _ = m.append(0, 1)
    assert m.num_free() == 61 and s == blocks[2] * 16 + 5


def pin_decode_allocates_at_block_starts(cls):
    # 2.2: one token per step takes a block only at positions 0, bs, 2 bs, ...
    for bs in (1, 4, 16):
        m = cls(200, bs, 200)
        m.add(7)
        taken_at = []
        for p in range(100):
            before = m.num_free()
            m.append(7, 1)
            if m.num_free() != before:
                assert before - m.num_free() == 1
                taken_at.append(p)
        assert taken_at == list(range(0, 100, bs))


def pin_lifo_hand_trace(cls):
    # 2.1: the free list starts 0..3 and pop() takes from its end.
    m = cls(4, 2, 4)
    m.add("A")
    assert m.append("A", 3) == ([6, 7, 4], None)          # blocks 3, 2
    m.add("B")
    assert m.append("B", 1) == ([2], None)                # block 1
    m.free("A")                                           # free list 0, 3, 2
    assert m.num_free() == 3
    m.add("C")
    assert m.append("C", 2) == ([4, 5], None)             # block 2 again
    assert m.append("C", 1) == ([6], None)                # then block 3
    assert m.table(["B", "C"], pad_block=-1) == ([[1, -1, -1, -1], [2, 3, -1, -1]], [1, 3])


def pin_full_changes_nothing(cls):
    m = cls(2, 2, 4)
    m.add(1)
    m.append(1, 4)
    with pytest.raises(ManagerError) as e:
        m.append(1, 1)
    assert e.value.kind == "full"
    assert m.length_of(1) == 4 and m.num_free() == 0 and m.blocks_of(1) == [1, 0]
    m2 = cls(3, 2, 4)
    m2.add(1)
    m2.append(1, 2)
    with pytest.raises(ManagerError):
        m2.append(1, 5)                                   # needs 3 more, 2 free
    assert m2.num_free() == 2 and m2.length_of(1) == 2 and m2.holder_counts() == [0, 0, 1]


def pin_too_long(cls):
    m = cls(16, 4, 2)
    m.add(0)
    m.append(0, 8)
    with pytest.raises(ManagerError) as e:
        m.append(0, 1)
    assert e.value.kind == "shape" and m.length_of(0) == 8 and m.num_free() == 14


def pin_shared_prefix_release(cls):
    # 5.2: freeing one of two sequences that share blocks returns none of them; freeing
    # the second returns all.
    m = cls(8, 4, 4)
    m.add(0)
    m.append(0, 8)
    m.fork(0, 1)
    assert [m.holders(b) for b in m.blocks_of(0)] == [2, 2]
    m.free(0)
    assert m.num_free() == 6 and [m.holders(b) for b in m.blocks_of(1)] == [1, 1]
    m.free(1)
    assert m.num_free() == 8 and m.holder_counts() == [0] * 8


def pin_copy_on_write(cls):
    # A fork in the middle of a block: the first writer copies the shared block.
    m = cls(8, 4, 4)
    m.add(0)
    m.append(0, 6)                                        # blocks 7, 6; 2 rows in 6
    m.fork(0, 1)
    slots, copy = m.append(1, 1)
    assert copy == (6, 5) and slots == [5 * 4 + 2]
    assert m.blocks_of(1) == [7, 5] and m.blocks_of(0) == [7, 6]
    assert m.holders(6) == 1 and m.holders(7) == 2
    slots, copy = m.append(0, 1)                          # block 6 no longer shared
    assert copy is None and slots == [6 * 4 + 2]
    m.fork(0, 2)                                          # block 6 shared again, 3 rows
    assert m.append(0, 1) == ([4 * 4 + 3], (6, 4))        # the writer moves to block 4
    assert m.blocks_of(2) == [7, 6] and m.holders(6) == 1
    m3 = cls(8, 4, 4)
    m3.add(0)
    m3.append(0, 8)
    m3.fork(0, 1)
    assert m3.append(1, 1)[1] is None                     # full last block: no copy


def run_dual_track(cls, seed, num_blocks=48, bs=4, mbs=12, ops=400):
    """Random adds, forks, appends and frees; a store maps slot -> token id; the rows of a
    copy on write are copied before the new tokens are written.  After every operation each
    live sequence read through its table must equal its own history."""
    rng = random.Random(seed)
    m = cls(num_blocks, bs, mbs)
    store, hist, next_id, token = {}, {}, 0, 0
    for _ in range(ops):
        live = list(hist)
        r = rng.random()
        if r < 0.15 or not live:
            m.add(next_id)
            hist[next_id] = []
            next_id += 1
        elif r < 0.3:
            parent = rng.choice(live)
            m.fork(parent, next_id)
            hist[next_id] = list(hist[parent])
            next_id += 1
        elif r < 0.45:
            s = rng.choice(live)
            m.free(s)
            del hist[s]
        else:
            s = rng.choice(live)
            n = rng.choice([1, 1, 1, 2, 3, 5, 9])
            try:
                slots, copy = m.append(s, n)
            except ManagerError:
                continue
            if copy is not None:
                src, dst = copy
                for o in range(bs):
                    if src * bs + o in store:
                        store[dst * bs + o] = store[src * bs + o]
            for sl in slots:
                store[sl] = token
                hist[s].append(token)
                token += 1
        check_invariants(m, list(hist))
        for s, h in hist.items():
            rows, lens = m.table([s], pad_block=-1)
            assert lens == [len(h)]
            got = [store.get(rows[0][p // bs] * bs + p % bs) for p in range(len(h))]
            assert got == h, (seed, s)
    return token


def pin_dual_track(cls):
    total = 0
    for seed in range(6):
        total += run_dual_track(cls, seed)
    assert total > 500          # the walk really wrote tokens


PINS = [pin_pages_37_tokens, pin_decode_allocates_at_block_starts, pin_lifo_hand_trace,
        pin_full_changes_nothing, pin_too_long, pin_shared_prefix_release, pin_copy_on_write,
        pin_dual_track]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_model_pin(pin):
    pin(BlockManagerModel)


# ----------------------------------------------------------------------------- mutants
class FifoFreeList(BlockManagerModel):
    def _grab(self):
        blk = self._spare.pop(0)
        self._holders[blk] = 1
        return blk


class FreeIgnoresCounts(BlockManagerModel):
    def free(self, seq):
        rec = self._record(seq)
        del self._seqs[seq]
        for blk in rec.blocks:
            self._holders[blk] = max(self._holders[blk] - 1, 0)
            if blk not in self._spare:
                self._spare.append(blk)


class ForkKeepsCounts(BlockManagerModel):
    def fork(self, parent, child):
        src = self._seqs[parent]
        self._seqs[child] = SeqRecord(list(src.blocks), src.length)


class NoCopyOnWrite(BlockManagerModel):
    def _plan(self, rec, num_tokens):
        fresh, shared_tail = super()._plan(rec, num_tokens)
        return (fresh[1:] if shared_tail else fresh), False


class EagerNextBlock(BlockManagerModel):
    """Takes the next block when a block's last row is written."""
    def append(self, seq, num_tokens):
        slots, copy = super().append(seq, num_tokens)
        rec = self._seqs[seq]
        if num_tokens and rec.length % self.block_size == 0 and self._spare:
            rec.blocks.append(self._grab())
        return slots, copy


class OffsetOffByOne(BlockManagerModel):
    def append(self, seq, num_tokens):
        slots, copy = super().append(seq, num_tokens)
        bs = self.block_size
        return [(s // bs) * bs + (s % bs + 1) % bs for s in slots], copy


class FailureLeaksBlocks(BlockManagerModel):
    def append(self, seq, num_tokens):
        try:
            return super().append(seq, num_tokens)
        except ManagerError as e:
            if e.kind == "full" and self._spare:
                self._seqs[seq].blocks.append(self._grab())
            raise


MUTANTS = [FifoFreeList, FreeIgnoresCounts, ForkKeepsCounts, NoCopyOnWrite, EagerNextBlock,
           OffsetOffByOne, FailureLeaksBlocks]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda c: c.__name__)
def test_mutant_is_caught(mutant):
    caught = 0
    for pin in PINS:
        try:
            pin(mutant)
        except (AssertionError, ManagerError, KeyError, IndexError, ValueError):
            caught += 1
    assert caught > 0, f"no pin catches {mutant.__name__}"
