"""Pins of the oracle's address map, slot_mapping and cache write against the pages'
printed worked examples (tests/golden/*.json carry the citations)."""
import json
import os

import numpy as np
import pytest

from oracle import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_address_map_worked_example():
    g = gold("index_examples.json")["address_map"]
    table = np.array(g["identity_table"], np.int32)
    assert table.shape == (g["batch_size"], g["blocks_per_seq"])
    assert g["blocks_per_seq"] == g["max_seq_len"] // g["block_size"]
    nb = table.size
    slot = oracle.slot_of(table, g["batch_idx"], g["seq_pos"], g["block_size"], nb)
    assert slot == g["slot"]
    assert slot == g["physical_block"] * g["block_size"] + g["offset"]
    # logical block and offset separately: a table whose entries are all distinct shows
    # which entry was used; a different block only moves the slot by whole blocks
    t2 = table.copy()
    t2[g["batch_idx"], g["logical_block"]] = 0
    assert oracle.slot_of(t2, g["batch_idx"], g["seq_pos"], g["block_size"], nb) == g["offset"]


def test_decode_step_index_example():
    g = gold("index_examples.json")["decode_step_index"]
    bs = g["block_size"]
    table = np.array([[7, 9, 11, 13]], np.int32)
    slot = oracle.slot_of(table, 0, g["token_pos"], bs, 16)
    assert slot == table[0, g["logical_block"]] * bs + g["offset"]
    # a new block is needed for the next token exactly when the offset is bs-1
    for pos in range(0, 3 * bs):
        here = oracle.slot_of(table, 0, pos, bs, 16) // bs
        nxt = oracle.slot_of(table, 0, pos + 1, bs, 16) // bs
        assert (here != nxt) == (pos % bs == g["new_block_when_offset"])


def test_blocks_for_length_example():
    g = gold("index_examples.json")["blocks_for_length"]
    bs = g["block_size"]
    table = np.array([g["physical_blocks"]], np.int32)
    # every position of the 37-token sequence is served by the 3-entry table ...
    for pos in range(g["length"]):
        s = oracle.slot_of(table, 0, pos, bs, 32)
        assert s >= 0 and s // bs == g["physical_blocks"][pos // bs]
    # ... and its last token lands in the third block
    assert oracle.slot_of(table, 0, g["length"] - 1, bs, 32) // bs == g["physical_blocks"][2]
    # 3 blocks are not enough one block further on
    assert oracle.slot_of(table, 0, g["logical_blocks"] * bs, bs, 32) == -1
    # reading 1 (0-based positions): appending to the 37-token sequence writes
    # position 37 -> logical block 2, offset 5
    s = oracle.slot_mapping(table, [37], [0, 1], bs, 32)
    assert s.tolist() == [g["physical_blocks"][2] * bs + 5]


def test_two_request_example():
    g = gold("index_examples.json")["two_requests"]
    bs = g["block_size"]
    table = np.full((2, 2), 3, np.int32)
    table[0, :2] = g["block_table"]["A"]
    table[1, :1] = g["block_table"]["B"]
    lens = [g["lengths"]["A"], g["lengths"]["B"]]
    cu = oracle.pack(lens)[0]
    slots = oracle.slot_mapping(table, [0, 0], cu, bs, len(g["free_list"]))
    want = [blk * bs + off for blk, off in g["placement"]["A"] + g["placement"]["B"]]
    assert slots.tolist() == want


def test_slot_mapping_identity_table_examples():
    g = gold("slot_mapping_examples.json")
    msl, bs, B = g["max_seq_len"], g["block_size"], g["batch_size"]
    table = np.arange(B * (msl // bs), dtype=np.int32).reshape(B, -1)
    nb = table.size
    # prefill: every sequence writes its whole prompt starting at position 0
    kv = g["prefill"]["kv_len"]
    cu = np.concatenate([[0], np.cumsum(kv)]).astype(np.int32)
    slots = oracle.slot_mapping(table, [0] * B, cu, bs, nb)
    want = np.concatenate([np.arange(a, e) for a, e in g["prefill"]["ranges"]])
    assert len(slots) == g["prefill"]["count"]
    assert np.array_equal(slots, want)
    # decode: one token per sequence at position kv_len
    dec = g["decode"]["kv_len"]
    slots = oracle.slot_mapping(table, dec, np.arange(B + 1, dtype=np.int32), bs, nb)
    assert slots.reshape(B, 1).tolist() == g["decode"]["slot_mapping"]
    offs = np.array(g["decode"]["kv_len_offset"]).reshape(-1)
    assert (slots == np.array(dec) + offs).all()


def test_sequential_formula_is_identity_table_special_case():
    """Skill page 3.3: with the identity table, slot = b * max_seq_len + pos."""
    rng = np.random.default_rng(0)
    for bs in (1, 2, 16, 128):
        msl = 512
        B = 3
        table = np.arange(B * (msl // bs), dtype=np.int32).reshape(B, -1)
        for _ in range(50):
            b = int(rng.integers(B))
            pos = int(rng.integers(msl))
            assert oracle.slot_of(table, b, pos, bs, table.size) == b * msl + pos


def test_slot_mapping_rejects_bad_tables():
    table = np.array([[0, 1], [1, 2]], np.int32)
    # both sequences write position 16 -> logical block 1: sequence 0 -> block 1,
    # sequence 1 -> block 2: fine.  Position 0 of seq 1 -> block 1, offset 0 = slot 16,
    # which sequence 0's position 16 also uses: duplicate.
    with pytest.raises(oracle.OracleError):
        oracle.slot_mapping(table, [16, 0], [0, 1, 2], 16, 3)
    with pytest.raises(oracle.OracleError):        # past max_blocks_per_seq
        oracle.slot_mapping(table, [32, 0], [0, 1, 2], 16, 3)
    with pytest.raises(oracle.OracleError):        # physical id out of the pool
        oracle.slot_mapping(np.array([[5]], np.int32), [0], [0, 1], 16, 3)


def test_write_matches_atb_contiguous_form():
    """Paged write with the identity table == ATB write loop (ai6s.net 4.2) into a
    contiguous [batch, max_seq_len] cache: byte-identical."""
    rng = np.random.default_rng(1)
    B, msl, bs, H, D = 3, 64, 16, 2, 8
    table = np.arange(B * (msl // bs), dtype=np.int32).reshape(B, -1)
    nb = table.size
    before = np.array([5, 0, 40], np.int32)
    n = np.array([3, 17, 1], np.int32)
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    cache = rng.standard_normal((nb, bs, H, D)).astype(np.float32)
    new = rng.standard_normal((int(cu[-1]), H, D)).astype(np.float32)
    slots = oracle.slot_mapping(table, before, cu, bs, nb)
    paged = oracle.kv_write(cache, new, slots)
    contig = oracle.kv_write_contiguous(cache.reshape(B, msl, H, D), new, n, before + n)
    assert paged.tobytes() == contig.tobytes()
    # only the written rows changed
    changed = np.nonzero((paged != cache).reshape(nb * bs, -1).any(axis=1))[0]
    assert set(changed.tolist()) <= set(slots.tolist())


def test_write_rejects_bad_slots():
    cache = np.zeros((2, 4, 1, 4), np.float32)
    rows = np.ones((2, 1, 4), np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.kv_write(cache, rows, [3, 3])
    with pytest.raises(oracle.OracleError):
        oracle.kv_write(cache, rows, [0, 8])
