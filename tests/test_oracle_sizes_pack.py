"""Pins of the oracle's packing and size formulas against the pages' printed numbers,
and of the attention gather against the KV-size formula (it must read exactly
L' x 2 x H x d x B bytes of cache per layer: every visible row once, nothing else)."""
import json
import math
import os

import numpy as np
import torch

from oracle import oracle
from paged_kv_cache_133_amd import workloads as wl
from tests.helpers import case_numpy

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_kv_size_formula_worked_example():
    g = gold("sizes.json")["kv_size_formula"]
    assert oracle.kv_cache_bytes(g["layers"], g["tokens"], g["heads"], g["head_dim"],
                                 g["elem_bytes"]) == g["bytes"]


def test_llama7b_per_token_bytes():
    g = gold("sizes.json")["llama7b_per_token"]
    assert g["heads"] * g["head_dim"] == g["hidden"]
    assert oracle.kv_cache_bytes(1, 1, g["heads"], g["head_dim"], g["elem_bytes"]) == \
        g["bytes_per_layer_token"]
    assert oracle.kv_cache_bytes(g["layers"], 1, g["heads"], g["head_dim"],
                                 g["elem_bytes"]) == g["bytes_per_token"]
    assert oracle.kv_cache_bytes(g["layers"], g["tokens"], g["heads"], g["head_dim"],
                                 g["elem_bytes"]) == g["bytes_request"]


def test_page_table_rows():
    """A request of N tokens is served by exactly ceil(N / bs) table entries."""
    g = gold("sizes.json")["page_table_rows"]
    N = g["tokens"]
    for bs_s, rows in g["rows"].items():
        bs = int(bs_s)
        nb = rows + 1
        full = np.arange(rows, dtype=np.int32)[None, :]
        assert oracle.slot_of(full, 0, N - 1, bs, nb) >= 0
        short = full[:, :rows - 1]
        assert oracle.slot_of(short, 0, N - 1, bs, nb) == -1


def test_packing_examples():
    g = gold("packing.json")
    for key in ("three_requests", "four_requests"):
        offs, pos = oracle.pack(g[key]["lengths"])
        assert offs.tolist() == g[key]["seq_offset"]
        # position ids restart at 0 in every sequence
        for b, n in enumerate(g[key]["lengths"]):
            assert pos[offs[b]:offs[b + 1]].tolist() == list(range(n))
    f = g["four_requests"]
    assert oracle.pack(f["lengths"])[0][-1] == f["packed"]
    assert len(f["lengths"]) * max(f["lengths"]) == f["padded"]


def test_length_conventions():
    g = gold("packing.json")["length_conventions"]
    assert oracle.pack(g["kv_len"])[0][1:].tolist() == g["tnd_cumsum"]
    assert oracle.pack([1, 1])[0][1:].tolist() == g["decode_q_cumsum"]


def test_attention_reads_exactly_the_kv_size_formula():
    """One layer of the ai6s.net worked example (H=16, d=128, S=1024, 2-byte elements):
    the gather touches S rows of K and V per sequence; x 32 layers = 268,435,456 B."""
    g = gold("sizes.json")["kv_size_formula"]
    w = wl.custom(batch=1, num_q_heads=g["heads"], num_kv_heads=g["heads"],
                  head_dim=g["head_dim"], block_size=16, dtype="bf16")
    c = wl.make_case(w, [g["tokens"] - 1], [1], seed=3)
    h = case_numpy(c)
    out = oracle.decode_step(h, causal=False)
    _, _, touched = oracle.paged_attention(h["q"], out["cache_k"], out["cache_v"],
                                           h["block_table"], h["cu_q"], h["lens_after"],
                                           w.scale, False, want_touched=True)
    rows = int(touched.sum())
    assert rows == g["tokens"]
    per_layer = rows * w.num_kv_heads * (w.head_dim + w.head_dim_v) * w.elem_bytes
    assert per_layer * g["layers"] == g["bytes"]


def test_attention_touches_only_visible_rows():
    """Touched rows are exactly L'_b rows inside each sequence's own blocks, for tables
    whose unused entries hold INT32_MAX (never read)."""
    w = wl.custom(batch=3, num_q_heads=2, num_kv_heads=1, head_dim=8, block_size=4)
    c = wl.make_case(w, [0, 5, 11], [1, 1, 1], seed=5, max_blocks_per_seq=6)
    h = case_numpy(c)
    for b in range(w.batch):
        h["block_table"][b, c.need[b]:] = np.iinfo(np.int32).max
    r = oracle.decode_step(h, causal=False)
    _, _, touched = oracle.paged_attention(h["q"], r["cache_k"], r["cache_v"],
                                           h["block_table"], h["cu_q"], h["lens_after"],
                                           w.scale, False, want_touched=True)
    t = touched.reshape(c.num_blocks, w.block_size)
    for b in range(w.batch):
        for j in range(int(c.need[b])):
            P = int(c.block_table[b, j])
            valid = min(w.block_size, int(c.lens_after[b]) - j * w.block_size)
            assert t[P, :valid].all() and not t[P, valid:].any()
    assert int(touched.sum()) == int(c.lens_after.sum())
