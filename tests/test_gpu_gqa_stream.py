"""GPU parity of the bf16 GQA decode on the matrix cores (4..16 query heads per kv head)
against the fp64 oracle, through the C ABI: the range-streaming kernel (ranges of tiles
that cross sequence ends, many short sequences per range, fewer tiles than ranges, block
sizes down to one wave load) and the per-split kernel it leaves the other shapes to
(blocks smaller than a wave load, more than 1024 sequences).  Needs an MI355X."""
import numpy as np
import pytest
import torch

import paged_kv_cache_133_amd as pkv
from paged_kv_cache_133_amd import workloads as wl
from tests.gpu_common import compare_outputs, compare_writes, gpu_step, oracle_step, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# (Hq, Hkv, D, block_size, lengths after the step)
CASES = [
    (32, 8, 128, 4, [1, 2, 31, 32, 33, 64, 65, 100, 5, 300]),          # G 4, one wave load per block
    (40, 8, 128, 8, [700, 1, 1, 1, 40, 2, 96, 33]),                    # G 5: partial query rows
    (28, 4, 64, 16, [3, 1500, 17, 64, 1, 250]),                        # G 7, D 64
    (64, 4, 128, 32, [2047, 2048, 2049, 31, 1]),                       # G 16
    (16, 2, 64, 8, [9, 10, 11]),                                       # fewer tiles than ranges
    (16, 2, 128, 256, [5000, 6, 4100, 257, 255, 256]),
    (32, 4, 128, 2, [300, 2, 3, 77]),                                  # blocks < one wave load
    (16, 4, 64, 4, [129, 1, 64, 500]),                                 # D 64: 8 rows per wave load
    # longest sequence >= 8192 keys: the compact layout (two stages, 4 workgroups per CU)
    (32, 4, 128, 16, [8200, 1, 33, 9000, 31, 64]),                     # G 8
    (64, 4, 64, 32, [8192, 5, 3000, 1, 8300]),                         # G 16, D 64
    (16, 4, 128, 128, [12000, 2, 7, 100, 129]),                        # G 4, large blocks
]


def _case(Hq, Hkv, D, bs, L, seed):
    w = wl.custom(batch=len(L), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                  dtype="bf16")
    return wl.make_case(w, np.array(L) - 1, [1] * len(L), seed=seed, device=DEV)


@pytest.mark.parametrize("case", CASES, ids=lambda s: "hq%d_hkv%d_d%d_bs%d" % s[:4])
def test_gqa_mfma_decode(case):
    Hq, Hkv, D, bs, L = case
    say(f"gqa mfma decode: {case[:4]} L={L}")
    c = _case(Hq, Hkv, D, bs, L, seed=Hq + bs)
    g = gpu_step(c)
    o = oracle_step(c)
    compare_writes(c, g, o)
    err = compare_outputs(c, g, o, tokens=o["tokens"], label=str(case[:4]))
    say(f"  max-abs error {err:.3e}")


@pytest.mark.parametrize("case", CASES[:5] + CASES[-3:], ids=lambda s: "hq%d_hkv%d_d%d_bs%d" % s[:4])
def test_gqa_mfma_decode_append(case):
    """Write-and-attend in one pass: pool bytes, slots, outputs and lse as the oracle's."""
    Hq, Hkv, D, bs, L = case
    say(f"gqa mfma decode_append: {case[:4]} L={L}")
    c = _case(Hq, Hkv, D, bs, L, seed=3 * Hq + bs)
    o = oracle_step(c)
    B = len(L)
    k, v = c.cache_k.clone(), c.cache_v.clone()
    slots = torch.full((B,), -3, dtype=torch.int64, device=DEV)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    out, _ = pkv.paged_attn_decode_append(c.q, c.new_k, c.new_v, k, v, c.table_tensor(DEV),
                                          c.lens_after_tensor(DEV), c.max_len_after, c.w.scale,
                                          lse=lse, slots_out=slots)
    torch.cuda.synchronize()
    g = {"slots": slots, "cache_k": k, "cache_v": v, "out": out, "lse": lse}
    compare_writes(c, g, o)
    compare_outputs(c, g, o, tokens=o["tokens"], label=f"append {case[:4]}")


def test_gqa_mfma_many_sequences_sampled():
    """300 sequences of mixed lengths (many per range, ranges cutting through long ones)
    and 1100 short ones (past the range kernel's limit): sampled rows against the oracle."""
    rng = np.random.default_rng(11)
    for B, hi, bs in ((300, 3000, 16), (1100, 90, 16)):
        L = rng.integers(1, hi, size=B)
        L[::37] = 1
        w = wl.custom(batch=B, num_q_heads=32, num_kv_heads=4, head_dim=128, block_size=bs,
                      dtype="bf16")
        say(f"gqa mfma many sequences: B={B} max L={int(L.max())}")
        c = wl.make_case(w, L - 1, [1] * B, seed=B, device=DEV)
        g = gpu_step(c)
        rows = sorted({0, 1, B // 2, B - 1, int(np.argmax(L)), int(np.argmin(L)), 37, 74})
        o = oracle_step(c, rows=rows)
        compare_writes(c, g, o)
        compare_outputs(c, g, o, tokens=o["tokens"], label=f"B={B}")


def test_gqa_mfma_split_and_combine_equal_decode():
    """_split + _combine called separately == one decode call, bit for bit (the
    range-streaming kernel leaves its tile prefix in the workspace for the combine)."""
    from paged_kv_cache_133_amd import _lib
    c = _case(32, 4, 128, 16, [3000, 17, 1200, 1, 64], seed=9)
    g = gpu_step(c)
    out2 = torch.empty_like(g["out"])
    lse2 = torch.empty_like(g["lse"])
    split, combine, _, _ = _lib.prepare_decode(c.q, g["cache_k"], g["cache_v"], c.table_tensor(DEV),
                                               c.lens_after_tensor(DEV), c.max_len_after, c.w.scale,
                                               out=out2, lse=lse2)
    split()
    combine()
    torch.cuda.synchronize()
    assert torch.equal(g["out"].view(torch.int16), out2.view(torch.int16))
    assert torch.equal(g["lse"], lse2)


def test_gqa_compact_many_short_sequences():
    """The compact layout (one sequence of 5000 keys) with 400 sequences of 1..70 keys:
    many one- and two-tile segments per range; every row checked, writes included."""
    rng = np.random.default_rng(8)
    L = [int(x) for x in rng.integers(1, 71, size=400)] + [5000]
    say(f"gqa compact layout, many short sequences (B={len(L)})")
    c = _case(32, 4, 128, 16, L, seed=13)
    g = gpu_step(c)
    o = oracle_step(c)
    compare_writes(c, g, o)
    compare_outputs(c, g, o, tokens=o["tokens"], label="compact many short")
