"""GPU parity of the MFMA paths against the fp64 oracle, through the C ABI: the
MLA-absorbed decode (key = nope || rope, value = nope) and the packed varlen causal
chunk (bottom-right causal, self included).  Needs an MI355X."""
import numpy as np
import pytest
import torch

import paged_kv_cache_133_amd as pkv
from paged_kv_cache_133_amd import workloads as wl
from tests.gpu_common import compare_outputs, compare_writes, gpu_step, oracle_step, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


# 160 and 256 heads: two workgroups (head groups of 128) per (sequence, split)
@pytest.mark.parametrize("hq,bs", [(128, 128), (64, 16), (32, 1), (96, 64), (16, 32), (160, 16), (256, 64)])
def test_mla_decode_parity_small(hq, bs):
    w = wl.custom(mode="mla", batch=5, num_q_heads=hq, num_kv_heads=1, head_dim=512,
                  head_dim_rope=64, block_size=bs, dtype="bf16")
    # L' on block/tile edges (1, 32, 33, bs-1, bs+1) and one sequence over several splits
    L = [0, 31, 32, max(bs - 2, 3), 2600]
    say(f"mla parity: hq={hq} bs={bs} L={L}")
    c = wl.make_case(w, L, [1] * 5, seed=hq + bs, device=DEV)
    g = gpu_step(c)
    o = oracle_step(c)
    compare_writes(c, g, o)
    err = compare_outputs(c, g, o, tokens=o["tokens"], label=f"mla hq={hq} bs={bs}")
    say(f"  max-abs error {err:.3e}")


def test_mla_full_workload():
    """B = 64, 128 heads, lengths U{2048..8192}: every sequence against the oracle, and
    both written pools (nope and rope) byte for byte."""
    w = wl.MLA
    say("mla full workload (all rows)")
    c = wl.make_workload_case(w, seed=0, device=DEV)
    g = gpu_step(c)
    o = oracle_step(c)
    compare_writes(c, g, o)
    err = compare_outputs(c, g, o, tokens=o["tokens"], label="mla full")
    say(f"  {w.batch} rows, lens {int(c.lens_after.min())}..{int(c.lens_after.max())}, "
        f"max-abs error {err:.3e}")


def _mla_append(c, cap=None):
    """pkv_paged_attn_decode_mla_append on fresh copies of the case's pools."""
    k, rope = c.cache_k.clone(), c.cache_rope.clone()
    B = c.w.batch
    slots = torch.full((B,), -5, dtype=torch.int64, device=DEV)
    lse = torch.empty((B, c.w.num_q_heads), dtype=torch.float32, device=DEV)
    out, _ = pkv.paged_attn_decode_mla_append(c.q, c.q_rope, c.new_k, c.new_rope, k, rope,
                                              c.table_tensor(DEV), c.lens_after_tensor(DEV),
                                              c.max_len_after if cap is None else cap,
                                              c.w.scale, lse=lse, slots_out=slots)
    torch.cuda.synchronize()
    return {"slots": slots, "cache_k": k, "cache_v": k, "cache_rope": rope, "out": out,
            "lse": lse}


@pytest.mark.parametrize("hq,bs", [(128, 128), (64, 16), (32, 1), (16, 32)])
def test_mla_decode_append_parity_small(hq, bs):
    """The latent write folded into the MLA split pass: the slots, both written pools and
    the outputs equal the oracle's slot_mapping + write + attention, and they equal the
    separate write + decode bit for bit (the new key sits on a tile edge in some rows)."""
    w = wl.custom(mode="mla", batch=6, num_q_heads=hq, num_kv_heads=1, head_dim=512,
                  head_dim_rope=64, block_size=bs, dtype="bf16")
    L = [0, 31, 32, 63, max(bs - 1, 3), 2600]
    say(f"mla append parity: hq={hq} bs={bs} L={L}")
    c = wl.make_case(w, L, [1] * 6, seed=hq * 7 + bs, device=DEV)
    g = _mla_append(c)
    o = oracle_step(c)
    compare_writes(c, g, o)
    err = compare_outputs(c, g, o, tokens=o["tokens"], label=f"mla append hq={hq} bs={bs}")
    say(f"  max-abs error {err:.3e}")
    ref = gpu_step(c)
    assert torch.equal(g["out"].view(torch.int16), ref["out"].view(torch.int16))
    assert torch.equal(g["lse"], ref["lse"])


def test_mla_decode_append_full_workload():
    """B = 64, 128 heads, lengths U{2048..8192} through the fused MLA step: every row against
    the oracle, the slots exactly, both pools byte for byte."""
    say("mla append full workload (all rows)")
    c = wl.make_workload_case(wl.MLA, seed=0, device=DEV)
    g = _mla_append(c)
    o = oracle_step(c)
    compare_writes(c, g, o)
    err = compare_outputs(c, g, o, tokens=o["tokens"], label="mla append full")
    say(f"  max-abs error {err:.3e}")


def test_mla_decode_append_overlength_row_writes_nothing():
    """A row longer than max_seq_len_kv writes nothing (slot -1, pools unchanged there) and
    attends to its first max_seq_len_kv keys, like the plain MLA decode with that bound."""
    from oracle import oracle
    from tests.helpers import case_numpy, host
    w = wl.custom(mode="mla", batch=3, num_q_heads=64, num_kv_heads=1, head_dim=512,
                  head_dim_rope=64, block_size=16, dtype="bf16")
    cap = 200
    say("mla append over-length row")
    c = wl.make_case(w, [99, 299, 49], [1] * 3, seed=93, device=DEV)
    h = case_numpy(c)
    all_slots = oracle.slot_mapping(h["block_table"], h["lens_before"], h["cu_q"],
                                    h["block_size"], h["num_blocks"])
    keep = np.array([0, 2])
    ref_k = oracle.kv_write(h["cache_k"], h["new_k"][keep], all_slots[keep])
    ref_r = oracle.kv_write(h["cache_rope"], h["new_rope"][keep], all_slots[keep])
    g = _mla_append(c, cap=cap)
    exp_slots = all_slots.copy()
    exp_slots[1] = -1
    assert np.array_equal(g["slots"].cpu().numpy(), exp_slots)
    assert host(g["cache_k"]).tobytes() == ref_k.tobytes()
    assert host(g["cache_rope"]).tobytes() == ref_r.tobytes()
    plain, _ = pkv.paged_attn_decode(c.q, g["cache_k"], g["cache_k"], c.table_tensor(DEV),
                                     c.lens_after_tensor(DEV), cap, w.scale, q_rope=c.q_rope,
                                     k_rope_cache=g["cache_rope"])
    torch.cuda.synchronize()
    assert torch.equal(g["out"].view(torch.int16), plain.view(torch.int16))
    lens = np.minimum(c.lens_after, cap).astype(np.int32)
    ref_out, _ = oracle.paged_attention(h["q"], ref_k, ref_k, c.block_table,
                                        np.arange(4, dtype=np.int32), lens, w.scale, False,
                                        q_rope=h["q_rope"], k_rope=ref_r)
    err = float(np.abs(g["out"].float().cpu().numpy().astype(np.float64) - ref_out).max())
    assert err <= 2e-2, err


def test_mla_split_and_combine_equal_decode():
    w = wl.custom(mode="mla", batch=3, num_q_heads=128, num_kv_heads=1, head_dim=512,
                  head_dim_rope=64, block_size=128, dtype="bf16")
    c = wl.make_case(w, [3000, 100, 1500], [1] * 3, seed=5, device=DEV)
    g = gpu_step(c)
    from paged_kv_cache_133_amd import _lib
    out2 = torch.empty_like(g["out"])
    lse2 = torch.empty_like(g["lse"])
    split, combine, _, _ = _lib.prepare_decode(c.q, g["cache_k"], g["cache_k"], c.table_tensor(DEV),
                                               c.lens_after_tensor(DEV), c.max_len_after, w.scale,
                                               q_rope=c.q_rope, k_rope_cache=g["cache_rope"],
                                               out=out2, lse=lse2)
    split()
    combine()
    torch.cuda.synchronize()
    assert torch.equal(g["out"].view(torch.int16), out2.view(torch.int16))
    assert torch.equal(g["lse"], lse2)


def test_mla_deterministic_and_permutation_invariant():
    w = wl.custom(mode="mla", batch=3, num_q_heads=128, num_kv_heads=1, head_dim=512,
                  head_dim_rope=64, block_size=16, dtype="bf16")
    L = [1200, 5, 700]
    a = wl.make_case(w, L, [1] * 3, seed=9, device=DEV, perm_seed=1)
    b = wl.make_case(w, L, [1] * 3, seed=9, device=DEV, perm_seed=2)
    for src, dst in ((a.cache_k, b.cache_k), (a.cache_rope, b.cache_rope)):
        dst.fill_(float("nan"))
        for s in range(w.batch):
            for j in range(int(a.need[s])):
                dst[int(b.block_table[s, j])] = src[int(a.block_table[s, j])]
    ga, gb, ga2 = gpu_step(a), gpu_step(b), gpu_step(a)
    assert torch.equal(ga["out"].view(torch.int16), gb["out"].view(torch.int16))
    assert torch.equal(ga["out"].view(torch.int16), ga2["out"].view(torch.int16))


VARLEN_SHAPES = [  # (Hq, Hkv, D, bs)
    (32, 8, 128, 128), (8, 8, 128, 16), (16, 1, 64, 32), (12, 4, 64, 1), (48, 3, 128, 64),
]


@pytest.mark.parametrize("shape", VARLEN_SHAPES, ids=lambda s: "hq%d_hkv%d_d%d_bs%d" % s)
@pytest.mark.parametrize("causal", [True, False])
def test_varlen_parity_small(shape, causal):
    Hq, Hkv, D, bs = shape
    w = wl.custom(mode="varlen", batch=5, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                  block_size=bs, dtype="bf16")
    # prefixes 0 (plain causal self-attention), on block edges, and chunks that span
    # several query blocks with ragged tails
    L = [0, bs - 1, 37, 2 * bs, 300]
    n = [45, 1, 70, 9, 130]
    say(f"varlen parity: {shape} causal={causal} L={L} n={n}")
    c = wl.make_case(w, L, n, seed=Hq * 3 + D + bs, device=DEV)
    g = gpu_step(c, causal=causal)
    o = oracle_step(c, causal=causal)
    compare_writes(c, g, o)
    err = compare_outputs(c, g, o, tokens=o["tokens"], label=f"varlen {shape} causal={causal}")
    say(f"  max-abs error {err:.3e}")


def test_varlen_full_workload():
    """16 sequences, lognormal chunk lengths, prefixes U{0..4096}: every query row of
    every sequence against the oracle, and both written pools byte for byte."""
    w = wl.VARLEN
    say("varlen full workload (all rows)")
    c = wl.make_workload_case(w, seed=0, device=DEV)
    g = gpu_step(c, causal=True)
    o = oracle_step(c, causal=True)
    compare_writes(c, g, o)
    err = compare_outputs(c, g, o, tokens=o["tokens"], label="varlen full")
    say(f"  {c.num_tokens} rows, n {int(c.n_new.min())}..{int(c.n_new.max())}, "
        f"max-abs error {err:.3e}")


def test_varlen_single_token_rows_equal_decode():
    """A chunk of one token per sequence is a decode step: varlen == decode output."""
    w = wl.custom(mode="varlen", batch=4, num_q_heads=16, num_kv_heads=4, head_dim=128,
                  block_size=16, dtype="bf16")
    c = wl.make_case(w, [100, 0, 31, 640], [1, 1, 1, 1], seed=12, device=DEV)
    g = gpu_step(c, causal=True)
    dec, _ = pkv.paged_attn_decode(c.q, g["cache_k"], g["cache_v"], c.table_tensor(DEV),
                                   c.lens_after_tensor(DEV), c.max_len_after, w.scale)
    torch.cuda.synchronize()
    diff = (g["out"].float() - dec.float()).abs().max().item()
    assert diff <= 2e-2
