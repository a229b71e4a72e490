"""GPU parity of the decode path (slot_mapping + cache write + split-KV attention +
combine) against the fp64 oracle, through the C ABI.  Needs an MI355X."""
import numpy as np
import pytest
import torch

from paged_kv_cache_133_amd import workloads as wl
from tests.gpu_common import compare_outputs, compare_writes, gpu_step, oracle_step, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# (Hq, Hkv, D, block_size, dtype): every group size class, both head dims, both dtypes,
# block sizes from 1 to 256
SHAPES = [
    (4, 1, 64, 16, "f32"),
    (8, 8, 128, 16, "bf16"),
    (16, 2, 128, 128, "bf16"),
    (12, 4, 64, 4, "bf16"),
    (16, 1, 64, 1, "f32"),
    (6, 6, 128, 2, "f32"),
    (32, 2, 128, 256, "bf16"),
    (2, 1, 128, 32, "f32"),
    (16, 16, 64, 64, "bf16"),
    # one query head per kv head, odd head counts: one kv head per workgroup (even counts
    # take adjacent pairs)
    (5, 5, 128, 8, "bf16"),
    (3, 3, 64, 16, "f32"),
]


def lengths_for(bs, rng, B=6, long=1300):
    """L_b before the step: values whose L' = L+1 sits at 0, 1 and bs-1 (mod bs), one
    sequence of a single token and one long enough for several splits."""
    L = [bs - 1, bs, 2 * bs - 2 if bs > 1 else 2, 0, long, int(rng.integers(1, 700))]
    return np.array(L[:B])


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "hq%d_hkv%d_d%d_bs%d_%s" % s)
def test_decode_parity_small(shape):
    Hq, Hkv, D, bs, dt = shape
    rng = np.random.default_rng(Hq * 7 + bs)
    w = wl.custom(batch=6, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                  dtype=dt)
    L = lengths_for(bs, rng)
    say(f"decode parity small: shape={shape} L={L.tolist()}")
    c = wl.make_case(w, L, [1] * 6, seed=int(rng.integers(1 << 30)), device=DEV)
    g = gpu_step(c)
    o = oracle_step(c)
    compare_writes(c, g, o)
    err = compare_outputs(c, g, o, tokens=o["tokens"], label=str(shape))
    say(f"  max-abs error {err:.3e}")


@pytest.mark.parametrize("name", ["tiny_gqa_f32", "llama7b_mha_bf16"])
def test_decode_parity_full_workload(name):
    """The full-size workload through slot_mapping + kv_cache_write + paged_attn_decode
    (the bench's `separate` path); every output row is checked."""
    w = wl.WORKLOADS[name]
    say(f"decode parity full: {name}")
    c = wl.make_workload_case(w, seed=0, device=DEV)
    g = gpu_step(c)
    o = oracle_step(c)
    compare_writes(c, g, o)
    err = compare_outputs(c, g, o, tokens=o["tokens"], label=name)
    say(f"  max-abs error {err:.3e}")


def test_decode_parity_gqa_long_full():
    """GQA 64/8, lengths up to 32K, every one of the 64 sequences against the oracle."""
    w = wl.GQA_LONG
    say("decode parity gqa_long (all rows)")
    c = wl.make_workload_case(w, seed=0, device=DEV)
    g = gpu_step(c)
    o = oracle_step(c)
    compare_writes(c, g, o)
    err = compare_outputs(c, g, o, tokens=o["tokens"], label="gqa_long")
    say(f"  {w.batch} rows, lens {int(c.lens_after.min())}..{int(c.lens_after.max())}, "
        f"max-abs error {err:.3e}")


def _append_full(name, seed=0):
    """One step of a full-size workload through paged_attn_decode_append (the bench's
    default, fused path: write folded into the split pass, then the combine) against the
    oracle's slot_mapping + write + attention: slots exactly, both whole pools byte for
    byte, every output row."""
    import paged_kv_cache_133_amd as pkv
    w = wl.WORKLOADS[name]
    say(f"decode_append full workload: {name} seed {seed}")
    c = wl.make_workload_case(w, seed=seed, device=DEV)
    o = oracle_step(c)
    k, v = c.cache_k.clone(), c.cache_v.clone()
    T = c.num_tokens
    slots = torch.full((T,), -5, dtype=torch.int64, device=DEV)
    lse = torch.empty((T, w.num_q_heads), dtype=torch.float32, device=DEV)
    out, _ = pkv.paged_attn_decode_append(c.q, c.new_k, c.new_v, k, v, c.table_tensor(DEV),
                                          c.lens_after_tensor(DEV), c.max_len_after, w.scale,
                                          lse=lse, slots_out=slots)
    torch.cuda.synchronize()
    g = {"slots": slots, "cache_k": k, "cache_v": v, "out": out, "lse": lse}
    compare_writes(c, g, o)
    err = compare_outputs(c, g, o, tokens=o["tokens"], label=f"decode_append {name}")
    say(f"  {w.batch} rows, max-abs error {err:.3e}")


def test_decode_append_full_workload_llama7b():
    _append_full("llama7b_mha_bf16")


def test_decode_append_full_workload_gqa_long():
    _append_full("gqa_long_bf16")


def test_decode_other_seeds_llama7b():
    for seed in (1, 2):
        say(f"decode parity llama7b seed {seed}")
        c = wl.make_workload_case(wl.LLAMA7B, seed=seed, device=DEV)
        g = gpu_step(c)
        o = oracle_step(c, rows=list(range(0, 32, 3)))
        compare_writes(c, g, o)
        compare_outputs(c, g, o, tokens=o["tokens"], label=f"llama7b seed {seed}")


def test_decode_is_deterministic_and_permutation_invariant():
    """Same logical content under two physical-block permutations: bitwise-equal output;
    and the same call twice gives the same bits."""
    w = wl.custom(batch=5, num_q_heads=16, num_kv_heads=4, head_dim=128, block_size=16,
                  dtype="bf16")
    L = [700, 15, 16, 1, 2000]
    say("decode permutation invariance")
    a = wl.make_case(w, L, [1] * 5, seed=21, device=DEV, perm_seed=1)
    b = wl.make_case(w, L, [1] * 5, seed=21, device=DEV, perm_seed=2)
    assert not np.array_equal(a.block_table, b.block_table)
    for src, dst in ((a.cache_k, b.cache_k), (a.cache_v, b.cache_v)):
        dst.fill_(float("nan"))
        for s in range(w.batch):
            for j in range(int(a.need[s])):
                dst[int(b.block_table[s, j])] = src[int(a.block_table[s, j])]
    ga = gpu_step(a)
    gb = gpu_step(b)
    ga2 = gpu_step(a)
    assert torch.equal(ga["out"].view(torch.int16), gb["out"].view(torch.int16))
    assert torch.equal(ga["lse"], gb["lse"])
    assert torch.equal(ga["out"].view(torch.int16), ga2["out"].view(torch.int16))


def test_decode_shared_prefix_blocks():
    """Two sequences read the same physical prefix blocks (a ref-counted shared prefix,
    source note 5.2): results match the oracle and a de-aliased copy bit for bit."""
    w = wl.custom(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                  dtype="bf16")
    L = [100, 90, 40]
    say("decode shared prefix")
    c = wl.make_case(w, L, [1] * 3, seed=33, device=DEV)
    # sequence 1 reuses sequence 0's first 4 blocks (64 tokens of identical prefix)
    spare = [int(x) for x in c.block_table[1, :4]]
    c.block_table[1, :4] = c.block_table[0, :4]
    g = gpu_step(c)
    o = oracle_step(c)
    compare_outputs(c, g, o, tokens=o["tokens"], label="shared prefix")
    # de-alias: copy the shared blocks into sequence 1's original blocks
    for j in range(4):
        c.cache_k[spare[j]] = c.cache_k[int(c.block_table[0, j])]
        c.cache_v[spare[j]] = c.cache_v[int(c.block_table[0, j])]
    c.block_table[1, :4] = spare
    g2 = gpu_step(c)
    assert torch.equal(g["out"].view(torch.int16), g2["out"].view(torch.int16))


def test_decode_without_lse_and_empty_batch():
    w = wl.custom(batch=2, num_q_heads=4, num_kv_heads=1, head_dim=64, block_size=16)
    c = wl.make_case(w, [37, 130], [1, 1], seed=0, device=DEV)
    g = gpu_step(c, want_lse=False)
    o = oracle_step(c)
    compare_outputs(c, g, o, tokens=o["tokens"], label="no lse")
    import paged_kv_cache_133_amd as pkv
    e = torch.empty((0, 4, 64), device=DEV)
    out, _ = pkv.paged_attn_decode(e, c.cache_k, c.cache_v, c.table_tensor(DEV)[:0],
                                   c.lens_after_tensor(DEV)[:0], 131, w.scale)
    torch.cuda.synchronize()
    assert out.shape == (0, 4, 64)


def test_append_matches_oracle_write():
    """slot_mapping + write fused in one launch: same slots and same pool bytes as the
    oracle, for one token per sequence and for multi-token chunks."""
    import paged_kv_cache_133_amd as pkv
    for w, L, n in [(wl.LLAMA7B, None, None),
                    (wl.custom(mode="varlen", batch=4, num_q_heads=8, num_kv_heads=2,
                               head_dim=128, block_size=16, dtype="bf16"),
                     [0, 15, 16, 300], [40, 1, 33, 17]),
                    (wl.custom(batch=3, num_q_heads=4, num_kv_heads=1, head_dim=64,
                               block_size=1, dtype="f32"), [5, 0, 9], [3, 2, 1])]:
        say(f"append parity: {w.name}")
        c = (wl.make_workload_case(w, seed=4, device=DEV) if L is None
             else wl.make_case(w, L, n, seed=4, device=DEV))
        o = oracle_step(c)
        k, v = c.cache_k.clone(), c.cache_v.clone()
        slots = torch.full((c.num_tokens,), -7, dtype=torch.int64, device=DEV)
        pkv.kv_cache_append(c.new_k, c.new_v, k, v, c.table_tensor(DEV), c.lens_before_tensor(DEV),
                            c.cu_q_tensor(DEV), c.max_new, slots_out=slots)
        torch.cuda.synchronize()
        g = {"slots": slots, "cache_k": k, "cache_v": v}
        compare_writes(c, g, o)


def test_two_launch_form_equals_decode():
    """_split + _combine called separately == pkv_paged_attn_decode, bit for bit, on a
    case with many splits."""
    from paged_kv_cache_133_amd import _lib
    w = wl.custom(batch=3, num_q_heads=16, num_kv_heads=2, head_dim=128, block_size=16,
                  dtype="bf16")
    c = wl.make_case(w, [3000, 17, 1200], [1, 1, 1], seed=7, device=DEV)
    say("split + combine vs decode")
    g = gpu_step(c)
    table, la = c.table_tensor(DEV), c.lens_after_tensor(DEV)
    out2 = torch.empty_like(g["out"])
    lse2 = torch.empty_like(g["lse"])
    split, combine, _, _ = _lib.prepare_decode(c.q, g["cache_k"], g["cache_v"], table, la,
                                               c.max_len_after, w.scale, out=out2, lse=lse2)
    split()
    combine()
    torch.cuda.synchronize()
    assert torch.equal(g["out"].view(torch.int16), out2.view(torch.int16))
    assert torch.equal(g["lse"], lse2)


def test_workspace_reuse():
    """The same workspace serves several decode calls in a row, with lengths that change
    between calls (no state survives from one call to the next)."""
    import paged_kv_cache_133_amd as pkv
    w = wl.custom(batch=4, num_q_heads=8, num_kv_heads=8, head_dim=128, block_size=16,
                  dtype="bf16")
    ws = pkv.new_decode_workspace(4, 8, 8, 128, 4096, DEV)
    for it, L in enumerate([[4000, 100, 2000, 3000], [257, 4095, 1, 600], [4095, 4095, 4095, 4095]]):
        say(f"workspace reuse call {it}: L={L}")
        c = wl.make_case(w, L, [1] * 4, seed=50 + it, device=DEV, max_blocks_per_seq=256)
        k, v = c.cache_k.clone(), c.cache_v.clone()
        table = c.table_tensor(DEV)
        slots = pkv.slot_mapping(table, c.lens_before_tensor(DEV), c.cu_q_tensor(DEV), 16, 4)
        pkv.kv_cache_write(c.new_k, c.new_v, k, v, slots)
        lse = torch.empty((4, 8), dtype=torch.float32, device=DEV)
        out, _ = pkv.paged_attn_decode(c.q, k, v, table, c.lens_after_tensor(DEV), 4096, w.scale,
                                       lse=lse, workspace=ws)
        torch.cuda.synchronize()
        o = oracle_step(c)
        compare_outputs(c, {"out": out, "lse": lse}, o, tokens=o["tokens"], label=f"reuse {it}")


@pytest.mark.parametrize("shape", [(32, 32, 128, 16, "bf16"), (8, 2, 64, 1, "f32"),
                                   (16, 2, 128, 128, "bf16"), (4, 1, 128, 32, "f32"),
                                   (6, 6, 128, 1, "f32"), (5, 5, 64, 16, "bf16")],
                         ids=lambda s: "hq%d_hkv%d_d%d_bs%d_%s" % s)
def test_decode_append_matches_oracle(shape):
    """Write-and-attend in one pass: the written pool, the slots and the outputs equal the
    oracle's slot_mapping + write + attention; and they equal append + decode bit for bit."""
    import paged_kv_cache_133_amd as pkv
    Hq, Hkv, D, bs, dt = shape
    w = wl.custom(batch=6, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                  dtype=dt)
    L = lengths_for(bs, np.random.default_rng(3))
    say(f"decode_append parity: {shape} L={L.tolist()}")
    c = wl.make_case(w, L, [1] * 6, seed=77, device=DEV)
    o = oracle_step(c)
    table, la = c.table_tensor(DEV), c.lens_after_tensor(DEV)
    k, v = c.cache_k.clone(), c.cache_v.clone()
    slots = torch.full((6,), -3, dtype=torch.int64, device=DEV)
    lse = torch.empty((6, Hq), dtype=torch.float32, device=DEV)
    out, _ = pkv.paged_attn_decode_append(c.q, c.new_k, c.new_v, k, v, table, la,
                                          c.max_len_after, w.scale, lse=lse, slots_out=slots)
    torch.cuda.synchronize()
    g = {"slots": slots, "cache_k": k, "cache_v": v, "out": out, "lse": lse}
    compare_writes(c, g, o)
    compare_outputs(c, g, o, tokens=o["tokens"], label=f"decode_append {shape}")
    ref = gpu_step(c)
    assert torch.equal(out.view(torch.int16) if dt == "bf16" else out.view(torch.int32),
                       ref["out"].view(torch.int16) if dt == "bf16" else ref["out"].view(torch.int32))
    assert torch.equal(lse, ref["lse"])


@pytest.mark.parametrize("shape", [(8, 8, 128, 16, "bf16"), (4, 1, 64, 16, "f32"),
                                   (16, 2, 128, 16, "bf16"), (16, 2, 128, 2, "bf16"),
                                   (3, 3, 128, 16, "bf16")],
                         ids=lambda s: "hq%d_hkv%d_d%d_bs%d_%s" % s)
def test_decode_append_overlength_row_writes_nothing(shape):
    """A row whose length exceeds max_seq_len_kv (a broken precondition) appends nothing in
    the fused write-and-attend call: its slot is reported as -1, the pools keep their bytes
    there, and it attends to its first max_seq_len_kv cached keys, exactly as the plain
    decode does.  The other rows are written and attended as usual."""
    import paged_kv_cache_133_amd as pkv
    from oracle import oracle
    from tests.helpers import case_numpy, host
    Hq, Hkv, D, bs, dt = shape
    w = wl.custom(batch=3, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                  dtype=dt)
    L = [99, 299, 49]            # L' = 100, 300, 50
    cap = 200                    # row 1 is over the bound
    say(f"decode_append over-length row: {shape}")
    c = wl.make_case(w, L, [1] * 3, seed=91, device=DEV)
    h = case_numpy(c)
    all_slots = oracle.slot_mapping(h["block_table"], h["lens_before"], h["cu_q"],
                                    h["block_size"], h["num_blocks"])
    keep = np.array([0, 2])
    ref_k = oracle.kv_write(h["cache_k"], h["new_k"][keep], all_slots[keep])
    ref_v = oracle.kv_write(h["cache_v"], h["new_v"][keep], all_slots[keep])
    k, v = c.cache_k.clone(), c.cache_v.clone()
    table, la = c.table_tensor(DEV), c.lens_after_tensor(DEV)
    slots = torch.full((3,), -9, dtype=torch.int64, device=DEV)
    out, _ = pkv.paged_attn_decode_append(c.q, c.new_k, c.new_v, k, v, table, la, cap, w.scale,
                                          slots_out=slots)
    torch.cuda.synchronize()
    exp_slots = all_slots.copy()
    exp_slots[1] = -1
    assert np.array_equal(slots.cpu().numpy(), exp_slots)
    assert host(k).tobytes() == ref_k.tobytes()
    assert host(v).tobytes() == ref_v.tobytes()
    # the plain decode over the written pools with the same bound: the same bits
    plain, _ = pkv.paged_attn_decode(c.q, k, v, table, la, cap, w.scale)
    torch.cuda.synchronize()
    ity = torch.int16 if dt == "bf16" else torch.int32
    assert torch.equal(out.view(ity), plain.view(ity))
    # and the oracle over those pools, row 1 cut to its first `cap` keys
    lens = np.minimum(c.lens_after, cap).astype(np.int32)
    ref_out, _ = oracle.paged_attention(h["q"], ref_k, ref_v, c.block_table,
                                        np.arange(4, dtype=np.int32), lens, w.scale, False)
    err = float(np.abs(out.float().cpu().numpy().astype(np.float64) - ref_out).max())
    assert err <= {"f32": 1e-5, "bf16": 2e-2}[dt], err
