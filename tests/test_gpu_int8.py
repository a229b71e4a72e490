"""GPU parity of the INT8 KV cache against the oracle, through the C ABI: the quantizing
write bit for bit (codes and fp32 scales, all other bytes unchanged, out-of-pool slots
skipped), and decode over the int8 caches against fp64 attention over the exactly
dequantized rows.  Needs an MI355X."""
import numpy as np
import pytest
import torch

import paged_kv_cache_133_amd as pkv
from oracle import oracle
from paged_kv_cache_133_amd import _lib
from paged_kv_cache_133_amd import workloads as wl
from tests.gpu_common import LSE_REL, lse_error, say
from tests.helpers import host

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.mark.parametrize("dtype,hkv,d,bs", [("bf16", 8, 128, 16), ("f32", 1, 64, 1),
                                            ("bf16", 4, 64, 128), ("f32", 2, 128, 32)])
def test_int8_write_bit_exact(dtype, hkv, d, bs):
    td = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    g = torch.Generator().manual_seed(hkv * d + bs)
    T = 29
    nb = max(8, (2 * T + bs - 1) // bs)
    k_new = (torch.randn(T, hkv, d, generator=g) * torch.rand(T, hkv, 1, generator=g) * 50).to(td)
    v_new = (torch.randn(T, hkv, d, generator=g) * 0.01).to(td)
    k_new[3] = 0                                   # zero rows: scale 0, zero codes
    v_new[7, 0] = 0
    slots = torch.randperm(nb * bs, generator=g)[:T].to(torch.int64)
    slots[11] = -1
    slots[12] = nb * bs
    kc = torch.randint(-128, 128, (nb, bs, hkv, d), generator=g, dtype=torch.int8)
    vc = torch.randint(-128, 128, (nb, bs, hkv, d), generator=g, dtype=torch.int8)
    ks = torch.randn(nb, hkv, bs, generator=g)     # [block][kv head][offset]
    vs = torch.randn(nb, hkv, bs, generator=g)
    say(f"int8 write {dtype} hkv={hkv} d={d} bs={bs}")
    dk, dv, dks, dvs = kc.to(DEV), vc.to(DEV), ks.to(DEV), vs.to(DEV)
    pkv.kv_cache_write_int8(k_new.to(DEV), v_new.to(DEV), dk, dv, dks, dvs, slots.to(DEV))
    torch.cuda.synchronize()
    ok = ((slots >= 0) & (slots < nb * bs)).numpy()
    sl = slots.numpy()[ok]
    for new, cache, scale, gc, gs in ((k_new, kc, ks, dk, dks), (v_new, vc, vs, dv, dvs)):
        q, s = oracle.quantize_rows(host(new))                     # [T, hkv, d], [T, hkv]
        exp_c = cache.numpy().reshape(nb * bs, hkv, d).copy()
        exp_s = scale.permute(0, 2, 1).numpy().reshape(nb * bs, hkv).copy()   # per slot
        exp_c[sl] = q[ok]
        exp_s[sl] = s[ok]
        assert np.array_equal(gc.cpu().numpy().reshape(nb * bs, hkv, d), exp_c)
        got_s = gs.cpu().permute(0, 2, 1).contiguous().numpy().reshape(nb * bs, hkv)
        assert np.array_equal(got_s.view(np.uint32), exp_s.view(np.uint32))


def _int8_case(Hq, Hkv, D, bs, L, seed):
    """A decode case whose pool rows are int8 codes and scales (the oracle's quantization of
    a bf16 pool), with the step's new rows written by the GPU's quantizing write."""
    w = wl.custom(batch=len(L), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                  dtype="bf16")
    c = wl.make_case(w, np.array(L) - 1, [1] * len(L), seed=seed, device=DEV, poison=False)
    nb = c.num_blocks
    kq, ksc = oracle.quantize_rows(host(c.cache_k))
    vq, vsc = oracle.quantize_rows(host(c.cache_v))
    # scales per (slot, kv head) from the oracle, stored [block][kv head][offset]
    dev = {"kc": torch.from_numpy(kq).to(DEV), "vc": torch.from_numpy(vq).to(DEV),
           "ks": torch.from_numpy(ksc).permute(0, 2, 1).contiguous().to(DEV),
           "vs": torch.from_numpy(vsc).permute(0, 2, 1).contiguous().to(DEV)}
    table = c.table_tensor(DEV)
    slots = pkv.slot_mapping(table, c.lens_before_tensor(DEV), c.cu_q_tensor(DEV), bs, c.num_tokens)
    pkv.kv_cache_write_int8(c.new_k, c.new_v, dev["kc"], dev["vc"], dev["ks"], dev["vs"], slots)
    torch.cuda.synchronize()
    # the oracle's view of the written caches
    sl = slots.cpu().numpy()
    nq, ns = oracle.quantize_rows(host(c.new_k))
    kq = kq.reshape(nb * bs, Hkv, D)
    kq[sl] = nq
    ksc = ksc.reshape(nb * bs, Hkv)
    ksc[sl] = ns
    nq, ns = oracle.quantize_rows(host(c.new_v))
    vq = vq.reshape(nb * bs, Hkv, D)
    vq[sl] = nq
    vsc = vsc.reshape(nb * bs, Hkv)
    vsc[sl] = ns
    assert np.array_equal(dev["kc"].cpu().numpy().reshape(nb * bs, Hkv, D), kq)
    assert np.array_equal(dev["vs"].cpu().permute(0, 2, 1).contiguous().numpy().reshape(nb * bs, Hkv), vsc)
    assert np.array_equal(dev["ks"].cpu().permute(0, 2, 1).contiguous().numpy().reshape(nb * bs, Hkv), ksc)
    kdeq = oracle.dequantize_rows(kq, ksc).reshape(nb, bs, Hkv, D)
    vdeq = oracle.dequantize_rows(vq, vsc).reshape(nb, bs, Hkv, D)
    return c, dev, table, kdeq, vdeq


def _check(c, out, lse, kdeq, vdeq, window, rows=None):
    idx = np.arange(c.w.batch) if rows is None else np.asarray(rows)
    q = oracle.widen(host(c.q))[idx]
    cu = np.arange(len(idx) + 1, dtype=np.int32)
    o, ol = oracle.paged_attention(q, kdeq, vdeq, c.block_table[idx], cu, c.lens_after[idx],
                                   c.w.scale, False, window=window)
    got = out.float().cpu().numpy()[idx]
    err = np.abs(got - o).max()
    assert err <= 2e-2, f"max-abs error {err:.3e}"
    _check_lse(c, lse.cpu().numpy()[idx], ol)
    return err


def _check_lse(c, got, ol):
    """Both INT8 kernels (1..4 and 5..16 query heads per kv head) sum fp32 weights."""
    lerr = lse_error(got, ol)
    assert lerr <= LSE_REL, f"lse error {lerr:.3e}"


@pytest.mark.parametrize("shape", [(32, 32, 128, 16), (8, 2, 64, 1), (16, 4, 128, 128),
                                   (4, 1, 128, 32), (12, 4, 64, 64),
                                   # MHA: kv head pairs (even counts) and single heads
                                   (6, 6, 64, 1), (3, 3, 128, 16),
                                   # 5..16 query heads per kv head: the range-streaming kernel
                                   (32, 4, 128, 16), (64, 4, 64, 16), (40, 8, 128, 8),
                                   (16, 2, 128, 128), (48, 4, 64, 32)],
                         ids=lambda s: "hq%d_hkv%d_d%d_bs%d" % s)
@pytest.mark.parametrize("window", [0, 100])
def test_int8_decode(shape, window):
    Hq, Hkv, D, bs = shape
    L = [1, 31, 32, 33, 300, 1500, 3000]
    say(f"int8 decode {shape} window {window}")
    c, dev, table, kdeq, vdeq = _int8_case(Hq, Hkv, D, bs, L, seed=Hq + bs + window)
    lse = torch.empty((len(L), Hq), dtype=torch.float32, device=DEV)
    out, _ = pkv.paged_attn_decode_int8(c.q, dev["kc"], dev["vc"], dev["ks"], dev["vs"], table,
                                        c.lens_after_tensor(DEV), c.max_len_after, c.w.scale,
                                        lse=lse, window=window)
    torch.cuda.synchronize()
    say(f"  max-abs error {_check(c, out, lse, kdeq, vdeq, window):.3e}")


def test_int8_headline_workload():
    """The INT8 headline workload at full size (B = 32, 32 heads, lengths 513..2049): the
    whole pool quantized by the oracle, the step's rows by the GPU writer, decode on the GPU;
    every sequence checked."""
    w = wl.WORKLOADS["llama7b_mha_int8"]
    L, _ = wl.sample_lengths(w, 0)
    say("int8 headline workload (all rows)")
    c, dev, table, kdeq, vdeq = _int8_case(w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size,
                                           list(np.asarray(L) + 1), seed=0)
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=DEV)
    out, _ = pkv.paged_attn_decode_int8(c.q, dev["kc"], dev["vc"], dev["ks"], dev["vs"], table,
                                        c.lens_after_tensor(DEV), c.max_len_after, c.w.scale,
                                        lse=lse)
    torch.cuda.synchronize()
    _check(c, out, lse, kdeq, vdeq, 0)


@pytest.mark.parametrize("shape", [(32, 4, 128, 16), (64, 4, 64, 16), (12, 4, 128, 32)],
                         ids=lambda s: "hq%d_hkv%d_d%d_bs%d" % s)
def test_int8_decode_padding_rows(shape):
    """Rows with seq_lens_kv = 0 (padding): output 0 and lse -inf; the others as the oracle
    says (both kernels: 12:4 the split one, 8 and 16 per kv head the range one)."""
    Hq, Hkv, D, bs = shape
    L = [40, 700, 9, 2100, 64, 33]
    say(f"int8 decode padding rows {shape}")
    c, dev, table, kdeq, vdeq = _int8_case(Hq, Hkv, D, bs, L, seed=Hq + D)
    lens = c.lens_after_tensor(DEV).clone()
    pad = [0, 3]
    lens[pad] = 0
    lse = torch.full((len(L), Hq), 7.0, dtype=torch.float32, device=DEV)
    out, _ = pkv.paged_attn_decode_int8(c.q, dev["kc"], dev["vc"], dev["ks"], dev["vs"], table,
                                        lens, c.max_len_after, c.w.scale, lse=lse)
    torch.cuda.synchronize()
    got, got_lse = out.float().cpu(), lse.cpu()
    for b in pad:
        assert (got[b] == 0).all() and torch.isneginf(got_lse[b]).all()
    _check(c, out, lse, kdeq, vdeq, 0, rows=[1, 2, 4, 5])


def test_int8_two_passes_equal_one_ranges():
    """The range pass and the combine as two calls give the one-call result bit for bit
    (8 query heads per kv head)."""
    L = [3000, 5, 1400, 64, 65, 2222, 1, 800]
    c, dev, table, kdeq, vdeq = _int8_case(32, 4, 128, 16, L, seed=11)
    la = c.lens_after_tensor(DEV)
    args = (c.q, dev["kc"], dev["vc"], dev["ks"], dev["vs"], table, la, c.max_len_after, c.w.scale)
    lse1 = torch.empty((len(L), 32), dtype=torch.float32, device=DEV)
    out1, _ = pkv.paged_attn_decode_int8(*args, lse=lse1)
    lse2 = torch.empty_like(lse1)
    first, second, out2 = _lib.prepare_decode_int8(*args, lse=lse2)
    first()
    second()
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse1.view(torch.int32), lse2.view(torch.int32))
    _check(c, out1, lse1, kdeq, vdeq, 0)


def test_int8_gqa_long_workload_sampled():
    """The long-context GQA workload over the INT8 cache at full size (B = 64, 64 q / 8 kv
    heads, bs 128, lengths log-uniform [1024, 32768]).  The pool is seeded random codes and
    scales (quantizing 600M elements on the host would take minutes; the writer has its own
    bit-exact tests); the oracle dequantizes the blocks of four sequences and checks them."""
    w = wl.WORKLOADS["gqa_long_int8"]
    L, _ = wl.sample_lengths(w, 0)
    say("int8 gqa_long workload (sampled sequences)")
    c = wl.make_case(w, L, [1] * w.batch, seed=0, device=DEV, poison=False)
    nb, bs, hkv, d = c.cache_k.shape
    gen = torch.Generator(device=DEV).manual_seed(1234)
    codes = [torch.randint(-127, 128, (nb, bs, hkv, d), generator=gen, device=DEV, dtype=torch.int8)
             for _ in range(2)]
    scales = [torch.rand((nb, hkv, bs), generator=gen, device=DEV) * 0.03 + 1e-3 for _ in range(2)]
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=DEV)
    out, _ = pkv.paged_attn_decode_int8(c.q, codes[0], codes[1], scales[0], scales[1],
                                        c.table_tensor(DEV), c.lens_after_tensor(DEV),
                                        c.max_len_after, c.w.scale, lse=lse)
    torch.cuda.synchronize()
    order = np.argsort(c.lens_after)
    rows = sorted({int(order[0]), int(order[-1]), int(order[len(order) // 2]), 3})
    # a compact pool of the sampled sequences' blocks, the table renumbered into it
    used = [c.block_table[b][:(int(c.lens_after[b]) + bs - 1) // bs] for b in rows]
    blocks = np.concatenate(used).astype(np.int64)
    sel = torch.from_numpy(blocks).to(DEV)
    deq = []
    for cd, sc in zip(codes, scales):
        q8 = cd[sel].cpu().numpy()                                   # [n, bs, hkv, d]
        s32 = sc[sel].permute(0, 2, 1).contiguous().cpu().numpy()    # [n, bs, hkv]
        deq.append(oracle.dequantize_rows(q8, s32))
    table = np.zeros((len(rows), max(len(u) for u in used)), np.int32)
    k = 0
    for i, u in enumerate(used):
        table[i, :len(u)] = np.arange(k, k + len(u))
        k += len(u)
    cu = np.arange(len(rows) + 1, dtype=np.int32)
    o, ol = oracle.paged_attention(oracle.widen(host(c.q))[rows], deq[0], deq[1], table, cu,
                                   c.lens_after[rows], c.w.scale, False)
    err = float(np.abs(out.float().cpu().numpy()[rows] - o).max())
    assert err <= 2e-2, f"max-abs error {err:.3e}"
    _check_lse(c, lse.cpu().numpy()[rows], ol)
    say(f"  max-abs error {err:.3e}")


def test_int8_ranges_many_short_sequences():
    """300 sequences of 1..70 keys and one of 6000 at 8 query heads per kv head: ranges hold
    many one- and two-tile segments in a row, so the next segment's query fragments are
    issued while the previous segment is still in use; every row checked."""
    rng = np.random.default_rng(5)
    L = [int(x) for x in rng.integers(1, 71, size=300)] + [6000]
    say(f"int8 ranges, many short sequences (B={len(L)})")
    c, dev, table, kdeq, vdeq = _int8_case(32, 4, 128, 16, L, seed=21)
    lse = torch.empty((len(L), 32), dtype=torch.float32, device=DEV)
    out, _ = pkv.paged_attn_decode_int8(c.q, dev["kc"], dev["vc"], dev["ks"], dev["vs"], table,
                                        c.lens_after_tensor(DEV), c.max_len_after, c.w.scale, lse=lse)
    torch.cuda.synchronize()
    say(f"  max-abs error {_check(c, out, lse, kdeq, vdeq, 0):.3e}")


def _code_pools(c):
    """Two device copies of the INT8 pools (codes, [block][kv head][offset] scales): the
    oracle's quantization of the case's bf16 pools."""
    kq, ksc = oracle.quantize_rows(host(c.cache_k))
    vq, vsc = oracle.quantize_rows(host(c.cache_v))
    one = lambda: {"kc": torch.from_numpy(kq).to(DEV), "vc": torch.from_numpy(vq).to(DEV),  # noqa: E731
                   "ks": torch.from_numpy(ksc).permute(0, 2, 1).contiguous().to(DEV),
                   "vs": torch.from_numpy(vsc).permute(0, 2, 1).contiguous().to(DEV)}
    return one(), one()


@pytest.mark.parametrize("shape", [(32, 32, 128, 16), (8, 2, 64, 1), (16, 4, 128, 128),
                                   (4, 1, 128, 32), (12, 4, 64, 64), (6, 6, 64, 1),
                                   (3, 3, 128, 16),
                                   # 5..16 query heads per kv head: the range-streaming kernel
                                   # writes the new key before its last tile reads it back
                                   (32, 4, 128, 16), (64, 4, 64, 16), (40, 8, 128, 8),
                                   (16, 2, 128, 128)],
                         ids=lambda s: "hq%d_hkv%d_d%d_bs%d" % s)
@pytest.mark.parametrize("window", [0, 100])
def test_int8_decode_append(shape, window):
    """Quantize, write and attend to the step's token in one pass: the slots, the written codes
    and scales (whole pools) and the outputs equal slot_mapping + the quantizing write +
    decode_int8 bit for bit, and the output matches the oracle over the dequantized pools."""
    Hq, Hkv, D, bs = shape
    L = [1, 31, 32, 33, 300, 1500, 3000]
    say(f"int8 decode_append {shape} window {window}")
    w = wl.custom(batch=len(L), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                  dtype="bf16")
    c = wl.make_case(w, np.array(L) - 1, [1] * len(L), seed=Hq * 5 + bs + window, device=DEV,
                     poison=False)
    a, s = _code_pools(c)
    table, la = c.table_tensor(DEV), c.lens_after_tensor(DEV)
    B = len(L)
    slots_a = torch.full((B,), -2, dtype=torch.int64, device=DEV)
    lse_a = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    out_a, _ = pkv.paged_attn_decode_int8_append(c.q, c.new_k, c.new_v, a["kc"], a["vc"], a["ks"],
                                                 a["vs"], table, la, c.max_len_after, w.scale,
                                                 lse=lse_a, slots_out=slots_a, window=window)
    slots_s = pkv.slot_mapping(table, c.lens_before_tensor(DEV), c.cu_q_tensor(DEV), bs, B)
    pkv.kv_cache_write_int8(c.new_k, c.new_v, s["kc"], s["vc"], s["ks"], s["vs"], slots_s)
    lse_s = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    out_s, _ = pkv.paged_attn_decode_int8(c.q, s["kc"], s["vc"], s["ks"], s["vs"], table, la,
                                          c.max_len_after, w.scale, lse=lse_s, window=window)
    torch.cuda.synchronize()
    assert torch.equal(slots_a, slots_s)
    for key in ("kc", "vc"):
        assert torch.equal(a[key], s[key]), key
    for key in ("ks", "vs"):
        assert torch.equal(a[key].view(torch.int32), s[key].view(torch.int32)), key
    assert torch.equal(out_a.view(torch.int16), out_s.view(torch.int16))
    assert torch.equal(lse_a.view(torch.int32), lse_s.view(torch.int32))
    nb = c.num_blocks
    kdeq = oracle.dequantize_rows(a["kc"].cpu().numpy().reshape(nb * bs, Hkv, D),
                                  a["ks"].cpu().permute(0, 2, 1).contiguous().numpy().reshape(nb * bs, Hkv))
    vdeq = oracle.dequantize_rows(a["vc"].cpu().numpy().reshape(nb * bs, Hkv, D),
                                  a["vs"].cpu().permute(0, 2, 1).contiguous().numpy().reshape(nb * bs, Hkv))
    err = _check(c, out_a, lse_a, kdeq.reshape(nb, bs, Hkv, D), vdeq.reshape(nb, bs, Hkv, D), window)
    say(f"  max-abs error {err:.3e}")


def test_int8_decode_append_headline_and_overlength_row():
    """The INT8 headline workload (B = 32, 32 heads, lengths 513..2049) through the fused
    call the bench times, against the separate write + decode bit for bit; then a row over
    the length bound: nothing written for it (slot -1) and the same output as decode_int8."""
    w = wl.WORKLOADS["llama7b_mha_int8"]
    L, _ = wl.sample_lengths(w, 0)
    Lp = np.asarray(L) + 1
    say("int8 decode_append headline")
    wc = wl.custom(batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                   head_dim=w.head_dim, block_size=w.block_size, dtype="bf16")
    c = wl.make_case(wc, Lp - 1, [1] * w.batch, seed=0, device=DEV, poison=False)
    table, la = c.table_tensor(DEV), c.lens_after_tensor(DEV)
    for cap in (c.max_len_after, int(np.sort(Lp)[-2])):     # the second bound cuts the longest row
        a, s = _code_pools(c)
        slots_a = torch.full((w.batch,), -2, dtype=torch.int64, device=DEV)
        out_a, _ = pkv.paged_attn_decode_int8_append(c.q, c.new_k, c.new_v, a["kc"], a["vc"], a["ks"],
                                                     a["vs"], table, la, cap, w.scale,
                                                     slots_out=slots_a)
        slots_s = pkv.slot_mapping(table, c.lens_before_tensor(DEV), c.cu_q_tensor(DEV),
                                   w.block_size, w.batch)
        over = la > cap
        slots_s[over] = -1
        keep = ~over
        pkv.kv_cache_write_int8(c.new_k[keep], c.new_v[keep], s["kc"], s["vc"], s["ks"], s["vs"],
                                slots_s[keep])
        out_s, _ = pkv.paged_attn_decode_int8(c.q, s["kc"], s["vc"], s["ks"], s["vs"], table, la, cap,
                                              w.scale)
        torch.cuda.synchronize()
        say(f"  bound {cap}: {int(over.sum())} rows over it")
        assert torch.equal(slots_a, slots_s)
        for key in ("kc", "vc", "ks", "vs"):
            assert torch.equal(a[key].view(torch.int8) if key in ("kc", "vc") else a[key].view(torch.int32),
                               s[key].view(torch.int8) if key in ("kc", "vc") else s[key].view(torch.int32)), key
        assert torch.equal(out_a.view(torch.int16), out_s.view(torch.int16))


@pytest.mark.parametrize("shape", [(32, 4, 128, 16), (16, 2, 128, 128)], ids=lambda s: "hq%d_hkv%d_d%d_bs%d" % s)
def test_int8_decode_append_ranges_overlength_row(shape):
    """The range-streaming form of the fused call with a length bound that cuts the longest
    row: nothing is written for it (slot -1), the other rows are, and the outputs equal the
    separate write + decode_int8 under the same bound bit for bit."""
    Hq, Hkv, D, bs = shape
    L = np.array([7, 300, 2999, 1500, 64, 1100, 33, 2048])
    say(f"int8 decode_append ranges over-length {shape}")
    w = wl.custom(batch=len(L), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                  dtype="bf16")
    c = wl.make_case(w, L - 1, [1] * len(L), seed=Hq + bs, device=DEV, poison=False)
    table, la = c.table_tensor(DEV), c.lens_after_tensor(DEV)
    B = len(L)
    cap = int(np.sort(L)[-2])
    a, s = _code_pools(c)
    slots_a = torch.full((B,), -2, dtype=torch.int64, device=DEV)
    out_a, _ = pkv.paged_attn_decode_int8_append(c.q, c.new_k, c.new_v, a["kc"], a["vc"], a["ks"],
                                                 a["vs"], table, la, cap, w.scale, slots_out=slots_a)
    slots_s = pkv.slot_mapping(table, c.lens_before_tensor(DEV), c.cu_q_tensor(DEV), bs, B)
    over = la > cap
    slots_s[over] = -1
    keep = ~over
    pkv.kv_cache_write_int8(c.new_k[keep], c.new_v[keep], s["kc"], s["vc"], s["ks"], s["vs"],
                            slots_s[keep])
    out_s, _ = pkv.paged_attn_decode_int8(c.q, s["kc"], s["vc"], s["ks"], s["vs"], table, la, cap,
                                          w.scale)
    torch.cuda.synchronize()
    assert int(over.sum()) == 1
    assert torch.equal(slots_a, slots_s)
    for key in ("kc", "vc"):
        assert torch.equal(a[key], s[key]), key
    for key in ("ks", "vs"):
        assert torch.equal(a[key].view(torch.int32), s[key].view(torch.int32)), key
    assert torch.equal(out_a.view(torch.int16), out_s.view(torch.int16))
