"""GPU parity of the INT8 MLA latent cache against the oracle, through the C ABI: the
quantizing writer bit for bit (nope and rope rows each with their own scale, other bytes
unchanged, out-of-pool slots skipped), and the MLA-absorbed decode over the codes against
fp64 attention over the exactly dequantized rows (key = nope || rope, value = nope).  Needs an
MI355X."""
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


@pytest.mark.parametrize("dtype,bs", [("bf16", 16), ("f32", 4), ("bf16", 128)])
def test_int8_mla_write_bit_exact(dtype, bs):
    td = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    g = torch.Generator().manual_seed(bs)
    T, nb = 37, 12
    nope = (torch.randn(T, 512, generator=g) * torch.rand(T, 1, generator=g) * 20).to(td)
    rope = (torch.randn(T, 64, generator=g) * 3).to(td)
    nope[5] = 0                                          # zero row: scale 0, zero codes
    slots = torch.randperm(nb * bs, generator=g)[:T].to(torch.int64)
    slots[3], slots[9] = -1, nb * bs                     # skipped
    nc = torch.randint(-128, 128, (nb, bs, 512), generator=g, dtype=torch.int8)
    rc = torch.randint(-128, 128, (nb, bs, 64), generator=g, dtype=torch.int8)
    ns = torch.randn(nb, bs, generator=g)
    rs = torch.randn(nb, bs, generator=g)
    say(f"int8 mla write {dtype} bs={bs}")
    d = [t.to(DEV) for t in (nc, rc, ns, rs)]
    pkv.kv_cache_write_int8_mla(nope.to(DEV), rope.to(DEV), *d, slots.to(DEV))
    torch.cuda.synchronize()
    ok = ((slots >= 0) & (slots < nb * bs)).numpy()
    sl = slots.numpy()[ok]
    for new, codes, scales, gc, gs, w in ((nope, nc, ns, d[0], d[2], 512), (rope, rc, rs, d[1], d[3], 64)):
        q, s = oracle.quantize_rows(host(new))           # [T, w], [T]
        exp_c = codes.numpy().reshape(nb * bs, w).copy()
        exp_s = scales.numpy().reshape(nb * bs).copy()
        exp_c[sl] = q[ok]
        exp_s[sl] = s[ok]
        assert np.array_equal(gc.cpu().numpy().reshape(nb * bs, w), exp_c)
        assert np.array_equal(gs.cpu().numpy().reshape(nb * bs).view(np.uint32), exp_s.view(np.uint32))


def _int8_mla_case(hq, bs, L, seed):
    """An MLA case whose pools are the oracle's quantization of a bf16 pool, with the step's
    new rows written by the GPU's quantizing writer.  A length of 0 marks a padding row: the
    case still gives it one row (q has one row per sequence), and the lengths the kernel gets
    (returned) say 0 there.  Returns the case, the device arrays, the dequantized pools (fp64)
    and the lengths."""
    w = wl.custom(mode="mla", batch=len(L), num_q_heads=hq, num_kv_heads=1, head_dim=512,
                  head_dim_rope=64, block_size=bs, dtype="bf16")
    c = wl.make_case(w, np.maximum(np.array(L) - 1, 0), [1] * len(L), seed=seed, device=DEV,
                     poison=False)
    lens = np.where(np.array(L) > 0, c.lens_after, 0).astype(np.int32)
    nb = c.num_blocks
    nq, nsc = oracle.quantize_rows(host(c.cache_k).reshape(nb, bs, 512))
    rq, rsc = oracle.quantize_rows(host(c.cache_rope).reshape(nb, bs, 64))
    dev = {"nc": torch.from_numpy(nq).to(DEV), "rc": torch.from_numpy(rq).to(DEV),
           "ns": torch.from_numpy(nsc).to(DEV), "rs": torch.from_numpy(rsc).to(DEV)}
    table = c.table_tensor(DEV)
    if c.num_tokens:
        slots = pkv.slot_mapping(table, c.lens_before_tensor(DEV), c.cu_q_tensor(DEV), bs, c.num_tokens)
        pkv.kv_cache_write_int8_mla(c.new_k.reshape(-1, 512), c.new_rope.reshape(-1, 64), dev["nc"],
                                    dev["rc"], dev["ns"], dev["rs"], slots)
        torch.cuda.synchronize()
        sl = slots.cpu().numpy()
        a, b = oracle.quantize_rows(host(c.new_k).reshape(-1, 512))
        nq.reshape(nb * bs, 512)[sl] = a
        nsc.reshape(nb * bs)[sl] = b
        a, b = oracle.quantize_rows(host(c.new_rope).reshape(-1, 64))
        rq.reshape(nb * bs, 64)[sl] = a
        rsc.reshape(nb * bs)[sl] = b
    assert np.array_equal(dev["nc"].cpu().numpy(), nq) and np.array_equal(dev["rs"].cpu().numpy(), rsc)
    kdeq = oracle.dequantize_rows(nq, nsc).reshape(nb, bs, 1, 512)
    rdeq = oracle.dequantize_rows(rq, rsc).reshape(nb, bs, 1, 64)
    return c, dev, table, kdeq, rdeq, lens


def _check(c, out, lse, kdeq, rdeq, lens_all, rows=None):
    idx = np.arange(c.w.batch) if rows is None else np.asarray(rows)
    lens = lens_all[idx]
    live = idx[lens > 0]
    got = out.float().cpu().numpy()
    got_lse = lse.cpu().numpy()
    for b in idx[lens == 0]:                            # padding rows: 0 and -inf
        assert (got[b] == 0).all() and np.isneginf(got_lse[b]).all()
    if len(live) == 0:
        return 0.0
    cu = np.arange(len(live) + 1, dtype=np.int32)
    o, ol = oracle.paged_attention(oracle.widen(host(c.q))[live], kdeq, kdeq, c.block_table[live], cu,
                                   lens_all[live], c.w.scale, False,
                                   q_rope=oracle.widen(host(c.q_rope))[live], k_rope=rdeq)
    err = float(np.abs(got[live] - o).max())
    assert err <= 2e-2, f"max-abs error {err:.3e}"
    lerr = lse_error(got_lse[live], ol)
    assert lerr <= LSE_REL, f"lse error {lerr:.3e}"
    return err


@pytest.mark.parametrize("hq,bs", [(128, 16), (64, 4), (16, 128), (32, 8), (192, 32)])
def test_int8_mla_decode_parity(hq, bs):
    L = [0, 1, 31, 32, 33, bs - 1 if bs > 1 else 2, 700, 2600]
    say(f"int8 mla decode hq={hq} bs={bs} L={L}")
    c, dev, table, kdeq, rdeq, lens = _int8_mla_case(hq, bs, L, seed=hq + bs)
    assert c.q.shape[0] == len(L)
    lse = torch.full((len(L), hq), 3.0, dtype=torch.float32, device=DEV)
    out, _ = pkv.paged_attn_decode_mla_int8(c.q, c.q_rope, dev["nc"], dev["rc"], dev["ns"], dev["rs"],
                                            table, torch.from_numpy(lens).to(DEV), c.max_len_after,
                                            c.w.scale, lse=lse)
    torch.cuda.synchronize()
    say(f"  max-abs error {_check(c, out, lse, kdeq, rdeq, lens):.3e}")


def test_int8_mla_two_passes_equal_one():
    c, dev, table, kdeq, rdeq, lens = _int8_mla_case(128, 64, [3000, 5, 1400, 64, 65], seed=4)
    la = torch.from_numpy(lens).to(DEV)
    args = (c.q, c.q_rope, dev["nc"], dev["rc"], dev["ns"], dev["rs"], table, la, c.max_len_after, c.w.scale)
    lse1 = torch.empty((5, 128), dtype=torch.float32, device=DEV)
    out1, _ = pkv.paged_attn_decode_mla_int8(*args, lse=lse1)
    lse2 = torch.empty_like(lse1)
    first, second, out2 = _lib.prepare_decode_mla_int8(*args, lse=lse2)
    first()
    second()
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse1.view(torch.int32), lse2.view(torch.int32))
    _check(c, out1, lse1, kdeq, rdeq, lens)


def test_int8_mla_full_workload():
    """The MLA workload's shape at full size (64 sequences of U{2048..8192}, 128 heads, bs
    128) over the INT8 latent cache; the oracle checks every sequence."""
    w = wl.WORKLOADS["mla_absorbed_bf16"]
    L, _ = wl.sample_lengths(w, 0)
    Lp = [int(x) + 1 for x in L]
    say("int8 mla full-size workload (all rows)")
    c, dev, table, kdeq, rdeq, lens = _int8_mla_case(128, 128, Lp, seed=0)
    lse = torch.empty((len(Lp), 128), dtype=torch.float32, device=DEV)
    out, _ = pkv.paged_attn_decode_mla_int8(c.q, c.q_rope, dev["nc"], dev["rc"], dev["ns"], dev["rs"],
                                            table, torch.from_numpy(lens).to(DEV), c.max_len_after,
                                            c.w.scale, lse=lse)
    torch.cuda.synchronize()
    say(f"  max-abs error {_check(c, out, lse, kdeq, rdeq, lens):.3e}")


def _int8_mla_pools(c):
    """Two device copies of the INT8 latent pools: the oracle's quantization of the case's
    bf16 pools (the step's rows not yet written)."""
    nb, bs = c.num_blocks, c.w.block_size
    nq, nsc = oracle.quantize_rows(host(c.cache_k).reshape(nb, bs, 512))
    rq, rsc = oracle.quantize_rows(host(c.cache_rope).reshape(nb, bs, 64))
    one = lambda: {"nc": torch.from_numpy(nq).to(DEV), "rc": torch.from_numpy(rq).to(DEV),  # noqa: E731
                   "ns": torch.from_numpy(nsc).to(DEV), "rs": torch.from_numpy(rsc).to(DEV)}
    return one(), one()


@pytest.mark.parametrize("hq,bs,cut", [(128, 16, False), (64, 4, False), (192, 32, False),
                                       (128, 128, False), (128, 64, True)])
def test_int8_mla_decode_append(hq, bs, cut):
    """Quantize, write and attend to the step's latent row in one pass: the slots, the whole
    code and scale pools and the outputs equal slot_mapping + the quantizing writer +
    decode_mla_int8 bit for bit; the output matches the oracle over the written pools.  With
    `cut`, the length bound excludes the longest row: it writes nothing (slot -1)."""
    L = np.array([1, 31, 32, 33, 700, 2600, 1500, 64])
    say(f"int8 mla decode_append hq={hq} bs={bs} cut={cut}")
    w = wl.custom(mode="mla", batch=len(L), num_q_heads=hq, num_kv_heads=1, head_dim=512,
                  head_dim_rope=64, block_size=bs, dtype="bf16")
    c = wl.make_case(w, L - 1, [1] * len(L), seed=hq + bs + cut, device=DEV, poison=False)
    table, la = c.table_tensor(DEV), c.lens_after_tensor(DEV)
    B = len(L)
    cap = int(np.sort(L)[-2]) if cut else c.max_len_after
    a, s = _int8_mla_pools(c)
    nope_new, rope_new = c.new_k.reshape(B, 512), c.new_rope.reshape(B, 64)
    slots_a = torch.full((B,), -2, dtype=torch.int64, device=DEV)
    lse_a = torch.empty((B, hq), dtype=torch.float32, device=DEV)
    out_a, _ = pkv.paged_attn_decode_mla_int8_append(c.q, c.q_rope, nope_new, rope_new, a["nc"], a["rc"],
                                                     a["ns"], a["rs"], table, la, cap, w.scale,
                                                     lse=lse_a, slots_out=slots_a)
    slots_s = pkv.slot_mapping(table, c.lens_before_tensor(DEV), c.cu_q_tensor(DEV), bs, B)
    over = la > cap
    slots_s[over] = -1
    keep = ~over
    pkv.kv_cache_write_int8_mla(nope_new[keep], rope_new[keep], s["nc"], s["rc"], s["ns"], s["rs"],
                                slots_s[keep])
    lse_s = torch.empty((B, hq), dtype=torch.float32, device=DEV)
    out_s, _ = pkv.paged_attn_decode_mla_int8(c.q, c.q_rope, s["nc"], s["rc"], s["ns"], s["rs"], table,
                                              la, cap, w.scale, lse=lse_s)
    torch.cuda.synchronize()
    assert int(over.sum()) == (1 if cut else 0)
    assert torch.equal(slots_a, slots_s)
    for key in ("nc", "rc"):
        assert torch.equal(a[key], s[key]), key
    for key in ("ns", "rs"):
        assert torch.equal(a[key].view(torch.int32), s[key].view(torch.int32)), key
    assert torch.equal(out_a.view(torch.int16), out_s.view(torch.int16))
    assert torch.equal(lse_a.view(torch.int32), lse_s.view(torch.int32))
    if not cut:
        nb = c.num_blocks
        kdeq = oracle.dequantize_rows(a["nc"].cpu().numpy(), a["ns"].cpu().numpy()).reshape(nb, bs, 1, 512)
        rdeq = oracle.dequantize_rows(a["rc"].cpu().numpy(), a["rs"].cpu().numpy()).reshape(nb, bs, 1, 64)
        say(f"  max-abs error {_check(c, out_a, lse_a, kdeq, rdeq, c.lens_after.astype(np.int32)):.3e}")
