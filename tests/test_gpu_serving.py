"""GPU tests of the serving pieces around the attention kernels, through the C ABI:
block copies (copy on write), padding rows (seq_lens_kv = 0) on every decode path, and a
decode loop driven by the host block manager (forks, copies on write, frees, block reuse)
whose recorded steps are replayed with new tables and checked, replay by replay, against
the same calls made eagerly, against the oracle, and against a plain per-sequence history
of the written rows ("Paged KV Cache and Packed Sequence", 5.2-5.4).  Needs an MI355X."""
import random

import numpy as np
import pytest
import torch

import paged_kv_cache_133_amd as pkv
from oracle import oracle
from paged_kv_cache_133_amd.step import GraphDecodeStep
from tests.gpu_common import ATOL, LSE_REL, lse_error, say
from tests.helpers import host

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _bits(t):
    """The tensor's raw bits on the host (so that -0.0, NaN and -inf compare exactly)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    return t


@pytest.mark.parametrize("shape,dtype", [((40, 16, 8, 128), torch.bfloat16),
                                         ((9, 1, 1, 1), torch.float32),
                                         ((33, 4, 2, 64), torch.int8)],
                         ids=["bf16_blocks", "f32_scales_4B", "int8_blocks"])
def test_copy_blocks(shape, dtype):
    g = torch.Generator().manual_seed(shape[0])
    if dtype == torch.int8:
        pool = torch.randint(-128, 128, shape, generator=g, dtype=torch.int8)
    else:
        pool = torch.randn(shape, generator=g).to(dtype)
    nb = shape[0]
    # destinations distinct and never a source (the documented precondition); plus a
    # same-block pair and two pairs outside the pool, which are skipped
    pairs = [(1, 0), (5, 7), (nb - 1, 3), (2, 2), (-1, 6), (6, nb), (8, 4)]
    dst = [t for s_, t in pairs if 0 <= s_ < nb and 0 <= t < nb and s_ != t]
    assert len(set(dst)) == len(dst) and not set(dst) & {s_ for s_, t in pairs}
    say(f"copy_blocks {shape} {dtype}")
    d = pool.to(DEV)
    pkv.kv_cache_copy_blocks(d, torch.tensor(pairs, dtype=torch.int64, device=DEV))
    torch.cuda.synchronize()
    want = pool.clone()
    for s, t in pairs:
        if 0 <= s < nb and 0 <= t < nb and s != t:
            want[t] = pool[s]
    assert torch.equal(_bits(d), _bits(want))


def _padding_case(hq, hkv, d, bs, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    lens = [0, 37, 0, 300, 1, 0]
    B = len(lens)
    mbs = -(-max(lens) // bs) + 1
    nb = B * mbs + 3
    perm = torch.randperm(nb, generator=g)[:B * mbs].view(B, mbs).to(torch.int32)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kc = torch.randn(nb, bs, hkv, d, generator=g).to(tdt)
    vc = torch.randn(nb, bs, hkv, d, generator=g).to(tdt)
    q = torch.randn(B, hq, d, generator=g).to(tdt)
    kn = torch.randn(B, hkv, d, generator=g).to(tdt)
    vn = torch.randn(B, hkv, d, generator=g).to(tdt)
    return lens, perm, kc, vc, q, kn, vn


@pytest.mark.parametrize("hq,hkv,d,bs,dtype", [(8, 8, 128, 16, "bf16"), (8, 2, 128, 16, "bf16"),
                                               (16, 1, 64, 32, "bf16"), (4, 2, 64, 1, "f32"),
                                               (32, 2, 128, 64, "bf16")],
                         ids=lambda v: str(v))
def test_padding_rows(hq, hkv, d, bs, dtype):
    """Rows with seq_lens_kv = 0: out 0, lse -inf, no cache row written, slot -1; the other
    rows as the oracle says (decode with the new rows written, and plain decode)."""
    lens, table, kc, vc, q, kn, vn = _padding_case(hq, hkv, d, bs, dtype, seed=hq * d + bs)
    B = len(lens)
    say(f"padding rows hq={hq} hkv={hkv} d={d} bs={bs} {dtype}")
    dk, dv = kc.to(DEV), vc.to(DEV)
    lens_d = torch.tensor(lens, dtype=torch.int32, device=DEV)
    table_d = table.to(DEV)
    scale = d ** -0.5
    lse = torch.full((B, hq), 7.0, dtype=torch.float32, device=DEV)
    slots = torch.full((B,), 12345, dtype=torch.int64, device=DEV)
    out = torch.full((B, hq, d), 3.0, dtype=q.dtype, device=DEV)
    pkv.paged_attn_decode_append(q.to(DEV), kn.to(DEV), vn.to(DEV), dk, dv, table_d, lens_d,
                                 table.shape[1] * bs, scale, out=out, lse=lse, slots_out=slots)
    torch.cuda.synchronize()
    # expected writes: position L - 1 of each non-empty row
    want_k, want_v = kc.clone(), vc.clone()
    want_slots = []
    for b, L in enumerate(lens):
        if L == 0:
            want_slots.append(-1)
            continue
        blk, off = int(table[b, (L - 1) // bs]), (L - 1) % bs
        want_k[blk, off], want_v[blk, off] = kn[b], vn[b]
        want_slots.append(blk * bs + off)
    assert slots.cpu().tolist() == want_slots
    assert torch.equal(_bits(dk), _bits(want_k)) and torch.equal(_bits(dv), _bits(want_v))
    # the oracle on the rows that hold a sequence; padding rows by their definition
    live = [b for b, L in enumerate(lens) if L]
    pad = [b for b, L in enumerate(lens) if not L]
    o_out, o_lse = oracle.paged_attention(host(q)[live], host(want_k), host(want_v),
                                          table.numpy()[live],
                                          np.arange(len(live) + 1, dtype=np.int32),
                                          np.array(lens, np.int32)[live], scale, False)
    got = out.float().cpu().numpy()
    got_lse = lse.cpu().numpy()
    assert (got[pad] == 0).all() and np.isneginf(got_lse[pad]).all()
    err = float(np.abs(got[live] - o_out).max())
    assert err <= ATOL[dtype], err
    assert lse_error(got_lse[live], o_lse) <= LSE_REL
    # plain decode over the written caches: the same outputs
    out2, _ = pkv.paged_attn_decode(q.to(DEV), dk, dv, table_d, lens_d, table.shape[1] * bs, scale)
    torch.cuda.synchronize()
    got2 = out2.float().cpu().numpy()
    assert float(np.abs(got2[live] - o_out).max()) <= ATOL[dtype]
    assert (got2[pad] == 0).all()


def test_padding_rows_int8():
    lens = [0, 200, 0, 33]
    B, hq, hkv, d, bs = 4, 8, 2, 128, 16
    g = torch.Generator().manual_seed(5)
    mbs = 16
    nb = B * mbs
    table = torch.randperm(nb, generator=g).view(B, mbs).to(torch.int32)
    kc = torch.randint(-127, 128, (nb, bs, hkv, d), generator=g, dtype=torch.int8)
    vc = torch.randint(-127, 128, (nb, bs, hkv, d), generator=g, dtype=torch.int8)
    ks = torch.rand(nb, bs, hkv, generator=g) * 0.02
    vs = torch.rand(nb, bs, hkv, generator=g) * 0.02
    q = torch.randn(B, hq, d, generator=g).to(torch.bfloat16)
    say("padding rows int8")
    lse = torch.full((B, hq), 7.0, dtype=torch.float32, device=DEV)
    blockwise = lambda s: s.permute(0, 2, 1).contiguous().to(DEV)   # [block][kv head][offset]  # noqa: E731
    out, _ = pkv.paged_attn_decode_int8(q.to(DEV), kc.to(DEV), vc.to(DEV), blockwise(ks), blockwise(vs),
                                        table.to(DEV), torch.tensor(lens, dtype=torch.int32, device=DEV),
                                        mbs * bs, d ** -0.5, lse=lse)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert (got[[0, 2]] == 0).all() and np.isneginf(lse.cpu().numpy()[[0, 2]]).all()
    kd = oracle.dequantize_rows(kc.numpy().reshape(-1, hkv, d), ks.numpy().reshape(-1, hkv))
    vd = oracle.dequantize_rows(vc.numpy().reshape(-1, hkv, d), vs.numpy().reshape(-1, hkv))
    live = [1, 3]
    o_out, _ = oracle.paged_attention(oracle.widen(host(q))[live], kd.reshape(nb, bs, hkv, d),
                                      vd.reshape(nb, bs, hkv, d), table.numpy()[live],
                                      np.arange(len(live) + 1, dtype=np.int32),
                                      np.array(lens, np.int32)[live], d ** -0.5, False)
    assert float(np.abs(got[live] - o_out).max()) <= 2e-2


def _rows_through_table(cache, table_row, n, bs):
    idx = torch.arange(n)
    return cache[table_row[idx // bs].long(), idx % bs]


@pytest.mark.parametrize("hq,hkv,d", [(8, 2, 128), (4, 4, 64)], ids=["gqa_g4", "mha_d64"])
def test_serving_loop_graph_replays(hq, hkv, d):
    """Block manager -> host tables -> recorded decode step, 24 replays.  Each replay equals
    the eager call bit for bit (outputs, lse, slots, caches); every 6th step also matches
    the oracle; the caches read through the tables equal each sequence's own history."""
    bs, nb, mbs, B, steps = 16, 160, 40, 6, 24
    rng = random.Random(hq * 100 + d)
    gen = torch.Generator(device=DEV).manual_seed(hq + d)
    dt = torch.bfloat16
    scale = d ** -0.5
    kA = torch.zeros(nb, bs, hkv, d, dtype=dt, device=DEV)
    vA = torch.zeros_like(kA)
    kB, vB = torch.zeros_like(kA), torch.zeros_like(kA)
    bm = pkv.BlockManager(nb, bs, mbs)
    step = GraphDecodeStep(kA, vA, B, mbs, hq, scale)
    hist = {}            # seq id -> [(k rows, v rows)] of every token, in order (CPU)
    rows = [None] * B    # batch row -> seq id or None (padding)
    next_id = 0

    def prefill(row, n):
        nonlocal next_id
        sid = next_id
        next_id += 1
        bm.add(sid)
        slots, copy = bm.append(sid, n)
        assert copy is None
        kn = torch.randn(n, hkv, d, generator=gen, device=DEV).to(dt)
        vn = torch.randn(n, hkv, d, generator=gen, device=DEV).to(dt)
        sl = torch.from_numpy(slots).to(DEV)
        for kc, vc in ((kA, vA), (kB, vB)):
            pkv.kv_cache_write(kn, vn, kc, vc, sl)
        hist[sid] = [kn.cpu(), vn.cpu()]
        rows[row] = sid

    for r in range(4):
        prefill(r, rng.randint(1, 300))
    wsB = pkv.new_decode_workspace(B, hq, hkv, d, mbs * bs, DEV)
    outB = torch.empty(B, hq, d, dtype=dt, device=DEV)
    lseB = torch.empty(B, hq, dtype=torch.float32, device=DEV)
    slotsB = torch.empty(B, dtype=torch.int64, device=DEV)
    copies_seen = 0
    for t in range(steps):
        # host side of the step: forks, frees, new sequences, then one token per sequence
        free_rows = [r for r in range(B) if rows[r] is None]
        if t % 5 == 1 and free_rows:
            parent = rows[rng.choice([r for r in range(B) if rows[r] is not None])]
            child = next_id
            next_id += 1
            bm.fork(parent, child)
            hist[child] = [x.clone() for x in hist[parent]]
            rows[free_rows[0]] = child
        elif t % 7 == 3:
            r = rng.choice([r for r in range(B) if rows[r] is not None])
            bm.free(rows[r])
            del hist[rows[r]]
            rows[r] = None
        elif t % 9 == 4 and free_rows:
            prefill(free_rows[0], rng.randint(1, 200))
        # one native call: a token for every live row, the fixed-batch table and lengths
        # straight into the pinned buffer the next replay uploads, and the copies on write
        tab, lens = step.host_tables()
        ids = [-1 if rows[r] is None else rows[r] for r in range(B)]
        _, _, _, cp = bm.decode_step(ids, table=tab, seq_lens=lens)
        pairs = [tuple(x) for x in cp.tolist()]
        copies_seen += len(pairs)
        live = [r for r in range(B) if rows[r] is not None]
        # eager work between replays: copies on write, this step's inputs
        if pairs:
            pd = torch.tensor(pairs, dtype=torch.int64, device=DEV)
            for c in (kA, vA, kB, vB):
                pkv.kv_cache_copy_blocks(c, pd)
        step.q.copy_(torch.randn(B, hq, d, generator=gen, device=DEV).to(dt))
        step.k_new.copy_(torch.randn(B, hkv, d, generator=gen, device=DEV).to(dt))
        step.v_new.copy_(torch.randn(B, hkv, d, generator=gen, device=DEV).to(dt))
        table_d = torch.from_numpy(tab.copy()).to(DEV)
        lens_d = torch.from_numpy(lens.copy()).to(DEV)
        say(f"serving step {t}: live rows {live}, lens {lens.tolist()}, copies {pairs}")
        step.launch()
        pkv.paged_attn_decode_append(step.q, step.k_new, step.v_new, kB, vB, table_d, lens_d,
                                     mbs * bs, scale, out=outB, lse=lseB, workspace=wsB,
                                     slots_out=slotsB)
        torch.cuda.synchronize()
        assert torch.equal(_bits(step.out), _bits(outB)), t
        assert torch.equal(_bits(step.lse), _bits(lseB)), t
        assert torch.equal(step.slots, slotsB), t
        assert torch.equal(_bits(kA), _bits(kB)) and torch.equal(_bits(vA), _bits(vB)), t
        kn, vn = step.k_new.cpu(), step.v_new.cpu()
        for r in live:
            h = hist[rows[r]]
            h[0] = torch.cat([h[0], kn[r:r + 1]])
            h[1] = torch.cat([h[1], vn[r:r + 1]])
        pad = [r for r in range(B) if rows[r] is None]
        assert (step.slots.cpu()[pad] == -1).all() and (step.out.cpu()[pad].float() == 0).all()
        # dual track: every live sequence read back through its table
        kh, vh = kA.cpu(), vA.cpu()
        for r in live:
            n = int(lens[r])
            trow = torch.from_numpy(tab[r].copy())
            assert torch.equal(_bits(_rows_through_table(kh, trow, n, bs)), _bits(hist[rows[r]][0])), (t, r)
            assert torch.equal(_bits(_rows_through_table(vh, trow, n, bs)), _bits(hist[rows[r]][1])), (t, r)
        if t % 6 == 5:
            o_out, _ = oracle.paged_attention(host(step.q)[live], host(kA), host(vA), tab[live],
                                              np.arange(len(live) + 1, dtype=np.int32),
                                              lens[live], scale, False)
            err = float(np.abs(step.out.float().cpu().numpy()[live] - o_out).max())
            say(f"  oracle max-abs error {err:.3e}")
            assert err <= ATOL["bf16"]
    assert copies_seen > 0, "the walk never exercised a copy on write"
    step.close()
    bm.close()


def test_runner_capture_errors_and_plain_replays():
    """The runner refuses a second open capture and a launch of an unrecorded graph; a
    recorded step replayed many times with eager work between equals the eager call."""
    import ctypes
    from paged_kv_cache_133_amd._lib import PagedKVError, _check, lib
    say("runner capture errors and replays")
    bs, hq, hkv, d, B, mbs = 16, 8, 2, 128, 3, 8
    g = torch.Generator(device=DEV).manual_seed(3)
    k = torch.randn(40, bs, hkv, d, generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn(40, bs, hkv, d, generator=g, device=DEV).to(torch.bfloat16)
    step = GraphDecodeStep(k.clone(), v.clone(), B, mbs, hq, 0.088)
    s = torch.cuda.Stream(DEV)
    sh = ctypes.c_void_p(s.cuda_stream)
    assert lib().pkv_runner_capture_begin(step._r, 0, sh) == -2       # graph 0 exists
    assert lib().pkv_runner_capture_begin(step._r, 2, sh) == -2
    assert lib().pkv_runner_capture_end(step._r, sh) == -2             # none open
    kk, vv = k.clone(), v.clone()
    table = torch.arange(B * mbs, dtype=torch.int32).view(B, mbs) + 5
    for rep, lens in enumerate(([1, 17, 100], [2, 18, 101], [0, 19, 102], [4, 0, 103], [5, 1, 104])):
        tab, ln = step.host_tables()
        tab[:] = table.numpy()
        ln[:] = lens
        step.q.copy_(torch.randn(B, hq, d, generator=g, device=DEV).to(torch.bfloat16))
        step.k_new.copy_(torch.randn(B, hkv, d, generator=g, device=DEV).to(torch.bfloat16))
        step.v_new.copy_(torch.randn(B, hkv, d, generator=g, device=DEV).to(torch.bfloat16))
        step.launch()
        out, lse = pkv.paged_attn_decode_append(
            step.q, step.k_new, step.v_new, kk, vv, table.to(DEV),
            torch.tensor(lens, dtype=torch.int32, device=DEV), mbs * bs, 0.088,
            lse=torch.empty(B, hq, dtype=torch.float32, device=DEV))
        torch.cuda.synchronize()
        assert torch.equal(_bits(step.out), _bits(out)), rep
        assert torch.equal(_bits(step.lse), _bits(lse)), rep
    step.close()
    with pytest.raises(PagedKVError):
        _check(lib().pkv_runner_launch(None, None))


@pytest.mark.parametrize("n", [1, 3, 4, 5, 1027, 4868])
def test_upload_kernel_copies_pinned_buffer(n):
    """pkv_upload_kernel (the copy the step runner records): n int32 words from a pinned host
    tensor into a device tensor, 16-byte words plus a 4-byte tail; the words after the
    copy stay untouched."""
    import ctypes
    from paged_kv_cache_133_amd._lib import _check, lib
    say(f"upload kernel: {n} words")
    src = torch.arange(n, dtype=torch.int32).mul_(7919).add_(13).pin_memory()
    dst = torch.full((n + 8,), -1, dtype=torch.int32, device=DEV)
    _check(lib().pkv_upload_kernel(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()),
                                   n * 4, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))
    torch.cuda.synchronize()
    assert torch.equal(dst[:n].cpu(), src)
    assert (dst[n:] == -1).all()
