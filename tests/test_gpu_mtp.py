"""GPU parity of the multi-token decode (MTP: next_n + 1 causal query tokens per sequence,
pkv_paged_attn_decode_mtp) against the oracle's causal varlen attention, through the C ABI:
small shapes on block and tile edges, windows, padding rows, the two-pass form, agreement
with the varlen kernel, and the full-size MTP workload on sampled sequences.  Needs an
MI355X."""
import numpy as np
import pytest
import torch

import paged_kv_cache_133_amd as pkv
from paged_kv_cache_133_amd import _lib
from paged_kv_cache_133_amd import workloads as wl
from tests.gpu_common import ATOL, compare_outputs, compare_writes, oracle_step, say, LSE_REL, lse_error

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def mtp_step(c, qn, window=0, two_pass=False, lens=None):
    """slot_mapping + cache write of the step's qn new rows per sequence, then the MTP
    decode (one call, or the range pass and the combine pass as two calls)."""
    w = c.w
    table = c.table_tensor(DEV)
    cu = c.cu_q_tensor(DEV)
    la = c.lens_after_tensor(DEV) if lens is None else lens
    slots = pkv.slot_mapping(table, c.lens_before_tensor(DEV), cu, w.block_size, c.num_tokens)
    k, v = c.cache_k.clone(), c.cache_v.clone()
    pkv.kv_cache_write(c.new_k, c.new_v, k, v, slots)
    lse = torch.full((c.num_tokens, w.num_q_heads), 5.0, dtype=torch.float32, device=DEV)
    if two_pass:
        first, second, out = _lib.prepare_decode_mtp(c.q, k, v, table, la, qn, c.max_len_after,
                                                     w.scale, lse=lse, window=window)
        first()
        second()
    else:
        out, _ = pkv.paged_attn_decode_mtp(c.q, k, v, table, la, qn, c.max_len_after, w.scale,
                                           lse=lse, window=window)
    torch.cuda.synchronize()
    return {"slots": slots, "cache_k": k, "cache_v": v, "out": out, "lse": lse}


SHAPES = [  # hq, hkv, d, bs, qn  (columns qn * hq / hkv)
    (32, 8, 128, 16, 2),     # G 4, 8 columns: the MTP workload's shape
    (16, 8, 128, 4, 3),      # G 2, 6 columns, the smallest block for d 128
    (8, 8, 64, 8, 4),        # MHA, 4 columns, d 64
    (32, 2, 128, 64, 1),     # G 16, one token: plain decode through the same kernel
    (16, 4, 64, 32, 4),      # G 4, all 16 columns
    (64, 8, 128, 128, 2),    # G 8, 16 columns, large blocks
]


def test_mtp_decode_long_context():
    """A sequence of more than 8192 keys puts the MTP decode in the compact layout (query
    fragments of (token, head) columns in registers)."""
    hq, hkv, d, bs, qn = 32, 8, 128, 16, 2
    w = wl.custom(mode="varlen", batch=5, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                  block_size=bs, dtype="bf16")
    L = [9000, 30, 1, 4000, 8191]
    say(f"mtp long context L={L}")
    c = wl.make_case(w, L, [qn] * len(L), seed=77, device=DEV)
    g = mtp_step(c, qn)
    o = oracle_step(c, causal=True)
    compare_writes(c, g, o)
    compare_outputs(c, g, o, tokens=o["tokens"], label="mtp long context")


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "hq%d_hkv%d_d%d_bs%d_qn%d" % s)
@pytest.mark.parametrize("window", [0, 100])
def test_mtp_decode_parity(shape, window):
    hq, hkv, d, bs, qn = shape
    w = wl.custom(mode="varlen", batch=8, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                  block_size=bs, dtype="bf16")
    # lengths before the step: empty prefix, block and tile edges, several tiles, long
    L = [0, bs - 1, 31, 32 - qn, 33, 300, 1200, 2047]
    say(f"mtp parity {shape} window {window} L={L}")
    c = wl.make_case(w, L, [qn] * len(L), seed=hq + d + bs + qn + window, device=DEV)
    g = mtp_step(c, qn, window)
    o = oracle_step(c, causal=True, window=window)
    compare_writes(c, g, o)
    err = compare_outputs(c, g, o, tokens=o["tokens"], label=f"mtp {shape} window {window}")
    say(f"  max-abs error {err:.3e}")


def test_mtp_two_pass_equals_one_and_matches_varlen():
    hq, hkv, d, bs, qn = 32, 8, 128, 16, 2
    w = wl.custom(mode="varlen", batch=12, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                  block_size=bs, dtype="bf16")
    rng = np.random.default_rng(7)
    L = [int(x) for x in rng.integers(1, 3000, size=12)]
    say(f"mtp two-pass / varlen L={L}")
    c = wl.make_case(w, L, [qn] * 12, seed=5, device=DEV)
    one = mtp_step(c, qn)
    two = mtp_step(c, qn, two_pass=True)
    assert torch.equal(one["out"].view(torch.int16), two["out"].view(torch.int16))
    assert torch.equal(one["lse"].view(torch.int32), two["lse"].view(torch.int32))
    table, cu, la = c.table_tensor(DEV), c.cu_q_tensor(DEV), c.lens_after_tensor(DEV)
    lse_v = torch.empty_like(one["lse"])
    out_v, _ = pkv.paged_attn_varlen(c.q, one["cache_k"], one["cache_v"], table, cu, la, qn,
                                     w.scale, causal=True, lse=lse_v)
    torch.cuda.synchronize()
    assert float((out_v.float() - one["out"].float()).abs().max()) <= ATOL["bf16"]
    # two kernels, each within LSE_REL of the exact value
    assert lse_error(lse_v.cpu().numpy(), one["lse"].cpu().numpy()) <= 2 * LSE_REL


def test_mtp_padding_rows():
    """Sequences with seq_lens_kv = 0 (padding): their qn rows are 0 with lse -inf; the
    others as the oracle says."""
    hq, hkv, d, bs, qn = 32, 8, 128, 16, 2
    w = wl.custom(mode="varlen", batch=5, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                  block_size=bs, dtype="bf16")
    c = wl.make_case(w, [40, 300, 7, 1000, 64], [qn] * 5, seed=9, device=DEV)
    lens = c.lens_after_tensor(DEV).clone()
    lens[[0, 2]] = 0
    say("mtp padding rows")
    g = mtp_step(c, qn, lens=lens)
    out, lse = g["out"].float().cpu(), g["lse"].cpu()
    for b in (0, 2):
        rows = slice(b * qn, b * qn + qn)
        assert (out[rows] == 0).all() and torch.isneginf(lse[rows]).all()
    live = [1, 3, 4]
    o = oracle_step(c, causal=True, rows=live)
    compare_outputs(c, g, o, tokens=o["tokens"], label="mtp padding")


def test_mtp_full_workload():
    """The full-size MTP workload (32 sequences of U{512..2048} + 2, 32 q / 8 kv heads,
    bs 16); the oracle checks every sequence."""
    w = wl.WORKLOADS["mtp_decode_bf16"]
    say("full mtp workload via decode_mtp (all rows)")
    c = wl.make_workload_case(w, seed=0, device=DEV)
    o = oracle_step(c, causal=True)
    g = mtp_step(c, 2)
    compare_writes(c, g, o)
    compare_outputs(c, g, o, tokens=o["tokens"], label="mtp workload")
