"""GPU parity of the sliding-window (band) forms against the fp64 oracle, through the C
ABI: every decode kernel (vector-ALU split kernel, GQA range-streaming and per-split MFMA
kernels, write-and-attend), the varlen chunk (causal and not), and MTP-shaped decode
(next_n + 1 causal query tokens per sequence through the varlen path).  Needs an MI355X."""
import numpy as np
import pytest
import torch

import paged_kv_cache_133_amd as pkv
from paged_kv_cache_133_amd import workloads as wl
from tests.gpu_common import compare_outputs, compare_writes, gpu_step, oracle_step, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

LENS = [1, 31, 32, 33, 300, 1500, 3000]     # after the step
# (Hq, Hkv, D, block_size, dtype): VALU (fp32 GQA, bf16 MHA), range streaming, per split
SHAPES = [(4, 1, 64, 16, "f32"), (8, 8, 128, 16, "bf16"), (32, 4, 128, 16, "bf16"),
          (32, 4, 128, 2, "bf16"), (48, 4, 64, 128, "bf16"), (5, 5, 64, 16, "bf16")]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "hq%d_hkv%d_d%d_bs%d_%s" % s)
@pytest.mark.parametrize("window", [1, 33, 256, 1000, 4096])
def test_decode_window(shape, window):
    Hq, Hkv, D, bs, dt = shape
    w = wl.custom(batch=len(LENS), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                  dtype=dt)
    say(f"decode window {window}: {shape}")
    c = wl.make_case(w, np.array(LENS) - 1, [1] * len(LENS), seed=window + Hq, device=DEV)
    g = gpu_step(c, window=window)
    o = oracle_step(c, window=window)
    compare_writes(c, g, o)
    compare_outputs(c, g, o, tokens=o["tokens"], label=f"window {window} {shape}")


@pytest.mark.parametrize("shape", [(32, 4, 128, 16, "bf16"), (64, 4, 64, 32, "bf16")],
                         ids=lambda s: "hq%d_hkv%d_d%d_bs%d_%s" % s)
@pytest.mark.parametrize("window", [4096, 5000])
def test_decode_window_long(shape, window):
    """Windows of 4096+ keys over sequences to 9000: the range kernel's compact layout."""
    Hq, Hkv, D, bs, dtype = shape
    w = wl.custom(batch=5, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs, dtype=dtype)
    L = [9000, 40, 5000, 4100, 1]
    say(f"decode window {window} long: {shape}")
    c = wl.make_case(w, np.array(L) - 1, [1] * len(L), seed=window + D, device=DEV)
    g = gpu_step(c, window=window)
    o = oracle_step(c, window=window)
    compare_writes(c, g, o)
    compare_outputs(c, g, o, tokens=o["tokens"], label=f"window {window} long {shape}")


@pytest.mark.parametrize("shape", SHAPES[1:4], ids=lambda s: "hq%d_hkv%d_d%d_bs%d_%s" % s)
def test_decode_append_window(shape):
    """Write-and-attend with a window: pool bytes, slots, outputs and lse as the oracle's."""
    Hq, Hkv, D, bs, dt = shape
    window = 100
    w = wl.custom(batch=len(LENS), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                  dtype=dt)
    c = wl.make_case(w, np.array(LENS) - 1, [1] * len(LENS), seed=7, device=DEV)
    o = oracle_step(c, window=window)
    B = len(LENS)
    k, v = c.cache_k.clone(), c.cache_v.clone()
    slots = torch.full((B,), -3, dtype=torch.int64, device=DEV)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    out, _ = pkv.paged_attn_decode_append(c.q, c.new_k, c.new_v, k, v, c.table_tensor(DEV),
                                          c.lens_after_tensor(DEV), c.max_len_after, w.scale,
                                          lse=lse, slots_out=slots, window=window)
    torch.cuda.synchronize()
    g = {"slots": slots, "cache_k": k, "cache_v": v, "out": out, "lse": lse}
    compare_writes(c, g, o)
    compare_outputs(c, g, o, tokens=o["tokens"], label=f"append window {shape}")


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("window", [1, 40, 300])
@pytest.mark.parametrize("shape", [(32, 8, 128, 16), (16, 4, 64, 64)], ids=lambda s: "hq%d_hkv%d_d%d_bs%d" % s)
def test_varlen_window(shape, window, causal):
    Hq, Hkv, D, bs = shape
    w = wl.custom(mode="varlen", batch=4, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                  block_size=bs, dtype="bf16")
    say(f"varlen window {window} causal {causal}: {shape}")
    c = wl.make_case(w, [0, 70, 300, 1000], [45, 1, 130, 200], seed=window, device=DEV)
    g = gpu_step(c, causal=causal, window=window)
    o = oracle_step(c, causal=causal, window=window)
    compare_writes(c, g, o)
    compare_outputs(c, g, o, tokens=o["tokens"], label=f"varlen window {window} causal {causal}")


def test_mtp_decode_through_varlen():
    """MTP decode: next_n + 1 = 2 new tokens per sequence, causal, written then attended
    in one varlen call; also with a window."""
    w = wl.custom(mode="varlen", batch=6, num_q_heads=32, num_kv_heads=8, head_dim=128,
                  block_size=16, dtype="bf16")
    c = wl.make_case(w, [0, 15, 16, 511, 1200, 2047], [2] * 6, seed=12, device=DEV)
    for window in (0, 64):
        say(f"mtp decode window {window}")
        g = gpu_step(c, causal=True, window=window)
        o = oracle_step(c, causal=True, window=window)
        compare_writes(c, g, o)
        compare_outputs(c, g, o, tokens=o["tokens"], label=f"mtp window {window}")


@pytest.mark.parametrize("name", ["swa_decode_bf16", "mtp_decode_bf16"])
def test_window_and_mtp_workloads(name):
    """The full-size band and MTP workloads as the bench runs them (write-and-attend for the
    band, write + varlen for MTP); the oracle checks every sequence."""
    w = wl.WORKLOADS[name]
    say(f"full workload {name} (all rows)")
    c = wl.make_workload_case(w, seed=0, device=DEV)
    o = oracle_step(c, causal=w.mode == "varlen", window=w.window)
    if w.mode == "varlen":
        g = gpu_step(c, causal=True, window=w.window)
    else:
        B = w.batch
        k, v = c.cache_k.clone(), c.cache_v.clone()
        slots = torch.full((B,), -3, dtype=torch.int64, device=DEV)
        lse = torch.empty((B, w.num_q_heads), dtype=torch.float32, device=DEV)
        out, _ = pkv.paged_attn_decode_append(c.q, c.new_k, c.new_v, k, v, c.table_tensor(DEV),
                                              c.lens_after_tensor(DEV), c.max_len_after, w.scale,
                                              lse=lse, slots_out=slots, window=w.window)
        torch.cuda.synchronize()
        g = {"slots": slots, "cache_k": k, "cache_v": v, "out": out, "lse": lse}
    compare_writes(c, g, o)
    compare_outputs(c, g, o, tokens=o["tokens"], label=name)
