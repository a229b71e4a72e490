"""The measurement aids through the C ABI: the stream read and the gather read run, return
PKV_OK and leave the sink alone on an all-zero source (their XOR never matches the constant
that would make them write).  Needs an MI355X."""
import pytest
import torch

import paged_kv_cache_133_amd as pkv
from paged_kv_cache_133_amd import _lib
from paged_kv_cache_133_amd import workloads as wl
from tests.gpu_common import say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def test_stream_read_runs():
    src = torch.zeros(1 << 20, dtype=torch.uint8, device=DEV)
    sink = torch.zeros(4, dtype=torch.int32, device=DEV)
    say("stream_read 1 MiB")
    for grid in (1, 7, 1024):
        _lib.prepare_stream_read(src, sink, grid)()
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0


@pytest.mark.parametrize("bs", [1, 16, 128])
def test_gather_read_runs(bs):
    w = wl.custom(mode="decode", batch=3, num_q_heads=4, num_kv_heads=2, head_dim=64,
                  block_size=bs, dtype="bf16")
    c = wl.make_case(w, [0, 300, 1500], [1, 1, 1], seed=5, device=DEV)
    k = torch.zeros_like(c.cache_k)
    v = torch.zeros_like(c.cache_v)
    sink = torch.zeros(4, dtype=torch.int32, device=DEV)
    table = c.table_tensor(DEV)
    la = c.lens_after_tensor(DEV)
    row = k[0, 0].numel() * k.element_size()
    say(f"gather_read bs={bs} row={row}")
    for slice_bytes, split in ((128, 256), (row, 16), (row, 1024), (16, 1)):
        _lib.prepare_gather_read(k, v, table, la, c.max_len_after, slice_bytes, split, sink)()
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0
    with pytest.raises(pkv.PagedKVError):
        _lib.prepare_gather_read(k, v, table, la, c.max_len_after, 48, 256, sink)()
