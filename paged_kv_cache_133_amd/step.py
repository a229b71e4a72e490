"""A decode step recorded once and replayed with new host-built tables.

"Paged KV Cache and Packed Sequence", 5.3: the block table changes every step, so the
recorded step must not hold it; the host builds it (BlockManager.table) into a tensor that
is copied to the device before each replay, and with two such buffers the copy for the next
step runs while this step's attention does.  Here:

  * two pinned host buffers and two device buffers, each [batch * max_blocks_per_seq +
    batch] int32 (the table, then seq_lens_kv);
  * two graphs, graph j recording pkv_paged_attn_decode_ex (write of the new rows and
    attention) over device buffer j, on a stream of its own;
  * launch(): the upload of buffer j runs on a copy stream once the graph that last read
    device buffer j is done, and graph j waits for that upload only, so the upload of step
    t+1 overlaps the attention of step t when the host runs ahead.

The batch is fixed at capture; rows without a sequence are padding rows (length 0: output
0, lse -inf, nothing written, slot -1).  Inputs q, k_new and v_new are the step's own
device tensors, written by the caller before launch() on the current stream.
"""
from __future__ import annotations

import ctypes

import torch

from ._lib import _check, lib, new_decode_workspace, paged_attn_decode_append, upload


class GraphDecodeStep:
    def __init__(self, k_cache: torch.Tensor, v_cache: torch.Tensor, batch: int,
                 max_blocks_per_seq: int, num_q_heads: int, softmax_scale: float,
                 window: int = 0):
        dev = k_cache.device
        nb, bs, hkv, d = k_cache.shape
        self.device, self.batch, self.mbs = dev, batch, max_blocks_per_seq
        self.max_len = max_blocks_per_seq * bs
        n = batch * max_blocks_per_seq + batch
        self.staging = [torch.zeros(n, dtype=torch.int32, pin_memory=True) for _ in range(2)]
        self._host = [s.numpy() for s in self.staging]
        self.dev = [torch.zeros(n, dtype=torch.int32, device=dev) for _ in range(2)]
        self.q = torch.zeros(batch, num_q_heads, d, dtype=k_cache.dtype, device=dev)
        self.k_new = torch.zeros(batch, hkv, d, dtype=k_cache.dtype, device=dev)
        self.v_new = torch.zeros_like(self.k_new)
        self.out = torch.zeros_like(self.q)
        self.lse = torch.zeros(batch, num_q_heads, dtype=torch.float32, device=dev)
        self.slots = torch.zeros(batch, dtype=torch.int64, device=dev)
        self.workspace = new_decode_workspace(batch, num_q_heads, hkv, d, self.max_len, dev)
        self.main = torch.cuda.Stream(dev)
        self.copy = torch.cuda.Stream(dev)
        self._main_h = ctypes.c_void_p(self.main.cuda_stream)
        self.uploaded = [torch.cuda.Event() for _ in range(2)]
        self.consumed = [torch.cuda.Event() for _ in range(2)]
        self.graphs = []
        self.main.wait_stream(torch.cuda.current_stream(dev))
        for j in range(2):
            table, lens = self.device_views(j)
            with torch.cuda.stream(self.main):
                _check(lib().pkv_graph_begin(self._main_h))
                g = ctypes.c_void_p()
                try:
                    paged_attn_decode_append(self.q, self.k_new, self.v_new, k_cache, v_cache,
                                             table, lens, self.max_len, softmax_scale,
                                             out=self.out, lse=self.lse,
                                             workspace=self.workspace, slots_out=self.slots,
                                             window=window)
                except BaseException:
                    lib().pkv_graph_end(self._main_h, ctypes.byref(g))
                    lib().pkv_graph_destroy(g)
                    self.close()
                    raise
                _check(lib().pkv_graph_end(self._main_h, ctypes.byref(g)))
            self.graphs.append(g)
        self.t = 0

    def device_views(self, j: int):
        cut = self.batch * self.mbs
        return self.dev[j][:cut].view(self.batch, self.mbs), self.dev[j][cut:]

    def host_tables(self):
        """(table [batch][max_blocks_per_seq], seq_lens [batch]) numpy views of the pinned
        buffer the next launch() uploads; fill both before calling it.  Waits until the
        upload that last read this buffer has run."""
        j = self.t % 2
        self.uploaded[j].synchronize()
        cut = self.batch * self.mbs
        v = self._host[j]
        return v[:cut].reshape(self.batch, self.mbs), v[cut:]

    def launch(self, timing=None):
        """Upload the host tables and replay the step; the current stream then waits for
        it (out, lse and slots are ready for work enqueued on it afterwards).  timing: an
        optional dict of two timing-event pairs, "upload" (recorded on the copy stream
        around the upload) and "graph" (on the step's stream around the replay)."""
        j = self.t % 2
        cur = torch.cuda.current_stream(self.device)
        self.copy.wait_event(self.consumed[j])
        if timing:
            timing["upload"][0].record(self.copy)
        with torch.cuda.stream(self.copy):
            upload(self.dev[j], self.staging[j])
        if timing:
            timing["upload"][1].record(self.copy)
        self.uploaded[j].record(self.copy)
        self.main.wait_stream(cur)
        self.main.wait_event(self.uploaded[j])
        if timing:
            timing["graph"][0].record(self.main)
        _check(lib().pkv_graph_launch(self.graphs[j], self._main_h))
        if timing:
            timing["graph"][1].record(self.main)
        self.consumed[j].record(self.main)
        cur.wait_stream(self.main)
        self.t += 1

    def close(self):
        for g in getattr(self, "graphs", []):
            lib().pkv_graph_destroy(g)
        self.graphs = []

    __del__ = close
