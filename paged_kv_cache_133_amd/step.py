"""A decode step recorded once and replayed with new host-built tables (pkv_runner_*).

"Paged KV Cache and Packed Sequence", 5.3: the block table changes every step, so the
recorded step must not hold it; the host builds it (BlockManager.decode_step) into a
buffer that is copied to the device at the start of each replay, and with two such buffers
the host fills the next one while this step runs.  Here:

  * two pinned host buffers and two device buffers, each [batch * max_blocks_per_seq +
    batch] int32 (the table, then seq_lens_kv), owned by this object;
  * two graphs in a native step runner, graph j recording a copy kernel (pinned host
    buffer j -> device buffer j) and pkv_paged_attn_decode_append (write of the new rows
    and attention) over device buffer j;
  * launch(): one library call that replays graph j on the current stream.

The batch is fixed at capture; rows without a sequence are padding rows (length 0: output
0, lse -inf, nothing written, slot -1).  Inputs q, k_new and v_new are the step's own
device tensors, written by the caller before launch() on the current stream.
"""
from __future__ import annotations

import ctypes

import torch

from ._lib import PagedKVError, _check, _stream, lib, new_decode_workspace, \
    paged_attn_decode_append


class GraphDecodeStep:
    def __init__(self, k_cache: torch.Tensor, v_cache: torch.Tensor, batch: int,
                 max_blocks_per_seq: int, num_q_heads: int, softmax_scale: float,
                 window: int = 0):
        dev = k_cache.device
        nb, bs, hkv, d = k_cache.shape
        self.device, self.batch, self.mbs = dev, batch, max_blocks_per_seq
        self.max_len = max_blocks_per_seq * bs
        n = batch * max_blocks_per_seq + batch
        self.nbytes = n * 4
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
        vp = ctypes.c_void_p
        self._r = lib().pkv_runner_create(vp(self.dev[0].data_ptr()), vp(self.dev[1].data_ptr()),
                                          vp(self.staging[0].data_ptr()),
                                          vp(self.staging[1].data_ptr()), self.nbytes)
        if not self._r:
            msg = lib().pkv_last_error()
            raise PagedKVError(-8, msg.decode() if msg else "")
        cap = torch.cuda.Stream(dev)
        cap_h = vp(cap.cuda_stream)
        cap.wait_stream(torch.cuda.current_stream(dev))
        for j in range(2):
            table, lens = self.device_views(j)
            with torch.cuda.stream(cap):
                _check(lib().pkv_runner_capture_begin(self._r, j, cap_h))
                try:
                    paged_attn_decode_append(self.q, self.k_new, self.v_new, k_cache, v_cache,
                                             table, lens, self.max_len, softmax_scale,
                                             out=self.out, lse=self.lse,
                                             workspace=self.workspace, slots_out=self.slots,
                                             window=window)
                finally:
                    rc = lib().pkv_runner_capture_end(self._r, cap_h)
                _check(rc)
        torch.cuda.current_stream(dev).wait_stream(cap)

    def device_views(self, j: int):
        cut = self.batch * self.mbs
        return self.dev[j][:cut].view(self.batch, self.mbs), self.dev[j][cut:]

    def host_tables(self):
        """(table [batch][max_blocks_per_seq], seq_lens [batch]) numpy views of the pinned
        buffer the next launch() copies in; fill both before calling it.  Waits until the
        replay that last read this buffer (two steps back) has run."""
        p = lib().pkv_runner_host_buffer(self._r)
        if not p:
            _check(-8)
        j = 0 if p == self.staging[0].data_ptr() else 1
        cut = self.batch * self.mbs
        v = self._host[j]
        return v[:cut].reshape(self.batch, self.mbs), v[cut:]

    def launch(self):
        """Replay the step on the current stream: the table copy, then write-and-attend."""
        _check(lib().pkv_runner_launch(self._r, _stream(self.device)))

    def graph(self, j: int):
        """Executable graph j (its table copy and the step; pkv_graph_launch)."""
        return lib().pkv_runner_graph(self._r, j)

    def close(self):
        if getattr(self, "_r", None):
            lib().pkv_runner_destroy(self._r)
            self._r = None

    __del__ = close
