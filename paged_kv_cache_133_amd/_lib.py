"""ctypes binding of libpagedkv.so: argument marshalling only.

Every function takes torch tensors that already live on the GPU, reads their shapes,
passes raw device pointers and torch's current HIP stream to the C ABI
(include/pagedkv.h), and raises PagedKVError with the library's message on a
non-zero status.  torch supplies device memory (outputs, workspace) and streams;
all computation happens in the library's kernels.  There is no fallback: without the
built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

# PKV_LIBRARY_PATH names another build of the library (the host-sanitizer test loads a
# host-only ASan/UBSan build this way); by default the one built next to this file.
LIB_PATH = (os.environ.get("PKV_LIBRARY_PATH")
            or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedkv.so"))

PKV_F32, PKV_BF16 = 0, 1
STATUS = {0: "PKV_OK", -1: "PKV_ERR_NULL", -2: "PKV_ERR_SHAPE", -3: "PKV_ERR_DTYPE",
          -4: "PKV_ERR_UNSUPPORTED", -5: "PKV_ERR_ALIGN", -6: "PKV_ERR_SCALE",
          -7: "PKV_ERR_WORKSPACE", -8: "PKV_ERR_HIP"}
EXPORTS = ("pkv_version", "pkv_last_error", "pkv_slot_mapping", "pkv_kv_cache_write",
           "pkv_kv_cache_append", "pkv_kv_cache_write_int8", "pkv_kv_rmsnorm_rope_cache",
           "pkv_decode_workspace_size", "pkv_paged_attn_decode_int8",
           "pkv_paged_attn_decode",
           "pkv_paged_attn_decode_split", "pkv_paged_attn_decode_combine",
           "pkv_paged_attn_decode_append", "pkv_paged_attn_decode_append_noalloc",
           "pkv_paged_attn_decode_ex", "pkv_paged_attn_varlen",
           "pkv_paged_attn_varlen_ex", "pkv_bm_create", "pkv_bm_destroy", "pkv_bm_num_free",
           "pkv_bm_add", "pkv_bm_fork", "pkv_bm_append", "pkv_bm_decode_step", "pkv_bm_free",
           "pkv_bm_length",
           "pkv_bm_ref_count", "pkv_bm_table", "pkv_kv_cache_copy_blocks", "pkv_upload",
           "pkv_graph_begin", "pkv_graph_end", "pkv_graph_launch", "pkv_graph_destroy",
           "pkv_runner_create", "pkv_runner_destroy", "pkv_runner_capture_begin",
           "pkv_runner_capture_end", "pkv_runner_graph", "pkv_runner_host_buffer",
           "pkv_runner_launch", "pkv_upload_kernel", "pkv_decode_mtp_workspace_size", "pkv_paged_attn_decode_mtp",
           "pkv_kv_cache_write_int8_mla", "pkv_paged_attn_decode_mla_int8", "pkv_stream_read",
           "pkv_paged_attn_decode_int8_append", "pkv_paged_attn_decode_mla_append",
           "pkv_gather_read", "pkv_paged_attn_decode_mla_int8_append",
           "pkv_paged_attn_varlen_append", "pkv_paged_attn_decode_mtp_append")


class PagedKVError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libpagedkv.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m paged_kv_cache_133_amd.build` (needs hipcc)")
    L = ctypes.CDLL(LIB_PATH)
    p, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                            ctypes.c_size_t)
    L.pkv_version.restype = ctypes.c_int
    L.pkv_version.argtypes = []
    L.pkv_last_error.restype = ctypes.c_char_p
    L.pkv_last_error.argtypes = []
    L.pkv_slot_mapping.restype = ctypes.c_int
    L.pkv_slot_mapping.argtypes = [p, p, p, p, i32, i64, i32, i32, p]
    L.pkv_kv_cache_write.restype = ctypes.c_int
    L.pkv_kv_cache_write.argtypes = [p, p, p, p, p, i64, i32, i32, i32, i32, i64, i32, p]
    L.pkv_kv_cache_append.restype = ctypes.c_int
    L.pkv_kv_cache_append.argtypes = [p, p, p, p, p, p, p, p, i32, i64, i32, i32, i32, i32, i32,
                                      i32, i64, i32, p]
    L.pkv_kv_cache_write_int8.restype = ctypes.c_int
    L.pkv_kv_cache_write_int8.argtypes = [p, p, p, p, p, p, p, i64, i32, i32, i32, i64, i32, p]
    L.pkv_paged_attn_decode_int8.restype = ctypes.c_int
    L.pkv_paged_attn_decode_int8.argtypes = [p, p, p, p, p, p, p, p, p, i32, i32, i32, i32, i32,
                                             i32, i32, i64, f32, i32, i32, p, sz, p]
    L.pkv_paged_attn_decode_mla_append.restype = ctypes.c_int
    L.pkv_paged_attn_decode_mla_append.argtypes = [p, p, p, p, p, p, p, p, p, p, p, i32, i32, i32,
                                                   i32, i32, i64, f32, i32, p, sz, p]
    L.pkv_paged_attn_decode_int8_append.restype = ctypes.c_int
    L.pkv_paged_attn_decode_int8_append.argtypes = [p, p, p, p, p, p, p, p, p, p, p, p, i32, i32, i32,
                                                    i32, i32, i32, i32, i64, f32, i32, i32, p, sz, p]
    L.pkv_kv_rmsnorm_rope_cache.restype = ctypes.c_int
    L.pkv_kv_rmsnorm_rope_cache.argtypes = [p, p, p, p, p, p, p, i64, i32, i32, i32, i64, f32, i32, p]
    L.pkv_decode_workspace_size.restype = sz
    L.pkv_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    for name in ("pkv_paged_attn_decode", "pkv_paged_attn_decode_split",
                 "pkv_paged_attn_decode_combine"):
        fn = getattr(L, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [p, p, p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                       i64, f32, i32, p, sz, p]
    L.pkv_paged_attn_decode_append.restype = ctypes.c_int
    L.pkv_paged_attn_decode_append.argtypes = [p, p, p, p, p, p, p, p, p, p, i32, i32, i32, i32,
                                               i32, i32, i32, i64, f32, i32, i32, p, sz, p]
    L.pkv_stream_read.restype = ctypes.c_int
    L.pkv_stream_read.argtypes = [p, i64, p, i32, p]
    L.pkv_gather_read.restype = ctypes.c_int
    L.pkv_gather_read.argtypes = [p, p, p, p, i32, i32, i32, i32, i64, i32, i32, i32, p, p]
    L.pkv_paged_attn_decode_append_noalloc.restype = ctypes.c_int
    L.pkv_paged_attn_decode_append_noalloc.argtypes = [p, p, p, p, p, p, p, p, p, p, i32, i32,
                                                       i32, i32, i32, i32, i32, i64, f32, i32, p]
    L.pkv_paged_attn_decode_ex.restype = ctypes.c_int
    L.pkv_paged_attn_decode_ex.argtypes = [p, p, p, p, p, p, p, p, p, p, i32, i32, i32, i32,
                                           i32, i32, i32, i64, f32, i32, i32, i32, p, sz, p]
    L.pkv_paged_attn_varlen.restype = ctypes.c_int
    L.pkv_paged_attn_varlen.argtypes = [p, p, p, p, p, p, p, p, i32, i64, i32, i32, i32, i32,
                                        i32, i32, i64, f32, i32, i32, p]
    L.pkv_paged_attn_varlen_ex.restype = ctypes.c_int
    L.pkv_paged_attn_varlen_ex.argtypes = [p, p, p, p, p, p, p, p, i32, i64, i32, i32, i32, i32,
                                           i32, i32, i64, f32, i32, i32, i32, p]
    L.pkv_paged_attn_varlen_append.restype = ctypes.c_int
    L.pkv_paged_attn_varlen_append.argtypes = [p, p, p, p, p, p, p, p, p, p, i32, i64, i32, i32,
                                               i32, i32, i32, i32, i64, f32, i32, i32, i32, p, p]
    L.pkv_bm_create.restype = p
    L.pkv_bm_create.argtypes = [i64, i32, i32]
    L.pkv_bm_destroy.restype = None
    L.pkv_bm_destroy.argtypes = [p]
    L.pkv_bm_num_free.restype = i64
    L.pkv_bm_num_free.argtypes = [p]
    for name in ("pkv_bm_add", "pkv_bm_free"):
        getattr(L, name).restype = ctypes.c_int
        getattr(L, name).argtypes = [p, i64]
    L.pkv_bm_fork.restype = ctypes.c_int
    L.pkv_bm_fork.argtypes = [p, i64, i64]
    L.pkv_bm_append.restype = ctypes.c_int
    L.pkv_bm_append.argtypes = [p, i64, i32, p, p, p]
    L.pkv_bm_decode_step.restype = ctypes.c_int
    L.pkv_bm_decode_step.argtypes = [p, p, i32, p, p, p, p, p, i32]
    L.pkv_bm_length.restype = ctypes.c_int
    L.pkv_bm_length.argtypes = [p, i64, p]
    L.pkv_bm_ref_count.restype = ctypes.c_int
    L.pkv_bm_ref_count.argtypes = [p, i32, p]
    L.pkv_bm_table.restype = ctypes.c_int
    L.pkv_bm_table.argtypes = [p, p, i32, p, p, i32]
    L.pkv_kv_cache_copy_blocks.restype = ctypes.c_int
    L.pkv_kv_cache_copy_blocks.argtypes = [p, i64, i64, p, i32, p]
    L.pkv_upload.restype = ctypes.c_int
    L.pkv_upload.argtypes = [p, p, sz, p]
    L.pkv_graph_begin.restype = ctypes.c_int
    L.pkv_graph_begin.argtypes = [p]
    L.pkv_graph_end.restype = ctypes.c_int
    L.pkv_graph_end.argtypes = [p, p]
    L.pkv_graph_launch.restype = ctypes.c_int
    L.pkv_graph_launch.argtypes = [p, p]
    L.pkv_graph_destroy.restype = ctypes.c_int
    L.pkv_graph_destroy.argtypes = [p]
    L.pkv_kv_cache_write_int8_mla.restype = ctypes.c_int
    L.pkv_kv_cache_write_int8_mla.argtypes = [p, p, p, p, p, p, p, i64, i32, i64, i32, p]
    L.pkv_paged_attn_decode_mla_int8.restype = ctypes.c_int
    L.pkv_paged_attn_decode_mla_int8.argtypes = [p, p, p, p, p, p, p, p, p, p, i32, i32, i32, i32,
                                                 i32, i64, f32, i32, p, sz, p]
    L.pkv_paged_attn_decode_mla_int8_append.restype = ctypes.c_int
    L.pkv_paged_attn_decode_mla_int8_append.argtypes = [p, p, p, p, p, p, p, p, p, p, p, p, p, i32,
                                                        i32, i32, i32, i32, i64, f32, i32, p, sz, p]
    L.pkv_decode_mtp_workspace_size.restype = sz
    L.pkv_decode_mtp_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    L.pkv_paged_attn_decode_mtp.restype = ctypes.c_int
    L.pkv_paged_attn_decode_mtp.argtypes = [p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32,
                                            i32, i32, i64, f32, i32, i32, i32, p, sz, p]
    L.pkv_paged_attn_decode_mtp_append.restype = ctypes.c_int
    L.pkv_paged_attn_decode_mtp_append.argtypes = [p, p, p, p, p, p, p, p, p, i32, i32, i32, i32,
                                                   i32, i32, i32, i32, i64, f32, i32, i32, i32, p,
                                                   sz, p, p]
    L.pkv_runner_create.restype = p
    L.pkv_runner_create.argtypes = [p, p, p, p, sz]
    L.pkv_runner_destroy.restype = ctypes.c_int
    L.pkv_runner_destroy.argtypes = [p]
    L.pkv_runner_capture_begin.restype = ctypes.c_int
    L.pkv_runner_capture_begin.argtypes = [p, i32, p]
    L.pkv_runner_capture_end.restype = ctypes.c_int
    L.pkv_runner_capture_end.argtypes = [p, p]
    L.pkv_runner_graph.restype = p
    L.pkv_runner_graph.argtypes = [p, i32]
    L.pkv_runner_host_buffer.restype = p
    L.pkv_runner_host_buffer.argtypes = [p]
    L.pkv_runner_launch.restype = ctypes.c_int
    L.pkv_runner_launch.argtypes = [p, p]
    L.pkv_upload_kernel.restype = ctypes.c_int
    L.pkv_upload_kernel.argtypes = [p, p, sz, p]
    _lib = L
    return L


def _check(rc: int):
    if rc != 0:
        msg = lib().pkv_last_error()
        raise PagedKVError(rc, msg.decode() if msg else "")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PKV_F32
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _batch_rows(B, block_table, seq_lens_kv, q_rope=None):
    """Host-side guard: one table row and one length per sequence (the library cannot see
    device array sizes; a mismatch would read past a tensor's end)."""
    if block_table.dim() != 2 or block_table.shape[0] != B or seq_lens_kv.shape[0] != B:
        raise ValueError(f"block_table {tuple(block_table.shape)} and seq_lens_kv "
                         f"{tuple(seq_lens_kv.shape)} need one row per sequence (batch {B})")
    if q_rope is not None and q_rope.shape[0] != B:
        raise ValueError(f"q_rope has {q_rope.shape[0]} rows, expected {B}")


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("tensors must live on the GPU")
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def version() -> int:
    return int(lib().pkv_version())


def slot_mapping(block_table: torch.Tensor, lens_before: torch.Tensor, cu_new: torch.Tensor,
                 block_size: int, num_tokens: int,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """int64 slot per new token (see pkv_slot_mapping)."""
    _dev(block_table, lens_before, cu_new, out)
    if out is None:
        out = torch.empty(num_tokens, dtype=torch.int64, device=block_table.device)
    _check(lib().pkv_slot_mapping(_ptr(out), _ptr(block_table), _ptr(lens_before), _ptr(cu_new),
                                  lens_before.shape[0], num_tokens, block_table.shape[1],
                                  block_size, _stream(block_table.device)))
    return out


def kv_cache_write(k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor,
                   v_cache: torch.Tensor, slots: torch.Tensor) -> None:
    """Scatter k_new/v_new rows into the caches at `slots` (see pkv_kv_cache_write)."""
    _dev(k_new, v_new, k_cache, v_cache, slots)
    nb, bs, hkv, dk = k_cache.shape
    dv = v_cache.shape[-1]
    _check(lib().pkv_kv_cache_write(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(slots), slots.shape[0], hkv, dk, dv, bs, nb,
                                    _dtype_code(k_cache), _stream(k_cache.device)))


def _append_args(k_new, v_new, k_cache, v_cache, block_table, lens_before, cu_new,
                 max_new_tokens, slots_out):
    _dev(k_new, v_new, k_cache, v_cache, block_table, lens_before, cu_new, slots_out)
    nb, bs, hkv, dk = k_cache.shape
    dv = v_cache.shape[-1]
    return (_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
            _ptr(lens_before), _ptr(cu_new), _ptr(slots_out), lens_before.shape[0],
            k_new.shape[0], max_new_tokens, block_table.shape[1], hkv, dk, dv, bs, nb,
            _dtype_code(k_cache), _stream(k_cache.device))


def kv_cache_append(k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor,
                    v_cache: torch.Tensor, block_table: torch.Tensor, lens_before: torch.Tensor,
                    cu_new: torch.Tensor, max_new_tokens: int,
                    slots_out: Optional[torch.Tensor] = None) -> Optional[torch.Tensor]:
    """slot_mapping + write in one launch (see pkv_kv_cache_append)."""
    _check(lib().pkv_kv_cache_append(*_append_args(k_new, v_new, k_cache, v_cache, block_table,
                                                   lens_before, cu_new, max_new_tokens,
                                                   slots_out)))
    return slots_out


def prepare_kv_cache_append(k_new, v_new, k_cache, v_cache, block_table, lens_before, cu_new,
                            max_new_tokens, slots_out=None):
    args = _append_args(k_new, v_new, k_cache, v_cache, block_table, lens_before, cu_new,
                        max_new_tokens, slots_out)
    return PreparedCall(lib().pkv_kv_cache_append, args,
                        (k_new, v_new, k_cache, v_cache, block_table, lens_before, cu_new,
                         slots_out))


def kv_rmsnorm_rope_cache(kv: torch.Tensor, gamma: torch.Tensor, cos: torch.Tensor,
                          sin: torch.Tensor, cache_nope: torch.Tensor, cache_rope: torch.Tensor,
                          slot_mapping: torch.Tensor, eps: float):
    """RMSNorm + RoPE + write of the MLA latent row (see pkv_kv_rmsnorm_rope_cache).
    kv [T, Dn + Dr], gamma [Dn], cos/sin [T, Dr/2] fp32, caches [nb, bs, 1, Dn/Dr].
    eps (the RMSNorm epsilon) has no default: the caller states the model's value."""
    _dev(kv, gamma, cos, sin, cache_nope, cache_rope, slot_mapping)
    nb, bs, _, dn = cache_nope.shape
    dr = cache_rope.shape[-1]
    _check(lib().pkv_kv_rmsnorm_rope_cache(_ptr(kv), _ptr(gamma), _ptr(cos), _ptr(sin),
                                           _ptr(cache_nope), _ptr(cache_rope), _ptr(slot_mapping),
                                           slot_mapping.shape[0], dn, dr, bs, nb, float(eps),
                                           _dtype_code(kv), _stream(kv.device)))


def _scale_shape(k_scale, v_scale, nb, hkv, bs):
    for s in (k_scale, v_scale):
        if tuple(s.shape) != (nb, hkv, bs) or s.dtype != torch.float32:
            raise ValueError(f"INT8 scale arrays are float32 [num_blocks, num_kv_heads, "
                             f"block_size] = {(nb, hkv, bs)}, got {tuple(s.shape)} {s.dtype}")


def kv_cache_write_int8(k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor,
                        v_cache: torch.Tensor, k_scale: torch.Tensor, v_scale: torch.Tensor,
                        slot_mapping: torch.Tensor):
    """Quantize and write one step's K/V rows into the INT8 cache (see
    pkv_kv_cache_write_int8).  Caches [nb, bs, Hkv, D] int8, scales [nb, Hkv, bs] fp32."""
    _dev(k_new, v_new, k_cache, v_cache, k_scale, v_scale, slot_mapping)
    nb, bs, hkv, d = k_cache.shape
    _scale_shape(k_scale, v_scale, nb, hkv, bs)
    _check(lib().pkv_kv_cache_write_int8(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                         _ptr(k_scale), _ptr(v_scale), _ptr(slot_mapping),
                                         slot_mapping.shape[0], hkv, d, bs, nb, _dtype_code(k_new),
                                         _stream(k_new.device)))


def _decode_int8_args(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens_kv,
                      max_seq_len_kv, softmax_scale, stages, out, lse, workspace, window):
    _dev(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens_kv, out, lse, workspace)
    B, hq, d = q.shape
    _batch_rows(B, block_table, seq_lens_kv)
    nb, bs, hkv, _ = k_cache.shape
    _scale_shape(k_scale, v_scale, nb, hkv, bs)
    if out is None:
        out = torch.empty((B, hq, d), dtype=q.dtype, device=q.device)
    if workspace is None:
        workspace = new_decode_workspace(B, hq, hkv, d, max_seq_len_kv, q.device)
    args = (_ptr(out), _ptr(lse), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
            _ptr(v_scale), _ptr(block_table), _ptr(seq_lens_kv), B, block_table.shape[1],
            max_seq_len_kv, hq, hkv, d, bs, nb, float(softmax_scale), int(window), stages,
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q.device))
    return args, out, workspace


def paged_attn_decode_int8(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens_kv,
                           max_seq_len_kv, softmax_scale, out=None, lse=None, workspace=None,
                           window=0):
    """Decode over the INT8 cache (see pkv_paged_attn_decode_int8).  Returns (out, lse)."""
    args, out, _ = _decode_int8_args(q, k_cache, v_cache, k_scale, v_scale, block_table,
                                     seq_lens_kv, max_seq_len_kv, softmax_scale, 3, out, lse,
                                     workspace, window)
    _check(lib().pkv_paged_attn_decode_int8(*args))
    return out, lse


def prepare_decode_int8(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens_kv,
                        max_seq_len_kv, softmax_scale, out=None, lse=None, workspace=None, window=0):
    """(split pass, combine pass) prepared calls of pkv_paged_attn_decode_int8."""
    calls = []
    for stages in (1, 2):
        args, out, workspace = _decode_int8_args(q, k_cache, v_cache, k_scale, v_scale, block_table,
                                                 seq_lens_kv, max_seq_len_kv, softmax_scale, stages,
                                                 out, lse, workspace, window)
        calls.append(PreparedCall(lib().pkv_paged_attn_decode_int8, args,
                                  (q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens_kv,
                                   out, lse, workspace)))
    return calls[0], calls[1], out


def _decode_int8_append_args(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_table,
                             seq_lens_kv, max_seq_len_kv, softmax_scale, stages, out, lse,
                             workspace, slots_out, window):
    _dev(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens_kv, out, lse,
         workspace, slots_out)
    B, hq, d = q.shape
    _batch_rows(B, block_table, seq_lens_kv)
    nb, bs, hkv, _ = k_cache.shape
    _scale_shape(k_scale, v_scale, nb, hkv, bs)
    if tuple(k_new.shape) != (B, hkv, d) or tuple(v_new.shape) != (B, hkv, d):
        raise ValueError(f"k_new/v_new must be [{B}, {hkv}, {d}]")
    if out is None:
        out = torch.empty((B, hq, d), dtype=q.dtype, device=q.device)
    if workspace is None:
        workspace = new_decode_workspace(B, hq, hkv, d, max_seq_len_kv, q.device)
    args = (_ptr(out), _ptr(lse), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
            _ptr(k_scale), _ptr(v_scale), _ptr(block_table), _ptr(seq_lens_kv), _ptr(slots_out), B,
            block_table.shape[1], max_seq_len_kv, hq, hkv, d, bs, nb, float(softmax_scale),
            int(window), stages, _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream(q.device))
    return args, out, workspace


def paged_attn_decode_int8_append(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_table,
                                  seq_lens_kv, max_seq_len_kv, softmax_scale, out=None, lse=None,
                                  workspace=None, slots_out=None, window=0):
    """Quantize, write and attend to this step's token in one pass over the INT8 cache (see
    pkv_paged_attn_decode_int8_append).  Returns (out, lse)."""
    args, out, _ = _decode_int8_append_args(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale,
                                            block_table, seq_lens_kv, max_seq_len_kv,
                                            softmax_scale, 3, out, lse, workspace, slots_out, window)
    _check(lib().pkv_paged_attn_decode_int8_append(*args))
    return out, lse


def prepare_decode_int8_append(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_table,
                               seq_lens_kv, max_seq_len_kv, softmax_scale, out=None, lse=None,
                               workspace=None, slots_out=None, window=0):
    """(split pass with the folded write, combine pass) prepared calls."""
    calls = []
    for stages in (1, 2):
        args, out, workspace = _decode_int8_append_args(q, k_new, v_new, k_cache, v_cache, k_scale,
                                                        v_scale, block_table, seq_lens_kv,
                                                        max_seq_len_kv, softmax_scale, stages, out,
                                                        lse, workspace, slots_out, window)
        calls.append(PreparedCall(lib().pkv_paged_attn_decode_int8_append, args,
                                  (q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_table,
                                   seq_lens_kv, out, lse, workspace, slots_out)))
    return calls[0], calls[1], out


def _decode_mla_append_args(q, q_rope, nope_new, rope_new, cache_nope, cache_rope, block_table,
                            seq_lens_kv, max_seq_len_kv, softmax_scale, stages, out, lse, workspace,
                            slots_out):
    _dev(q, q_rope, nope_new, rope_new, cache_nope, cache_rope, block_table, seq_lens_kv, out, lse,
         workspace, slots_out)
    B, hq, dn = q.shape
    _batch_rows(B, block_table, seq_lens_kv, q_rope)
    nb, bs = cache_nope.shape[:2]
    if nope_new.numel() != B * 512 or rope_new.numel() != B * 64:
        raise ValueError(f"nope_new / rope_new must hold {B} rows of 512 / 64")
    if out is None:
        out = torch.empty((B, hq, dn), dtype=q.dtype, device=q.device)
    if workspace is None:
        workspace = new_decode_workspace(B, hq, 1, dn, max_seq_len_kv, q.device)
    args = (_ptr(out), _ptr(lse), _ptr(q), _ptr(q_rope), _ptr(nope_new), _ptr(rope_new),
            _ptr(cache_nope), _ptr(cache_rope), _ptr(block_table), _ptr(seq_lens_kv),
            _ptr(slots_out), B, block_table.shape[1], max_seq_len_kv, hq, bs, nb,
            float(softmax_scale), stages, _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(q.device))
    return args, out, workspace


def paged_attn_decode_mla_append(q, q_rope, nope_new, rope_new, cache_nope, cache_rope,
                                 block_table, seq_lens_kv, max_seq_len_kv, softmax_scale, out=None,
                                 lse=None, workspace=None, slots_out=None):
    """MLA decode step that also writes the step's latent rows (see
    pkv_paged_attn_decode_mla_append).  Returns (out, lse)."""
    args, out, _ = _decode_mla_append_args(q, q_rope, nope_new, rope_new, cache_nope, cache_rope,
                                           block_table, seq_lens_kv, max_seq_len_kv, softmax_scale,
                                           3, out, lse, workspace, slots_out)
    _check(lib().pkv_paged_attn_decode_mla_append(*args))
    return out, lse


def prepare_decode_mla_append(q, q_rope, nope_new, rope_new, cache_nope, cache_rope, block_table,
                              seq_lens_kv, max_seq_len_kv, softmax_scale, out=None, lse=None,
                              workspace=None, slots_out=None):
    """(split pass with the folded write, combine pass) prepared calls."""
    calls = []
    for stages in (1, 2):
        args, out, workspace = _decode_mla_append_args(q, q_rope, nope_new, rope_new, cache_nope,
                                                       cache_rope, block_table, seq_lens_kv,
                                                       max_seq_len_kv, softmax_scale, stages, out,
                                                       lse, workspace, slots_out)
        calls.append(PreparedCall(lib().pkv_paged_attn_decode_mla_append, args,
                                  (q, q_rope, nope_new, rope_new, cache_nope, cache_rope,
                                   block_table, seq_lens_kv, out, lse, workspace, slots_out)))
    return calls[0], calls[1], out


def prepare_kv_cache_write_int8(k_new, v_new, k_cache, v_cache, k_scale, v_scale, slots):
    _dev(k_new, v_new, k_cache, v_cache, k_scale, v_scale, slots)
    nb, bs, hkv, d = k_cache.shape
    args = (_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
            _ptr(slots), slots.shape[0], hkv, d, bs, nb, _dtype_code(k_new), _stream(k_new.device))
    return PreparedCall(lib().pkv_kv_cache_write_int8, args,
                        (k_new, v_new, k_cache, v_cache, k_scale, v_scale, slots))


def new_decode_workspace(batch: int, num_q_heads: int, num_kv_heads: int, head_dim_v: int,
                         max_seq_len_kv: int, device) -> torch.Tensor:
    """A zero-filled decode workspace of the required size (at least 16 bytes)."""
    need = decode_workspace_size(batch, num_q_heads, num_kv_heads, head_dim_v, max_seq_len_kv)
    return torch.zeros(max(need, 16), dtype=torch.uint8, device=device)


def decode_workspace_size(batch: int, num_q_heads: int, num_kv_heads: int, head_dim_v: int,
                          max_seq_len_kv: int) -> int:
    return int(lib().pkv_decode_workspace_size(batch, num_q_heads, num_kv_heads, head_dim_v,
                                               max_seq_len_kv))


def _decode_args(q, k_cache, v_cache, block_table, seq_lens_kv, max_seq_len_kv, softmax_scale,
                 q_rope, k_rope_cache, out, lse, workspace):
    _dev(q, k_cache, v_cache, block_table, seq_lens_kv, q_rope, k_rope_cache, out, lse, workspace)
    B, hq, dqk = q.shape
    _batch_rows(B, block_table, seq_lens_kv, q_rope)
    nb, bs, hkv, _ = k_cache.shape
    dv = v_cache.shape[-1]
    dr = q_rope.shape[-1] if q_rope is not None else 0
    if out is None:
        out = torch.empty((B, hq, dv), dtype=q.dtype, device=q.device)
    if workspace is None:
        workspace = new_decode_workspace(B, hq, hkv, dv, max_seq_len_kv, q.device)
    args = (_ptr(out), _ptr(lse), _ptr(q), _ptr(q_rope), _ptr(k_cache), _ptr(v_cache),
            _ptr(k_rope_cache), _ptr(block_table), _ptr(seq_lens_kv), B, block_table.shape[1],
            max_seq_len_kv, hq, hkv, dqk, dv, dr, bs, nb, float(softmax_scale), _dtype_code(q),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q.device))
    return args, out, workspace


def paged_attn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      block_table: torch.Tensor, seq_lens_kv: torch.Tensor,
                      max_seq_len_kv: int, softmax_scale: float,
                      q_rope: Optional[torch.Tensor] = None,
                      k_rope_cache: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, window: int = 0):
    """Decode attention (see pkv_paged_attn_decode; window > 0: the sliding-window form
    pkv_paged_attn_decode_ex, MHA/GQA only).  Returns (out, lse or None)."""
    if window:
        if q_rope is not None or k_rope_cache is not None:
            raise ValueError("a sliding window is supported for MHA/GQA decode only")
        args, out, _ = _decode_append_args(q, None, None, k_cache, v_cache, block_table,
                                           seq_lens_kv, max_seq_len_kv, softmax_scale, 3, out,
                                           lse, workspace, None, window)
        _check(lib().pkv_paged_attn_decode_ex(*args))
        return out, lse
    args, out, _ = _decode_args(q, k_cache, v_cache, block_table, seq_lens_kv, max_seq_len_kv,
                                softmax_scale, q_rope, k_rope_cache, out, lse, workspace)
    _check(lib().pkv_paged_attn_decode(*args))
    return out, lse


class PreparedCall:
    """A library call with its arguments marshalled once (pointers, sizes, stream), for
    loops that launch the same step many times.  The tensors must stay alive."""

    def __init__(self, fn, args, keep):
        self._fn = fn
        self._args = args
        self._keep = keep

    def __call__(self):
        _check(self._fn(*self._args))


def prepare_decode(q, k_cache, v_cache, block_table, seq_lens_kv, max_seq_len_kv, softmax_scale,
                   q_rope=None, k_rope_cache=None, out=None, lse=None, workspace=None):
    """(split, combine, whole) prepared calls of one decode configuration."""
    args, out, workspace = _decode_args(q, k_cache, v_cache, block_table, seq_lens_kv,
                                        max_seq_len_kv, softmax_scale, q_rope, k_rope_cache,
                                        out, lse, workspace)
    keep = (q, k_cache, v_cache, block_table, seq_lens_kv, q_rope, k_rope_cache, out, lse,
            workspace)
    L = lib()
    return (PreparedCall(L.pkv_paged_attn_decode_split, args, keep),
            PreparedCall(L.pkv_paged_attn_decode_combine, args, keep),
            PreparedCall(L.pkv_paged_attn_decode, args, keep), out)


def _decode_append_args(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens_kv,
                        max_seq_len_kv, softmax_scale, stages, out, lse, workspace, slots_out,
                        window=0):
    """Arguments of pkv_paged_attn_decode_ex (k_new/v_new None: plain decode)."""
    _dev(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens_kv, out, lse, workspace,
         slots_out)
    B, hq, d = q.shape
    _batch_rows(B, block_table, seq_lens_kv)
    nb, bs, hkv, _ = k_cache.shape
    if out is None:
        out = torch.empty((B, hq, d), dtype=q.dtype, device=q.device)
    if workspace is None:
        workspace = new_decode_workspace(B, hq, hkv, d, max_seq_len_kv, q.device)
    args = (_ptr(out), _ptr(lse), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
            _ptr(block_table), _ptr(seq_lens_kv), _ptr(slots_out), B, block_table.shape[1],
            max_seq_len_kv, hq, hkv, d, bs, nb, float(softmax_scale), _dtype_code(q), int(window),
            stages, _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream(q.device))
    return args, out, workspace


def paged_attn_decode_append(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens_kv,
                             max_seq_len_kv, softmax_scale, out=None, lse=None, workspace=None,
                             slots_out=None, window=0):
    """Write this step's token and attend, in one pass (pkv_paged_attn_decode_ex with the new
    rows; window > 0 keeps each sequence's `window` most recent keys)."""
    if k_new is None or v_new is None:
        raise ValueError("paged_attn_decode_append needs k_new and v_new")
    args, out, _ = _decode_append_args(q, k_new, v_new, k_cache, v_cache, block_table,
                                       seq_lens_kv, max_seq_len_kv, softmax_scale, 3, out, lse,
                                       workspace, slots_out, window)
    _check(lib().pkv_paged_attn_decode_ex(*args))
    return out, lse


def paged_attn_decode_append_noalloc(q, k_new, v_new, k_cache, v_cache, block_table,
                                     seq_lens_kv, max_seq_len_kv, softmax_scale, out, lse=None,
                                     slots_out=None):
    """pkv_paged_attn_decode_append_noalloc: the write-and-attend decode step with the partial
    states in the library's fixed per-GPU scratch (no workspace; `out` is the caller's)."""
    _dev(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens_kv, out, lse, slots_out)
    B, hq, d = q.shape
    _batch_rows(B, block_table, seq_lens_kv)
    nb, bs, hkv, _ = k_cache.shape
    _check(lib().pkv_paged_attn_decode_append_noalloc(
        _ptr(out), _ptr(lse), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
        _ptr(block_table), _ptr(seq_lens_kv), _ptr(slots_out), B, block_table.shape[1],
        max_seq_len_kv, hq, hkv, d, bs, nb, float(softmax_scale), _dtype_code(q),
        _stream(q.device)))
    return out, lse


def prepare_stream_read(src: torch.Tensor, sink: torch.Tensor, grid: int):
    """pkv_stream_read over all of `src` (a measurement aid: the HBM read ceiling)."""
    _dev(src, sink)
    args = (_ptr(src), src.numel() * src.element_size(), _ptr(sink), int(grid), _stream(src.device))
    return PreparedCall(lib().pkv_stream_read, args, (src, sink))


def prepare_gather_read(k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                        seq_lens: torch.Tensor, max_seq_len_kv: int, slice_bytes: int,
                        split_tokens: int, sink: torch.Tensor):
    """pkv_gather_read: the K/V rows a decode over these arguments reads, read with no
    arithmetic (a measurement aid: the read floor of the decode's access pattern).  Caches
    [nb, bs, ...] contiguous; a row is everything after the block-size dimension."""
    _dev(k_cache, v_cache, block_table, seq_lens, sink)
    nb, bs = k_cache.shape[:2]
    row_bytes = k_cache[0, 0].numel() * k_cache.element_size()
    args = (_ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
            block_table.shape[0], block_table.shape[1], int(max_seq_len_kv), bs, nb, row_bytes,
            int(slice_bytes), int(split_tokens), _ptr(sink), _stream(k_cache.device))
    return PreparedCall(lib().pkv_gather_read, args, (k_cache, v_cache, block_table, seq_lens, sink))


def prepare_decode_append(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens_kv,
                          max_seq_len_kv, softmax_scale, out=None, lse=None, workspace=None,
                          slots_out=None, window=0):
    """(split pass, combine pass) prepared calls of the write-and-attend decode
    (pkv_paged_attn_decode_ex with the new rows)."""
    calls = []
    for stages in (1, 2):
        args, out, workspace = _decode_append_args(q, k_new, v_new, k_cache, v_cache,
                                                   block_table, seq_lens_kv, max_seq_len_kv,
                                                   softmax_scale, stages, out, lse, workspace,
                                                   slots_out, window)
        calls.append(PreparedCall(lib().pkv_paged_attn_decode_ex, args,
                                  (q, k_new, v_new, k_cache, v_cache, block_table, seq_lens_kv,
                                   out, lse, workspace, slots_out)))
    return calls[0], calls[1], out


def prepare_slot_mapping(block_table, lens_before, cu_new, block_size, num_tokens, out):
    _dev(block_table, lens_before, cu_new, out)
    args = (_ptr(out), _ptr(block_table), _ptr(lens_before), _ptr(cu_new), lens_before.shape[0],
            num_tokens, block_table.shape[1], block_size, _stream(block_table.device))
    return PreparedCall(lib().pkv_slot_mapping, args, (block_table, lens_before, cu_new, out))


def prepare_kv_cache_write(k_new, v_new, k_cache, v_cache, slots):
    _dev(k_new, v_new, k_cache, v_cache, slots)
    nb, bs, hkv, dk = k_cache.shape
    dv = v_cache.shape[-1]
    args = (_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(slots), slots.shape[0],
            hkv, dk, dv, bs, nb, _dtype_code(k_cache), _stream(k_cache.device))
    return PreparedCall(lib().pkv_kv_cache_write, args, (k_new, v_new, k_cache, v_cache, slots))


def kv_cache_write_int8_mla(kv_nope, k_rope, nope_codes, rope_codes, nope_scale, rope_scale,
                            slot_mapping):
    """Quantize and write MLA latent rows into the INT8 latent cache
    (pkv_kv_cache_write_int8_mla): codes [nb, bs, 512] / [nb, bs, 64] int8, scales [nb, bs]."""
    _dev(kv_nope, k_rope, nope_codes, rope_codes, nope_scale, rope_scale, slot_mapping)
    nb, bs = nope_codes.shape[0], nope_codes.shape[1]
    _mla_int8_shapes(nope_codes, rope_codes, nope_scale, rope_scale)
    _check(lib().pkv_kv_cache_write_int8_mla(_ptr(kv_nope), _ptr(k_rope), _ptr(nope_codes),
                                             _ptr(rope_codes), _ptr(nope_scale), _ptr(rope_scale),
                                             _ptr(slot_mapping), slot_mapping.shape[0], bs, nb,
                                             _dtype_code(kv_nope), _stream(kv_nope.device)))


def _mla_int8_shapes(nope_codes, rope_codes, nope_scale, rope_scale):
    nb, bs = nope_codes.shape[0], nope_codes.shape[1]
    want = ((nope_codes, (nb, bs, 512), torch.int8), (rope_codes, (nb, bs, 64), torch.int8),
            (nope_scale, (nb, bs), torch.float32), (rope_scale, (nb, bs), torch.float32))
    for t, shape, dt in want:
        if tuple(t.shape) != shape or t.dtype != dt:
            raise ValueError(f"INT8 MLA cache arrays: expected {shape} {dt}, got {tuple(t.shape)} {t.dtype}")


def _decode_mla_int8_args(q, q_rope, nope_codes, rope_codes, nope_scale, rope_scale, block_table,
                          seq_lens_kv, max_seq_len_kv, softmax_scale, stages, out, lse, workspace):
    _dev(q, q_rope, nope_codes, rope_codes, nope_scale, rope_scale, block_table, seq_lens_kv, out,
         lse, workspace)
    _mla_int8_shapes(nope_codes, rope_codes, nope_scale, rope_scale)
    B, hq, _ = q.shape
    _batch_rows(B, block_table, seq_lens_kv)
    nb, bs = nope_codes.shape[0], nope_codes.shape[1]
    if out is None:
        out = torch.empty((B, hq, 512), dtype=q.dtype, device=q.device)
    if workspace is None:
        workspace = new_decode_workspace(B, hq, 1, 512, max_seq_len_kv, q.device)
    args = (_ptr(out), _ptr(lse), _ptr(q), _ptr(q_rope), _ptr(nope_codes), _ptr(rope_codes),
            _ptr(nope_scale), _ptr(rope_scale), _ptr(block_table), _ptr(seq_lens_kv), B,
            block_table.shape[1], max_seq_len_kv, hq, bs, nb, float(softmax_scale), stages,
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q.device))
    return args, out, workspace


def paged_attn_decode_mla_int8(q, q_rope, nope_codes, rope_codes, nope_scale, rope_scale,
                               block_table, seq_lens_kv, max_seq_len_kv, softmax_scale, out=None,
                               lse=None, workspace=None):
    """MLA-absorbed decode over the INT8 latent cache (pkv_paged_attn_decode_mla_int8)."""
    args, out, _ = _decode_mla_int8_args(q, q_rope, nope_codes, rope_codes, nope_scale, rope_scale,
                                         block_table, seq_lens_kv, max_seq_len_kv, softmax_scale,
                                         3, out, lse, workspace)
    _check(lib().pkv_paged_attn_decode_mla_int8(*args))
    return out, lse


def prepare_decode_mla_int8(q, q_rope, nope_codes, rope_codes, nope_scale, rope_scale, block_table,
                            seq_lens_kv, max_seq_len_kv, softmax_scale, out=None, lse=None,
                            workspace=None):
    """(split pass, combine pass) prepared calls of pkv_paged_attn_decode_mla_int8."""
    calls = []
    for stages in (1, 2):
        args, out, workspace = _decode_mla_int8_args(q, q_rope, nope_codes, rope_codes, nope_scale,
                                                     rope_scale, block_table, seq_lens_kv,
                                                     max_seq_len_kv, softmax_scale, stages, out,
                                                     lse, workspace)
        calls.append(PreparedCall(lib().pkv_paged_attn_decode_mla_int8, args,
                                  (q, q_rope, nope_codes, rope_codes, nope_scale, rope_scale,
                                   block_table, seq_lens_kv, out, lse, workspace)))
    return calls[0], calls[1], out


def _decode_mla_int8_append_args(q, q_rope, nope_new, rope_new, nope_codes, rope_codes, nope_scale,
                                 rope_scale, block_table, seq_lens_kv, max_seq_len_kv, softmax_scale,
                                 stages, out, lse, workspace, slots_out):
    _dev(q, q_rope, nope_new, rope_new, nope_codes, rope_codes, nope_scale, rope_scale, block_table,
         seq_lens_kv, out, lse, workspace, slots_out)
    _mla_int8_shapes(nope_codes, rope_codes, nope_scale, rope_scale)
    B, hq, _ = q.shape
    _batch_rows(B, block_table, seq_lens_kv)
    if nope_new.dtype != torch.bfloat16 or rope_new.dtype != torch.bfloat16:
        raise ValueError("the new latent rows must be bf16")
    if tuple(nope_new.shape[-1:]) != (512,) or tuple(rope_new.shape[-1:]) != (64,) or \
            nope_new.numel() != B * 512 or rope_new.numel() != B * 64:
        raise ValueError("nope_new must hold [B, 512] and rope_new [B, 64] values")
    nb, bs = nope_codes.shape[0], nope_codes.shape[1]
    if out is None:
        out = torch.empty((B, hq, 512), dtype=q.dtype, device=q.device)
    if workspace is None:
        workspace = new_decode_workspace(B, hq, 1, 512, max_seq_len_kv, q.device)
    args = (_ptr(out), _ptr(lse), _ptr(q), _ptr(q_rope), _ptr(nope_new), _ptr(rope_new),
            _ptr(nope_codes), _ptr(rope_codes), _ptr(nope_scale), _ptr(rope_scale),
            _ptr(block_table), _ptr(seq_lens_kv), _ptr(slots_out), B, block_table.shape[1],
            max_seq_len_kv, hq, bs, nb, float(softmax_scale), stages, _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(q.device))
    return args, out, workspace


def paged_attn_decode_mla_int8_append(q, q_rope, nope_new, rope_new, nope_codes, rope_codes,
                                      nope_scale, rope_scale, block_table, seq_lens_kv,
                                      max_seq_len_kv, softmax_scale, out=None, lse=None,
                                      workspace=None, slots_out=None):
    """MLA decode over the INT8 latent cache that also quantizes and writes the step's latent
    rows (pkv_paged_attn_decode_mla_int8_append).  Returns (out, lse)."""
    args, out, _ = _decode_mla_int8_append_args(q, q_rope, nope_new, rope_new, nope_codes,
                                                rope_codes, nope_scale, rope_scale, block_table,
                                                seq_lens_kv, max_seq_len_kv, softmax_scale, 3, out,
                                                lse, workspace, slots_out)
    _check(lib().pkv_paged_attn_decode_mla_int8_append(*args))
    return out, lse


def prepare_decode_mla_int8_append(q, q_rope, nope_new, rope_new, nope_codes, rope_codes,
                                   nope_scale, rope_scale, block_table, seq_lens_kv,
                                   max_seq_len_kv, softmax_scale, out=None, lse=None,
                                   workspace=None, slots_out=None):
    """(split pass with the folded quantizing write, combine pass) prepared calls."""
    calls = []
    for stages in (1, 2):
        args, out, workspace = _decode_mla_int8_append_args(
            q, q_rope, nope_new, rope_new, nope_codes, rope_codes, nope_scale, rope_scale,
            block_table, seq_lens_kv, max_seq_len_kv, softmax_scale, stages, out, lse, workspace,
            slots_out)
        calls.append(PreparedCall(lib().pkv_paged_attn_decode_mla_int8_append, args,
                                  (q, q_rope, nope_new, rope_new, nope_codes, rope_codes,
                                   nope_scale, rope_scale, block_table, seq_lens_kv, out, lse,
                                   workspace, slots_out)))
    return calls[0], calls[1], out


def prepare_kv_cache_write_int8_mla(kv_nope, k_rope, nope_codes, rope_codes, nope_scale, rope_scale,
                                    slots):
    _dev(kv_nope, k_rope, nope_codes, rope_codes, nope_scale, rope_scale, slots)
    _mla_int8_shapes(nope_codes, rope_codes, nope_scale, rope_scale)
    nb, bs = nope_codes.shape[0], nope_codes.shape[1]
    args = (_ptr(kv_nope), _ptr(k_rope), _ptr(nope_codes), _ptr(rope_codes), _ptr(nope_scale),
            _ptr(rope_scale), _ptr(slots), slots.shape[0], bs, nb, _dtype_code(kv_nope),
            _stream(kv_nope.device))
    return PreparedCall(lib().pkv_kv_cache_write_int8_mla, args,
                        (kv_nope, k_rope, nope_codes, rope_codes, nope_scale, rope_scale, slots))


def _decode_mtp_args(q, k_cache, v_cache, block_table, seq_lens_kv, num_q_tokens,
                     max_seq_len_kv, softmax_scale, stages, out, lse, workspace, window):
    """Arguments of pkv_paged_attn_decode_mtp."""
    _dev(q, k_cache, v_cache, block_table, seq_lens_kv, out, lse, workspace)
    rows, hq, d = q.shape
    B = seq_lens_kv.shape[0]
    _batch_rows(B, block_table, seq_lens_kv)
    if rows != B * num_q_tokens:
        raise ValueError(f"q has {rows} rows, expected batch * num_q_tokens = {B * num_q_tokens}")
    nb, bs, hkv, _ = k_cache.shape
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        need = int(lib().pkv_decode_mtp_workspace_size(B, num_q_tokens, hq, hkv, d, max_seq_len_kv))
        workspace = torch.zeros(max(need, 16), dtype=torch.uint8, device=q.device)
    args = (_ptr(out), _ptr(lse), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
            _ptr(seq_lens_kv), B, num_q_tokens, block_table.shape[1], max_seq_len_kv, hq, hkv, d,
            bs, nb, float(softmax_scale), _dtype_code(q), int(window), stages, _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(q.device))
    return args, out, workspace


def paged_attn_decode_mtp(q, k_cache, v_cache, block_table, seq_lens_kv, num_q_tokens,
                          max_seq_len_kv, softmax_scale, out=None, lse=None, workspace=None,
                          window=0):
    """Decode of num_q_tokens causal query tokens per sequence (pkv_paged_attn_decode_mtp);
    q [batch * num_q_tokens][Hq][D].  Returns (out, lse)."""
    args, out, _ = _decode_mtp_args(q, k_cache, v_cache, block_table, seq_lens_kv, num_q_tokens,
                                    max_seq_len_kv, softmax_scale, 3, out, lse, workspace, window)
    _check(lib().pkv_paged_attn_decode_mtp(*args))
    return out, lse


def prepare_decode_mtp(q, k_cache, v_cache, block_table, seq_lens_kv, num_q_tokens,
                       max_seq_len_kv, softmax_scale, out=None, lse=None, workspace=None, window=0):
    """(range pass, combine pass) prepared calls of pkv_paged_attn_decode_mtp."""
    calls = []
    for stages in (1, 2):
        args, out, workspace = _decode_mtp_args(q, k_cache, v_cache, block_table, seq_lens_kv,
                                                num_q_tokens, max_seq_len_kv, softmax_scale,
                                                stages, out, lse, workspace, window)
        calls.append(PreparedCall(lib().pkv_paged_attn_decode_mtp, args,
                                  (q, k_cache, v_cache, block_table, seq_lens_kv, out, lse,
                                   workspace)))
    return calls[0], calls[1], out


def _decode_mtp_append_args(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens_kv,
                            num_q_tokens, max_seq_len_kv, softmax_scale, stages, out, lse,
                            workspace, window, slots_out):
    """Arguments of pkv_paged_attn_decode_mtp_append."""
    args, out, workspace = _decode_mtp_args(q, k_cache, v_cache, block_table, seq_lens_kv,
                                            num_q_tokens, max_seq_len_kv, softmax_scale, stages,
                                            out, lse, workspace, window)
    _dev(k_new, v_new, slots_out)
    rows = q.shape[0]
    hkv, d = k_cache.shape[2], k_cache.shape[3]
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if tuple(t.shape) != (rows, hkv, d) or t.dtype != q.dtype:
            raise ValueError(f"{name} must be a {q.dtype} tensor of shape {(rows, hkv, d)}")
    if slots_out is not None and (tuple(slots_out.shape) != (rows,) or slots_out.dtype != torch.int64):
        raise ValueError(f"slots_out must be int64 of shape {(rows,)}")
    # (out, lse, q, k_cache, v_cache, table, lens, ...) -> (out, lse, q, k_new, v_new, k_cache, ...)
    args = args[:3] + (_ptr(k_new), _ptr(v_new)) + args[3:-1] + (_ptr(slots_out), args[-1])
    return args, out, workspace


def paged_attn_decode_mtp_append(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens_kv,
                                 num_q_tokens, max_seq_len_kv, softmax_scale, out=None, lse=None,
                                 workspace=None, window=0, slots_out=None):
    """MTP decode with the step's rows written in the pass (pkv_paged_attn_decode_mtp_append);
    k_new, v_new [batch * num_q_tokens][Hkv][D].  Returns (out, lse)."""
    args, out, _ = _decode_mtp_append_args(q, k_new, v_new, k_cache, v_cache, block_table,
                                           seq_lens_kv, num_q_tokens, max_seq_len_kv,
                                           softmax_scale, 3, out, lse, workspace, window, slots_out)
    _check(lib().pkv_paged_attn_decode_mtp_append(*args))
    return out, lse


def prepare_decode_mtp_append(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens_kv,
                              num_q_tokens, max_seq_len_kv, softmax_scale, out=None, lse=None,
                              workspace=None, window=0, slots_out=None):
    """(range pass with the writes, combine pass) prepared calls of
    pkv_paged_attn_decode_mtp_append."""
    calls = []
    for stages in (1, 2):
        args, out, workspace = _decode_mtp_append_args(q, k_new, v_new, k_cache, v_cache,
                                                       block_table, seq_lens_kv, num_q_tokens,
                                                       max_seq_len_kv, softmax_scale, stages, out,
                                                       lse, workspace, window, slots_out)
        calls.append(PreparedCall(lib().pkv_paged_attn_decode_mtp_append, args,
                                  (q, k_new, v_new, k_cache, v_cache, block_table, seq_lens_kv,
                                   out, lse, workspace, slots_out)))
    return calls[0], calls[1], out


def _varlen_args(q, k_cache, v_cache, block_table, cu_seqlens_q, seq_lens_kv, max_seqlen_q,
                 softmax_scale, causal, out, lse, window=0):
    """Arguments of pkv_paged_attn_varlen_ex."""
    _dev(q, k_cache, v_cache, block_table, cu_seqlens_q, seq_lens_kv, out, lse)
    T, hq, d = q.shape
    nb, bs, hkv, _ = k_cache.shape
    if out is None:
        out = torch.empty_like(q)
    args = (_ptr(out), _ptr(lse), _ptr(q), _ptr(cu_seqlens_q), _ptr(seq_lens_kv), _ptr(k_cache),
            _ptr(v_cache), _ptr(block_table), seq_lens_kv.shape[0], T, max_seqlen_q,
            block_table.shape[1], hq, hkv, d, bs, nb, float(softmax_scale), int(bool(causal)),
            int(window), _dtype_code(q), _stream(q.device))
    return args, out


def paged_attn_varlen(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      block_table: torch.Tensor, cu_seqlens_q: torch.Tensor,
                      seq_lens_kv: torch.Tensor, max_seqlen_q: int, softmax_scale: float,
                      causal: bool = True, out: Optional[torch.Tensor] = None,
                      lse: Optional[torch.Tensor] = None, window: int = 0):
    """Packed varlen attention over the paged cache (pkv_paged_attn_varlen_ex; window > 0
    keeps each row's `window` most recent visible keys)."""
    args, out = _varlen_args(q, k_cache, v_cache, block_table, cu_seqlens_q, seq_lens_kv,
                             max_seqlen_q, softmax_scale, causal, out, lse, window)
    _check(lib().pkv_paged_attn_varlen_ex(*args))
    return out, lse


def prepare_varlen(q, k_cache, v_cache, block_table, cu_seqlens_q, seq_lens_kv, max_seqlen_q,
                   softmax_scale, causal=True, out=None, lse=None, window=0):
    args, out = _varlen_args(q, k_cache, v_cache, block_table, cu_seqlens_q, seq_lens_kv,
                             max_seqlen_q, softmax_scale, causal, out, lse, window)
    return PreparedCall(lib().pkv_paged_attn_varlen_ex, args,
                        (q, k_cache, v_cache, block_table, cu_seqlens_q, seq_lens_kv, out, lse))


def _varlen_append_args(q, k_new, v_new, k_cache, v_cache, block_table, cu_seqlens_q,
                        seq_lens_kv, max_seqlen_q, softmax_scale, causal, out, lse, window,
                        slots_out):
    """Arguments of pkv_paged_attn_varlen_append."""
    _dev(q, k_new, v_new, k_cache, v_cache, block_table, cu_seqlens_q, seq_lens_kv, out, lse,
         slots_out)
    T, hq, d = q.shape
    nb, bs, hkv, _ = k_cache.shape
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if tuple(t.shape) != (T, hkv, d) or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {q.dtype} tensor of shape {(T, hkv, d)}")
    if slots_out is not None and (tuple(slots_out.shape) != (T,) or slots_out.dtype != torch.int64):
        raise ValueError(f"slots_out must be int64 of shape {(T,)}")
    if out is None:
        out = torch.empty_like(q)
    args = (_ptr(out), _ptr(lse), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(cu_seqlens_q),
            _ptr(seq_lens_kv), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
            seq_lens_kv.shape[0], T, max_seqlen_q, block_table.shape[1], hq, hkv, d, bs, nb,
            float(softmax_scale), int(bool(causal)), int(window), _dtype_code(q),
            _ptr(slots_out), _stream(q.device))
    return args, out


def paged_attn_varlen_append(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                             k_cache: torch.Tensor, v_cache: torch.Tensor,
                             block_table: torch.Tensor, cu_seqlens_q: torch.Tensor,
                             seq_lens_kv: torch.Tensor, max_seqlen_q: int, softmax_scale: float,
                             causal: bool = True, out: Optional[torch.Tensor] = None,
                             lse: Optional[torch.Tensor] = None, window: int = 0,
                             slots_out: Optional[torch.Tensor] = None):
    """The chunk's cache write folded into the varlen pass (pkv_paged_attn_varlen_append):
    new rows at positions seq_lens_kv[b] - n_b + i, then attention over every key."""
    args, out = _varlen_append_args(q, k_new, v_new, k_cache, v_cache, block_table,
                                    cu_seqlens_q, seq_lens_kv, max_seqlen_q, softmax_scale,
                                    causal, out, lse, window, slots_out)
    _check(lib().pkv_paged_attn_varlen_append(*args))
    return out, lse


def prepare_varlen_append(q, k_new, v_new, k_cache, v_cache, block_table, cu_seqlens_q,
                          seq_lens_kv, max_seqlen_q, softmax_scale, causal=True, out=None,
                          lse=None, window=0, slots_out=None):
    args, out = _varlen_append_args(q, k_new, v_new, k_cache, v_cache, block_table,
                                    cu_seqlens_q, seq_lens_kv, max_seqlen_q, softmax_scale,
                                    causal, out, lse, window, slots_out)
    return PreparedCall(lib().pkv_paged_attn_varlen_append, args,
                        (q, k_new, v_new, k_cache, v_cache, block_table, cu_seqlens_q,
                         seq_lens_kv, out, lse, slots_out))


# ---------------------------------------------------------------------- block management
class BlockManager:
    """Host block manager of one cache pool (pkv_bm_*): LIFO free list, per-block reference
    counts, copy on write of a shared partly filled last block.  Sequences are int ids."""

    def __init__(self, num_blocks: int, block_size: int, max_blocks_per_seq: int):
        self._h = lib().pkv_bm_create(num_blocks, block_size, max_blocks_per_seq)
        if not self._h:
            msg = lib().pkv_last_error()
            raise PagedKVError(-2, msg.decode() if msg else "")
        self.num_blocks, self.block_size = num_blocks, block_size
        self.max_blocks_per_seq = max_blocks_per_seq

    def close(self):
        if getattr(self, "_h", None):
            lib().pkv_bm_destroy(self._h)
            self._h = None

    __del__ = close

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    @property
    def num_free(self) -> int:
        return int(lib().pkv_bm_num_free(self._h))

    def add(self, seq: int):
        _check(lib().pkv_bm_add(self._h, seq))

    def fork(self, parent: int, child: int):
        _check(lib().pkv_bm_fork(self._h, parent, child))

    def append(self, seq: int, num_tokens: int = 1):
        """Extend seq; returns (slots int64 [num_tokens], copy) with copy = (src, dst) block
        of a copy on write, or None."""
        import numpy as np
        slots = np.empty(max(num_tokens, 0), dtype=np.int64)
        copy = np.empty(2, dtype=np.int64)
        n = ctypes.c_int32(0)
        _check(lib().pkv_bm_append(self._h, seq, num_tokens, slots.ctypes.data_as(ctypes.c_void_p),
                                   copy.ctypes.data_as(ctypes.c_void_p), ctypes.byref(n)))
        return slots, ((int(copy[0]), int(copy[1])) if n.value else None)

    def decode_step(self, seqs, table=None, seq_lens=None, slots=None, pad_block: int = 0):
        """One token for each row's sequence (negative id: padding row) and the step's table,
        lengths and slots (pkv_bm_decode_step).  Arrays may be the caller's (C-contiguous
        int32 table [n][max_blocks_per_seq] and seq_lens [n], int64 slots [n]).  Returns
        (table, seq_lens, slots, copies) with copies an int64 [k][2] array of
        copy-on-write (source, destination) blocks."""
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        n = ids.shape[0]
        if table is None:
            table = np.empty((n, self.max_blocks_per_seq), dtype=np.int32)
        if seq_lens is None:
            seq_lens = np.empty(n, dtype=np.int32)
        if slots is None:
            slots = np.empty(n, dtype=np.int64)
        for a, shape, dt in ((table, (n, self.max_blocks_per_seq), np.int32),
                             (seq_lens, (n,), np.int32), (slots, (n,), np.int64)):
            if a.dtype != dt or tuple(a.shape) != shape or not a.flags["C_CONTIGUOUS"]:
                raise ValueError(f"expected a C-contiguous {dt.__name__} array of shape {shape}")
        copies = np.empty((max(n, 1), 2), dtype=np.int64)
        k = ctypes.c_int32(0)
        vp = ctypes.c_void_p
        _check(lib().pkv_bm_decode_step(self._h, ids.ctypes.data_as(vp), n,
                                        slots.ctypes.data_as(vp), copies.ctypes.data_as(vp),
                                        ctypes.byref(k), table.ctypes.data_as(vp),
                                        seq_lens.ctypes.data_as(vp), pad_block))
        return table, seq_lens, slots, copies[:k.value]

    def free(self, seq: int):
        _check(lib().pkv_bm_free(self._h, seq))

    def length(self, seq: int) -> int:
        v = ctypes.c_int64(0)
        _check(lib().pkv_bm_length(self._h, seq, ctypes.byref(v)))
        return int(v.value)

    def ref_count(self, block: int) -> int:
        v = ctypes.c_int32(0)
        _check(lib().pkv_bm_ref_count(self._h, block, ctypes.byref(v)))
        return int(v.value)

    def table(self, seqs, pad_block: int = 0, table=None, seq_lens=None):
        """Fixed-width int32 block table [len(seqs)][max_blocks_per_seq] and int32 lengths
        (numpy arrays, or the caller's writable C-contiguous int32 arrays)."""
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        n = ids.shape[0]
        if table is None:
            table = np.empty((n, self.max_blocks_per_seq), dtype=np.int32)
        if seq_lens is None:
            seq_lens = np.empty(n, dtype=np.int32)
        for a, shape in ((table, (n, self.max_blocks_per_seq)), (seq_lens, (n,))):
            if a.dtype != np.int32 or tuple(a.shape) != shape or not a.flags["C_CONTIGUOUS"]:
                raise ValueError(f"expected a C-contiguous int32 array of shape {shape}")
        _check(lib().pkv_bm_table(self._h, ids.ctypes.data_as(ctypes.c_void_p), n,
                                  table.ctypes.data_as(ctypes.c_void_p),
                                  seq_lens.ctypes.data_as(ctypes.c_void_p), pad_block))
        return table, seq_lens


def kv_cache_copy_blocks(pool: torch.Tensor, pairs: torch.Tensor):
    """Copy whole blocks of pool [num_blocks][...] (pkv_kv_cache_copy_blocks); pairs is an
    int64 [n][2] device tensor of (source, destination) blocks."""
    _dev(pool, pairs)
    if pairs.dtype != torch.int64 or pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be an int64 [n][2] tensor")
    block_bytes = pool[0].numel() * pool.element_size()
    _check(lib().pkv_kv_cache_copy_blocks(_ptr(pool), block_bytes, pool.shape[0], _ptr(pairs),
                                          pairs.shape[0], _stream(pool.device)))


def upload(dst: torch.Tensor, src: torch.Tensor):
    """Host -> device copy on the current stream (pkv_upload); src pinned for capture."""
    _dev(dst)
    if src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous host tensor")
    nbytes = src.numel() * src.element_size()
    if nbytes > dst.numel() * dst.element_size():
        raise ValueError("dst is smaller than src")
    _check(lib().pkv_upload(_ptr(dst), _ptr(src), nbytes, _stream(dst.device)))


class CapturedStep:
    """Graph of the library calls made inside `with step.capture(): ...` on a created
    stream (pkv_graph_*); replay() launches it on that stream."""

    def __init__(self, device=None):
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None else device
        self.stream = torch.cuda.Stream(self.device)
        self._g = None

    def capture(self):
        import contextlib

        @contextlib.contextmanager
        def cm():
            if self._g is not None:
                raise RuntimeError("already captured")
            s = ctypes.c_void_p(self.stream.cuda_stream)
            self.stream.wait_stream(torch.cuda.current_stream(self.device))
            with torch.cuda.stream(self.stream):
                _check(lib().pkv_graph_begin(s))
                try:
                    yield self
                except BaseException:
                    g = ctypes.c_void_p()
                    lib().pkv_graph_end(s, ctypes.byref(g))
                    lib().pkv_graph_destroy(g)
                    raise
                g = ctypes.c_void_p()
                _check(lib().pkv_graph_end(s, ctypes.byref(g)))
                self._g = g
        return cm()

    def replay(self):
        """Launch on the step's stream after the current stream's prior work; the current
        stream then waits for it."""
        cur = torch.cuda.current_stream(self.device)
        self.stream.wait_stream(cur)
        _check(lib().pkv_graph_launch(self._g, ctypes.c_void_p(self.stream.cuda_stream)))
        cur.wait_stream(self.stream)

    def close(self):
        if getattr(self, "_g", None) is not None:
            lib().pkv_graph_destroy(self._g)
            self._g = None

    __del__ = close
