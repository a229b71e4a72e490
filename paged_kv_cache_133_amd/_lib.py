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

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedkv.so")

PKV_F32, PKV_BF16 = 0, 1
STATUS = {0: "PKV_OK", -1: "PKV_ERR_NULL", -2: "PKV_ERR_SHAPE", -3: "PKV_ERR_DTYPE",
          -4: "PKV_ERR_UNSUPPORTED", -5: "PKV_ERR_ALIGN", -6: "PKV_ERR_SCALE",
          -7: "PKV_ERR_WORKSPACE", -8: "PKV_ERR_HIP"}
EXPORTS = ("pkv_version", "pkv_last_error", "pkv_slot_mapping", "pkv_kv_cache_write",
           "pkv_kv_cache_append", "pkv_kv_cache_write_int8", "pkv_kv_rmsnorm_rope_cache",
           "pkv_decode_workspace_size", "pkv_paged_attn_decode_int8",
           "pkv_paged_attn_decode",
           "pkv_paged_attn_decode_split", "pkv_paged_attn_decode_combine",
           "pkv_paged_attn_decode_append", "pkv_paged_attn_decode_ex", "pkv_paged_attn_varlen",
           "pkv_paged_attn_varlen_ex")


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
    L.pkv_paged_attn_decode_ex.restype = ctypes.c_int
    L.pkv_paged_attn_decode_ex.argtypes = [p, p, p, p, p, p, p, p, p, p, i32, i32, i32, i32,
                                           i32, i32, i32, i64, f32, i32, i32, i32, p, sz, p]
    L.pkv_paged_attn_varlen.restype = ctypes.c_int
    L.pkv_paged_attn_varlen.argtypes = [p, p, p, p, p, p, p, p, i32, i64, i32, i32, i32, i32,
                                        i32, i32, i64, f32, i32, i32, p]
    L.pkv_paged_attn_varlen_ex.restype = ctypes.c_int
    L.pkv_paged_attn_varlen_ex.argtypes = [p, p, p, p, p, p, p, p, i32, i64, i32, i32, i32, i32,
                                           i32, i32, i64, f32, i32, i32, i32, p]
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
                          slot_mapping: torch.Tensor, eps: float = 1e-6):
    """RMSNorm + RoPE + write of the MLA latent row (see pkv_kv_rmsnorm_rope_cache).
    kv [T, Dn + Dr], gamma [Dn], cos/sin [T, Dr/2] fp32, caches [nb, bs, 1, Dn/Dr]."""
    _dev(kv, gamma, cos, sin, cache_nope, cache_rope, slot_mapping)
    nb, bs, _, dn = cache_nope.shape
    dr = cache_rope.shape[-1]
    _check(lib().pkv_kv_rmsnorm_rope_cache(_ptr(kv), _ptr(gamma), _ptr(cos), _ptr(sin),
                                           _ptr(cache_nope), _ptr(cache_rope), _ptr(slot_mapping),
                                           slot_mapping.shape[0], dn, dr, bs, nb, float(eps),
                                           _dtype_code(kv), _stream(kv.device)))


def kv_cache_write_int8(k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor,
                        v_cache: torch.Tensor, k_scale: torch.Tensor, v_scale: torch.Tensor,
                        slot_mapping: torch.Tensor):
    """Quantize and write one step's K/V rows into the INT8 cache (see
    pkv_kv_cache_write_int8).  Caches [nb, bs, Hkv, D] int8, scales [nb, bs, Hkv] fp32."""
    _dev(k_new, v_new, k_cache, v_cache, k_scale, v_scale, slot_mapping)
    nb, bs, hkv, d = k_cache.shape
    _check(lib().pkv_kv_cache_write_int8(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                         _ptr(k_scale), _ptr(v_scale), _ptr(slot_mapping),
                                         slot_mapping.shape[0], hkv, d, bs, nb, _dtype_code(k_new),
                                         _stream(k_new.device)))


def _decode_int8_args(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens_kv,
                      max_seq_len_kv, softmax_scale, stages, out, lse, workspace, window):
    _dev(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens_kv, out, lse, workspace)
    B, hq, d = q.shape
    nb, bs, hkv, _ = k_cache.shape
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
