"""Python face of the fp64 CPU oracle (numpy in, numpy out).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's CPU-baseline
leg may import this module; the product path never does.  It shares no code with
the HIP library.  The hot-path arithmetic lives in pkv_oracle.c; this file marshals
arrays, computes the upstream RMSNorm + RoPE of the MLA latent row in numpy fp64
(rmsnorm_rope), and holds the two host-side formulas the pages print in Python form:

  * packing (hotelren.com source note "Paged KV Cache and Packed Sequence",
    section 3.1): seq_offset is the prefix sum of the lengths with a leading 0,
    position_ids restart at 0 inside every sequence;
  * the KV-size formula (ai6s.net article, section 3.1): total bytes =
    layers * tokens * 2 * heads * head_dim * bytes_per_element.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pkv_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
# The mutation test points this at a deliberately broken build of the oracle.
_LIB_OVERRIDE = os.environ.get("PKV_ORACLE_LIB_OVERRIDE")

F32, BF16, F64 = 0, 1, 2
ERRORS = {-1: "bad argument", -2: "block table cannot serve a position",
          -3: "slot out of range", -4: "duplicate slot", -5: "bad lengths", -6: "out of memory"}


class OracleError(RuntimeError):
    pass


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (C99, OpenMP, no fast-math)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(LIB):
                build(force=True)
            L = ctypes.CDLL(LIB)
        p, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.orc_max_threads.restype = ctypes.c_int
        L.orc_max_threads.argtypes = []
        L.orc_slot_of.restype = i64
        L.orc_slot_of.argtypes = [p, i32, i32, i64, i32, i64]
        L.orc_slot_mapping.argtypes = [p, i32, i32, p, p, i32, i64, p]
        L.orc_kv_write.argtypes = [p, i64, i64, p, p, i64]
        L.orc_kv_write_contiguous.argtypes = [p, i32, i64, i64, p, p, p]
        L.orc_paged_attention.argtypes = [p, p, i32, p, p, p, p, i32, i32, p, p, i32, i32,
                                          i32, i32, i32, i32, i64, f64, i32, i32, p, p, p,
                                          i32]
        L.orc_merge_states.argtypes = [p, p, p, i32, i64, i32, p, p]
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int):
    if rc != 0:
        raise OracleError(f"oracle error {rc}: {ERRORS.get(rc, 'unknown')}")


def _c(a, dtype=None):
    a = np.asarray(a) if dtype is None else np.asarray(a, dtype=dtype)
    return np.ascontiguousarray(a)


def _storage(a: np.ndarray) -> tuple[np.ndarray, int]:
    """Raw storage of a value array and its dtype code: float32, bf16 as uint16 bits, or
    float64 (values widened on the host, e.g. dequantized int8)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.float64:
        return a, F64
    if a.dtype in (np.uint16, np.int16):
        return a.view(np.uint16), BF16
    raise TypeError(f"oracle takes float32, float64 or bf16-as-uint16 arrays, got {a.dtype}")


def max_threads() -> int:
    """Threads the oracle's parallel loop uses."""
    return int(lib().orc_max_threads())


# --------------------------------------------------------------------------- index map
def slot_of(block_table, b: int, pos: int, block_size: int, num_blocks: int) -> int:
    t = _c(block_table, np.int32)
    return int(lib().orc_slot_of(_ptr(t), t.shape[1], b, pos, block_size, num_blocks))


def slot_mapping(block_table, lens_before, cu_new, block_size: int, num_blocks: int) -> np.ndarray:
    t = _c(block_table, np.int32)
    L = _c(lens_before, np.int32)
    cu = _c(cu_new, np.int32)
    out = np.zeros(int(cu[-1]) if len(cu) else 0, np.int64)
    _check(lib().orc_slot_mapping(_ptr(t), len(L), t.shape[1], _ptr(L), _ptr(cu), block_size,
                                  num_blocks, _ptr(out)))
    return out


# --------------------------------------------------------------------------- write
def kv_write(cache: np.ndarray, rows: np.ndarray, slots) -> np.ndarray:
    """Return a copy of `cache` ([nb, bs, ...]) with rows[t] written at slots[t]."""
    out = np.array(cache, copy=True, order="C")
    kv_write_into(out, rows, slots)
    return out


def kv_write_into(cache: np.ndarray, rows: np.ndarray, slots) -> None:
    """Write rows[t] at slots[t] of `cache` ([nb, bs, ...], C-contiguous) in place."""
    assert cache.flags["C_CONTIGUOUS"] and cache.flags["WRITEABLE"]
    rows = np.ascontiguousarray(rows)
    s = _c(slots, np.int64)
    num_slots = cache.shape[0] * cache.shape[1]
    row_bytes = cache.nbytes // num_slots if num_slots else 0
    assert rows.dtype == cache.dtype and rows.nbytes == len(s) * row_bytes
    if len(s):
        _check(lib().orc_kv_write(_ptr(cache), num_slots, row_bytes, _ptr(rows), _ptr(s), len(s)))


def kv_write_contiguous(cache: np.ndarray, newkv: np.ndarray, seqlen, token_offset) -> np.ndarray:
    """ATB-form write into a contiguous [batch, max_seq_len, ...] cache (returns a copy)."""
    out = np.array(cache, copy=True, order="C")
    newkv = np.ascontiguousarray(newkv)
    sl = _c(seqlen, np.int32)
    to = _c(token_offset, np.int32)
    row_bytes = out.nbytes // (out.shape[0] * out.shape[1])
    _check(lib().orc_kv_write_contiguous(_ptr(out), len(sl), out.shape[1], row_bytes,
                                         _ptr(newkv), _ptr(sl), _ptr(to)))
    return out


# --------------------------------------------------------------------------- attention
def paged_attention(q, k_cache, v_cache, block_table, cu_q, seq_lens_kv, scale: float,
                    causal: bool, q_rope=None, k_rope=None, want_touched: bool = False,
                    threads: int = 0, window: int = 0):
    """fp64 paged attention; returns (out [T,Hq,Dv] f64, lse [T,Hq] f64[, touched]).
    window > 0: each row sees only its `window` most recent visible positions (the band of
    sparse_mode 4 with pre_tokens = window - 1; "KVCache Optimization Skill", Appendix C)."""
    qs, dt = _storage(q)
    ks, dk = _storage(k_cache)
    vs, dv = _storage(v_cache)
    assert dt == dk == dv
    qr = kr = None
    Dr = 0
    if q_rope is not None or k_rope is not None:
        qr, d1 = _storage(q_rope)
        kr, d2 = _storage(k_rope)
        assert d1 == d2 == dt
        Dr = qr.shape[-1]
    T, Hq, Dqk = qs.shape
    nb, bs, Hkv, _ = ks.shape
    Dv = vs.shape[-1]
    t = _c(block_table, np.int32)
    cu = _c(cu_q, np.int32)
    sl = _c(seq_lens_kv, np.int32)
    out = np.zeros((T, Hq, Dv), np.float64)
    lse = np.zeros((T, Hq), np.float64)
    touched = np.zeros(nb * bs, np.uint8) if want_touched else None
    _check(lib().orc_paged_attention(_ptr(qs), _ptr(qr), dt, _ptr(ks), _ptr(vs), _ptr(kr),
                                     _ptr(t), len(sl), t.shape[1], _ptr(cu), _ptr(sl), Hq, Hkv,
                                     Dqk, Dv, Dr, bs, nb, float(scale), int(bool(causal)),
                                     int(window), _ptr(out), _ptr(lse), _ptr(touched),
                                     int(threads)))
    if want_touched:
        return out, lse, touched
    return out, lse


def merge_states(m, l, o):
    """Merge S partial states: m, l [S, rows], o [S, rows, D] -> (out [rows, D], lse [rows])."""
    m = _c(m, np.float64)
    l = _c(l, np.float64)
    o = _c(o, np.float64)
    S, rows, D = o.shape
    out = np.zeros((rows, D), np.float64)
    lse = np.zeros(rows, np.float64)
    _check(lib().orc_merge_states(_ptr(m), _ptr(l), _ptr(o), S, rows, D, _ptr(out), _ptr(lse)))
    return out, lse


# --------------------------------------------------------------------------- upstream of the write
def widen(a: np.ndarray) -> np.ndarray:
    """fp64 copy of fp32 values or of bf16 bit patterns (uint16 storage; exact)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def rmsnorm_rope(kv, gamma, cos, sin, head_dim_nope: int, eps: float):
    """The fused normalise-rotate step in front of the MLA cache write ("KVCache
    Optimization Skill", Mode 3 and its fused write npu_kv_rmsnorm_rope_cache, which the
    pages name without defining; the readings below are this build's).  For every token
    row kv[t] = [c (head_dim_nope) | k_pe (head_dim_rope)]:
      nope[t] = c / sqrt(mean(c^2) + eps) * gamma                         (RMSNorm)
      rope[t] = [x1 cos - x2 sin | x2 cos + x1 sin], x1 = k_pe[:Dr/2], x2 = k_pe[Dr/2:]
    (rotary embedding in the half-split form: pair (x1[i], x2[i]) turned by the angle whose
    cosine and sine are cos[t, i] and sin[t, i]).  fp64, unrounded; returns (nope, rope)."""
    x = widen(kv)
    g = widen(gamma)
    c = np.asarray(cos, np.float64)
    s_ = np.asarray(sin, np.float64)
    xn, xr = x[:, :head_dim_nope], x[:, head_dim_nope:]
    rms = np.sqrt((xn * xn).mean(axis=1) + float(eps))
    nope = xn / rms[:, None] * g[None, :]
    h = xr.shape[1] // 2
    x1, x2 = xr[:, :h], xr[:, h:]
    rope = np.concatenate([x1 * c - x2 * s_, x2 * c + x1 * s_], axis=1)
    return nope, rope


# --------------------------------------------------------------------------- int8 cache
def quantize_rows(x):
    """Symmetric int8 codes of each row (last axis) with one fp32 scale per row: the INT8
    KV cache with per-(token, kv head) scales.  The pages name the knobs (antiquant_scale,
    dequant_scale_key/value: "KVCache Optimization Skill", Layer 3 notes; ai6s.net article,
    low-precision and quantized caches) but not the scheme; the reading taken:
      s = max|x| / 127            (fp32 division)
      q = round_half_even(x / s)  (fp32 division), clamped to [-127, 127];  s = 0 -> q = 0
    The codes are integers decided in floating point, so this follows the fp32 operations
    of the GPU writer exactly (IEEE division, ties to even).  Returns (q int8, s float32)."""
    xf = widen(x).astype(np.float32)          # exact for fp32 and bf16 inputs
    amax = np.max(np.abs(xf), axis=-1)
    s = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    q = np.rint((xf / safe[..., None]).astype(np.float32))
    q = np.where((s > 0)[..., None], q, 0.0)
    return np.clip(q, -127, 127).astype(np.int8), s


def dequantize_rows(q, s):
    """q * s in fp64 (exact: a 7-bit code times a 24-bit mantissa)."""
    return np.asarray(q, np.float64) * np.asarray(s, np.float64)[..., None]


# --------------------------------------------------------------------------- host formulas
def pack(lengths):
    """(seq_offset [B+1] with leading 0, position_ids) for packed sequences."""
    offs = [0]
    pos = []
    for n in lengths:
        offs.append(offs[-1] + int(n))
        pos.extend(range(int(n)))
    return np.array(offs, np.int64), np.array(pos, np.int64)


def kv_cache_bytes(layers: int, tokens: int, heads: int, head_dim: int, elem_bytes: int) -> int:
    """layers x tokens x 2 (K and V) x heads x head_dim x bytes per element."""
    return layers * tokens * 2 * heads * head_dim * elem_bytes


# --------------------------------------------------------------------------- one step
def decode_step(case_np: dict, causal: bool, threads: int = 0, window: int = 0):
    """Whole step on host arrays: slot_mapping, cache writes, then attention.

    case_np holds numpy arrays: block_table, lens_before, cu_q, lens_after, cache_k,
    cache_v (may be the same object: MLA), cache_rope, q, q_rope, new_k, new_v,
    new_rope, block_size, num_blocks, scale.  Returns a dict with slots, the written
    caches, out and lse.
    """
    c = case_np
    slots = slot_mapping(c["block_table"], c["lens_before"], c["cu_q"], c["block_size"],
                         c["num_blocks"])
    mla = c.get("cache_rope") is not None
    k = kv_write(c["cache_k"], c["new_k"], slots)
    if mla:
        rope = kv_write(c["cache_rope"], c["new_rope"], slots)
        v = k
    else:
        rope = None
        v = kv_write(c["cache_v"], c["new_v"], slots)
    out, lse = paged_attention(c["q"], k, v, c["block_table"], c["cu_q"], c["lens_after"],
                               c["scale"], causal, q_rope=c.get("q_rope"), k_rope=rope,
                               threads=threads, window=window)
    return {"slots": slots, "cache_k": k, "cache_v": v, "cache_rope": rope, "out": out,
            "lse": lse}
