"""Seeded synthetic inputs for paged-attention decode (shared by the tests, bench and smoke).

This module draws inputs only.  It holds none of the method's arithmetic: it never
computes a slot from a position, never gathers through a block table and never
computes attention.  It decides lengths, assigns physical blocks to logical blocks
(the job of a block manager), fills the pool and draws queries and new K/V rows.

Shapes follow the pages' problem statement ("KVCache Optimization Skill", section
"Layer 3: In-depth Principles", 3.1): a cache is [num_blocks, block_size,
num_kv_heads, head_dim]; the block table is int32 [batch, max_blocks_per_seq]; one
K cache and one V cache per layer (one layer here).  For the MLA-absorbed shape the
pages' "Mode 3: MLA compressed cache" gives cache_nope [.., 1, kv_lora_rank=512] and
cache_rope [.., 1, qk_rope_head_dim=64].

Recipe (all five workloads):
  * numpy Generator(PCG64(seed)) draws lengths and the physical-block permutation;
  * the pool holds ceil(1.1 * total blocks needed) blocks (the tiny case: exactly 32);
    the first sum(need) entries of permutation(num_blocks) are handed out sequence
    by sequence in logical order; need_b = ceil(L'_b / block_size);
  * a torch Generator on the target device draws, in this order, pool K, pool V
    [, pool rope], q [, q_rope], new K, new V — each fp32 N(0, 1), then cast
    (round-to-nearest-even) to the workload dtype;
  * poison: every pool row that does not hold a cached prefix token is NaN (spare
    blocks, rows past the prefix inside an assigned block, and the rows the step
    itself is about to write); table entries past need_b point at a NaN-filled spare
    block, so a kernel that reads them produces NaN instead of faulting.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    mode: str                 # "decode" (MHA/GQA), "mla" or "varlen"
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int             # query/key width (the nope part for MLA)
    head_dim_v: int           # value/output width
    head_dim_rope: int        # 0 unless MLA
    block_size: int
    dtype: str                # "f32" or "bf16"
    scale: float
    max_blocks_per_seq: int
    description: str = ""
    window: int = 0           # sliding window (keys each query row sees; 0: all)
    kv_dtype: str = ""        # "int8": the cache holds int8 codes + fp32 row scales
    q_tokens: int = 0         # > 0: every sequence has this many causal query tokens (MTP)

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


# The five configurations of the benchmark, in order.
TINY = Workload("tiny_gqa_f32", "decode", 2, 4, 1, 64, 64, 0, 16, "f32", 1.0 / 8.0, 9,
                "B=2, kv lengths {37,130} before the step, bs 16, pool of 32 blocks, "
                "GQA 4:1, head_dim 64, fp32")
LLAMA7B = Workload("llama7b_mha_bf16", "decode", 32, 32, 32, 128, 128, 0, 16, "bf16",
                   1.0 / math.sqrt(128.0), 129,
                   "Llama-7B-shaped MHA decode layer: B=32, 32 heads, head_dim 128, "
                   "bs 16, kv lengths U{512..2048}, bf16")
GQA_LONG = Workload("gqa_long_bf16", "decode", 64, 64, 8, 128, 128, 0, 128, "bf16",
                    1.0 / math.sqrt(128.0), 257,
                    "GQA long-context decode: B=64, 64 q / 8 kv heads, head_dim 128, "
                    "bs 128, kv lengths log-uniform [1024, 32768], bf16")
MLA = Workload("mla_absorbed_bf16", "mla", 64, 128, 1, 512, 512, 64, 128, "bf16",
               1.0 / math.sqrt(576.0), 65,
               "MLA-absorbed decode: B=64, 128 q heads on 1 latent head, nope 512 + "
               "rope 64, bs 128, kv lengths U{2048..8192}, bf16")
VARLEN = Workload("varlen_causal_bf16", "varlen", 16, 32, 8, 128, 128, 0, 128, "bf16",
                  1.0 / math.sqrt(128.0), 56,
                  "packed varlen causal chunk: 16 sequences, new lengths lognormal "
                  "(median 300, sigma 1, clipped [50,3000]), prefix U{0..4096}, "
                  "32 q / 8 kv heads, head_dim 128, bs 128, bf16")

# Two more for the band and MTP rows (beyond the five above): a Mistral-7B-shaped
# sliding-window decode (window 4096 on long contexts) and an MTP decode step with
# next_n = 1 (two causal query tokens per sequence through the varlen path).
SWA_DECODE = Workload("swa_decode_bf16", "decode", 32, 32, 8, 128, 128, 0, 16, "bf16",
                      1.0 / math.sqrt(128.0), 2049,
                      "sliding-window GQA decode: B=32, 32 q / 8 kv heads, head_dim 128, bs 16, "
                      "kv lengths log-uniform [1024, 32768], window 4096, bf16", window=4096)
MTP_DECODE = Workload("mtp_decode_bf16", "varlen", 32, 32, 8, 128, 128, 0, 16, "bf16",
                      1.0 / math.sqrt(128.0), 129,
                      "MTP decode (next_n = 1): B=32, 2 causal query tokens per sequence, "
                      "32 q / 8 kv heads, head_dim 128, bs 16, kv lengths U{512..2048} before "
                      "the step, bf16", q_tokens=2)

# The headline shape over an INT8 cache (the same lengths as the bf16 headline).
LLAMA7B_INT8 = Workload("llama7b_mha_int8", "decode", 32, 32, 32, 128, 128, 0, 16, "bf16",
                        1.0 / math.sqrt(128.0), 129,
                        "Llama-7B-shaped MHA decode layer over an INT8 KV cache (codes + fp32 "
                        "scale per token and head): B=32, 32 heads, head_dim 128, bs 16, kv "
                        "lengths U{512..2048}, bf16 queries", kv_dtype="int8")

# The long-context GQA shape over an INT8 cache (the same lengths as the bf16 one).
GQA_LONG_INT8 = Workload("gqa_long_int8", "decode", 64, 64, 8, 128, 128, 0, 128, "bf16",
                         1.0 / math.sqrt(128.0), 257,
                         "GQA long-context decode over an INT8 KV cache (codes + fp32 scale per "
                         "token and head): B=64, 64 q / 8 kv heads, head_dim 128, bs 128, kv "
                         "lengths log-uniform [1024, 32768], bf16 queries", kv_dtype="int8")

# The MLA shape over an INT8 latent cache (the same lengths as the bf16 MLA workload).
MLA_INT8 = Workload("mla_absorbed_int8", "mla", 64, 128, 1, 512, 512, 64, 128, "bf16",
                    1.0 / math.sqrt(576.0), 65,
                    "MLA-absorbed decode over an INT8 latent cache (nope and rope codes, one fp32 "
                    "scale each per token): B=64, 128 q heads, bs 128, lengths U{2048..8192}, bf16 "
                    "queries", kv_dtype="int8")

WORKLOADS = {w.name: w for w in (TINY, LLAMA7B, GQA_LONG, MLA, VARLEN, SWA_DECODE, MTP_DECODE,
                                 LLAMA7B_INT8, GQA_LONG_INT8, MLA_INT8)}


def sample_lengths(w: Workload, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """Lengths before the step (L_b) and new tokens per sequence (n_b) for a workload."""
    rng = np.random.Generator(np.random.PCG64(seed))
    B = w.batch
    if w is TINY or w.name == TINY.name:
        return np.array([37, 130], np.int64), np.ones(2, np.int64)
    if w.name in (LLAMA7B.name, "llama7b_mha_int8"):
        return rng.integers(512, 2048, size=B, endpoint=True), np.ones(B, np.int64)
    if w.name in (GQA_LONG.name, "gqa_long_int8"):
        u = rng.uniform(math.log(1024.0), math.log(32768.0), size=B)
        return np.clip(np.round(np.exp(u)), 1024, 32768).astype(np.int64), np.ones(B, np.int64)
    if w.name in (MLA.name, "mla_absorbed_int8"):
        return rng.integers(2048, 8192, size=B, endpoint=True), np.ones(B, np.int64)
    if w.name == SWA_DECODE.name:
        u = rng.uniform(math.log(1024.0), math.log(32768.0), size=B)
        return np.clip(np.round(np.exp(u)), 1024, 32768).astype(np.int64), np.ones(B, np.int64)
    if w.name == MTP_DECODE.name:
        return rng.integers(512, 2048, size=B, endpoint=True), np.full(B, 2, np.int64)
    if w.name == VARLEN.name:
        n = np.clip(np.round(rng.lognormal(math.log(300.0), 1.0, size=B)), 50, 3000)
        L = rng.integers(0, 4096, size=B, endpoint=True)
        return L.astype(np.int64), n.astype(np.int64)
    raise ValueError(f"no length recipe for workload {w.name}")


@dataclass
class Case:
    """One synthetic step: host metadata (numpy) plus device/host tensors (torch)."""
    w: Workload
    seed: int
    lens_before: np.ndarray       # int32 [B]  L_b
    n_new: np.ndarray             # int32 [B]  n_b
    lens_after: np.ndarray        # int32 [B]  L'_b = L_b + n_b
    cu_q: np.ndarray              # int32 [B+1], leading 0
    num_blocks: int
    block_table: np.ndarray       # int32 [B, MBS]
    poison_block: int
    need: np.ndarray              # int64 [B] blocks assigned per sequence
    cache_k: torch.Tensor         # [nb, bs, Hkv, Dk]   (cache_nope for MLA)
    cache_v: torch.Tensor         # [nb, bs, Hkv, Dv]   (is cache_k for MLA)
    cache_rope: Optional[torch.Tensor]  # [nb, bs, 1, Dr] or None
    q: torch.Tensor               # [T, Hq, Dk]
    q_rope: Optional[torch.Tensor]      # [T, Hq, Dr] or None
    new_k: torch.Tensor           # [T, Hkv, Dk]
    new_v: Optional[torch.Tensor] # [T, Hkv, Dv] (None for MLA)
    new_rope: Optional[torch.Tensor]    # [T, 1, Dr] (MLA only)
    extra: dict = field(default_factory=dict)

    @property
    def num_tokens(self) -> int:
        return int(self.cu_q[-1])

    @property
    def max_len_after(self) -> int:
        return int(self.lens_after.max()) if len(self.lens_after) else 0

    @property
    def max_new(self) -> int:
        return int(self.n_new.max()) if len(self.n_new) else 0

    def table_tensor(self, device) -> torch.Tensor:
        return torch.from_numpy(self.block_table).to(device)

    def lens_after_tensor(self, device) -> torch.Tensor:
        return torch.from_numpy(self.lens_after).to(device)

    def lens_before_tensor(self, device) -> torch.Tensor:
        return torch.from_numpy(self.lens_before).to(device)

    def cu_q_tensor(self, device) -> torch.Tensor:
        return torch.from_numpy(self.cu_q).to(device)


def _randn(shape, gen, device, dtype):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(dtype)


def make_case(w: Workload, lens_before, n_new, seed: int = 0, device="cpu",
              num_blocks: Optional[int] = None, max_blocks_per_seq: Optional[int] = None,
              poison: bool = True, perm_seed: Optional[int] = None) -> Case:
    """Build one step's inputs for explicit lengths.

    lens_before: L_b per sequence (tokens already cached); n_new: tokens written this
    step.  Physical blocks come from a seeded permutation of the pool.
    """
    L = np.asarray(lens_before, np.int64)
    n = np.asarray(n_new, np.int64)
    B = len(L)
    assert len(n) == B and (L >= 0).all() and (n >= 0).all()
    bs = w.block_size
    Lp = L + n
    need = -(-Lp // bs)                       # blocks a block manager hands out
    total = int(need.sum())
    if num_blocks is None:
        num_blocks = max(int(math.ceil(1.1 * total)), total + 1)
    assert num_blocks > total, "pool needs at least one spare (poison) block"
    mbs = int(max_blocks_per_seq if max_blocks_per_seq is not None else max(1, need.max(initial=1)))
    assert (need <= mbs).all()
    rng = np.random.Generator(np.random.PCG64(seed if perm_seed is None else perm_seed))
    perm = rng.permutation(num_blocks)
    poison_block = int(perm[total])
    table = np.full((B, mbs), poison_block, np.int32)
    # prefix rows held by each physical block (0 for spares and fully-new blocks)
    held = np.zeros(num_blocks, np.int64)
    k = 0
    for b in range(B):
        for j in range(int(need[b])):
            P = int(perm[k]); k += 1
            table[b, j] = P
            held[P] = min(bs, max(0, int(L[b]) - j * bs))
    cu = np.zeros(B + 1, np.int32)
    cu[1:] = np.cumsum(n)
    T = int(cu[-1])

    dt = w.torch_dtype
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    Hkv, Hq = w.num_kv_heads, w.num_q_heads
    if w.mode == "mla":
        cache_k = _randn((num_blocks, bs, 1, w.head_dim), gen, device, dt)
        cache_rope = _randn((num_blocks, bs, 1, w.head_dim_rope), gen, device, dt)
        cache_v = cache_k
        q = _randn((T, Hq, w.head_dim), gen, device, dt)
        q_rope = _randn((T, Hq, w.head_dim_rope), gen, device, dt)
        new_k = _randn((T, 1, w.head_dim), gen, device, dt)
        new_rope = _randn((T, 1, w.head_dim_rope), gen, device, dt)
        new_v = None
    else:
        cache_k = _randn((num_blocks, bs, Hkv, w.head_dim), gen, device, dt)
        cache_v = _randn((num_blocks, bs, Hkv, w.head_dim_v), gen, device, dt)
        cache_rope = None
        q = _randn((T, Hq, w.head_dim), gen, device, dt)
        q_rope = None
        new_k = _randn((T, Hkv, w.head_dim), gen, device, dt)
        new_v = _randn((T, Hkv, w.head_dim_v), gen, device, dt)
        new_rope = None
    if poison:
        rows = torch.arange(bs, device=device)[None, :]
        bad = rows >= torch.from_numpy(held).to(device)[:, None]      # [nb, bs]
        for c in (cache_k, cache_v, cache_rope):
            if c is not None:
                c[bad] = float("nan")
    return Case(w, seed, L.astype(np.int32), n.astype(np.int32), Lp.astype(np.int32), cu,
                num_blocks, table, poison_block, need, cache_k, cache_v, cache_rope,
                q, q_rope, new_k, new_v, new_rope)


def make_workload_case(w: Workload, seed: int = 0, device="cpu", poison: bool = True) -> Case:
    """The full-size case of one of the five benchmark workloads."""
    L, n = sample_lengths(w, seed)
    nb = 32 if w.name == TINY.name else None
    return make_case(w, L, n, seed=seed, device=device, num_blocks=nb,
                     max_blocks_per_seq=w.max_blocks_per_seq, poison=poison)


def custom(mode="decode", batch=2, num_q_heads=4, num_kv_heads=1, head_dim=64,
           head_dim_v=None, head_dim_rope=0, block_size=16, dtype="f32",
           scale=None, name="custom") -> Workload:
    """A small workload of arbitrary shape for parity and pin tests."""
    hv = head_dim if head_dim_v is None else head_dim_v
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim + head_dim_rope)
    return Workload(name, mode, batch, num_q_heads, num_kv_heads, head_dim, hv,
                    head_dim_rope, block_size, dtype, scale, 0)
