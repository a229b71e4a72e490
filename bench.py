#!/usr/bin/env python3
"""Paged-attention decode benchmark on one MI355X.

One step = one decode layer of the Llama-7B-shaped workload (B = 32 sequences, 32 query
heads = 32 kv heads, head_dim 128, block_size 16, bf16, kv lengths U{512..2048} before
the step, physical blocks shuffled in a pool of total need + 10 %):
    slot_mapping + cache write of the new K/V rows + split-KV attention (one launch,
    pkv_paged_attn_decode_append), then the split combine (second launch),
all through the C ABI of libpagedkv.so on torch's current stream, with every input
already resident in HBM.  --path append / separate time the same step as three / four
launches (kv_cache_append or slot_mapping + kv_cache_write, split, combine).  Several copies of the K/V pool are rotated so that each step
reads a pool that left the 256 MB Infinity Cache long ago.

Before the W warm-up steps, whole steps run untimed for at least --settle-ms (200 ms) of
wall time, until the GPU clock has settled; then exactly K steps are timed, HIP events
only at the two ends of the timed region.

Prints one JSON line: KV-read GB/s (value), µs per step, the roofline of the dominant
kernel (the split-KV attention pass: K launches of it alone, back to back on the stream
it runs on, HIP events at the two ends, after the timed steps) and the fp64 CPU oracle
timed on this host as a baseline.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--seed S]
  python bench.py --calibrate-copy MIB     # plain copy of known size, for counter scaling
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged-decode KV-read HBM GB/s (% of peak) + µs/step, Llama-7B-shape B=32, 1 GPU"
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E, vendor figure
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, vendor figure
CSRC = "paged_kv_cache_133_amd/csrc/"
MFMA_SOURCES = [CSRC + "mfma_common.h", CSRC + "pkv_device.h"]


def dominant_kernel(w, path="fused"):
    """The attention kernel a workload's step runs (the library's dispatch rule) and the
    sources its traffic counters depend on."""
    if w.mode == "mla":
        return "mla_wide_kernel", [CSRC + "mla_wide.hip"] + MFMA_SOURCES
    if w.q_tokens:      # multi-token decode: the range-streaming kernel
        return "gqa_stream_kernel", [CSRC + "gqa_attn.hip"] + MFMA_SOURCES
    if w.mode == "varlen":
        name = "varlen_append_kernel<128>" if path == "fused" else "varlen_kernel<128>"
        return name, [CSRC + "varlen_attn.hip"] + MFMA_SOURCES
    group = w.num_q_heads // w.num_kv_heads
    if w.kv_dtype == "int8":
        if group > 4:   # the range-streaming kernel over the codes
            return "gqa_stream_kernel", [CSRC + "gqa_attn.hip"] + MFMA_SOURCES
        return "decode_int8_kernel", [CSRC + "int8_kv.hip", CSRC + "pkv_device.h"]
    if w.dtype == "bf16" and 4 <= group <= 16:
        rows_per_wave_load = 1024 // (2 * w.head_dim)
        name = ("gqa_stream_kernel" if w.block_size >= rows_per_wave_load and w.batch <= 1024
                else "gqa_decode_kernel")
        return name, [CSRC + "gqa_attn.hip"] + MFMA_SOURCES
    return "decode_split_kernel", [CSRC + "decode.hip", CSRC + "pkv_device.h"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed whole steps for at least this long before the warm-up steps")
    ap.add_argument("--workload", default="llama7b_mha_bf16")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--replicas", type=int, default=0, help="K/V pool copies rotated (0: auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=5.0,
                    help="minimum wall time of the CPU-oracle sample")
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="skip the second timed region (the dominant kernel alone) and the roofline")
    ap.add_argument("--path", choices=("fused", "append", "separate"), default="fused",
                    help="fused: decode_append (write folded into the split pass), combine; "
                         "append: kv_cache_append (slot_mapping + write), split, combine; "
                         "separate: slot_mapping, write, split, combine")
    ap.add_argument("--serving", action="store_true",
                    help="serving loop instead: host block manager, recorded decode step "
                         "replayed with double-buffered table uploads, per block size")
    ap.add_argument("--block-sizes", default="16,32,64,128",
                    help="block sizes of the --serving sweep")
    ap.add_argument("--table-capacity", type=float, default=1.0,
                    help="--serving: max_blocks_per_seq as this multiple of what the longest "
                         "sequence reaches during the run (the recorded step's length bound)")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="only measure the practical HBM read ceiling (pkv_stream_read over "
                         "0.7-4 GB at several grid sizes), a device copy, and the read floor "
                         "of the headline decode's access pattern (pkv_gather_read)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (for counter scaling)")
    return ap.parse_args()


def kernel_source_hash(sources) -> str:
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str, kernel: str, sources):
    """(HBM bytes per launch of the dominant kernel, where the figure comes from): the
    committed rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE runs, scaled by a copy
    of known size), or (None, reason) if it is missing or was taken on other kernel sources.
    The counters are not read in this run."""
    rel = os.path.join("profiles", f"traffic_{kernel.split('<')[0]}_{workload}.txt")
    path = os.path.join(ROOT, rel)
    if not os.path.exists(path):
        return None, f"no counter summary {rel}"
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash(sources):
        return None, f"{rel} was taken on other kernel sources"
    try:
        return float(vals["hbm_bytes_per_launch"]), f"committed counter summary {rel}"
    except (KeyError, ValueError):
        return None, f"{rel} holds no hbm_bytes_per_launch"


def visible_keys(case):
    """Per sequence: (keys some query row sees, visible (query row, key) pairs), with
    bottom-right causal rows for varlen and the workload's sliding window."""
    import numpy as np
    w = case.w
    L = case.lens_before.astype("int64")
    n = case.n_new.astype("int64")
    Lp = L + n
    if w.mode == "varlen":
        # row i sees keys [0, L + i]: i + L + 1 of them, at most `window`
        rows = [np.arange(int(k)) + int(b) + 1 for b, k in zip(L, n)]
        if w.window:
            rows = [np.minimum(r, w.window) for r in rows]
        pairs = np.array([int(r.sum()) for r in rows], np.int64)
        first = np.maximum(0, L + 1 - w.window) if w.window else np.zeros_like(L)
        keys = Lp - first
    else:
        keys = np.minimum(Lp, w.window) if w.window else Lp
        pairs = keys.copy()
    return keys, pairs


def algorithmic_flops(case):
    """Flops of the attention kernel: 2 (Dqk + Dv) per visible (query row, key) pair."""
    w = case.w
    pairs = int(visible_keys(case)[1].sum())
    return pairs * w.num_q_heads * 2 * (w.head_dim + w.head_dim_rope + w.head_dim_v)


def algorithmic_bytes(case, path="fused"):
    """(kv_read, split_kernel, step) algorithmic bytes of one step."""
    w = case.w
    e = w.elem_bytes
    Lp = visible_keys(case)[0]                     # keys some row of the sequence sees
    B, T = w.batch, case.num_tokens
    if w.mode == "mla" and w.kv_dtype == "int8":
        row = w.head_dim + w.head_dim_rope + 8      # nope and rope codes + their two scales
        kv = int(Lp.sum()) * row
        # the quantizing writer reads the new rows in the query dtype, writes codes and scales
        new_rows = (T * (w.head_dim + w.head_dim_rope) * e + T * row) // 2
    elif w.mode == "mla":
        row = w.head_dim + w.head_dim_rope          # nope read once (key and value) + rope
        new_rows = T * (w.head_dim + w.head_dim_rope) * e
        kv = int(Lp.sum()) * row * e
    elif w.kv_dtype == "int8":
        # one-byte codes of K and V plus one fp32 scale each per (token, kv head)
        row = w.num_kv_heads * (w.head_dim + w.head_dim_v + 8)
        kv = int(Lp.sum()) * row
        # the quantizing write reads the new rows in the query dtype, writes codes and scales
        new_rows = (T * w.num_kv_heads * (w.head_dim + w.head_dim_v) * e + T * row) // 2
    else:
        row = w.num_kv_heads * (w.head_dim + w.head_dim_v)
        new_rows = T * w.num_kv_heads * (w.head_dim + w.head_dim_v) * e
        kv = int(Lp.sum()) * row * e
    q_bytes = T * w.num_q_heads * (w.head_dim + w.head_dim_rope) * e
    out_bytes = T * w.num_q_heads * w.head_dim_v * e
    table = 4 * int((-(-Lp // w.block_size)).sum())
    split = kv + q_bytes + out_bytes + table + 4 * B
    if w.mode == "varlen" and path == "fused":
        # the fused pass also stores the chunk's new rows (its reads of them replace cache
        # reads already counted in kv); the decode passes' one row per sequence is left out
        split += new_rows
    # slot_mapping: table entry, L_b, cu; slot written; write: new rows read + written
    step = split + 2 * new_rows + 4 * B * 3 + 8 * T
    return kv, split, step


def calibrate_copy(mib: int):
    import torch
    n = mib * (1 << 20)
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "launches": 5}), flush=True)


def settle_clock(ms: float, buf=None):
    """Untimed HBM reads (pkv_stream_read over 1 GiB, or `buf`) for at least `ms` of wall
    time: from idle the GPU's clock takes tens of milliseconds to settle under load."""
    import torch
    from paged_kv_cache_133_amd import _lib
    if ms <= 0:
        return
    dev = torch.device("cuda:0")
    if buf is None:
        buf = torch.zeros(1 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    call = _lib.prepare_stream_read(buf, sink, 2048)
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            call()
        torch.cuda.synchronize()


def read_ceiling(launches: int = 20, settle_ms: float = 200.0):
    """--read-ceiling: pkv_stream_read (16-byte non-temporal loads, grid-stride) over 0.7,
    1.5 and 4 GB at 1K-16K workgroups, rotating over a 4 GiB buffer so that no launch finds
    its bytes in the 256 MB Infinity Cache, and a torch device copy of 1 GiB; events at the
    two ends of each run of launches.  Prints one JSON line."""
    import torch
    from paged_kv_cache_133_amd import _lib
    _lib.lib()
    dev = torch.device("cuda:0")
    total = 4 << 30
    buf = torch.zeros(total, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    settle_clock(settle_ms, buf)
    rows = []
    for size in (700_000_000, 1_500_000_000, total):
        size -= size % 4096
        nrot = max(1, total // size)
        for grid in (1024, 2048, 4096, 8192, 16384):
            calls = [_lib.prepare_stream_read(buf[r * size:(r + 1) * size], sink, grid)
                     for r in range(nrot)]
            for i in range(3):
                calls[i % nrot]()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            for i in range(launches):
                calls[i % nrot]()
            b.record()
            torch.cuda.synchronize()
            us = a.elapsed_time(b) * 1e3 / launches
            rows.append({"bytes": size, "grid": grid, "us_per_launch": round(us, 2),
                         "GB_per_s": round(size / (us * 1e-6) / 1e9, 1)})
    del buf
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(launches):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / launches
    del src, dst
    best = max(rows, key=lambda r: r["GB_per_s"])
    print(json.dumps({"read_ceiling_GB_per_s": best["GB_per_s"], "best": best,
                      "frac_of_8TBps": round(best["GB_per_s"] / PEAK_HBM_GBPS, 4),
                      "copy_1GiB": {"us_per_copy": round(us, 2),
                                    "GB_per_s_read_plus_write": round(2 * n / (us * 1e-6) / 1e9, 1)},
                      "gather": gather_floor(launches=launches),
                      "runs": rows}), flush=True)


def gather_floor(launches: int = 20, replicas: int = 3):
    """The read floor of the headline decode's own access pattern: pkv_gather_read over the
    llama7b_mha_bf16 case (seed 0; the same table, lengths after the step and pools, rotated
    over `replicas` copies) reads exactly the K/V rows the decode reads, with no arithmetic.
    Slices of 512 B (the rows of the pair of heads one decode workgroup reads) and splits of
    256 rows are the decode's own pattern; other slices and splits show how much of the floor
    is the pattern's."""
    import torch
    from paged_kv_cache_133_amd import _lib
    from paged_kv_cache_133_amd import workloads as wl
    dev = torch.device("cuda:0")
    w = wl.LLAMA7B
    case = wl.make_workload_case(w, seed=0, device=dev)
    table = case.table_tensor(dev)
    la = case.lens_after_tensor(dev)
    pools = [(case.cache_k, case.cache_v)] + [(case.cache_k.clone(), case.cache_v.clone())
                                              for _ in range(replicas - 1)]
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    row = w.num_kv_heads * w.head_dim * case.cache_k.element_size()
    kv_bytes = int(la.sum().item()) * row * 2
    runs = []
    for slice_bytes, split in ((512, 256), (256, 256), (256, 128), (256, 512), (1024, 128),
                               (2048, 64), (row, 16)):
        calls = [_lib.prepare_gather_read(k, v, table, la, case.max_len_after, slice_bytes, split,
                                          sink) for k, v in pools]
        for i in range(2 * replicas):
            calls[i % replicas]()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(launches):
            calls[i % replicas]()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / launches
        runs.append({"slice_bytes": slice_bytes, "split_tokens": split, "us_per_launch": round(us, 2),
                     "GB_per_s": round(kv_bytes / (us * 1e-6) / 1e9, 1)})
    return {"workload": w.name, "kv_read_bytes": kv_bytes, "decode_pattern": runs[0],
            "best": max(runs, key=lambda r: r["GB_per_s"]), "runs": runs}


def cpu_baseline(case, kv_bytes, min_seconds):
    """The fp64 oracle on this host, on host copies of the same inputs.  One step is
    slot_mapping, the in-place cache writes of the step's rows, then attention for every
    sequence; the pools are copied to the host once, outside the timing (writing the same
    rows to the same slots again changes nothing).  INT8 workloads also quantize the new
    rows and dequantize the pools, as the oracle computes them.  Timed with all of the
    oracle's threads (median of at least 3 runs, at least min_seconds in all), then with
    one thread, on the whole step when that takes under ~10 s, else on every k-th
    sequence (the KV bytes of those sequences over their time)."""
    from oracle import oracle
    import numpy as np
    import torch

    def host(t):
        if t is None:
            return None
        t = t.detach().cpu().contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    c = case
    w = c.w
    h = {"block_table": c.block_table, "lens_before": c.lens_before, "cu_q": c.cu_q,
         "lens_after": c.lens_after, "cache_k": host(c.cache_k), "cache_v": host(c.cache_v),
         "cache_rope": host(c.cache_rope), "q": host(c.q), "q_rope": host(c.q_rope),
         "new_k": host(c.new_k), "new_v": host(c.new_v), "new_rope": host(c.new_rope)}
    int8 = w.kv_dtype == "int8"
    mla = w.mode == "mla"
    causal = w.mode == "varlen"
    if int8:
        # the oracle's own quantization of the pools (outside the timed step)
        pk, sk = oracle.quantize_rows(h["cache_k"])
        pv, sv = oracle.quantize_rows(h["cache_rope" if mla else "cache_v"])
        pools = [(pk, sk, h["new_k"]), (pv, sv, h["new_rope" if mla else "new_v"])]
    else:
        pools = [(h["cache_k"], h["new_k"]), (h["cache_rope" if mla else "cache_v"],
                                               h["new_rope" if mla else "new_v"])]

    def step(rows, threads):
        slots = oracle.slot_mapping(h["block_table"], h["lens_before"], h["cu_q"],
                                    w.block_size, c.num_blocks)
        if int8:
            caches = []
            for codes, scales, new in pools:
                qn, sn = oracle.quantize_rows(new)
                oracle.kv_write_into(codes, qn, slots)
                oracle.kv_write_into(scales, sn, slots)
                caches.append(oracle.dequantize_rows(codes, scales))
            q = oracle.widen(h["q"])
            q_rope = oracle.widen(h["q_rope"]) if mla else None
        else:
            for pool, new in pools:
                oracle.kv_write_into(pool, new, slots)
            caches = [p for p, _ in pools]
            q, q_rope = h["q"], h["q_rope"]
        k = caches[0]
        v, rope = (k, caches[1]) if mla else (caches[1], None)
        tok = np.concatenate([np.arange(c.cu_q[b], c.cu_q[b + 1]) for b in rows]).astype(np.int64)
        n = c.cu_q[rows + 1] - c.cu_q[rows]
        cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
        oracle.paged_attention(q[tok], k, v, c.block_table[rows], cu, c.lens_after[rows], w.scale,
                               causal, q_rope=q_rope[tok] if q_rope is not None else None,
                               k_rope=rope, threads=threads, window=w.window)

    all_rows = np.arange(w.batch)
    threads = oracle.max_threads()
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        step(all_rows, threads)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start >= min_seconds and len(times) >= 3:
            break
    med = statistics.median(times)
    # one thread: the whole step, or every k-th sequence so that it takes ~10 s at most
    keys = visible_keys(c)[0].astype(np.float64)
    k_every = max(1, int(np.ceil(med * threads / 10.0)))
    rows1 = all_rows[::k_every]
    t1 = time.perf_counter()
    step(rows1, 1)
    t1 = time.perf_counter() - t1
    bytes1 = kv_bytes * float(keys[rows1].sum() / keys.sum())
    sample1 = ("the whole step" if k_every == 1 else
               f"the step's writes and the attention of one sequence in {k_every} "
               f"({len(rows1)} of {w.batch}, {bytes1 / 1e6:.1f} MB of KV)")
    return {"value": round(kv_bytes / med / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"whole {w.name} step (slot_mapping, in-place K/V writes, fp64 attention "
                       f"over all {w.batch} sequences; pools copied to the host once, outside "
                       f"the timing), median of {len(times)} runs, {med * 1e3:.1f} ms/step"),
            "value_1_thread": round(bytes1 / t1 / 1e9, 4),
            "sample_1_thread": f"{sample1}: {t1 * 1e3:.1f} ms"}


def step_description(w, path):
    """What one timed step launches, for the JSON line."""
    if int8_workload(w) and w.mode == "mla":
        if path == "fused":
            return ("paged_attn_decode_mla_int8_append: MLA split pass that also quantizes and "
                    "writes the new latent row (slot_mapping + quantizing write of nope and rope "
                    "+ split-KV attention), then combine")
        return ("slot_mapping, kv_cache_write_int8_mla (quantizing write of nope and rope), "
                "decode_mla_int8 split pass, combine")
    if int8_workload(w):
        ranges = w.num_q_heads // w.num_kv_heads > 4
        if path == "fused":
            return ("paged_attn_decode_int8_append: %s pass that also quantizes and writes the "
                    "new token (slot_mapping + quantizing write + attention), then combine"
                    % ("range" if ranges else "split"))
        return ("slot_mapping, kv_cache_write_int8 (quantizing write), decode_int8 %s pass, combine"
                % ("range" if ranges else "split"))
    if w.q_tokens:
        if path == "fused":
            return ("paged_attn_decode_mtp_append: range pass that also writes the step's %d rows "
                    "per sequence (slot_mapping + write + attention), then combine" % w.q_tokens)
        return ("kv_cache_append (slot_mapping + write of the step's %d rows per sequence), "
                "decode_mtp range pass, combine" % w.q_tokens)
    if w.mode == "varlen":
        if path == "fused":
            return ("paged_attn_varlen_append: varlen causal attention pass that also writes the "
                    "chunk's new rows (slot_mapping + write + attention, one launch)")
        return "kv_cache_append (slot_mapping + write), varlen causal attention"
    if w.mode == "mla":
        return {"separate": "slot_mapping, kv_cache_write (nope + rope), MLA split pass, combine",
                "append": "kv_cache_append (nope + rope), MLA split pass, combine"}.get(
            path, "paged_attn_decode_mla_append: MLA split pass that also writes the new latent "
                  "row (slot_mapping + write of nope and rope + split-KV attention), then combine")
    return {"fused": "paged_attn_decode_append: split pass that also writes the new "
                     "token (slot_mapping + write + split-KV attention), then combine",
            "append": "kv_cache_append (slot_mapping + write), decode split, combine",
            "separate": "slot_mapping, kv_cache_write, decode split, combine"}[path]


def int8_workload(w):
    return w.kv_dtype == "int8"


def serving(args):
    """--serving: the decode layer of a workload as a serving loop runs it, once per block
    size ("Paged KV Cache and Packed Sequence", 5.3-5.4).  The sequences start at the
    workload's lengths, their blocks taken from the host block manager one block per
    sequence in turn (so that neighbouring blocks belong to different sequences, as under
    continuous batching).  A loop step is pkv_bm_decode_step writing the next table into a
    pinned buffer (host time) and one pkv_runner_launch (replay of the recorded step: the
    table copy kernel, then write-and-attend).  Timed beside it, each back to back on one
    stream: the table copy kernel alone, the replay alone, and the same step (without the
    copy) run eagerly.
    Prints one JSON line with a row per block size."""
    import numpy as np
    import torch
    import paged_kv_cache_133_amd as pkv
    from paged_kv_cache_133_amd import _lib
    from paged_kv_cache_133_amd import workloads as wl
    from paged_kv_cache_133_amd.step import GraphDecodeStep

    w = wl.WORKLOADS[args.workload]
    if w.mode != "decode" or w.kv_dtype:
        print("bench.py --serving runs MHA/GQA decode workloads", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    L0, _ = wl.sample_lengths(w, args.seed)
    B, hq, hkv, d = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
    row_bytes = hkv * d * w.elem_bytes
    gen = torch.Generator(device=dev).manual_seed(args.seed)
    K = args.steps
    total = args.warmup + 2 * K
    ev = lambda: torch.cuda.Event(enable_timing=True)   # noqa: E731
    cur = lambda: ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)   # noqa: E731

    def timed(fn, n):
        """Mean µs of fn() run n times back to back (after one untimed call)."""
        fn()
        a, b = ev(), ev()
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n * 1e3

    rows = []
    for bs in [int(x) for x in args.block_sizes.split(",")]:
        final = L0 + total + 2
        mbs = int(math.ceil(final.max() / bs * args.table_capacity))
        nb = int(sum(math.ceil(x / bs) for x in final)) + 8
        k = torch.randn(nb, bs, hkv, d, generator=gen, device=dev).to(w.torch_dtype)
        v = torch.randn(nb, bs, hkv, d, generator=gen, device=dev).to(w.torch_dtype)
        bm = pkv.BlockManager(nb, bs, mbs)
        left = [int(x) for x in L0]
        for b in range(B):
            bm.add(b)
        while any(left):
            for b in range(B):
                n = min(left[b], bs)
                if n:
                    bm.append(b, n)
                    left[b] -= n
        step = GraphDecodeStep(k, v, B, mbs, hq, w.scale, window=w.window)
        step.q.copy_(torch.randn(B, hq, d, generator=gen, device=dev).to(w.torch_dtype))
        step.k_new.copy_(torch.randn(B, hkv, d, generator=gen, device=dev).to(w.torch_dtype))
        step.v_new.copy_(step.k_new)
        ids = np.arange(B, dtype=np.int64)

        def loop_step():
            tab, lens = step.host_tables()
            bm.decode_step(ids, table=tab, seq_lens=lens)
            step.launch()

        settle_clock(args.settle_ms)
        for _ in range(args.warmup):
            loop_step()
        torch.cuda.synchronize()
        tokens_before = sum(bm.length(b) for b in range(B))
        # the serving loop: host work and launches, K steps
        t0, t1 = ev(), ev()
        host_s = 0.0
        t0.record()
        wall0 = time.perf_counter()
        for _ in range(K):
            h0 = time.perf_counter()
            tab, lens = step.host_tables()
            bm.decode_step(ids, table=tab, seq_lens=lens)
            host_s += time.perf_counter() - h0
            step.launch()
        t1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        loop_gpu = t0.elapsed_time(t1) / K * 1e3
        # pieces alone, on the tables of the last step (lengths stay put: the same slot is
        # rewritten each time)
        j_last = (K + args.warmup - 1) % 2
        up = timed(lambda: _lib._check(_lib.lib().pkv_upload_kernel(
            ctypes.c_void_p(step.dev[j_last].data_ptr()),
            ctypes.c_void_p(step.staging[j_last].data_ptr()), step.nbytes, cur())), K)
        graph = step.graph(j_last)
        gr = timed(lambda: _lib._check(_lib.lib().pkv_graph_launch(graph, cur())), K)
        table_d, lens_d = (x.clone() for x in step.device_views(j_last))
        ws = pkv.new_decode_workspace(B, hq, hkv, d, mbs * bs, dev)
        out = torch.empty_like(step.out)
        eager = timed(lambda: pkv.paged_attn_decode_append(step.q, step.k_new, step.v_new, k, v,
                                                           table_d, lens_d, mbs * bs, w.scale,
                                                           out=out, workspace=ws), K)
        kv_tokens = tokens_before + B * (K + 1) / 2.0
        held = sum(math.ceil(bm.length(b) / bs) for b in range(B))
        rows.append({"block_size": bs, "max_blocks_per_seq": mbs,
                     "table_capacity": args.table_capacity,
                     "table_bytes": step.nbytes,
                     "host_table_us": round(host_s / K * 1e6, 2),
                     "upload_us": round(up, 2), "graph_replay_us": round(gr, 2),
                     "eager_step_us": round(eager, 2),
                     "loop_gpu_us_per_step": round(loop_gpu, 2),
                     "loop_wall_us_per_step": round(wall / K * 1e6, 2),
                     "kv_read_gbps_loop": round(kv_tokens * 2 * row_bytes / (loop_gpu * 1e-6) / 1e9, 1),
                     "slack_tokens": held * bs - sum(bm.length(b) for b in range(B))})
        print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
        step.close()
        bm.close()
        del k, v, step
        torch.cuda.empty_cache()
    line = {"metric": "serving decode step per block size (host table, upload, graph replay)",
            "unit": "us", "n_gpus": 1, "steps": K, "warmup": args.warmup,
            "dtype": w.dtype, "data": "synthetic",
            "config": {"workload": w.name, "batch": B, "num_q_heads": hq, "num_kv_heads": hkv,
                       "head_dim": d, "window": w.window, "seed": args.seed},
            "results": rows}
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.read_ceiling:
        read_ceiling(settle_ms=args.settle_ms)
        return
    if args.serving:
        import torch
        if not torch.cuda.is_available():
            print("bench.py needs a GPU", file=sys.stderr)
            sys.exit(1)
        serving(args)
        return
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import paged_kv_cache_133_amd as pkv
    from paged_kv_cache_133_amd import _lib
    from paged_kv_cache_133_amd import workloads as wl

    pkv.lib()   # fails loudly if the HIP library is missing
    w = wl.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    case = wl.make_workload_case(w, seed=args.seed, device=dev)
    kv_bytes, split_bytes, step_bytes = algorithmic_bytes(case, args.path)
    int8 = w.kv_dtype == "int8"
    if int8 and w.mode == "mla":
        # The INT8 latent pools: nope and rope rows of the bf16 pools quantized by the writer.
        nbs = case.num_blocks * w.block_size
        nb_, bs_ = case.cache_k.shape[:2]
        pool_i8 = {"k": torch.empty((nb_, bs_, 512), dtype=torch.int8, device=dev),
                   "v": torch.empty((nb_, bs_, 64), dtype=torch.int8, device=dev)}
        pool_sc = {n: torch.empty((nb_, bs_), dtype=torch.float32, device=dev) for n in ("k", "v")}
        pkv.kv_cache_write_int8_mla(case.cache_k.reshape(nbs, 512), case.cache_rope.reshape(nbs, 64),
                                    pool_i8["k"], pool_i8["v"], pool_sc["k"], pool_sc["v"],
                                    torch.arange(nbs, dtype=torch.int64, device=dev))
        pool_bytes = sum(t.numel() * t.element_size() for t in (*pool_i8.values(), *pool_sc.values()))
    elif int8:
        # The INT8 pools: every row of the bf16 pool quantized by the library's writer.
        nbs = case.num_blocks * w.block_size
        pool_i8 = {n: torch.empty(case.cache_k.shape, dtype=torch.int8, device=dev) for n in ("k", "v")}
        nb_, bs_, hkv_ = case.cache_k.shape[:3]
        pool_sc = {n: torch.empty((nb_, hkv_, bs_), dtype=torch.float32, device=dev)
                   for n in ("k", "v")}
        pkv.kv_cache_write_int8(case.cache_k.reshape(nbs, w.num_kv_heads, w.head_dim),
                                case.cache_v.reshape(nbs, w.num_kv_heads, w.head_dim_v),
                                pool_i8["k"], pool_i8["v"], pool_sc["k"], pool_sc["v"],
                                torch.arange(nbs, dtype=torch.int64, device=dev))
        pool_bytes = sum(t.numel() * t.element_size() for t in (*pool_i8.values(), *pool_sc.values()))
    else:
        pool_bytes = sum(t.numel() * t.element_size()
                         for t in {id(x): x for x in (case.cache_k, case.cache_v, case.cache_rope)
                                   if x is not None}.values())
    R = args.replicas or max(2, min(64, math.ceil(2.0e9 / pool_bytes)))
    mla = w.mode == "mla"

    table = case.table_tensor(dev)
    lb = case.lens_before_tensor(dev)
    la = case.lens_after_tensor(dev)
    cu = case.cu_q_tensor(dev)
    T = case.num_tokens
    slots = torch.empty(T, dtype=torch.int64, device=dev)
    out = torch.empty((T, w.num_q_heads, w.head_dim_v), dtype=w.torch_dtype, device=dev)
    lse = torch.empty((T, w.num_q_heads), dtype=torch.float32, device=dev)
    need = pkv.decode_workspace_size(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim_v,
                                     case.max_len_after)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=dev)
    ws_mtp = None
    if w.q_tokens:
        need = int(_lib.lib().pkv_decode_mtp_workspace_size(w.batch, w.q_tokens, w.num_q_heads,
                                                            w.num_kv_heads, w.head_dim_v,
                                                            case.max_len_after))
        ws_mtp = torch.zeros(max(need, 16), dtype=torch.uint8, device=dev)
    slot_call = _lib.prepare_slot_mapping(table, lb, cu, w.block_size, T, slots)
    fused = args.path == "fused"
    reps = []
    # INT8: the quantizing write folds into the attention pass (the fused path); the
    # separate path runs slot_mapping and the quantizing writer first.
    int8_fused = int8 and fused
    slot_first = args.path == "separate" or (int8 and not int8_fused)
    for r in range(R):
        if int8 and mla:
            nc, rc, ns, rs = (pool_i8["k"], pool_i8["v"], pool_sc["k"], pool_sc["v"]) if r == 0 else (
                pool_i8["k"].clone(), pool_i8["v"].clone(), pool_sc["k"].clone(), pool_sc["v"].clone())
            if int8_fused:
                split, combine, _ = _lib.prepare_decode_mla_int8_append(
                    case.q, case.q_rope, case.new_k.reshape(T, 512), case.new_rope.reshape(T, 64),
                    nc, rc, ns, rs, table, la, case.max_len_after, w.scale, out=out, lse=lse,
                    workspace=ws, slots_out=slots)
                reps.append((None, split, combine))
                continue
            write = _lib.prepare_kv_cache_write_int8_mla(case.new_k.reshape(T, 512),
                                                         case.new_rope.reshape(T, 64), nc, rc, ns,
                                                         rs, slots)
            split, combine, _ = _lib.prepare_decode_mla_int8(case.q, case.q_rope, nc, rc, ns, rs,
                                                             table, la, case.max_len_after, w.scale,
                                                             out=out, lse=lse, workspace=ws)
            reps.append((write, split, combine))
            continue
        if int8:
            ki8, vi8, ksc, vsc = (pool_i8["k"], pool_i8["v"], pool_sc["k"], pool_sc["v"]) if r == 0 else (
                pool_i8["k"].clone(), pool_i8["v"].clone(), pool_sc["k"].clone(), pool_sc["v"].clone())
            if int8_fused:
                split, combine, _ = _lib.prepare_decode_int8_append(
                    case.q, case.new_k, case.new_v, ki8, vi8, ksc, vsc, table, la,
                    case.max_len_after, w.scale, out=out, lse=lse, workspace=ws, slots_out=slots,
                    window=w.window)
                reps.append((None, split, combine))
                continue
            write = _lib.prepare_kv_cache_write_int8(case.new_k, case.new_v, ki8, vi8, ksc, vsc, slots)
            split, combine, _ = _lib.prepare_decode_int8(case.q, ki8, vi8, ksc, vsc, table, la,
                                                         case.max_len_after, w.scale, out=out,
                                                         lse=lse, workspace=ws, window=w.window)
            reps.append((write, split, combine))
            continue
        k = case.cache_k if r == 0 else case.cache_k.clone()
        rope = None
        if mla:
            v = k
            rope = case.cache_rope if r == 0 else case.cache_rope.clone()
            pair = (case.new_k, case.new_rope, k, rope)
        else:
            v = case.cache_v if r == 0 else case.cache_v.clone()
            pair = (case.new_k, case.new_v, k, v)
        if w.q_tokens and fused:
            attn, combine, _ = _lib.prepare_decode_mtp_append(case.q, case.new_k, case.new_v, k, v,
                                                              table, la, w.q_tokens,
                                                              case.max_len_after, w.scale, out=out,
                                                              lse=lse, workspace=ws_mtp,
                                                              window=w.window, slots_out=slots)
            reps.append((None, attn, combine))
            continue
        if w.q_tokens:
            write = _lib.prepare_kv_cache_append(*pair, table, lb, cu, case.max_new, slots)
            attn, combine, _ = _lib.prepare_decode_mtp(case.q, k, v, table, la, w.q_tokens,
                                                       case.max_len_after, w.scale, out=out,
                                                       lse=lse, workspace=ws_mtp, window=w.window)
            reps.append((write, attn, combine))
            continue
        if w.mode == "varlen":
            if fused:
                attn = _lib.prepare_varlen_append(case.q, case.new_k, case.new_v, k, v, table, cu,
                                                  la, case.max_new, w.scale, causal=True, out=out,
                                                  lse=lse, window=w.window, slots_out=slots)
                reps.append((None, attn, None))
                continue
            write = _lib.prepare_kv_cache_append(*pair, table, lb, cu, case.max_new, slots)
            attn = _lib.prepare_varlen(case.q, k, v, table, cu, la, case.max_new, w.scale,
                                       causal=True, out=out, lse=lse, window=w.window)
            reps.append((write, attn, None))
            continue
        if fused and mla:
            split, combine, _ = _lib.prepare_decode_mla_append(case.q, case.q_rope, case.new_k,
                                                               case.new_rope, k, rope, table, la,
                                                               case.max_len_after, w.scale,
                                                               out=out, lse=lse, workspace=ws,
                                                               slots_out=slots)
            reps.append((None, split, combine))
            continue
        if fused and not mla:
            split, combine, _ = _lib.prepare_decode_append(case.q, case.new_k, case.new_v, k, v,
                                                           table, la, case.max_len_after, w.scale,
                                                           out=out, lse=lse, workspace=ws,
                                                           slots_out=slots, window=w.window)
            reps.append((None, split, combine))
            continue
        if w.window:
            print("bench.py: sliding-window workloads run the fused path only", file=sys.stderr)
            sys.exit(2)
        if args.path == "separate":
            write = _lib.prepare_kv_cache_write(*pair, slots)
        else:
            write = _lib.prepare_kv_cache_append(*pair, table, lb, cu, case.max_new, slots)
        split, combine, whole, _ = _lib.prepare_decode(case.q, k, v, table, la,
                                                       case.max_len_after, w.scale,
                                                       q_rope=case.q_rope, k_rope_cache=rope,
                                                       out=out, lse=lse, workspace=ws)
        reps.append((write, split, combine))
    torch.cuda.synchronize()

    def step(i):
        write, attn, combine = reps[i % R]
        if slot_first:
            slot_call()
        if write is not None:
            write()
        attn()
        if combine is not None:
            combine()

    # Clock settling: from idle the GPU's clock takes tens of milliseconds to reach its
    # steady level under this load (measured: a few warm-up steps leave the long-context
    # and varlen steps 15-20 % slower than a settled run), so whole steps run untimed for
    # at least --settle-ms of wall time before the W warm-up steps.
    settle_steps = 0
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(8):
            step(settle_steps)
            settle_steps += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(settle_steps + i)
    torch.cuda.synchronize()
    # Timed region: K whole steps, events only at its two ends.
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(args.steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    us_step = ms_step * 1e3
    value = kv_bytes / (ms_step * 1e-3) / 1e9

    roofline = None
    flops = algorithmic_flops(case)
    if not args.no_kernel_events:
        # The dominant kernel's launch time: a second timed region of K launches of that
        # kernel alone, back to back over the rotated pools, on the stream the library
        # launches on (torch's current stream), events only at the two ends.  (Events
        # around every launch add their own overhead to each duration.)
        for i in range(2):
            reps[i % R][1]()
        k0 = torch.cuda.Event(enable_timing=True)
        k1 = torch.cuda.Event(enable_timing=True)
        k0.record()
        for i in range(args.steps):
            reps[i % R][1]()
        k1.record()
        torch.cuda.synchronize()
        split_ms = k0.elapsed_time(k1) / args.steps
        gbps = split_bytes / (split_ms * 1e-3) / 1e9
        tflops = flops / (split_ms * 1e-3) / 1e12
        # The bound is whichever resource the launch would saturate first at peak.
        mfma_bound = flops / (PEAK_BF16_TFLOPS * 1e12) > split_bytes / (PEAK_HBM_GBPS * 1e9)
        kname, ksources = dominant_kernel(w, args.path)
        traffic, traffic_src = read_traffic(w.name, kname, ksources)
        if mfma_bound:
            roofline = {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4)}
        else:
            roofline = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS,
                        "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4)}
        roofline.update({"traffic": traffic, "traffic_source": traffic_src, "kernel": kname,
                         "kernel_us": round(split_ms * 1e3, 2),
                         "kernel_us_method": (f"{args.steps} launches of the kernel alone, back "
                                              "to back on its stream, HIP events at the two ends"),
                         "algorithmic_bytes_per_launch": split_bytes,
                         "algorithmic_flops_per_launch": flops,
                         "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4),
                         "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4)})

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(case, kv_bytes, args.cpu_seconds)

    cfg = {"workload": w.name, "batch": w.batch, "num_q_heads": w.num_q_heads,
           "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "head_dim_v": w.head_dim_v,
           "head_dim_rope": w.head_dim_rope, "block_size": w.block_size, "window": w.window,
           "kv_dtype": w.kv_dtype or w.dtype,
           "num_blocks": case.num_blocks, "seed": args.seed,
           "kv_tokens": int(case.lens_after.sum()), "max_kv_len": case.max_len_after,
           "pool_replicas": R,
           "path": args.path,
           "step": step_description(w, args.path)}
    line = {"metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
            "settle": {"ms": args.settle_ms, "steps": settle_steps,
                       "what": "untimed whole steps before the warm-up, until the GPU clock has settled"},
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": w.dtype, "data": "synthetic", "config": cfg,
            "us_per_step": round(us_step, 2),
            "pct_of_peak_hbm": round(100.0 * value / PEAK_HBM_GBPS, 2),
            "algorithmic_bytes_per_step": step_bytes, "kv_read_bytes_per_step": kv_bytes,
            "roofline": roofline, "cpu_baseline": cpu}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
