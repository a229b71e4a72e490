"""Test-side helpers: host copies of a case, and the textbook (unpaged) attention pin.

The brute-force attention here is written independently of the oracle: it builds each
sequence's logical K/V by concatenating that sequence's physical blocks in block-table
order (the defining property of a block table), appends the new rows, and applies
numpy softmax attention with an explicit mask.  It reads no slot formula.
"""
import numpy as np
import torch
from scipy.special import logsumexp


def host(t):
    """A torch tensor as a numpy array the oracle accepts (f32, or bf16 bits as uint16)."""
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_f64(t):
    if t is None:
        return None
    return t.detach().cpu().to(torch.float64).numpy()


def case_numpy(case):
    c = case
    return {
        "block_table": c.block_table, "lens_before": c.lens_before, "cu_q": c.cu_q,
        "lens_after": c.lens_after, "cache_k": host(c.cache_k),
        "cache_v": host(c.cache_v), "cache_rope": host(c.cache_rope), "q": host(c.q),
        "q_rope": host(c.q_rope), "new_k": host(c.new_k), "new_v": host(c.new_v),
        "new_rope": host(c.new_rope), "block_size": c.w.block_size,
        "num_blocks": c.num_blocks, "scale": c.w.scale,
    }


def logical_rows(pool, table_row, need, prefix_len, new_rows):
    """Logical [L', ...] rows of one sequence: its blocks in table order, cut at the prefix,
    then the new rows."""
    blocks = [pool[int(table_row[j])] for j in range(int(need))]
    if blocks:
        flat = np.concatenate(blocks, axis=0)[:prefix_len]
    else:
        flat = pool[:0, 0]
    return np.concatenate([flat, new_rows], axis=0)


def brute_attention(case, causal, window=0):
    """Textbook attention in fp64 over contiguous per-sequence K/V.  Returns (out, lse).
    window > 0 keeps, for each row, only the `window` most recent of its visible keys."""
    c = case
    w = c.w
    kp = as_f64(c.cache_k)
    vp = kp if w.mode == "mla" else as_f64(c.cache_v)
    rp = as_f64(c.cache_rope)
    q = as_f64(c.q)
    qr = as_f64(c.q_rope)
    nk = as_f64(c.new_k)
    nv = nk if w.mode == "mla" else as_f64(c.new_v)
    nr = as_f64(c.new_rope)
    T, Hq, _ = q.shape
    G = w.num_q_heads // w.num_kv_heads
    out = np.zeros((T, Hq, w.head_dim_v))
    lse = np.zeros((T, Hq))
    for b in range(w.batch):
        a, e = int(c.cu_q[b]), int(c.cu_q[b + 1])
        L = int(c.lens_before[b])
        K = logical_rows(kp, c.block_table[b], c.need[b], L, nk[a:e])
        V = logical_rows(vp, c.block_table[b], c.need[b], L, nv[a:e])
        R = logical_rows(rp, c.block_table[b], c.need[b], L, nr[a:e]) if rp is not None else None
        n = e - a
        Lp = L + n
        for h in range(Hq):
            g = h // G
            s = q[a:e, h, :] @ K[:, g, :].T
            if R is not None:
                s = s + qr[a:e, h, :] @ R[:, g, :].T
            s = s * w.scale
            # row i may see keys 0 .. hi_i: hi_i = Lp - n + i (causal) or Lp - 1
            hi = (Lp - n + np.arange(n)) if causal else np.full(n, Lp - 1)
            keep = np.arange(Lp)[None, :] <= hi[:, None]
            if window > 0:
                keep &= np.arange(Lp)[None, :] > (hi - window)[:, None]
            s = np.where(keep, s, -np.inf)
            z = logsumexp(s, axis=1)
            p = np.exp(s - z[:, None])
            out[a:e, h, :] = p @ V[:, g, :w.head_dim_v]
            lse[a:e, h] = z
    return out, lse
