"""GPU parity of the fused RMSNorm + RoPE + cache write of the MLA latent row against the
fp64 oracle, through the C ABI: written rows within one rounding to the cache dtype of the
exact values, every other byte of both pools unchanged, slots outside the pool skipped.
Needs an MI355X."""
import numpy as np
import pytest
import torch

import paged_kv_cache_133_amd as pkv
from oracle import oracle
from tests.gpu_common import say
from tests.helpers import host

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.mark.parametrize("dtype,dn,dr,bs", [("bf16", 512, 64, 64), ("bf16", 128, 32, 16),
                                            ("f32", 512, 64, 1), ("f32", 96, 16, 128)])
def test_norm_rope_write(dtype, dn, dr, bs):
    torch.manual_seed(dn + dr + bs)
    td = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    T = 37
    nb = max(12, (2 * T + bs - 1) // bs)     # a pool with room for every token
    g = torch.Generator().manual_seed(3)
    kv = (torch.randn(T, dn + dr, generator=g) * 3.0).to(td)
    gamma = (1.0 + 0.2 * torch.randn(dn, generator=g)).to(td)
    ang = torch.rand(T, dr // 2, generator=g, dtype=torch.float64) * 6.0 - 3.0
    cos, sin = torch.cos(ang).float(), torch.sin(ang).float()
    slots = torch.randperm(nb * bs, generator=g)[:T].to(torch.int64)
    slots[5] = -1                     # skipped
    slots[9] = nb * bs                # outside the pool: skipped
    cache_nope = torch.randn(nb, bs, 1, dn, generator=g).to(td)
    cache_rope = torch.randn(nb, bs, 1, dr, generator=g).to(td)
    before = (host(cache_nope).copy(), host(cache_rope).copy())
    say(f"norm_rope write {dtype} dn={dn} dr={dr} bs={bs}")
    cn, cr = cache_nope.to(DEV), cache_rope.to(DEV)
    pkv.kv_rmsnorm_rope_cache(kv.to(DEV), gamma.to(DEV), cos.to(DEV), sin.to(DEV), cn, cr,
                              slots.to(DEV), eps=1e-6)
    torch.cuda.synchronize()
    nope_x, rope_x = oracle.rmsnorm_rope(host(kv), host(gamma), cos.numpy(), sin.numpy(), dn, 1e-6)
    gn = oracle.widen(host(cn)).reshape(nb * bs, dn)
    gr = oracle.widen(host(cr)).reshape(nb * bs, dr)
    ok = (slots >= 0) & (slots < nb * bs)
    sl = slots[ok].numpy()
    # written rows: within one rounding of the exact value (bf16: half an ulp, 2^-8
    # relative; fp32: the fp32 arithmetic, 2e-5 relative)
    rel = 2.0 ** -8 if dtype == "bf16" else 2e-5
    for got, exact in ((gn[sl], nope_x[ok.numpy()]), (gr[sl], rope_x[ok.numpy()])):
        err = np.abs(got - exact) - (rel * np.abs(exact) + 1e-6)
        assert err.max() <= 0, f"max excess {err.max():.3e}"
    # every other row byte-identical
    mask = np.ones(nb * bs, bool)
    mask[sl] = False
    assert np.array_equal(host(cn).reshape(nb * bs, -1)[mask], before[0].reshape(nb * bs, -1)[mask])
    assert np.array_equal(host(cr).reshape(nb * bs, -1)[mask], before[1].reshape(nb * bs, -1)[mask])
