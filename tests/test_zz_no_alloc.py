"""sp_region_bwd_noalloc (the backward with the library's static device
scratch as its workspace) against sp_region_bwd with a caller-allocated
workspace: bit for bit on two calls in a row, the second on a smaller shard,
plus the size limit and the argument checks."""
import numpy as np
import pytest

import layernorm_sp_region_amd as spr
import workloads as W

pytestmark = pytest.mark.gpu


def _shard(cuda_device, name, h, t, s, norm, dres, seed):
    import torch
    w = W.custom(name, h=h, t=t, s=s, norm=norm, p_drop=0.1, seed=seed, bias=False)
    inp = W.make_inputs(w)
    tt = lambda a: W.as_torch(a, cuda_device)
    fo = spr.fwd(tt(inp["partials"]), tt(inp["gamma"]), tt(inp["beta"]), residual=tt(inp["residual"]), b=1, s=s,
                 t=t, rank=1, eps=w.eps, p_drop=w.p_drop, seed=inp["seed"], norm=norm)
    dr = tt(W.make_inputs(w, seed=seed + 1)["dy"]) if dres else None
    torch.cuda.synchronize()
    return dict(w=w, s=s, t=t, norm=norm, dy=tt(inp["dy"]), z=fo.z, mean=fo.mean, rstd=fo.rstd,
                gamma=tt(inp["gamma"]), dres=dr)


def _outs(c, cuda_device, fill):
    import torch
    T, h = c["z"].shape
    ln = c["norm"] == "layernorm"
    return spr.BwdOut(torch.full((T, h), fill, dtype=c["z"].dtype, device=cuda_device),
                      torch.full((h,), fill, device=cuda_device),
                      torch.full((h,), fill, device=cuda_device) if ln else None)


def _both(c, cuda_device):
    import torch
    kw = dict(b=1, s=c["s"], t=c["t"], norm=c["norm"], dres_in=c["dres"])
    ref = spr.bwd(c["dy"], c["z"], c["mean"], c["rstd"], c["gamma"], out=_outs(c, cuda_device, 0.0), **kw)
    got = spr.bwd_noalloc(c["dy"], c["z"], c["mean"], c["rstd"], c["gamma"], out=_outs(c, cuda_device, 7.0), **kw)
    torch.cuda.synchronize()
    for k in ("dx", "dgamma", "dbeta"):
        a, b = getattr(ref, k), getattr(got, k)
        if a is None:
            assert b is None
            continue
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), k


def test_noalloc_matches_workspace_backward_twice(cuda_device):
    # The 70B shard's backward first, then a smaller, ragged-width shard with
    # an extra residual-stream gradient, then RMSNorm: each bit for bit the
    # caller-workspace call's outputs (the scratch keeps the previous call's
    # partials, which the kernels overwrite).
    _both(_shard(cuda_device, "na_big", 8192, 8, 8 * 2048, "layernorm", False, 41), cuda_device)
    _both(_shard(cuda_device, "na_small", 1032, 4, 4 * 37, "layernorm", True, 42), cuda_device)
    _both(_shard(cuda_device, "na_rms", 4096, 2, 2 * 300, "rmsnorm", False, 43), cuda_device)


def test_noalloc_limit_and_checks(cuda_device):
    import torch
    # The smallest shard at h = 16384 whose workspace exceeds the static
    # scratch is refused before any launch, outputs untouched.
    h = 16384
    T = next(T for T in range(1, 4096) if spr.workspace_bytes(T, h) > spr.NOALLOC_SCRATCH_BYTES)
    assert spr.workspace_bytes(T - 1, h) <= spr.NOALLOC_SCRATCH_BYTES
    z = torch.zeros((T, h), dtype=torch.bfloat16, device=cuda_device)
    stats = torch.ones(T, device=cuda_device)
    gamma = torch.ones(h, dtype=torch.bfloat16, device=cuda_device)
    out = spr.BwdOut(torch.full_like(z, 3.0), torch.full((h,), 3.0, device=cuda_device),
                     torch.full((h,), 3.0, device=cuda_device))
    with pytest.raises(spr.SpRegionError) as e:
        spr.bwd_noalloc(z, z, stats, stats, gamma, b=1, s=4 * T, t=4, out=out)
    assert e.value.status == spr.SPR_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((out.dx == 3.0).all()) and bool((out.dgamma == 3.0).all()) and bool((out.dbeta == 3.0).all())
    # ... while the largest shard that fits runs, bit for bit as sp_region_bwd.
    _both(_shard(cuda_device, "na_edge", h, 4, 4 * (T - 1), "layernorm", False, 45), cuda_device)
    # Argument checks are sp_region_bwd's: LayerNorm without a mean.
    c = _shard(cuda_device, "na_chk", 256, 2, 2 * 8, "layernorm", False, 44)
    lib = spr.load_library()
    st = lib.sp_region_bwd_noalloc(1, c["s"], 256, 2, c["gamma"].data_ptr(), spr.SPR_LAYERNORM, spr.SPR_BF16,
                                   c["dy"].data_ptr(), c["z"].data_ptr(), None, c["rstd"].data_ptr(), None,
                                   c["z"].data_ptr(), c["rstd"].data_ptr(), None, None)
    assert st == spr.SPR_ERR_INVALID_ARG
