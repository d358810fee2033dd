"""GPU parity of the backward through the dropout and the slab sum
(sp_region_bwd_dropout) against the oracle's dropout_backward on the same
seeded inputs.

Bars: dpartial as dx (bf16: half an ulp of the float64 value plus a float32
slack of 4e-5*(1+|ref|), and 2e-2 absolute below 8; float32: 1e-4 relative),
exactly 0 wherever the forward dropped; dbias_j within 1e-4 * sum_i
|dpartial_ij|.  dx, dgamma and dbeta must equal sp_region_bwd's bit for bit.
"""
import numpy as np
import pytest

import layernorm_sp_region_amd as spr
import oracle.region as ref
import workloads as W
from test_gpu_parity import assert_out_close, inputs_for, log, to_np_f64

pytestmark = pytest.mark.gpu


def run_both(inp, w, rank, device, dres=None, recommended_stride=True):
    import torch
    t = lambda a: W.as_torch(a, device)
    P = t(inp["partials"])
    if recommended_stride:
        Pp = spr.empty_partials(P.shape[0], P.shape[1], P.shape[2], P.dtype, device)
        Pp.copy_(P)
        P = Pp
    cu = inp["cu_seqlens"]
    fo = spr.fwd(P, t(inp["gamma"]), t(inp["beta"]), bias=t(inp["bias"]), residual=t(inp["residual"]),
                 b=inp["b"], s=inp["s"], t=w.t, rank=rank, eps=w.eps, p_drop=w.p_drop, seed=inp["seed"],
                 norm=w.norm, cu_seqlens=cu)
    dy, gamma, dr = t(inp["dy"]), t(inp["gamma"]), t(dres)
    one = spr.bwd(dy, fo.z, fo.mean, fo.rstd, gamma, b=inp["b"], s=inp["s"], t=w.t, norm=w.norm, dres_in=dr)
    two = spr.bwd_dropout(dy, fo.z, fo.mean, fo.rstd, gamma, b=inp["b"], s=inp["s"], t=w.t, rank=rank,
                          p_drop=w.p_drop, seed=inp["seed"], norm=w.norm, cu_seqlens=cu, dres_in=dr)
    torch.cuda.synchronize()
    bits = lambda x: None if x is None else x.view(torch.int32 if x.dtype == torch.float32 else torch.int16).cpu()
    for name in ("dx", "dgamma", "dbeta"):
        a, b = getattr(one, name), getattr(two, name)
        assert (a is None) == (b is None), name
        if a is not None:
            assert torch.equal(bits(a), bits(b)), f"{name} differs from sp_region_bwd"
    return fo, two


def check(w, inp, rank, two, dres=None):
    o = ref.region_forward(inp["partials"], t=w.t, rank=rank, dtype=w.dtype, norm=w.norm, eps=w.eps,
                           p_drop=w.p_drop, seed=inp["seed"], gamma=inp["gamma"], beta=inp["beta"],
                           bias=inp["bias"], residual=inp["residual"], cu_seqlens=inp["cu_seqlens"])
    ob = ref.region_backward(inp["dy"], o["z"], inp["gamma"], dtype=w.dtype, norm=w.norm, eps=w.eps, dres_in=dres)
    od = ref.dropout_backward(ob["dx"], t=w.t, rank=rank, p_drop=w.p_drop, seed=inp["seed"],
                              cu_seqlens=inp["cu_seqlens"])
    got = to_np_f64(two.dpartial)
    assert np.all(got[~od["keep"]] == 0.0), "dpartial nonzero where the forward dropped"
    assert_out_close(got, od["dpartial"], w.dtype, "dpartial", 4e-5)
    assert_out_close(to_np_f64(two.dx), ob["dx"], w.dtype, "dx", 3e-5)
    err = np.abs(to_np_f64(two.dbias) - od["dbias"])
    assert np.all(err <= 1e-4 * od["C"]), f"dbias: worst err/C {np.max(err / np.maximum(od['C'], 1e-300)):.2e}"
    log(f"  dropout backward ok: dbias err/C max {np.max(err / np.maximum(od['C'], 1e-300)):.2e}, "
        f"dropped {(~od['keep']).mean():.4f}")


@pytest.mark.parametrize("name,rank", [("tiny", 3), ("page_demo", 7), ("shard70b", 0), ("ragged13b", 5)])
def test_workload_dropout_backward(cuda_device, name, rank):
    w = W.BY_NAME[name]
    log(f"[dropout-bwd] {name} rank={rank}")
    inp = inputs_for(w)
    _, two = run_both(inp, w, rank, cuda_device)
    check(w, inp, rank, two)


NO_DBIAS = [("page_demo", 2, False), ("tiny", 1, False),
            # ragged shard: the token index of each row from cu_seqlens (scalar loads)
            (W.custom("ragged_drop_small", h=1024, t=4, lengths=(40, 0, 96, 8, 200), norm="layernorm",
                      p_drop=0.3), 3, False),
            # odd t, b = 2, 65 vectors per row (a ragged last column block), extra gradient on z
            (W.custom("odd_t3_h520_dres", h=520, t=3, s=3 * 37, b=2, p_drop=0.25), 2, True),
            # float32 RMSNorm (dgamma only)
            (W.custom("f32_rms_h768", h=768, t=2, s=2 * 50, dtype="f32", norm="rmsnorm", p_drop=0.5), 1, False)]


@pytest.mark.parametrize("case,rank,with_dres", NO_DBIAS,
                         ids=[c if isinstance(c, str) else c.name for c, _, _ in NO_DBIAS])
def test_dropout_backward_without_dbias(cuda_device, case, rank, with_dres):
    """Without dbias, small shards take the one-launch backward (row blocks
    write dx and dpartial, column blocks sum dgamma/dbeta): dpartial and dx
    against the oracle, dgamma/dbeta bit for bit those of sp_region_bwd and
    of the two-launch path."""
    import torch
    w = W.BY_NAME[case] if isinstance(case, str) else case
    name = w.name
    log(f"[dropout-bwd no dbias] {name} rank={rank} dres={with_dres}")
    inp = inputs_for(w) if isinstance(case, str) else W.make_inputs(w)
    dres = None
    if with_dres:
        dres = W.make_inputs(W.custom(w.name + "_g", h=w.h, t=w.t, s=w.t * inp["T"], dtype=w.dtype, seed=98))["dy"]
    t = lambda a: W.as_torch(a, cuda_device)
    fo = spr.fwd(t(inp["partials"]), t(inp["gamma"]), t(inp["beta"]), bias=t(inp["bias"]),
                 residual=t(inp["residual"]), b=inp["b"], s=inp["s"], t=w.t, rank=rank, eps=w.eps, p_drop=w.p_drop,
                 seed=inp["seed"], norm=w.norm, cu_seqlens=inp["cu_seqlens"])
    dy, gamma = t(inp["dy"]), t(inp["gamma"])
    kw = dict(b=inp["b"], s=inp["s"], t=w.t, norm=w.norm, dres_in=t(dres))
    dkw = dict(kw, rank=rank, p_drop=w.p_drop, seed=inp["seed"], cu_seqlens=inp["cu_seqlens"], want_dbias=False)
    one = spr.bwd(dy, fo.z, fo.mean, fo.rstd, gamma, **kw)
    outs = {}
    try:
        for n in (1, 2):
            spr.set_bwd_launches(n)
            outs[n] = spr.bwd_dropout(dy, fo.z, fo.mean, fo.rstd, gamma, **dkw)
    finally:
        spr.set_bwd_launches(1)
    torch.cuda.synchronize()
    d = outs[1]
    assert d.dbias is None
    bits = lambda x: x.view(torch.int32 if x.dtype == torch.float32 else torch.int16).cpu()
    for k in ("dx", "dgamma", "dbeta"):
        a, b = getattr(one, k), getattr(d, k)
        assert (a is None) == (b is None), k
        if a is not None:
            assert torch.equal(bits(a), bits(b)), f"{k} differs from sp_region_bwd"
    for k in ("dx", "dpartial", "dgamma", "dbeta"):
        a, b = getattr(outs[2], k), getattr(d, k)
        if a is not None:
            assert torch.equal(bits(a), bits(b)), f"{k}: one launch against two"
    o = ref.region_forward(inp["partials"], t=w.t, rank=rank, dtype=w.dtype, norm=w.norm, eps=w.eps,
                           p_drop=w.p_drop, seed=inp["seed"], gamma=inp["gamma"], beta=inp["beta"],
                           bias=inp["bias"], residual=inp["residual"], cu_seqlens=inp["cu_seqlens"])
    ob = ref.region_backward(inp["dy"], o["z"], inp["gamma"], dtype=w.dtype, norm=w.norm, eps=w.eps, dres_in=dres)
    od = ref.dropout_backward(ob["dx"], t=w.t, rank=rank, p_drop=w.p_drop, seed=inp["seed"],
                              cu_seqlens=inp["cu_seqlens"])
    got = to_np_f64(d.dpartial)
    assert np.all(got[~od["keep"]] == 0.0), "dpartial nonzero where the forward dropped"
    assert_out_close(got, od["dpartial"], w.dtype, "dpartial", 4e-5)
    assert_out_close(to_np_f64(d.dx), ob["dx"], w.dtype, "dx", 3e-5)
    err = np.abs(to_np_f64(d.dgamma) - ob["dgamma"])
    assert np.all(err <= 1e-4 * ob["A"]), "dgamma"


EDGE = [
    # ragged shard with dropout on: the token index comes from cu_seqlens (scalar loads)
    (W.custom("ragged_drop", h=1024, t=4, lengths=(40, 0, 96, 8, 200), norm="layernorm", p_drop=0.3), 2, True),
    # odd t, 65 vectors per row (a partial wave), b = 2, extra gradient on z
    (W.custom("odd_t3_h520", h=520, t=3, s=3 * 37, b=2, p_drop=0.25), 1, True),
    # largest bf16 h: 4 vectors per thread (the register-heavy variant)
    (W.custom("hmax_bf16_t5", h=16384, t=5, s=5 * 16, p_drop=0.1), 4, True),
    # float32 RMSNorm, p = 0.5, no extra gradient
    (W.custom("f32_rms_p05", h=768, t=2, s=2 * 50, dtype="f32", norm="rmsnorm", p_drop=0.5), 1, False),
]


@pytest.mark.parametrize("w,rank,with_dres", EDGE, ids=[e[0].name for e in EDGE])
def test_edge_dropout_backward(cuda_device, w, rank, with_dres):
    log(f"[dropout-bwd-edge] {w.name} rank={rank} dres={with_dres}")
    inp = W.make_inputs(w)
    dres = None
    if with_dres:
        # a [T][h] gradient in the storage dtype (T rows of a uniform shard of the same width)
        dres = W.make_inputs(W.custom(w.name + "_g", h=w.h, t=w.t, s=w.t * inp["T"], dtype=w.dtype, seed=97))["dy"]
        assert dres.shape == (inp["T"], w.h)
    _, two = run_both(inp, w, rank, cuda_device, dres=dres)
    check(w, inp, rank, two, dres=dres)


def test_no_dropout_gives_dx(cuda_device):
    """p = 0: dpartial is dx's own bits (no mask, no scale)."""
    import torch
    w = W.BY_NAME["ragged13b"]
    inp = inputs_for(w)
    _, two = run_both(inp, w, 0, cuda_device, recommended_stride=False)
    assert w.p_drop == 0.0
    assert torch.equal(two.dx.view(torch.int16), two.dpartial.view(torch.int16))


def test_empty_shard_dropout_backward(cuda_device):
    import torch
    w = W.custom("empty", h=64, t=4, s=0)
    inp = W.make_inputs(w)
    t = lambda a: W.as_torch(a, cuda_device)
    z = torch.empty((0, 64), dtype=torch.bfloat16, device=cuda_device)
    st = torch.empty(0, device=cuda_device)
    out = spr.bwd_dropout(z, z, st, st, t(inp["gamma"]), b=1, s=0, t=4, rank=1, p_drop=0.2, seed=3)
    torch.cuda.synchronize()
    for g in (out.dgamma, out.dbeta, out.dbias):
        assert torch.all(g == 0)


def test_planned_buckets_end_to_end(cuda_device):
    """Host planning feeds the region: a mixed batch is bucketed at CV 0.15,
    each bucket that passes the gate is laid out for t = 4 (padded lengths,
    local cu_seqlens from the library), and the forward plus the dropout
    backward run on that layout match the oracle."""
    import torch
    from test_gpu_parity import compare, run_gpu
    lens = [37, 4096, 45, 3900, 41, 4200, 39, 4001, 0]
    order, starts = spr.bucket_by_tokens(lens)
    assert not spr.sp_gate(lens, 0.0) and len(starts) >= 3
    ran = 0
    for a, b in zip(starts, starts[1:]):
        bucket = [lens[i] for i in order[a:b]]
        if not spr.sp_gate(bucket, 0.05) or sum(bucket) == 0:
            continue
        padded, cu, T = spr.shard_layout(bucket, 4)
        w = W.custom(f"bucket{a}", h=512, t=4, lengths=tuple(padded), p_drop=0.2)
        inp = W.make_inputs(w)
        assert inp["T"] == T and [int(c) for c in inp["cu_seqlens"]] == cu
        log(f"[planned] bucket {bucket} -> T={T}")
        gpu = run_gpu(inp, w, 3, cuda_device)
        compare(w, inp, gpu, 3)
        _, two = run_both(inp, w, 3, cuda_device)
        check(w, inp, 3, two)
        torch.cuda.synchronize()
        ran += 1
    assert ran >= 2


@pytest.mark.parametrize("norm,slab_list", [("layernorm", False), ("rmsnorm", False), ("layernorm", True)])
def test_autograd_region_matches_torch_autograd(cuda_device, norm, slab_list):
    """spr.region under torch.autograd: the gradients of slabs, gamma, beta,
    bias and residual for loss = sum(y*gy) + sum(z*gz) against torch's own
    autograd in float64 on the CPU through the same forward (the oracle's
    keep mask, float32 scale).  slab_list: the slabs as t separate leaf
    tensors, each of which must receive its own gradient."""
    import torch
    import torch.nn.functional as F
    T, h, t, p, eps, seed = 24, 256, 3, 0.3, 1e-5, 0x1234
    rng = np.random.default_rng(21)
    P = rng.standard_normal((t, T, h)).astype(np.float32)
    res = rng.standard_normal((T, h)).astype(np.float32)
    bias = (0.1 * rng.standard_normal(h)).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, h).astype(np.float32)
    beta = (0.1 * rng.standard_normal(h)).astype(np.float32) if norm == "layernorm" else None
    gy = rng.standard_normal((T, h)).astype(np.float32)
    gz = rng.standard_normal((T, h)).astype(np.float32)
    keep = ref.region_forward(P, t=t, rank=1, dtype="f32", norm=norm, eps=eps, p_drop=p, seed=seed, gamma=gamma,
                              beta=beta, bias=bias, residual=res)["keep"]
    scale = float(ref.dropout_scale(p))

    c = lambda a: None if a is None else torch.from_numpy(a).double().requires_grad_(True)
    Pc, gc, bc, biasc, rc = c(P), c(gamma), c(beta), c(bias), c(res)
    acc = Pc.sum(0) + biasc
    z = rc + torch.where(torch.from_numpy(keep), acc * scale, torch.zeros_like(acc))
    if norm == "layernorm":
        y = F.layer_norm(z, (h,), gc, bc, eps)
    else:
        y = z * torch.rsqrt((z * z).mean(-1, keepdim=True) + eps) * gc
    (y * torch.from_numpy(gy).double()).sum().add((z * torch.from_numpy(gz).double()).sum()).backward()

    g = lambda a: None if a is None else torch.from_numpy(a).to(cuda_device).requires_grad_(True)
    Pg, gg, bg, biasg, rg = g(P), g(gamma), g(beta), g(bias), g(res)
    slabs = [g(np.ascontiguousarray(P[k])) for k in range(t)] if slab_list else None
    yg, zg = spr.region(slabs if slab_list else Pg, gg, bg, bias=biasg, residual=rg, b=1, s=t * T, t=t, rank=1,
                        eps=eps, p_drop=p, seed=seed, norm=norm)
    (yg * torch.from_numpy(gy).to(cuda_device)).sum().add((zg * torch.from_numpy(gz).to(cuda_device)).sum()).backward()
    torch.cuda.synchronize()
    if slab_list:
        assert Pg.grad is None
        Pg = type("Grads", (), {"grad": torch.stack([sk.grad for sk in slabs])})()
    for name, a, b in [("slabs", Pg, Pc), ("gamma", gg, gc), ("beta", bg, bc), ("bias", biasg, biasc),
                       ("residual", rg, rc)]:
        if a is None:
            continue
        got, want = a.grad.double().cpu(), b.grad
        tol = 1e-4 * max(1.0, float(want.abs().max()))
        assert float((got - want).abs().max()) <= tol, f"{name}: {float((got - want).abs().max()):.3e} > {tol:.3e}"
