"""GPU parity of the accumulating backward (sp_region_bwd_accumulate): the
parameter gradients are added into float32 main-grad buffers.

Bars: every accumulated element is, bit for bit, float32(old + sum) with sum
what the overwriting call (sp_region_bwd_dropout, or sp_region_bwd without
dpartial) writes on the same inputs, and dx / dpartial are that call's bits.
Against the oracle's accumulate_param_grads over its float64 sums, each
element is within 1e-4 of the sum's conditioning scale (A_j, B_j, C_j as in
the other backward tests) plus a float32 rounding of the result.
"""
import numpy as np
import pytest

import layernorm_sp_region_amd as spr
import oracle.region as ref
import workloads as W
from test_gpu_parity import inputs_for, log, to_np_f64

pytestmark = pytest.mark.gpu

NAMES = ("dgamma", "dbeta", "dbias")


def _bits(x):
    import torch
    return x.view(torch.int32 if x.dtype == torch.float32 else torch.int16).cpu()


def _main_buffers(h, device, seed):
    """Seeded float32 main gradients, with signed zeros among them."""
    import torch
    rng = np.random.default_rng(seed)
    out = {}
    for k in NAMES:
        v = (rng.standard_normal(h) * 10.0).astype(np.float32)
        v[:3] = np.array([0.0, -0.0, 1e-30], dtype=np.float32)
        out[k] = torch.from_numpy(v).to(device)
    return out


def _forward(inp, w, rank, device, gamma=None):
    t = lambda a: W.as_torch(a, device)
    g = t(inp["gamma"]) if gamma is None else gamma
    fo = spr.fwd(t(inp["partials"]), g, t(inp["beta"]), bias=t(inp["bias"]), residual=t(inp["residual"]),
                 b=inp["b"], s=inp["s"], t=w.t, rank=rank, eps=w.eps, p_drop=w.p_drop, seed=inp["seed"],
                 norm=w.norm, cu_seqlens=inp["cu_seqlens"])
    return fo, g


def _oracle_sums(inp, w, rank, gamma_np=None):
    gamma = inp["gamma"] if gamma_np is None else gamma_np
    o = ref.region_forward(inp["partials"], t=w.t, rank=rank, dtype=w.dtype, norm=w.norm, eps=w.eps,
                           p_drop=w.p_drop, seed=inp["seed"], gamma=gamma, beta=inp["beta"], bias=inp["bias"],
                           residual=inp["residual"], cu_seqlens=inp["cu_seqlens"])
    ob = ref.region_backward(inp["dy"], o["z"], gamma, dtype=w.dtype, norm=w.norm, eps=w.eps)
    od = ref.dropout_backward(ob["dx"], t=w.t, rank=rank, p_drop=w.p_drop, seed=inp["seed"],
                              cu_seqlens=inp["cu_seqlens"])
    sums = dict(dgamma=ob["dgamma"], dbeta=ob["dbeta"], dbias=od["dbias"])
    scales = dict(dgamma=ob["A"], dbeta=ob["B"], dbias=od["C"])
    return sums, scales


def _check_against_oracle(got, main0, sums, scales, what):
    """got, main0: dicts of [h] arrays; sums/scales: the oracle's float64 sums."""
    for k in got:
        if got[k] is None:
            continue
        want = ref.accumulate_param_grads({k: main0[k]}, {k: sums[k]})[k]
        err = np.abs(to_np_f64(got[k]) - want)
        bound = 1e-4 * scales[k] + 2.0 ** -23 * np.abs(want)
        assert np.all(err <= bound), f"{what} {k}: worst err/bound {np.max(err / np.maximum(bound, 1e-300)):.2e}"


@pytest.mark.parametrize("name,rank,through_dropout", [("tiny", 1, True), ("page_demo", 6, True),
                                                       ("ragged13b", 2, True), ("page_demo", 0, False),
                                                       ("shard70b", 0, True)])
def test_accumulate_equals_overwrite_plus_main(cuda_device, name, rank, through_dropout):
    import torch
    w = W.BY_NAME[name]
    log(f"[accumulate] {name} rank={rank} through_dropout={through_dropout}")
    inp = inputs_for(w)
    fo, gamma = _forward(inp, w, rank, cuda_device)
    dy = W.as_torch(inp["dy"], cuda_device)
    kw = dict(b=inp["b"], s=inp["s"], t=w.t, norm=w.norm)
    ln = w.norm == "layernorm"
    main0 = _main_buffers(w.h, cuda_device, seed=11)
    if through_dropout:
        dkw = dict(kw, rank=rank, p_drop=w.p_drop, seed=inp["seed"], cu_seqlens=inp["cu_seqlens"])
        over = spr.bwd_dropout(dy, fo.z, fo.mean, fo.rstd, gamma, **dkw)
        acc_out = spr.BwdDropoutOut(torch.empty_like(over.dx), torch.empty_like(over.dpartial),
                                    main0["dgamma"].clone(), main0["dbeta"].clone() if ln else None,
                                    main0["dbias"].clone())
        acc = spr.bwd_dropout(dy, fo.z, fo.mean, fo.rstd, gamma, **dkw, out=acc_out, accumulate=True)
        acts = ("dx", "dpartial")
    else:
        over = spr.bwd(dy, fo.z, fo.mean, fo.rstd, gamma, **kw)
        acc_out = spr.BwdOut(torch.empty_like(over.dx), main0["dgamma"].clone(),
                             main0["dbeta"].clone() if ln else None)
        acc = spr.bwd(dy, fo.z, fo.mean, fo.rstd, gamma, **kw, out=acc_out, accumulate=True)
        acts = ("dx",)
    torch.cuda.synchronize()
    for a in acts:
        assert torch.equal(_bits(getattr(acc, a)), _bits(getattr(over, a))), f"{a} differs from the overwriting call"
    got = {}
    for k in NAMES:
        if not hasattr(acc, k) or getattr(acc, k) is None:
            continue
        want = main0[k] + getattr(over, k)         # one IEEE float32 addition
        assert torch.equal(_bits(getattr(acc, k)), _bits(want)), f"{k} is not float32(old + sum)"
        got[k] = getattr(acc, k)
    sums, scales = _oracle_sums(inp, w, rank)
    _check_against_oracle(got, {k: main0[k].cpu().numpy() for k in got}, sums, scales, name)
    log(f"  accumulate ok: {sorted(got)}")


def test_micro_batches_accumulate(cuda_device):
    """Three micro-batches of different lengths (one of a single row, one
    ragged) sharing gamma: the buffers after three accumulating calls match
    the oracle's accumulation of the three backward passes."""
    import torch
    h, t, rank = 1032, 4, 3
    mbs = [W.custom("mb0", h=h, t=t, s=t * 37, b=2, p_drop=0.2, seed=21),
           W.custom("mb1", h=h, t=t, s=t, p_drop=0.2, seed=22),
           W.custom("mb2", h=h, t=t, lengths=(64, 0, 12, 100), p_drop=0.2, seed=23)]
    inps = [W.make_inputs(w) for w in mbs]
    gamma_np = inps[0]["gamma"]
    gamma = W.as_torch(gamma_np, cuda_device)
    main0 = _main_buffers(h, cuda_device, seed=12)
    bufs = {k: main0[k].clone() for k in NAMES}
    want = {k: main0[k].cpu().numpy() for k in NAMES}
    scale = {k: np.zeros(h) for k in NAMES}
    for w, inp in zip(mbs, inps):
        log(f"[accumulate] micro-batch {w.name}: T={inp['T']}")
        fo, _ = _forward(inp, w, rank, cuda_device, gamma=gamma)
        dy = W.as_torch(inp["dy"], cuda_device)
        out = spr.BwdDropoutOut(torch.empty_like(fo.z), torch.empty_like(fo.z), bufs["dgamma"], bufs["dbeta"],
                                bufs["dbias"])
        spr.bwd_dropout(dy, fo.z, fo.mean, fo.rstd, gamma, b=inp["b"], s=inp["s"], t=t, rank=rank,
                        p_drop=w.p_drop, seed=inp["seed"], cu_seqlens=inp["cu_seqlens"], out=out, accumulate=True)
        sums, scales = _oracle_sums(inp, w, rank, gamma_np=gamma_np)
        want = ref.accumulate_param_grads(want, sums)
        for k in NAMES:
            scale[k] += scales[k]
    torch.cuda.synchronize()
    for k in NAMES:
        err = np.abs(to_np_f64(bufs[k]) - want[k])
        # three float32 roundings of the running buffer, plus the sums' own bound
        bound = 1e-4 * scale[k] + 3 * 2.0 ** -23 * (np.abs(want[k]) + np.abs(main0[k].cpu().numpy()) + scale[k])
        assert np.all(err <= bound), f"{k}: worst err/bound {np.max(err / np.maximum(bound, 1e-300)):.2e}"


def test_empty_micro_batch_leaves_buffers(cuda_device):
    """T = 0 adds nothing: the buffers keep their bits, signed zeros included."""
    import torch
    h = 64
    main0 = _main_buffers(h, cuda_device, seed=13)
    bufs = {k: main0[k].clone() for k in NAMES}
    z = torch.empty((0, h), dtype=torch.bfloat16, device=cuda_device)
    st = torch.empty(0, device=cuda_device)
    gamma = torch.ones(h, dtype=torch.bfloat16, device=cuda_device)
    spr.bwd_dropout(z, z, st, st, gamma, b=1, s=0, t=4, rank=1, p_drop=0.2, seed=3, accumulate=True,
                    out=spr.BwdDropoutOut(z, z, bufs["dgamma"], bufs["dbeta"], bufs["dbias"]))
    spr.bwd(z, z, st, st, gamma, b=1, s=0, t=4, accumulate=True, out=spr.BwdOut(z, bufs["dgamma"], bufs["dbeta"]))
    torch.cuda.synchronize()
    for k in NAMES:
        assert torch.equal(_bits(bufs[k]), _bits(main0[k])), k
