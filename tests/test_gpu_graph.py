"""The region's entry points inside a captured HIP graph.

The library launches only kernels on the caller's stream -- no allocation,
no synchronisation, no memset -- so a caller can capture a whole forward +
backward step in a graph (torch.cuda.graph drives hipStreamBeginCapture) and
replay it without per-launch host work.  Each replay must reproduce the eager
call bit for bit (every kernel here is deterministic); eager work (zeroing
every output) runs between replays.
"""
import pytest

import layernorm_sp_region_amd as spr
import workloads as W
from test_gpu_parity import log

pytestmark = pytest.mark.gpu


def _bits(x):
    import torch
    return x.view(torch.int32 if x.dtype == torch.float32 else torch.int16).clone()


@pytest.mark.parametrize("name", ["page_demo", "shard70b"])
def test_captured_step_replays_bit_exact(cuda_device, name):
    import torch
    w = W.BY_NAME[name]
    log(f"[graph] {name}")
    inp = W.make_inputs(w)
    T, h = inp["T"], w.h
    t = lambda a: W.as_torch(a, cuda_device)
    P = spr.empty_partials(w.t, T, h, torch.bfloat16, cuda_device)
    P.copy_(t(inp["partials"]))
    gamma, beta, bias, res, dy = t(inp["gamma"]), t(inp["beta"]), t(inp["bias"]), t(inp["residual"]), t(inp["dy"])
    ln = w.norm == "layernorm"
    dt = gamma.dtype
    E = lambda *s, d=dt: torch.empty(s, dtype=d, device=cuda_device)
    fo = spr.FwdOut(E(T, h), E(T, h), E(T, d=torch.float32) if ln else None, E(T, d=torch.float32), None)
    bo = spr.BwdOut(E(T, h), E(h, d=torch.float32), E(h, d=torch.float32) if ln else None)
    do = spr.BwdDropoutOut(E(T, h), E(T, h), E(h, d=torch.float32), E(h, d=torch.float32) if ln else None,
                           E(h, d=torch.float32))
    ws = torch.empty(max(16, spr.dropout_workspace_bytes(T, h)), dtype=torch.uint8, device=cuda_device)
    kw = dict(b=inp["b"], s=inp["s"], t=w.t, norm=w.norm)

    def step():
        spr.fwd(P, gamma, beta, bias=bias, residual=res, rank=1, eps=w.eps, p_drop=w.p_drop, seed=inp["seed"],
                out=fo, **kw)
        spr.bwd(dy, fo.z, fo.mean, fo.rstd, gamma, workspace=ws, out=bo, **kw)
        spr.bwd_dropout(dy, fo.z, fo.mean, fo.rstd, gamma, rank=1, p_drop=w.p_drop, seed=inp["seed"],
                        workspace=ws, out=do, **kw)

    outs = [x for x in (*fo[:4], *bo, *do) if x is not None]
    step()
    torch.cuda.synchronize()
    eager = [_bits(x) for x in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                      # warm-up on the capture stream's side, as torch.cuda.graph expects
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for x in outs:
            x.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (x, ref) in enumerate(zip(outs, eager)):
            assert torch.equal(_bits(x), ref), f"replay {rep}: output {i} differs from the eager call"
    log(f"  {len(outs)} outputs bit-exact over 3 replays")
