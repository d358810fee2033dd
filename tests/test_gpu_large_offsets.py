"""Shards whose tensors exceed 4 GiB: every byte offset past 2^32 must be
formed in 64 bits (row offsets, slab offsets, the mask and the dropout
backward's outputs).

One uniform shard of T = 150000 rows at the widest bf16 h (16384), t = 2,
rank 1, dropout on: each [T][h] tensor is 4.9 GB, and slab 1 starts 4.9 GB
into the contiguous partials.  Inputs are drawn on the GPU (seeded); the
oracle runs on sampled rows, including both sides of the 4 GiB row boundary
(row 131072), which it reads back one by one: z bit-exact, the mask exact,
y / mean / rstd / dx / dpartial at the usual bars.  dbeta is checked at every
column against the float64 column sums of dy.
"""
import numpy as np
import pytest

import layernorm_sp_region_amd as spr
import oracle.region as ref
import workloads as W
from test_gpu_parity import assert_out_close, log, to_np_bits, to_np_f64

pytestmark = pytest.mark.gpu

T, H, TP, RANK, P_DROP, SEED, EPS = 150000, 16384, 2, 1, 0.1, 0x5EED0042, 1e-5


class _Rows:
    """A [T][h] device tensor as the oracle indexes it: x[r] copies rows r to
    the host (as storage bits)."""

    def __init__(self, x):
        self.x = x
        self.shape = tuple(x.shape)

    def __getitem__(self, r):
        import torch
        return to_np_bits(self.x[torch.as_tensor(np.asarray(r), device=self.x.device)])


class _Slabs:
    def __init__(self, p):
        self.p = p
        self.shape = tuple(p.shape)

    def __getitem__(self, k):
        return _Rows(self.p[k])


def test_tensors_beyond_4gib(cuda_device):
    import torch
    log(f"[large] T={T} h={H} t={TP}: {T * H * 2 / 2**30:.2f} GiB per [T][h] tensor")
    assert T * H * 2 > 2**32 and 131072 * H * 2 == 2**32
    P = W.device_normal((TP, T, H), seed=1, device=cuda_device, scale=float(np.sqrt(1 / 8)))
    res = W.device_normal((1, T, H), seed=2, device=cuda_device)[0]
    dy = W.device_normal((1, T, H), seed=3, device=cuda_device)[0]
    rng = np.random.default_rng(4)
    gamma = W._to_storage(rng.uniform(0.5, 1.5, size=H), "bf16")
    beta = W._to_storage(0.1 * rng.standard_normal(H), "bf16")
    bias = W._to_storage(0.02 * rng.standard_normal(H), "bf16")
    t = lambda a: W.as_torch(a, cuda_device)
    kw = dict(b=1, s=TP * T, t=TP, norm="layernorm")
    fo = spr.fwd(P, t(gamma), t(beta), bias=t(bias), residual=res, rank=RANK, eps=EPS, p_drop=P_DROP, seed=SEED,
                 return_mask=True, **kw)
    bo = spr.bwd_dropout(dy, fo.z, fo.mean, fo.rstd, t(gamma), rank=RANK, p_drop=P_DROP, seed=SEED, **kw)
    torch.cuda.synchronize()
    log("  kernels done")

    rows = np.unique(np.concatenate([[0, 1, 131071, 131072, 131073, T - 1],
                                     np.random.default_rng(5).integers(0, T, 26)]))
    o = ref.region_forward(_Slabs(P), t=TP, rank=RANK, dtype="bf16", norm="layernorm", eps=EPS, p_drop=P_DROP,
                           seed=SEED, gamma=gamma, beta=beta, bias=bias, residual=_Rows(res), rows=rows)
    ri = torch.as_tensor(rows, device=cuda_device)
    assert np.array_equal(to_np_bits(fo.z[ri]), o["z"]), "z differs from the oracle"
    assert np.array_equal(fo.mask[ri].cpu().numpy().astype(bool), o["keep"]), "mask differs"
    assert_out_close(to_np_f64(fo.y[ri]), o["y"], "bf16", "y", 1e-5)
    assert np.all(np.abs(to_np_f64(fo.rstd[ri]) - o["rstd"]) <= 1e-4 * o["rstd"]), "rstd"
    zabs = np.abs(o["z32"].astype(np.float64)).mean(axis=1)
    assert np.all(np.abs(to_np_f64(fo.mean[ri]) - o["mean"]) <= 1e-4 * zabs), "mean"

    dy_rows = to_np_bits(dy[ri])
    ob = ref.region_backward(dy_rows, o["z"], gamma, dtype="bf16", norm="layernorm", eps=EPS,
                             with_param_grads=False)
    assert_out_close(to_np_f64(bo.dx[ri]), ob["dx"], "bf16", "dx", 3e-5)
    od = ref.dropout_backward(ob["dx"], t=TP, rank=RANK, p_drop=P_DROP, seed=SEED, T=T, rows=rows)
    got = to_np_f64(bo.dpartial[ri])
    assert np.all(got[~od["keep"]] == 0.0), "dpartial nonzero where the forward dropped"
    assert_out_close(got, od["dpartial"], "bf16", "dpartial", 4e-5)
    log(f"  {len(rows)} sampled rows match the oracle (z bit-exact)")

    # dbeta_j = sum_i dy_ij: float64 column sums of the input, in row chunks
    ref_db = torch.zeros(H, dtype=torch.float64, device=cuda_device)
    ref_B = torch.zeros(H, dtype=torch.float64, device=cuda_device)
    for a in range(0, T, 16384):
        c = dy[a:a + 16384].double()
        ref_db += c.sum(0)
        ref_B += c.abs().sum(0)
    err = (bo.dbeta.double() - ref_db).abs()
    assert bool((err <= 1e-4 * ref_B).all()), f"dbeta: worst err/B {float((err / ref_B).max()):.2e}"
    log(f"  dbeta ok: worst err/B {float((err / ref_B).max()):.2e}")
    del P, res, dy, fo, bo
    torch.cuda.empty_cache()
