"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bars (per element):
  * z and the dropout mask: bit-exact.
  * bf16 y, dx: |err| <= 2e-2 for |ref| < 8, else half a bf16 ulp of ref +
    1e-3 (no bf16 output can be closer than half an ulp, which exceeds 2e-2
    from |ref| = 8 up); and a tighter derived bound: half a bf16 ulp of
    (|ref| + fp32 slack) + fp32 slack, slack = 1e-5*(1+|ref|) for y and
    3e-5*(1+|ref|) for dx.
  * float32 y, dx (fp32 shards): |err| <= 1e-4 * max(1, |ref|).
  * Rows whose mean is large against their spread (|mean| * rstd = kappa > 1)
    are ill-conditioned in float32: the statistics are float32, so z - mean
    carries an error of order u*|mean|, i.e. u*kappa relative to the row's
    spread.  For such rows (the hard-row tests) the float32 slacks above --
    the derived bf16 slack and the float32 bar -- scale by kappa.
  * rstd: relative 1e-4.  mean: |err| <= 1e-4 * mean_j|z_ij| (the mean of a
    zero-centred row cancels, so a relative bound on it is meaningless).
  * dgamma_j: |err| <= 1e-4 * sum_i|dy_ij xhat_ij|; dbeta_j: |err| <= 1e-4 *
    sum_i|dy_ij| (condition-scaled: both are sums of signed terms).
References are float64 and unrounded.
"""
import sys
import time

import numpy as np
import pytest

import layernorm_sp_region_amd as spr
import oracle.region as ref
import workloads as W
from oracle.bf16 import bf16_ulp

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_np_bits(x):
    import torch
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).cpu().numpy().view(np.uint16)
    return x.cpu().numpy()


def to_np_f64(x):
    return x.float().cpu().numpy().astype(np.float64)


def run_gpu(inp, w, rank, device, dres=None, padded_slabs=0, return_mask=True, recommended_stride=False):
    import torch
    t = lambda a: W.as_torch(a, device)
    P = inp["partials"]
    if recommended_stride:
        Pc = t(P)
        Pt = spr.empty_partials(P.shape[0], P.shape[1], P.shape[2], Pc.dtype, device)
        Pt.copy_(Pc)
        assert Pt.stride(0) == spr.partials_stride(P.shape[1], P.shape[2], Pc.dtype) > P.shape[1] * P.shape[2]
        del Pc
    elif padded_slabs:
        Pp = np.zeros((P.shape[0], P.shape[1] + padded_slabs, P.shape[2]), dtype=P.dtype)
        Pp[:, :P.shape[1]] = P
        Pt = t(Pp)[:, :P.shape[1], :]
    else:
        Pt = t(P)
    out = spr.fwd(Pt, t(inp["gamma"]), t(inp["beta"]), bias=t(inp["bias"]), residual=t(inp["residual"]),
                  b=inp["b"], s=inp["s"], t=w.t, rank=rank, eps=w.eps, p_drop=w.p_drop, seed=inp["seed"],
                  norm=w.norm, cu_seqlens=inp["cu_seqlens"], return_mask=return_mask)
    g = spr.bwd(t(inp["dy"]), out.z, out.mean, out.rstd, t(inp["gamma"]), b=inp["b"], s=inp["s"], t=w.t,
                norm=w.norm, dres_in=t(dres))
    torch.cuda.synchronize()
    return dict(z=to_np_bits(out.z), y=to_np_f64(out.y), mean=None if out.mean is None else to_np_f64(out.mean),
                rstd=to_np_f64(out.rstd), mask=None if out.mask is None else out.mask.cpu().numpy(),
                dx=to_np_f64(g.dx), dgamma=to_np_f64(g.dgamma), dbeta=None if g.dbeta is None else to_np_f64(g.dbeta))


def assert_out_close(got, want, dtype, what, slack, kappa=1.0):
    """kappa: per-row conditioning factor (a [rows][1] array or 1)."""
    err = np.abs(got - want)
    a = np.abs(want)
    if dtype == "f32":
        bound = 1e-4 * np.maximum(1.0, a) * kappa
        assert np.all(err <= bound), f"{what}: max err {err.max():.3e}"
        return
    stated = np.where(a < 8, 2e-2, 0.5 * bf16_ulp(want) + 1e-3)
    bad = err > stated
    assert not bad.any(), f"{what}: {bad.sum()} elements beyond the stated bound, max err {err.max():.3e}"
    sl = slack * (1.0 + a) * kappa
    tight = 0.5 * bf16_ulp(a + sl) + sl
    bad = err > tight
    assert not bad.any(), f"{what}: {bad.sum()} elements beyond half-ulp + fp32 slack, worst {err[bad].max():.3e}"


def compare(w, inp, gpu, rank, rows=None, dres=None, conditioned=False):
    """Oracle on the same inputs; rows (optional) restricts the per-row checks
    of y/dx to a sample, while z, the mask, the statistics and dgamma/dbeta
    are checked in full.  conditioned: scale the float32 slacks of each row
    by kappa = max(1, |mean|*rstd) (LayerNorm).  Returns the oracle's forward
    and backward results."""
    t0 = time.time()
    o = ref.region_forward(inp["partials"], t=w.t, rank=rank, dtype=w.dtype, norm=w.norm, eps=w.eps,
                           p_drop=w.p_drop, seed=inp["seed"], gamma=inp["gamma"], beta=inp["beta"],
                           bias=inp["bias"], residual=inp["residual"], cu_seqlens=inp["cu_seqlens"])
    z_bits = gpu["z"] if w.dtype == "bf16" else gpu["z"].view(np.uint32)
    o_bits = o["z"] if w.dtype == "bf16" else o["z"].view(np.uint32)
    nbad = int(np.sum(z_bits != o_bits))
    assert nbad == 0, f"z: {nbad} elements differ from the oracle"
    if gpu["mask"] is not None:
        assert np.array_equal(gpu["mask"].astype(bool), o["keep"]), "dropout mask differs"
    r = slice(None) if rows is None else rows
    kappa = 1.0
    if conditioned and w.norm == "layernorm":
        kappa = np.maximum(1.0, np.abs(o["mean"]) * o["rstd"])[r, None]
    assert_out_close(gpu["y"][r], o["y"][r], w.dtype, "y", 1e-5, kappa)
    assert np.all(np.abs(gpu["rstd"] - o["rstd"]) <= 1e-4 * o["rstd"]), "rstd"
    if w.norm == "layernorm":
        zabs = np.abs(o["z32"].astype(np.float64)).mean(axis=1)
        assert np.all(np.abs(gpu["mean"] - o["mean"]) <= 1e-4 * zabs), "mean"
    else:
        assert gpu["mean"] is None
    ob = ref.region_backward(inp["dy"], o["z"], inp["gamma"], dtype=w.dtype, norm=w.norm, eps=w.eps, dres_in=dres)
    assert_out_close(gpu["dx"][r], ob["dx"][r], w.dtype, "dx", 3e-5, kappa)
    assert np.all(np.abs(gpu["dgamma"] - ob["dgamma"]) <= 1e-4 * ob["A"]), "dgamma"
    if w.norm == "layernorm":
        assert np.all(np.abs(gpu["dbeta"] - ob["dbeta"]) <= 1e-4 * ob["B"]), "dbeta"
    else:
        assert gpu["dbeta"] is None
    dg_rel = float(np.max(np.abs(gpu["dgamma"] - ob["dgamma"]) / np.maximum(ob["A"], 1e-300))) if len(ob["A"]) else 0.0
    log(f"  oracle compare ok ({time.time() - t0:.1f}s): dgamma err/A max {dg_rel:.2e}")
    return o, ob


_INPUTS = {}


def inputs_for(w):
    if w.name not in _INPUTS:
        _INPUTS.clear()      # keep at most one large input set alive
        t0 = time.time()
        _INPUTS[w.name] = W.make_inputs(w)
        log(f"  inputs {w.name}: T={_INPUTS[w.name]['T']} h={w.h} t={w.t} ({time.time() - t0:.1f}s)")
    return _INPUTS[w.name]


# Each workload at the first and last rank; the slabs contiguous or at the
# recommended stride (the layout the benchmark times); the forward with the
# debug mask output (a separate kernel instantiation) and without it (the
# one the benchmark, region() and every mask-free caller run: its z must be
# bit-exact and its y/statistics within the bars on its own).
@pytest.mark.parametrize("name,rank,layout,mask", [
    ("tiny", 0, "contiguous", True), ("tiny", 3, "recommended", False),
    ("page_demo", 0, "recommended", False), ("page_demo", 7, "contiguous", True),
    ("shard70b", 0, "recommended", False), ("shard70b", 7, "contiguous", True),
    ("ragged13b", 0, "recommended", False), ("ragged13b", 7, "contiguous", True)])
def test_workload_parity(cuda_device, name, rank, layout, mask):
    w = W.BY_NAME[name]
    log(f"[parity] {name} rank={rank} slabs={layout} mask={mask}")
    inp = inputs_for(w)
    gpu = run_gpu(inp, w, rank, cuda_device, recommended_stride=layout == "recommended", return_mask=mask)
    assert (gpu["mask"] is None) == (not mask)
    compare(w, inp, gpu, rank)


def test_long_context_parity_sampled_rows(cuda_device):
    """The 128K-token shard (16384 rows, 2.1 GB of slabs), at the recommended
    slab stride with the mask-free forward the benchmark runs: z, statistics
    and dgamma/dbeta in full, y and dx on 64 sampled rows."""
    w = W.BY_NAME["long128k"]
    log("[parity] long128k rank=0 slabs=recommended mask=False")
    inp = inputs_for(w)
    gpu = run_gpu(inp, w, 0, cuda_device, recommended_stride=True, return_mask=False)
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, 1, inp["T"] // 2, inp["T"] - 1], rng.integers(0, inp["T"], 60)]))
    compare(w, inp, gpu, 0, rows=rows)
    _INPUTS.clear()


@pytest.mark.parametrize("h,T,dtype", [(16384, 4112, "bf16"), (4096, 8200, "f32")])
def test_streamed_y_on_large_outputs(cuda_device, h, T, dtype):
    """A shard whose z and y together pass 256 MB takes the forward variant
    that stores y nontemporally (bf16 at the widest h: two waves per row;
    float32 at h = 4096: one wave of 16 slots): z bit-exact and y/statistics
    within the bars on sampled rows against the oracle, and z/y bit for bit
    those of the mask-writing variant (ordinary stores) on every row."""
    import torch
    w = W.custom(f"h{h}_t2_{dtype}_streamed_y", h=h, t=2, s=2 * T, p_drop=0.1, dtype=dtype)
    assert 2 * T * h * (2 if dtype == "bf16" else 4) > 256 << 20
    log(f"[parity] {w.name} rank=1 mask=False (streamed y) and mask=True")
    inp = inputs_for(w)
    gpu = run_gpu(inp, w, 1, cuda_device, return_mask=False)
    rng = np.random.default_rng(12)
    rows = np.unique(np.concatenate([[0, 1, inp["T"] // 2, inp["T"] - 1], rng.integers(0, inp["T"], 28)]))
    compare(w, inp, gpu, 1, rows=rows)
    ref_gpu = run_gpu(inp, w, 1, cuda_device, return_mask=True)
    assert np.array_equal(gpu["z"], ref_gpu["z"])
    assert np.array_equal(gpu["y"], ref_gpu["y"])
    torch.cuda.empty_cache()
    _INPUTS.clear()


EDGE = [
    # odd t, a partial last wave of vectors (h = 520 bf16 -> 65 vectors), b > 1
    (W.custom("odd_t3_h520", h=520, t=3, s=3 * 37, b=2, p_drop=0.25), 2, {}),
    # t = 1 (no reduction), one vector per row, fp32, RMSNorm, p = 0.5
    (W.custom("t1_h4_f32_rms", h=4, t=1, s=5, dtype="f32", norm="rmsnorm", p_drop=0.5, bias=False), 0, {}),
    # largest bf16 h (16384): 4 vectors per thread forward, 2 per thread backward
    (W.custom("hmax_bf16_t5", h=16384, t=5, s=5 * 16, p_drop=0.1), 4, {}),
    # largest fp32 h (8192), t = 7, no dropout, no bias
    (W.custom("hmax_f32_t7", h=8192, t=7, s=7 * 12, dtype="f32", p_drop=0.0, bias=False), 6, {}),
    # packed ragged batch with an empty sequence and dropout on
    (W.custom("ragged_empty_seq", h=64, t=8, lengths=(16, 0, 40, 8), norm="rmsnorm", p_drop=0.3,
              bias=False, residual=False), 5, {}),
    # padded slab stride and an extra residual-stream gradient
    (W.custom("padded_slabs_dres", h=256, t=4, s=4 * 33, p_drop=0.2), 1, dict(padded=5, dres=True)),
    # 257 vectors per row: 8 slots per lane of LDS-resident z, all but one vector of the last 4 clamped
    (W.custom("h2056_257vec", h=2056, t=2, s=2 * 40, p_drop=0.15), 1, {}),
    # t = 6, h = 5120 (the ragged workload's width) uniform, LayerNorm without beta
    (W.custom("t6_h5120_nobeta", h=5120, t=6, s=6 * 20, p_drop=0.1, beta=False), 3, {}),
]


@pytest.mark.parametrize("w,rank,opt", EDGE, ids=[e[0].name for e in EDGE])
def test_edge_case_parity(cuda_device, w, rank, opt):
    log(f"[parity-edge] {w.name} rank={rank} {opt}")
    inp = W.make_inputs(w)
    dres = None
    if opt.get("dres"):
        dres = W.make_inputs(W.custom(w.name + "_dres", h=w.h, t=w.t, s=w.s, b=w.b, dtype=w.dtype, seed=99))["dy"]
    gpu = run_gpu(inp, w, rank, cuda_device, dres=dres, padded_slabs=opt.get("padded", 0))
    compare(w, inp, gpu, rank, dres=dres)


def test_empty_shard(cuda_device):
    import torch
    w = W.custom("empty", h=64, t=4, s=0)
    inp = W.make_inputs(w)
    t = lambda a: W.as_torch(a, cuda_device)
    out = spr.fwd(t(inp["partials"]), t(inp["gamma"]), t(inp["beta"]), bias=t(inp["bias"]),
                  residual=t(inp["residual"]), b=1, s=0, t=4, rank=0, eps=1e-5, p_drop=0.1, seed=1)
    assert out.z.shape == (0, 64)
    g = spr.bwd(t(inp["dy"]), out.z, out.mean, out.rstd, t(inp["gamma"]), b=1, s=0, t=4)
    torch.cuda.synchronize()
    assert torch.all(g.dgamma == 0) and torch.all(g.dbeta == 0)


def test_bitwise_reproducible(cuda_device):
    w = W.BY_NAME["page_demo"]
    inp = inputs_for(w)
    a = run_gpu(inp, w, 3, cuda_device)
    b = run_gpu(inp, w, 3, cuda_device)
    for k in ("z", "y", "mean", "rstd", "mask", "dx", "dgamma", "dbeta"):
        assert np.array_equal(a[k], b[k]), k


def test_time_next_call_stamps_one_call(cuda_device):
    """The profiling hook stamps the next region call's kernel start/end from
    the dispatch packets and then clears itself: a later call leaves the
    events alone."""
    import torch
    w = W.BY_NAME["page_demo"]
    inp = inputs_for(w)
    t = lambda a: W.as_torch(a, cuda_device)
    P, g, be, res = t(inp["partials"]), t(inp["gamma"]), t(inp["beta"]), t(inp["residual"])
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for e in ev:
        e.record()
    kw = dict(b=inp["b"], s=inp["s"], t=w.t, rank=0, eps=w.eps, p_drop=w.p_drop, seed=inp["seed"], norm=w.norm)
    spr.time_next_call(ev[0], ev[1])
    spr.fwd(P, g, be, residual=res, **kw)
    torch.cuda.synchronize()
    first = ev[0].elapsed_time(ev[1])
    assert 0.0 < first < 50.0, first             # one forward of a 512-row shard: microseconds
    spr.fwd(P, g, be, residual=res, **kw)        # hook cleared: events keep their stamps
    torch.cuda.synchronize()
    assert ev[0].elapsed_time(ev[1]) == first
    with pytest.raises(spr.SpRegionError):
        spr.time_next_call(ev[0], None)


def test_ranks_tile_unsharded_mask(cuda_device):
    """On the GPU, per-rank masks of a uniform shard tile the t = 1 mask of the
    whole sequence (same seed, global token index)."""
    import torch
    h, t, T = 256, 4, 24
    wr = W.custom("tile", h=h, t=t, s=t * T, p_drop=0.4, bias=False)
    inp = W.make_inputs(wr)
    tt = lambda a: W.as_torch(a, cuda_device)
    masks = []
    for r in range(t):
        o = spr.fwd(tt(inp["partials"]), tt(inp["gamma"]), tt(inp["beta"]), residual=tt(inp["residual"]),
                    b=1, s=t * T, t=t, rank=r, eps=1e-5, p_drop=0.4, seed=inp["seed"], return_mask=True)
        masks.append(o.mask)
    full_P = np.concatenate([inp["partials"][0]] * t)[None]
    full_res = np.concatenate([inp["residual"]] * t)
    o1 = spr.fwd(tt(full_P), tt(inp["gamma"]), tt(inp["beta"]), residual=tt(full_res), b=1, s=t * T, t=1,
                 rank=0, eps=1e-5, p_drop=0.4, seed=inp["seed"], return_mask=True)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(masks), o1.mask)


def test_oracle_philox_matches_rocrand_host_generator(cuda_device):
    """Library pin of the oracle's Philox-4x32-10 constants: rocRAND's host
    PHILOX4_32_10 generator (it needs a HIP device present, hence here) must
    produce the oracle's words for counters 0, 1, 2, ... under key = seed."""
    import ctypes
    from oracle.philox import philox4x32_10
    lib = ctypes.CDLL("librocrand.so")
    gen = ctypes.c_void_p()
    assert lib.rocrand_create_generator_host_blocking(ctypes.byref(gen), 404) == 0   # PHILOX4_32_10
    seed = 0x0123456789ABCDEF
    assert lib.rocrand_set_seed(gen, ctypes.c_ulonglong(seed)) == 0
    n = 4096
    outb = np.zeros(n, dtype=np.uint32)
    st = lib.rocrand_generate(gen, outb.ctypes.data_as(ctypes.c_void_p), ctypes.c_size_t(n))
    lib.rocrand_destroy_generator(gen)
    assert st == 0, f"rocrand_generate status {st}"
    ctr = np.arange(n // 4, dtype=np.uint64)
    words = philox4x32_10(ctr, 0, 0, 0, seed & 0xFFFFFFFF, seed >> 32)
    mine = np.stack(words, axis=-1).reshape(-1)
    log(f"  rocrand first words {[hex(x) for x in outb[:4]]}, oracle {[hex(x) for x in mine[:4]]}")
    assert np.array_equal(outb, mine)


# Every forward slot count (1, 2, 4, 8, 10, 12, 14, 16 vectors per lane, and
# two waves per row) in both dtypes, against the oracle, with ragged and
# uniform shards, both norms, with and without dropout/bias/residual.  Shards
# of at most 1024 rows split rows of 4 and 8 vectors per lane over 4 waves;
# the last three shapes keep one wave per row (more than 1024 rows).
SLOT_SHAPES = [
    # (h, dtype, norm, t, T-or-lengths, p, bias, residual)
    (64, "bf16", "layernorm", 3, 21, 0.3, True, True),           # 8 vectors: 1 slot
    (1032, "bf16", "rmsnorm", 2, 17, 0.0, False, True),          # 129 vectors: 4 slots
    (4104, "bf16", "layernorm", 4, (12, 0, 20), 0.2, True, False),   # 513 vectors: 10 slots, ragged
    (6144, "bf16", "layernorm", 5, 9, 0.1, True, True),          # 768 vectors: 12 slots
    (7168, "bf16", "rmsnorm", 7, 6, 0.25, False, True),          # 896 vectors: 14 slots
    (8200, "bf16", "layernorm", 2, 5, 0.1, True, True),          # 1025 vectors: two waves per row
    (2560, "f32", "layernorm", 3, 8, 0.15, True, True),          # 640 vectors: 10 slots
    (3072, "f32", "rmsnorm", 4, (8, 4), 0.4, False, True),       # 768 vectors: 12 slots, ragged
    (3584, "f32", "layernorm", 2, 7, 0.0, True, False),          # 896 vectors: 14 slots
    (4100, "f32", "layernorm", 1, 5, 0.2, False, True),          # 1025 vectors: two waves per row
    (1024, "bf16", "layernorm", 2, 1100, 0.1, True, True),       # 128 vectors: 2 slots, one wave per row
    (1024, "f32", "rmsnorm", 2, 1030, 0.2, False, True),         # 256 vectors: 4 slots, one wave per row
    (4096, "bf16", "layernorm", 2, 1040, 0.1, False, True),      # 512 vectors: 8 slots, one wave per row
]


@pytest.mark.parametrize("shape", SLOT_SHAPES, ids=[f"h{s[0]}_{s[1]}_{s[2]}_t{s[3]}" for s in SLOT_SHAPES])
def test_every_slot_count(cuda_device, shape):
    h, dtype, norm, t, rows, p, bias, res = shape
    if isinstance(rows, tuple):
        w = W.custom(f"slots_h{h}", h=h, t=t, dtype=dtype, norm=norm, p_drop=p, bias=bias, residual=res,
                     lengths=tuple(t * r for r in rows))
    else:
        w = W.custom(f"slots_h{h}", h=h, t=t, dtype=dtype, norm=norm, p_drop=p, bias=bias, residual=res, s=t * rows)
    rank = t - 1
    log(f"[parity-slots] h={h} {dtype} {norm} t={t} rows={rows} p={p} rank={rank}")
    inp = W.make_inputs(w)
    gpu = run_gpu(inp, w, rank, cuda_device, recommended_stride=True)
    compare(w, inp, gpu, rank)


@pytest.mark.parametrize("name", ["page_demo", "shard70b", "odd_t3_h520"])
def test_slab_pointer_table_matches_strided(cuda_device, name):
    """sp_region_fwd_slabs with the t slabs in t separate allocations (made in
    reverse order, so no stride relates them) gives the strided form's bits:
    z, y, mean, rstd and the mask; and it matches the oracle at the usual bars
    (z and the mask bit-exact), with and without the mask output."""
    import torch
    if name == "odd_t3_h520":
        w = W.custom("odd_t3_h520", h=520, t=3, s=3 * 37, b=2, p_drop=0.25)
        inp = W.make_inputs(w)
    else:
        w = W.BY_NAME[name]
        inp = inputs_for(w)
    log(f"[slab-table] {name}")
    t = lambda a: W.as_torch(a, cuda_device)
    P = t(inp["partials"])
    separate = [None] * w.t
    for k in reversed(range(w.t)):
        separate[k] = torch.empty_like(P[k]).copy_(P[k])
    kw = dict(bias=t(inp["bias"]), residual=t(inp["residual"]), b=inp["b"], s=inp["s"], t=w.t, rank=w.t - 1,
              eps=w.eps, p_drop=w.p_drop, seed=inp["seed"], norm=w.norm, cu_seqlens=inp["cu_seqlens"],
              return_mask=True)
    a = spr.fwd(P, t(inp["gamma"]), t(inp["beta"]), **kw)
    b = spr.fwd(separate, t(inp["gamma"]), t(inp["beta"]), **kw)
    torch.cuda.synchronize()
    for k in ("z", "y", "mean", "rstd", "mask"):
        x, y_ = getattr(a, k), getattr(b, k)
        if x is None:
            assert y_ is None
            continue
        assert torch.equal(x.view(torch.uint8), y_.view(torch.uint8)), k
    # ... and the pointer-table form against the oracle on its own, with the
    # mask-free kernel too (whose outputs must equal the masked one's).
    c = spr.fwd(separate, t(inp["gamma"]), t(inp["beta"]), **dict(kw, return_mask=False))
    g = spr.bwd(t(inp["dy"]), b.z, b.mean, b.rstd, t(inp["gamma"]), b=inp["b"], s=inp["s"], t=w.t, norm=w.norm)
    torch.cuda.synchronize()
    for k in ("z", "y", "mean", "rstd"):
        x, y_ = getattr(b, k), getattr(c, k)
        if x is not None:
            assert torch.equal(x.view(torch.uint8), y_.view(torch.uint8)), k + " (mask-free)"
    gpu = dict(z=to_np_bits(b.z), y=to_np_f64(b.y), mean=None if b.mean is None else to_np_f64(b.mean),
               rstd=to_np_f64(b.rstd), mask=b.mask.cpu().numpy(), dx=to_np_f64(g.dx), dgamma=to_np_f64(g.dgamma),
               dbeta=None if g.dbeta is None else to_np_f64(g.dbeta))
    compare(w, inp, gpu, w.t - 1)


# On small shards the backward is one launch whose column blocks sum
# dgamma/dbeta straight from dy and z (tiny, page_demo and the "direct"
# cases: at most 4 rows per row block, a ragged last vector of columns, dres,
# RMSNorm, a single row); otherwise, and always under set_bwd_launches(2),
# row blocks write partial sums and a second launch reduces them.  Both must
# give the same bits.
LAUNCH_CASES = ["tiny", "page_demo", "shard70b", "ragged13b",
                W.custom("wide_h16384_dres", h=16384, t=4, s=4 * 40, p_drop=0.2),
                W.custom("f32_h5120_rms_t3", h=5120, t=3, s=3 * 50, dtype="f32", norm="rmsnorm", p_drop=0.0,
                         bias=False),
                W.custom("direct_bf16_h4104_t2_dres", h=4104, t=2, s=2 * 50, p_drop=0.1),
                W.custom("direct_rms_f32_h2048", h=2048, t=4, s=4 * 37, dtype="f32", norm="rmsnorm", p_drop=0.0,
                         bias=False),
                W.custom("direct_one_row_bf16", h=1024, t=2, s=2, p_drop=0.1)]


@pytest.mark.parametrize("case", LAUNCH_CASES, ids=[c if isinstance(c, str) else c.name for c in LAUNCH_CASES])
def test_backward_launch_paths_bitwise_equal(cuda_device, case):
    import torch
    w = W.BY_NAME[case] if isinstance(case, str) else case
    inp = inputs_for(w) if isinstance(case, str) else W.make_inputs(w)
    log(f"[launch-paths] {w.name}")
    t = lambda a: W.as_torch(a, cuda_device)
    fo = spr.fwd(t(inp["partials"]), t(inp["gamma"]), t(inp["beta"]), bias=t(inp["bias"]),
                 residual=t(inp["residual"]), b=inp["b"], s=inp["s"], t=w.t, rank=1, eps=w.eps, p_drop=w.p_drop,
                 seed=inp["seed"], norm=w.norm, cu_seqlens=inp["cu_seqlens"])
    dres = t(W.make_inputs(w, seed=77)["dy"]) if "dres" in w.name else None
    kw = dict(b=inp["b"], s=inp["s"], t=w.t, norm=w.norm, dres_in=dres)
    dkw = dict(kw, rank=1, p_drop=w.p_drop, seed=inp["seed"], cu_seqlens=inp["cu_seqlens"],
               want_dbias=inp["bias"] is not None)
    # One workspace for every call, read by ordinary kernels in between (so
    # stale copies of its lines sit in the L2 caches when the next call
    # reuses it), and the default path run twice.
    T, h = fo.z.shape
    ws = torch.zeros(spr.dropout_workspace_bytes(T, h), dtype=torch.uint8, device=cuda_device)
    outs = {}
    try:
        for n in (2, 1, 1):
            spr.set_bwd_launches(n)
            g = spr.bwd(t(inp["dy"]), fo.z, fo.mean, fo.rstd, t(inp["gamma"]), workspace=ws, **kw)
            float(ws.float().sum())
            d = spr.bwd_dropout(t(inp["dy"]), fo.z, fo.mean, fo.rstd, t(inp["gamma"]), workspace=ws, **dkw)
            float(ws.float().sum())
            torch.cuda.synchronize()
            if n in outs:
                outs[3] = (g, d)
            else:
                outs[n] = (g, d)
    finally:
        spr.set_bwd_launches(1)
    for a, b in zip(outs[1], outs[3]):
        for k in a._fields:
            x, y = getattr(a, k), getattr(b, k)
            if x is not None:
                assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), k + " (one launch, repeated)"
    for a, b in zip(outs[1], outs[2]):
        for k in a._fields:
            x, y = getattr(a, k), getattr(b, k)
            if x is None:
                assert y is None, k
                continue
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), k
    with pytest.raises(spr.SpRegionError):
        spr.set_bwd_launches(3)


@pytest.mark.parametrize("launches", [1, 2])
def test_backward_reads_rewritten_inputs(cuda_device, launches):
    """The backward reads z, dy and its workspace as the previous kernels left
    them, although other kernels read the same memory (so L2 copies of the old
    contents exist) before it was rewritten: shard B's results must not carry
    any of shard A's values.  A 512 x 4096 shard (4 MB tensors, the size of
    one L2) and the same output and workspace buffers for both shards."""
    import torch
    wa = W.BY_NAME["page_demo"]
    wb = W.custom("page_demo_b", h=4096, t=8, s=4096, p_drop=0.1, bias=False, seed=123)
    ia, ib = inputs_for(wa), W.make_inputs(wb)
    t = lambda a: W.as_torch(a, cuda_device)
    T, h = ia["T"], wa.h
    out = spr.FwdOut(*(torch.empty((T, h), dtype=torch.bfloat16, device=cuda_device) for _ in range(2)),
                     torch.empty(T, device=cuda_device), torch.empty(T, device=cuda_device), None)
    dy = torch.empty((T, h), dtype=torch.bfloat16, device=cuda_device)
    ws = torch.zeros(spr.workspace_bytes(T, h), dtype=torch.uint8, device=cuda_device)
    bo = spr.BwdOut(torch.empty((T, h), dtype=torch.bfloat16, device=cuda_device), torch.empty(h, device=cuda_device),
                    torch.empty(h, device=cuda_device))
    kw = dict(b=1, s=4096, t=8, rank=2, eps=1e-5, p_drop=0.1, norm="layernorm")
    try:
        spr.set_bwd_launches(launches)
        for inp in (ia, ib):
            spr.fwd(t(inp["partials"]), t(inp["gamma"]), t(inp["beta"]), residual=t(inp["residual"]),
                    seed=inp["seed"], out=out, **kw)
            dy.copy_(t(inp["dy"]))
            spr.bwd(dy, out.z, out.mean, out.rstd, t(inp["gamma"]), b=1, s=4096, t=8, workspace=ws, out=bo)
            # Ordinary kernels read every buffer the next shard rewrites.
            float(out.z.float().sum() + dy.float().sum() + ws.float().sum() + bo.dx.float().sum())
        torch.cuda.synchronize()
    finally:
        spr.set_bwd_launches(1)
    gpu = dict(z=to_np_bits(out.z), y=to_np_f64(out.y), mean=to_np_f64(out.mean), rstd=to_np_f64(out.rstd),
               mask=None, dx=to_np_f64(bo.dx), dgamma=to_np_f64(bo.dgamma), dbeta=to_np_f64(bo.dbeta))
    compare(wb, ib, gpu, 2)
