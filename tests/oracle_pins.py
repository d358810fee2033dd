"""Checks that tie the region oracle to things other than itself.

Each ``check_*`` raises AssertionError on failure.  The pin tests call them
against the oracle as it is; the planted-mistake tests call them against an
oracle with one plausible mistake patched in, and expect them to fail.
Sources are the hpc.payai.win lesson 7 pages (LayerNorm formula of section 2,
token-wise SP region and g* of section 3, adjoint of section 3.B, seed-shared
full-tensor dropout mask of the answer to question 1)."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle.region as R
import oracle.region as oracle_region


def _rng(seed):
    return np.random.default_rng(seed)


def small_f32_case(seed=0, T=24, h=64, t=4, with_bias=True, with_res=True):
    rng = _rng(seed)
    P = rng.standard_normal((t, T, h)).astype(np.float32)
    res = rng.standard_normal((T, h)).astype(np.float32) if with_res else None
    bias = (0.02 * rng.standard_normal(h)).astype(np.float32) if with_bias else None
    gamma = rng.uniform(0.5, 1.5, h).astype(np.float32)
    beta = (0.1 * rng.standard_normal(h)).astype(np.float32)
    return P, res, bias, gamma, beta


def check_layernorm_matches_torch(seed=1, R=R):
    """t = 1, p = 0, no bias, no residual: the region is plain LayerNorm of the
    single slab; compare with torch's float64 layer_norm (library routine)."""
    rng = _rng(seed)
    T, h = 16, 96
    P = (3.0 * rng.standard_normal((1, T, h)) + 0.7).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, h).astype(np.float32)
    beta = rng.standard_normal(h).astype(np.float32)
    out = R.region_forward(P, t=1, rank=0, dtype="f32", norm="layernorm", eps=1e-5, p_drop=0.0,
                           seed=0, gamma=gamma, beta=beta)
    assert np.array_equal(out["z"], P[0]), "t=1, no bias/residual/dropout: z must be the slab"
    x = torch.from_numpy(P[0].astype(np.float64))
    ref = torch.nn.functional.layer_norm(x, (h,), torch.from_numpy(gamma.astype(np.float64)),
                                         torch.from_numpy(beta.astype(np.float64)),
                                         eps=float(np.float32(1e-5))).numpy()
    assert np.max(np.abs(out["y"] - ref)) < 1e-12
    var, mu = torch.var_mean(x, dim=1, unbiased=False)
    assert np.max(np.abs(out["mean"] - mu.numpy())) < 1e-12
    assert np.max(np.abs(out["rstd"] - 1.0 / np.sqrt(var.numpy() + float(np.float32(1e-5))))) < 1e-9


def check_rmsnorm_matches_torch(seed=2, R=R):
    rng = _rng(seed)
    T, h = 16, 80
    P = (2.0 * rng.standard_normal((1, T, h)) + 0.3).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, h).astype(np.float32)
    out = R.region_forward(P, t=1, rank=0, dtype="f32", norm="rmsnorm", eps=1e-6, p_drop=0.0,
                           seed=0, gamma=gamma)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(P[0].astype(np.float64)), (h,),
                                       torch.from_numpy(gamma.astype(np.float64)),
                                       eps=float(np.float32(1e-6))).numpy()
    assert out["mean"] is None
    assert np.max(np.abs(out["y"] - ref)) < 1e-12


def check_hand_case_h2(R=R):
    """h = 2, z = (0, 2): mean 1, population variance 1, so LayerNorm gives
    (-1, 1)/sqrt(1 + eps) before the affine map; RMS gives (0, 2)/sqrt(2 + eps).
    eps = 1 makes the placement of eps visible."""
    P = np.array([[[0.0, 2.0]]], dtype=np.float32)
    gamma = np.array([2.0, 3.0], dtype=np.float32)
    beta = np.array([0.5, -0.5], dtype=np.float32)
    for eps in (1.0, 1e-5):
        e = float(np.float32(eps))
        out = R.region_forward(P, t=1, rank=0, dtype="f32", norm="layernorm", eps=eps, p_drop=0.0,
                               seed=0, gamma=gamma, beta=beta)
        want = np.array([-2.0 / math.sqrt(1 + e) + 0.5, 3.0 / math.sqrt(1 + e) - 0.5])
        assert np.max(np.abs(out["y"][0] - want)) < 1e-14
        assert out["mean"][0] == 1.0
        out = R.region_forward(P, t=1, rank=0, dtype="f32", norm="rmsnorm", eps=eps, p_drop=0.0,
                               seed=0, gamma=gamma)
        want = np.array([0.0, 3.0 * 2.0 / math.sqrt(2 + e)])
        assert np.max(np.abs(out["y"][0] - want)) < 1e-14


def check_unit_affine_invariant(seed=3, dtype="bf16", R=R):
    """gamma = 1, beta = 0: per token, mean(y) = 0 and var(y) = s2/(s2 + eps)
    where s2 is the population variance of z."""
    rng = _rng(seed)
    T, h, t = 32, 512, 2
    P32 = (rng.standard_normal((t, T, h)) * rng.uniform(0.01, 5, (1, T, 1))).astype(np.float32)
    if dtype == "bf16":
        P = torch.from_numpy(P32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        gamma = np.full(h, 0x3F80, dtype=np.uint16)
        beta = np.zeros(h, dtype=np.uint16)
    else:
        P, gamma, beta = P32, np.ones(h, np.float32), np.zeros(h, np.float32)
    eps = 1e-2   # large enough that var(y) visibly differs from 1
    out = R.region_forward(P, t=t, rank=0, dtype=dtype, norm="layernorm", eps=eps, p_drop=0.0,
                           seed=0, gamma=gamma, beta=beta)
    z = out["z32"].astype(np.float64)
    s2 = np.var(z, axis=1)
    e = float(np.float32(eps))
    assert np.max(np.abs(out["y"].mean(axis=1))) < 1e-12
    assert np.max(np.abs(out["y"].var(axis=1) - s2 / (s2 + e))) < 1e-12


def check_z_within_exact_bound(seed=4, dtype="f32", p=0.1, R=R):
    """z against the exact real value residual + keep*(sum_k P_k + bias)/(1-p):
    the float32 chain of t+3 roundings is within (t+4)*2^-24 of the summed
    magnitudes, and one bf16 rounding adds at most half a bf16 ulp.  Dropped
    elements must equal the residual exactly."""
    P, res, bias, gamma, beta = small_f32_case(seed)
    t, T, h = P.shape
    if dtype == "bf16":
        cast = lambda a: torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        Ps, ress, biass, gs, bs = cast(P), cast(res), cast(bias), cast(gamma), cast(beta)
        val = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).double().numpy()
    else:
        Ps, ress, biass, gs, bs = P, res, bias, gamma, beta
        val = lambda a: a.astype(np.float64)
    seed_d = 77
    out = R.region_forward(Ps, t=t, rank=1, dtype=dtype, norm="layernorm", eps=1e-5, p_drop=p,
                           seed=seed_d, gamma=gs, beta=bs, bias=biass, residual=ress)
    Pv, rv, bv = val(Ps), val(ress), val(biass)
    keep = out["keep"]
    inv = 1.0 / (1.0 - float(np.float32(p)))
    exact = np.empty((T, h))
    mag = np.empty((T, h))
    for i in range(T):
        for j in range(h):
            terms = [Pv[k, i, j] for k in range(t)] + [bv[j]]
            s = math.fsum(terms)
            exact[i, j] = rv[i, j] + (s * inv if keep[i, j] else 0.0)
            mag[i, j] = abs(rv[i, j]) + inv * math.fsum(abs(x) for x in terms)
    bound = (t + 4) * 2.0 ** -24 * mag + 1e-30
    z = out["z32"].astype(np.float64)
    if dtype == "bf16":
        e_abs = np.abs(z - exact)
        a = np.abs(z)
        half_ulp = np.ldexp(1.0, (np.floor(np.log2(np.where(a > 0, a, 1.0))) - 8).astype(np.int64))
        assert np.all(e_abs <= half_ulp + bound * 1.01 + 1e-30)
    else:
        assert np.all(np.abs(z - exact) <= bound)
    assert np.array_equal(out["z32"][~keep], val(ress)[~keep].astype(np.float32))
    # The dropped fraction is near p (loose: small sample).
    frac = 1.0 - keep.mean()
    assert abs(frac - p) < 6 * math.sqrt(p * (1 - p) / keep.size) + 1e-12


def check_shard_invariance(seed=5, t=4, b=2, s_local=6, h=40, p=0.3, R=R):
    """Token-wise independence plus g* = sum-then-split: running every rank of a
    uniform [s/t][b][h] shard and concatenating equals the unsharded t = 1 run
    on the fp32 ascending-k sum of the full partial outputs -- bit for bit for
    z and the mask, exactly for y (same float64 operations)."""
    rng = _rng(seed)
    T = s_local * b
    Q = rng.standard_normal((t, t * T, h)).astype(np.float32)     # TP rank k's full row-linear output
    res = rng.standard_normal((t * T, h)).astype(np.float32)
    bias = (0.1 * rng.standard_normal(h)).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, h).astype(np.float32)
    beta = rng.standard_normal(h).astype(np.float32)
    kw = dict(dtype="f32", norm="layernorm", eps=1e-5, p_drop=p, seed=2024, gamma=gamma, beta=beta, bias=bias)
    S = Q[0].copy()
    for k in range(1, t):
        S = (S + Q[k]).astype(np.float32)
    full = R.region_forward(S[None], t=1, rank=0, residual=res, **kw)
    zs, ks, ys = [], [], []
    for r in range(t):
        sl = slice(r * T, (r + 1) * T)
        o = R.region_forward(np.ascontiguousarray(Q[:, sl]), t=t, rank=r, residual=res[sl], **kw)
        zs.append(o["z"]), ks.append(o["keep"]), ys.append(o["y"])
    assert np.array_equal(np.concatenate(zs), full["z"])
    assert np.array_equal(np.concatenate(ks), full["keep"])
    assert np.array_equal(np.concatenate(ys), full["y"])


def check_ragged_token_index(R=R):
    """Hand example: cu = [0, 2, 5], t = 2.  Sequence 0 has global length 4
    (start 0), sequence 1 global length 6 (start 4); rank 1 holds the second
    half of each: global tokens 2, 3 and 7, 8, 9."""
    assert list(R.token_index(5, 2, 1, np.array([0, 2, 5]))) == [2, 3, 7, 8, 9]
    assert list(R.token_index(5, 2, 0, np.array([0, 2, 5]))) == [0, 1, 4, 5, 6]
    assert list(R.token_index(5, 2, 1, None)) == [5, 6, 7, 8, 9]


def check_ragged_masks_tile_global(t=4, seed=6, R=R):
    """Per-rank masks of a packed ragged batch tile the mask of the unsharded
    packed batch: for every sequence, rank slices in rank order give the
    sequence's global rows in order (the mask covers the full tensor)."""
    rng = _rng(seed)
    lens = np.array([3, 0, 5, 1, 7])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, h, p, sd = int(cu[-1]), 24, 0.5, int(rng.integers(1 << 40))
    global_mask = R.keep_mask(sd, p, R.token_index(t * T, 1, 0, None), h)
    per_rank = [R.keep_mask(sd, p, R.token_index(T, t, r, cu), h) for r in range(t)]
    rebuilt = []
    for q in range(len(lens)):
        for r in range(t):
            rebuilt.append(per_rank[r][cu[q]:cu[q + 1]])
    assert np.array_equal(np.concatenate(rebuilt), global_mask)


def check_rows_subset(seed=7, R=R):
    P, res, bias, gamma, beta = small_f32_case(seed, T=20)
    kw = dict(t=4, rank=2, dtype="f32", norm="layernorm", eps=1e-5, p_drop=0.1, seed=5,
              gamma=gamma, beta=beta, bias=bias, residual=res)
    full = R.region_forward(P, chunk=7, **kw)
    rows = np.array([19, 0, 7, 3])
    sub = R.region_forward(P, rows=rows, **kw)
    assert np.array_equal(sub["z"], full["z"][rows])
    assert np.array_equal(sub["y"], full["y"][rows])
    assert np.array_equal(sub["keep"], full["keep"][rows])


def _loss(z64, dy64, gamma64, beta64, norm, eps, R=R):
    y, _, _ = R.normalize(z64, gamma64, beta64, norm, eps)
    return float(np.sum(dy64 * y))


def check_backward_finite_differences(norm="layernorm", seed=8, T=3, h=8, R=R):
    """Central differences in float64 of L = sum(dy * y) with respect to z,
    gamma and beta against the oracle's dx, dgamma, dbeta (brute force)."""
    rng = _rng(seed)
    z = rng.standard_normal((T, h)) * 1.7 + 0.4
    dy = rng.standard_normal((T, h))
    gamma = rng.uniform(0.5, 1.5, h)
    beta = rng.standard_normal(h) if norm == "layernorm" else None
    eps = 1e-3
    e = float(np.float32(eps))
    out = R.region_backward(dy, z, gamma, dtype="f64", norm=norm, eps=eps)
    d = 1e-6

    def fd(arr, idx, f):
        a0 = arr[idx]
        arr[idx] = a0 + d
        lp = f()
        arr[idx] = a0 - d
        lm = f()
        arr[idx] = a0
        return (lp - lm) / (2 * d)

    L = lambda: _loss(z, dy, gamma, beta, norm, e, R=oracle_region)
    dx_fd = np.array([[fd(z, (i, j), L) for j in range(h)] for i in range(T)])
    dg_fd = np.array([fd(gamma, j, L) for j in range(h)])
    scale = max(1.0, np.max(np.abs(dx_fd)))
    assert np.max(np.abs(out["dx"] - dx_fd)) < 1e-6 * scale
    assert np.max(np.abs(out["dgamma"] - dg_fd)) < 1e-6 * max(1.0, np.max(np.abs(dg_fd)))
    if beta is not None:
        db_fd = np.array([fd(beta, j, L) for j in range(h)])
        assert np.max(np.abs(out["dbeta"] - db_fd)) < 1e-6 * max(1.0, np.max(np.abs(db_fd)))


def check_backward_matches_torch_autograd(norm="layernorm", seed=9, T=48, h=256, R=R):
    """torch.autograd in float64 (library routine) on layer_norm / rms_norm,
    plus an extra gradient on z added to dx."""
    rng = _rng(seed)
    z = rng.standard_normal((T, h)) * 2.0 - 0.3
    dy = rng.standard_normal((T, h))
    dres = rng.standard_normal((T, h))
    gamma = rng.uniform(0.5, 1.5, h)
    beta = rng.standard_normal(h)
    eps = 1e-5
    e = float(np.float32(eps))
    zt = torch.from_numpy(z.copy()).requires_grad_(True)
    gt = torch.from_numpy(gamma.copy()).requires_grad_(True)
    bt = torch.from_numpy(beta.copy()).requires_grad_(True)
    if norm == "layernorm":
        y = torch.nn.functional.layer_norm(zt, (h,), gt, bt, eps=e)
    else:
        y = torch.nn.functional.rms_norm(zt, (h,), gt, eps=e)
    y.backward(torch.from_numpy(dy))
    out = R.region_backward(dy, z, gamma, dtype="f64", norm=norm, eps=eps, dres_in=dres)
    assert np.max(np.abs(out["dx"] - (zt.grad.numpy() + dres))) < 1e-10
    assert np.max(np.abs(out["dgamma"] - gt.grad.numpy())) < 1e-9
    if norm == "layernorm":
        assert np.max(np.abs(out["dbeta"] - bt.grad.numpy())) < 1e-9
    else:
        assert out["dbeta"] is None


def check_backward_scale_identities(norm="layernorm", seed=10, T=40, h=128, R=R):
    """Consequences of the normalisation being (almost) scale invariant:
    LayerNorm: sum_j dx_ij = 0 and sum_j dx_ij (z_ij - mu_i) = eps rstd_i^3 sum_j g_ij (z_ij - mu_i);
    RMSNorm:   sum_j dx_ij z_ij = eps rstd_i^3 sum_j g_ij z_ij,   with g = dy * gamma."""
    rng = _rng(seed)
    z = rng.standard_normal((T, h)) * rng.uniform(0.05, 3.0, (T, 1)) + 0.5
    dy = rng.standard_normal((T, h))
    gamma = rng.uniform(0.5, 1.5, h)
    eps = 0.05
    e = float(np.float32(eps))
    dx = R.region_backward(dy, z, gamma, dtype="f64", norm=norm, eps=eps)["dx"]
    g = dy * gamma
    if norm == "layernorm":
        mu = z.mean(axis=1, keepdims=True)
        c = z - mu
        rs = 1.0 / np.sqrt((c * c).mean(axis=1) + e)
        assert np.max(np.abs(dx.sum(axis=1))) < 1e-11 * np.max(np.abs(dx).sum(axis=1))
    else:
        c = z
        rs = 1.0 / np.sqrt((z * z).mean(axis=1) + e)
    lhs = (dx * c).sum(axis=1)
    rhs = e * rs ** 3 * (g * c).sum(axis=1)
    assert np.max(np.abs(lhs - rhs)) < 1e-10 * (1 + np.max(np.abs(rhs)))


def check_dbeta_is_column_sum(seed=11, T=64, h=32, R=R):
    rng = _rng(seed)
    z = rng.standard_normal((T, h)).astype(np.float32)
    dy = rng.standard_normal((T, h)).astype(np.float32)
    gamma = np.ones(h, np.float32)
    out = R.region_backward(dy, z, gamma, dtype="f32", norm="layernorm", eps=1e-5)
    for j in range(h):
        assert abs(out["dbeta"][j] - math.fsum(float(v) for v in dy[:, j])) <= 1e-12 * out["B"][j]


def check_dropout_backward_finite_differences(norm="layernorm", ragged=False, seed=12, T=3, h=8, t=2, rank=1,
                                              p=0.4, R=R):
    """Central differences in float64 through the whole region forward
    (dtype "f64": no rounding anywhere), of L = sum(dy * y) + sum(dres * z),
    with respect to one element of every slab, the bias and the residual,
    against the oracle's dropout_backward(region_backward(...)).  The mask is
    the forward's own; a ragged shard checks that both sides use the same
    global token index (brute force)."""
    rng = _rng(seed)
    P = rng.standard_normal((t, T, h))
    res = rng.standard_normal((T, h))
    bias = 0.3 * rng.standard_normal(h)
    gamma = rng.uniform(0.5, 1.5, h)
    beta = rng.standard_normal(h) if norm == "layernorm" else None
    dy = rng.standard_normal((T, h))
    dres = rng.standard_normal((T, h))
    cu = np.array([0, 1, T], dtype=np.int64) if ragged else None
    eps, sd = 1e-3, 0x1234_5678_9ABC
    kw = dict(t=t, rank=rank, dtype="f64", norm=norm, eps=eps, p_drop=p, seed=sd, gamma=gamma, beta=beta,
              cu_seqlens=cu)

    def L():
        o = oracle_region.region_forward(P, bias=bias, residual=res, **kw)
        return float(np.sum(dy * o["y"]) + np.sum(dres * o["z"]))

    fwd = R.region_forward(P, bias=bias, residual=res, **kw)
    assert 0 < (~fwd["keep"]).sum() < fwd["keep"].size        # some dropped, some kept
    bw = R.region_backward(dy, fwd["z"], gamma, dtype="f64", norm=norm, eps=eps, dres_in=dres)
    out = R.dropout_backward(bw["dx"], t=t, rank=rank, p_drop=p, seed=sd, cu_seqlens=cu)
    d = 1e-6

    def fd(arr, idx):
        a0 = arr[idx]
        arr[idx] = a0 + d
        lp = L()
        arr[idx] = a0 - d
        lm = L()
        arr[idx] = a0
        return (lp - lm) / (2 * d)

    for k in (0, t - 1):
        dp_fd = np.array([[fd(P, (k, i, j)) for j in range(h)] for i in range(T)])
        assert np.max(np.abs(out["dpartial"] - dp_fd)) < 1e-6 * max(1.0, np.max(np.abs(dp_fd))), f"slab {k}"
    db_fd = np.array([fd(bias, j) for j in range(h)])
    assert np.max(np.abs(out["dbias"] - db_fd)) < 1e-6 * max(1.0, np.max(np.abs(db_fd))), "dbias"
    dr_fd = np.array([[fd(res, (i, j)) for j in range(h)] for i in range(T)])
    assert np.max(np.abs(bw["dx"] - dr_fd)) < 1e-6 * max(1.0, np.max(np.abs(dr_fd))), "dresidual"


def check_dropout_backward_special_cases(seed=13, T=20, h=24, t=4, rank=2, R=R):
    """p = 0 leaves the gradient unchanged (no mask, no scale); with p > 0 the
    zero pattern of dpartial is the forward's dropped set and dbias is the
    exact column sum (math.fsum) of dpartial."""
    rng = _rng(seed)
    dx = rng.standard_normal((T, h))
    out0 = R.dropout_backward(dx, t=t, rank=rank, p_drop=0.0, seed=5)
    assert np.array_equal(out0["dpartial"], dx)
    P = rng.standard_normal((t, T, h)).astype(np.float32)
    gamma = np.ones(h, dtype=np.float32)
    fwd = oracle_region.region_forward(P, t=t, rank=rank, dtype="f32", norm="rmsnorm", eps=1e-5, p_drop=0.35,
                                       seed=77, gamma=gamma)
    out = R.dropout_backward(dx, t=t, rank=rank, p_drop=0.35, seed=77)
    assert np.array_equal(out["dpartial"] != 0.0, fwd["keep"])
    for j in range(h):
        assert out["dbias"][j] == math.fsum(out["dpartial"][:, j]) or \
            abs(out["dbias"][j] - math.fsum(out["dpartial"][:, j])) <= 1e-12 * out["C"][j]


def check_accumulate_split_batches(seed=14, T=23, h=40, t=2, rank=1, cuts=(0, 7, 8, 23), R=R):
    """Gradient accumulation: a batch's rows taken as micro-batches of
    unequal sizes (one of a single row), each micro-batch's parameter
    gradients added in turn into random float32 main buffers, equals those
    buffers plus the gradients of the whole batch in one backward -- the
    parameter gradient is a plain sum over tokens, so splitting the tokens
    splits the sum."""
    rng = _rng(seed)
    z = rng.standard_normal((T, h)).astype(np.float32)
    dy = rng.standard_normal((T, h)).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, h).astype(np.float32)
    main0 = {k: rng.standard_normal(h).astype(np.float32) for k in ("dgamma", "dbeta", "dbias")}

    def grads(rows):
        b = R.region_backward(dy, z, gamma, dtype="f32", norm="layernorm", eps=1e-5, rows=rows)
        d = R.dropout_backward(b["dx"], t=t, rank=rank, p_drop=0.3, seed=9, T=T, rows=rows)
        return dict(dgamma=b["dgamma"], dbeta=b["dbeta"], dbias=d["dbias"]), b["A"] + b["B"] + d["C"]

    acc = dict(main0)
    for a, b in zip(cuts[:-1], cuts[1:]):
        acc = R.accumulate_param_grads(acc, grads(np.arange(a, b))[0])
    full, scale = grads(np.arange(T))
    for k in main0:
        ref = main0[k].astype(np.float64) + full[k]
        assert np.max(np.abs(acc[k] - ref) / (scale + np.abs(main0[k]))) < 1e-12, k


def check_accumulate_identities(seed=15, h=24, R=R):
    """Zero buffers take the step's gradients exactly, a zero step leaves the
    buffers exactly, and a name without a buffer stays absent."""
    rng = _rng(seed)
    step = dict(dgamma=rng.standard_normal(h), dbeta=rng.standard_normal(h))
    main = dict(dgamma=rng.standard_normal(h).astype(np.float32), dbeta=None)
    out = R.accumulate_param_grads(dict(dgamma=np.zeros(h, np.float32), dbeta=np.zeros(h, np.float32)), step)
    assert np.array_equal(out["dgamma"], step["dgamma"]) and np.array_equal(out["dbeta"], step["dbeta"])
    out = R.accumulate_param_grads(main, dict(dgamma=np.zeros(h), dbeta=np.zeros(h)))
    assert np.array_equal(out["dgamma"], main["dgamma"].astype(np.float64)) and out["dbeta"] is None
