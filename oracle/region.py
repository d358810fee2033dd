"""CPU oracle of the sequence-parallel region (test infrastructure only).

What it computes, on one rank's shard of T = b*s/t rows by h channels:

  forward   z = residual + dropout(sum_k P_k + bias)        (one rank's g* output)
            y = LayerNorm(z) or RMSNorm(z)                   (per token, over all h)
  backward  dx = d(loss)/dz (+ an optional extra gradient on z), dgamma, dbeta;
            through the dropout: dpartial = d(loss)/dP_k (the same for every
            slab k) and dbias

Sources (hpc.payai.win, lesson 7 "Sequence parallelism"):
  * section 2 gives LayerNorm over the full hidden size: mean and population
    variance over h, eps inside the square root, then scale by gamma and shift
    by beta;
  * section 3 says the non-TP ops (LayerNorm, RMSNorm, dropout, residual) are
    token-wise, so a rank's sequence slice is computed on its own, and that the
    g* reduce-scatter both sums the row-linear partial outputs and leaves each
    rank its own s/t slice;
  * section 3.B: the backward is the adjoint of the forward;
  * answer to question 1: ranks must draw the dropout mask from the same seed,
    and the mask covers the whole (unsharded) tensor.

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):
  * order: bias is added to the partial sum, then dropout, then the residual;
  * the t partial slabs are summed in float32 in ascending k, then bias, the
    dropout scale and the residual are applied as separate float32 operations
    (no fused multiply-add), and z is rounded once to the storage dtype; the
    statistics and y use the stored (rounded) z;
  * dropout is inverted (kept values scaled by 1/(1-p)); the keep decision for
    channel j of global token g is word (j mod 4) of Philox-4x32-10 with
    counter (j div 4, lo32 g, hi32 g, 0) and key (lo32 seed, hi32 seed); the
    element is dropped iff that word < floor(p * 2^32), p taken as float32;
  * the global token index of local row i is r*T + i for a uniform shard, and
    t*cu[q] + r*len_q + (i - cu[q]) for row i of packed sequence q;
  * RMSNorm is z / sqrt(mean(z^2) + eps) * gamma, with no mean and no shift;
  * statistics, y and the whole backward are evaluated in float64.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .bf16 import bf16_to_f32, f32_to_bf16
from .philox import philox4x32_10

LAYERNORM = "layernorm"
RMSNORM = "rmsnorm"


def decode(a: Optional[np.ndarray], dtype: str) -> Optional[np.ndarray]:
    """Storage array -> float32 values ("f64" passes float64 values through,
    for the finite-difference pins of the backward)."""
    if a is None:
        return None
    if dtype == "bf16":
        return bf16_to_f32(a)
    if dtype == "f64":
        return np.asarray(a, dtype=np.float64)
    return np.asarray(a, dtype=np.float32)


def statistics(z64: np.ndarray, norm: str, eps64: float):
    """Per-token statistics over the last axis in float64.

    LayerNorm: mu = mean(z), var = mean((z - mu)^2) (population), rstd = 1/sqrt(var + eps).
    RMSNorm:   rstd = 1/sqrt(mean(z^2) + eps), no mean.
    Returns (mu or None, rstd, xhat) with xhat the normalised z before gamma/beta."""
    if norm == LAYERNORM:
        mu = z64.mean(axis=-1)
        var = ((z64 - mu[..., None]) ** 2).mean(axis=-1)
        rs = 1.0 / np.sqrt(var + eps64)
        return mu, rs, (z64 - mu[..., None]) * rs[..., None]
    rs = 1.0 / np.sqrt((z64 * z64).mean(axis=-1) + eps64)
    return None, rs, z64 * rs[..., None]


def normalize(z64: np.ndarray, gamma64: np.ndarray, beta64: Optional[np.ndarray], norm: str, eps64: float):
    """y = xhat * gamma (+ beta for LayerNorm).  Returns (y, mu or None, rstd)."""
    mu, rs, xhat = statistics(z64, norm, eps64)
    y = xhat * gamma64
    if beta64 is not None and norm == LAYERNORM:
        y = y + beta64
    return y, mu, rs


def encode(x32: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values -> storage array (bf16 bits rounded to nearest even);
    "f64" keeps float64 values."""
    if dtype == "bf16":
        return f32_to_bf16(x32)
    if dtype == "f64":
        return np.asarray(x32, dtype=np.float64)
    return np.asarray(x32, dtype=np.float32)


def token_index(T: int, t: int, rank: int, cu_seqlens: Optional[np.ndarray] = None) -> np.ndarray:
    """Global token index (row of the unsharded [s*b][h] view) of each local row.

    Uniform shard [s/t][b][h]: rank r holds global rows r*T .. r*T+T-1.
    Packed ragged batch: sequence q has local rows cu[q]..cu[q+1]-1 on every
    rank, global length t*len_q and global start t*cu[q]; rank r holds its
    r-th contiguous slice of len_q tokens.
    """
    i = np.arange(T, dtype=np.int64)
    if cu_seqlens is None:
        return rank * np.int64(T) + i
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    assert cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    g = np.empty(T, dtype=np.int64)
    for q in range(len(cu) - 1):
        a, b = cu[q], cu[q + 1]
        g[a:b] = t * a + rank * (b - a) + (i[a:b] - a)
    return g


def dropout_threshold(p: float) -> int:
    """floor(p * 2^32) with p rounded to float32 first."""
    p64 = float(np.float32(p))
    return int(np.floor(p64 * 4294967296.0))


def dropout_scale(p: float) -> np.float32:
    """float32(1 / (1 - p)), p rounded to float32 first."""
    return np.float32(1.0 / (1.0 - float(np.float32(p))))


def keep_mask(seed: int, p: float, gidx: np.ndarray, h: int) -> np.ndarray:
    """Boolean keep mask [len(gidx)][h]; all True when p == 0."""
    n = len(gidx)
    if p == 0.0:
        return np.ones((n, h), dtype=bool)
    thr = np.uint32(dropout_threshold(p))
    nblk = (h + 3) // 4
    g = np.asarray(gidx, dtype=np.uint64)
    c0 = np.arange(nblk, dtype=np.uint64)[None, :]
    c1 = (g & np.uint64(0xFFFFFFFF))[:, None]
    c2 = (g >> np.uint64(32))[:, None]
    words = philox4x32_10(c0, c1, c2, np.uint64(0), seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    u = np.stack(words, axis=-1).reshape(n, nblk * 4)[:, :h]   # u[:, j] = word j%4 of block j//4
    return u >= thr


def region_forward(partials, *, t, rank, dtype, norm, eps, p_drop, seed,
                   gamma, beta=None, bias=None, residual=None, cu_seqlens=None,
                   rows=None, chunk=256):
    """Forward of the region on one rank's shard.

    partials: [t][T][h] storage array (float32, or uint16 bf16 bits; float64
              values with dtype "f64", which runs the whole pre-norm sum in
              float64 with no rounding -- the mode the finite-difference
              pins of the backward differentiate).
    rows:     optional local row indices to evaluate (default all rows).
    Returns dict with z (storage), z32 (its float32 value), keep (bool),
    y, mean (None for RMSNorm), rstd -- y/mean/rstd in float64.
    """
    assert partials.shape[0] == t
    T, h = partials.shape[1], partials.shape[2]
    gidx_all = token_index(T, t, rank, cu_seqlens)
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    n = len(rows)
    g64 = decode(gamma, dtype).astype(np.float64)
    b64 = decode(beta, dtype).astype(np.float64) if beta is not None else None
    bias32 = decode(bias, dtype) if bias is not None else None
    scale = dropout_scale(p_drop)
    eps64 = float(np.float32(eps))

    acc_t = np.float64 if dtype == "f64" else np.float32   # arithmetic of the pre-norm sum
    z_out = np.empty((n, h), dtype={"f32": np.float32, "f64": np.float64}.get(dtype, np.uint16))
    z32_out = np.empty((n, h), dtype=acc_t)
    keep_out = np.empty((n, h), dtype=bool)
    y = np.empty((n, h), dtype=np.float64)
    mean = np.empty(n, dtype=np.float64) if norm == LAYERNORM else None
    rstd = np.empty(n, dtype=np.float64)

    for a in range(0, n, chunk):
        r = rows[a:a + chunk]
        acc = decode(partials[0][r], dtype).copy()                   # g*: sum of the t slabs
        for k in range(1, t):
            acc = (acc + decode(partials[k][r], dtype)).astype(acc_t)
        if bias32 is not None:
            acc = (acc + bias32[None, :]).astype(acc_t)
        keep = keep_mask(seed, p_drop, gidx_all[r], h)
        if p_drop > 0.0:
            d = np.where(keep, (acc * scale).astype(acc_t), acc_t(0.0)).astype(acc_t)
        else:
            d = acc
        if residual is not None:
            zf = (decode(residual[r], dtype) + d).astype(acc_t)
        else:
            zf = d
        zs = encode(zf, dtype)
        zv = decode(zs, dtype)
        z_out[a:a + len(r)] = zs
        z32_out[a:a + len(r)] = zv
        keep_out[a:a + len(r)] = keep

        yy, mu, rs = normalize(zv.astype(np.float64), g64, b64, norm, eps64)
        if mean is not None:
            mean[a:a + len(r)] = mu
        rstd[a:a + len(r)] = rs
        y[a:a + len(r)] = yy

    return dict(z=z_out, z32=z32_out, keep=keep_out, y=y, mean=mean, rstd=rstd, rows=rows)


def dropout_backward(dx, *, t, rank, p_drop, seed, cu_seqlens=None, T=None, rows=None):
    """Gradient of the slab sum and of the bias, given dx = d(loss)/dz (float64).

    The backward of each forward step is its adjoint (lesson 7, section 3.B):
    z = residual + dropout(a) with a = sum_k P_k + bias, and inverted dropout
    multiplies kept elements by scale = float32(1/(1-p)) and zeroes the rest,
    so d(loss)/da = dx * keep * scale, with the forward's own mask (same
    seed, same global token index).  The sum over the t slabs is linear with
    coefficient 1 for every slab, so d(loss)/dP_k is that same tensor for
    every k -- in the multi-GPU pipeline it is what the backward of g* (an
    all-gather, section 3.B) delivers to each rank's row-linear.  The bias
    gradient is its column sum over this rank's rows.

    dx:   float64 [n][h] for local rows `rows` (default all T rows, T = n).
    Returns dict: dpartial [n][h], dbias [h], C [h] = sum_i |dpartial_ij|
    (the conditioning scale of dbias), keep [n][h].
    """
    n, h = dx.shape
    T = n if T is None else T
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    assert len(rows) == n
    keep = keep_mask(seed, p_drop, token_index(T, t, rank, cu_seqlens)[rows], h)
    scale = float(dropout_scale(p_drop)) if p_drop > 0.0 else 1.0
    dpartial = np.where(keep, dx * scale, 0.0)
    return dict(dpartial=dpartial, dbias=dpartial.sum(axis=0), C=np.abs(dpartial).sum(axis=0), keep=keep)


def region_backward(dy, z, gamma, *, dtype, norm, eps, dres_in=None, rows=None, chunk=256,
                    with_param_grads=True):
    """Backward of the normalisation on z (float64 throughout).

    dx_ij = rstd_i * (g_ij - mean_j g_ij - xhat_ij * mean_j(g_ij * xhat_ij))   (LayerNorm)
    dx_ij = rstd_i * (g_ij - xhat_ij * mean_j(g_ij * xhat_ij))                  (RMSNorm)
    with g = dy * gamma and xhat the normalised z, plus dres_in when given.
    dgamma_j = sum_i dy_ij * xhat_ij and dbeta_j = sum_i dy_ij over this rank's
    rows; A_j = sum_i |dy_ij * xhat_ij| and B_j = sum_i |dy_ij| are returned as
    the conditioning scales of those sums.  Statistics are the oracle's own
    (recomputed from z), not the forward's saved ones.
    """
    T, h = z.shape
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    n = len(rows)
    g64 = decode(gamma, dtype).astype(np.float64)
    eps64 = float(np.float32(eps))
    dx = np.empty((n, h), dtype=np.float64)
    dgamma = np.zeros(h, dtype=np.float64)
    dbeta = np.zeros(h, dtype=np.float64)
    A = np.zeros(h, dtype=np.float64)
    B = np.zeros(h, dtype=np.float64)
    for a in range(0, n, chunk):
        r = rows[a:a + chunk]
        z64 = decode(z[r], dtype).astype(np.float64)
        dy64 = decode(dy[r], dtype).astype(np.float64)
        _, rs, xhat = statistics(z64, norm, eps64)
        g = dy64 * g64[None, :]
        c2 = (g * xhat).mean(axis=1)
        if norm == LAYERNORM:
            c1 = g.mean(axis=1)
            d = rs[:, None] * (g - c1[:, None] - xhat * c2[:, None])
        else:
            d = rs[:, None] * (g - xhat * c2[:, None])
        if dres_in is not None:
            d = d + decode(dres_in[r], dtype).astype(np.float64)
        dx[a:a + len(r)] = d
        if with_param_grads:
            dgamma += (dy64 * xhat).sum(axis=0)
            dbeta += dy64.sum(axis=0)
            A += np.abs(dy64 * xhat).sum(axis=0)
            B += np.abs(dy64).sum(axis=0)
    out = dict(dx=dx, rows=rows)
    if with_param_grads:
        out.update(dgamma=dgamma, dbeta=dbeta if norm == LAYERNORM else None, A=A, B=B)
    return out


def accumulate_param_grads(main, step):
    """Parameter gradients added into main-grad buffers (float64, unrounded).

    Gradient accumulation over micro-batches: the parameter gradient of a
    step is the sum over every token of every micro-batch, so each
    micro-batch's backward adds its own column sums (dgamma, dbeta, dbias of
    region_backward / dropout_backward) into buffers that persist across the
    micro-batches instead of replacing them.  The pages do not describe this
    step; it is the usual convention of mixed-precision training, where those
    buffers are float32.

    main: dict name -> [h] array (the buffers before the call) or None.
    step: dict name -> float64 [h] array (this micro-batch's sums) or None.
    Returns dict name -> float64 [h]: main + step for every name whose main
    buffer is given (a name without a buffer is not accumulated).
    """
    out = {}
    for name, buf in main.items():
        if buf is None:
            out[name] = None
            continue
        add = step.get(name)
        if add is None:
            raise ValueError(f"no gradient {name!r} to accumulate")
        out[name] = np.asarray(buf, dtype=np.float64) + np.asarray(add, dtype=np.float64)
    return out
