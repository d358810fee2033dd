"""Synthetic sequence-parallel shard workloads and their seeded inputs.

This module is shared by the oracle's tests, the GPU parity tests and the
benchmark.  It only *draws* inputs; it holds none of the region's arithmetic
(no sums, no dropout, no normalisation, no bf16 rounding of its own: the one
fp32 -> bf16 cast of the drawn inputs is done by torch's CPU conversion).

Shapes follow the pages' workloads:
  * ``tiny``      -- a small fp32 shard that a pure-Python oracle finishes fast;
  * ``page_demo`` -- the lesson's s = h = 4096, t = 8 shape-trace example
                     (hpc.payai.win lesson 7, code exercise and its answer);
  * ``shard70b``  -- the 70B worked example, h = 8192, s = 16384, t = 8, b = 1
                     (same lesson, worked example of section 4);
  * ``ragged13b`` -- a length-bucketed packed batch like the 13B replay of the
                     coreui.cn article (bucketing, length CV 0.18 gate);
  * ``long128k``  -- the 128K-context regime the guanweilu.cn explainer names.

Layout: one rank's shard is s-major ``[s/t][b][h]``, viewed as ``T = b*s/t``
rows of ``h`` channels.  A packed ragged batch is passed as ``b = 1`` with
``s = sum(s_i)``; ``cu_seqlens`` holds this rank's local row offsets.

Every array is returned as numpy: fp32 configs as float32, bf16 configs as
uint16 bit patterns (the exact bits both the oracle and the GPU consume).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

DTYPE_F32 = "f32"
DTYPE_BF16 = "bf16"
LAYERNORM = "layernorm"
RMSNORM = "rmsnorm"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int            # position in the workload list; seeds derive from it
    h: int
    t: int
    dtype: str
    norm: str
    eps: float
    p_drop: float
    has_bias: bool
    has_residual: bool
    has_beta: bool
    slab_scale: float     # partial slabs are N(0,1) * slab_scale
    s: int = 0            # uniform: global sequence length
    b: int = 1            # uniform: micro-batch size
    nseq: int = 0         # ragged: number of packed sequences
    mean_len: float = 0.0  # ragged: arithmetic mean of the global lengths
    len_cv: float = 0.0    # ragged: std/mean of the global lengths
    fixed_lengths: tuple = ()  # ragged: explicit global lengths (multiples of t, zeros allowed)
    seed_override: int = -1    # custom cases: input seed (else 1000 + index)

    @property
    def ragged(self) -> bool:
        return self.nseq > 0 or len(self.fixed_lengths) > 0

    @property
    def input_seed(self) -> int:
        return self.seed_override if self.seed_override >= 0 else 1000 + self.index

    @property
    def dropout_seed(self) -> int:
        if self.seed_override >= 0:      # custom cases: a seed with both 32-bit halves set
            return 0x9E3779B97F4A7C15 ^ self.seed_override
        return 0x5EED0000 + self.index

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == DTYPE_F32 else 2


_INV_SQRT8 = 1.0 / math.sqrt(8.0)

WORKLOADS = [
    Workload("tiny", 0, s=256, b=1, h=512, t=4, dtype=DTYPE_F32, norm=LAYERNORM,
             eps=1e-5, p_drop=0.1, has_bias=True, has_residual=True, has_beta=True,
             slab_scale=1.0),
    Workload("page_demo", 1, s=4096, b=1, h=4096, t=8, dtype=DTYPE_BF16, norm=LAYERNORM,
             eps=1e-5, p_drop=0.1, has_bias=False, has_residual=True, has_beta=True,
             slab_scale=_INV_SQRT8),
    Workload("shard70b", 2, s=16384, b=1, h=8192, t=8, dtype=DTYPE_BF16, norm=LAYERNORM,
             eps=1e-5, p_drop=0.1, has_bias=True, has_residual=True, has_beta=True,
             slab_scale=_INV_SQRT8),
    Workload("ragged13b", 3, h=5120, t=8, dtype=DTYPE_BF16, norm=RMSNORM,
             eps=1e-6, p_drop=0.0, has_bias=False, has_residual=False, has_beta=False,
             slab_scale=_INV_SQRT8, nseq=8, mean_len=4096.0, len_cv=0.18),
    Workload("long128k", 4, s=131072, b=1, h=8192, t=8, dtype=DTYPE_BF16, norm=LAYERNORM,
             eps=1e-5, p_drop=0.1, has_bias=False, has_residual=True, has_beta=True,
             slab_scale=_INV_SQRT8),
]
BY_NAME = {w.name: w for w in WORKLOADS}


def ragged_lengths(rng: np.random.Generator, w: Workload) -> np.ndarray:
    """Global lengths of the packed sequences: lognormal with the stated
    arithmetic mean and coefficient of variation, rounded to multiples of t
    (half-to-even) and at least t.  Explicit lengths are returned as given."""
    if w.fixed_lengths:
        lens = np.asarray(w.fixed_lengths, dtype=np.int64)
        assert np.all(lens % w.t == 0) and np.all(lens >= 0)
        return lens
    sigma_ln = math.sqrt(math.log1p(w.len_cv ** 2))
    mu_ln = math.log(w.mean_len) - 0.5 * sigma_ln ** 2
    x = rng.lognormal(mean=mu_ln, sigma=sigma_ln, size=w.nseq)
    return (w.t * np.maximum(1, np.rint(x / w.t))).astype(np.int64)


def _to_storage(x64: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 draw -> fp32 -> storage (fp32, or bf16 bits via torch's cast)."""
    x32 = x64.astype(np.float32)
    if dtype == DTYPE_F32:
        return x32
    import torch
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _draw(rng, shape, dtype, scale=1.0, loc=0.0, chunk_rows=1024) -> np.ndarray:
    """Normal(loc, scale) draws of ``shape`` in row chunks (same stream as one
    big draw), converted chunk by chunk to the storage dtype."""
    out = np.empty(shape, dtype=np.float32 if dtype == DTYPE_F32 else np.uint16)
    rows = shape[0]
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        x = rng.standard_normal((r1 - r0,) + tuple(shape[1:]))
        if scale != 1.0:
            x *= scale
        if loc != 0.0:
            x += loc
        out[r0:r1] = _to_storage(x, dtype)
    return out


def shard_geometry(w: Workload, lengths: Optional[np.ndarray] = None):
    """(b, s, T, cu_seqlens-or-None) of one rank's shard."""
    if w.ragged:
        assert lengths is not None
        local = lengths // w.t
        cu = np.zeros(len(lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(local)
        s = int(lengths.sum())
        return 1, s, int(cu[-1]), cu
    return w.b, w.s, w.b * w.s // w.t, None


def custom(name: str, *, h: int, t: int, dtype: str = DTYPE_BF16, norm: str = LAYERNORM, eps: float = 1e-5,
           p_drop: float = 0.1, bias: bool = True, residual: bool = True, beta: Optional[bool] = None,
           s: int = 0, b: int = 1, lengths: tuple = (), seed: int = 7, slab_scale: float = _INV_SQRT8) -> Workload:
    """An edge-case shard (odd t, ragged vector tails, empty sequences, ...)."""
    if beta is None:
        beta = norm == LAYERNORM
    return Workload(name, -1, h=h, t=t, dtype=dtype, norm=norm, eps=eps, p_drop=p_drop, has_bias=bias,
                    has_residual=residual, has_beta=beta, slab_scale=slab_scale, s=s, b=b,
                    fixed_lengths=tuple(lengths), seed_override=seed)


def make_inputs(w: Workload, seed: Optional[int] = None, with_dy: bool = True) -> Dict:
    """Seeded synthetic inputs of workload ``w``.

    Draw order is fixed: (ragged) lengths, slabs k = 0..t-1, residual, bias,
    gamma, beta, dy.  Absent tensors are not drawn.
    """
    rng = np.random.default_rng(w.input_seed if seed is None else seed)
    lengths = ragged_lengths(rng, w) if w.ragged else None
    b, s, T, cu = shard_geometry(w, lengths)
    h = w.h
    partials = np.empty((w.t, T, h), dtype=np.float32 if w.dtype == DTYPE_F32 else np.uint16)
    for k in range(w.t):
        partials[k] = _draw(rng, (T, h), w.dtype, scale=w.slab_scale)
    out = dict(workload=w, b=b, s=s, T=T, h=h, t=w.t, partials=partials,
               cu_seqlens=cu, lengths=lengths, seed=w.dropout_seed)
    out["residual"] = _draw(rng, (T, h), w.dtype) if w.has_residual else None
    out["bias"] = _to_storage(0.02 * rng.standard_normal(h), w.dtype) if w.has_bias else None
    out["gamma"] = _to_storage(rng.uniform(0.5, 1.5, size=h), w.dtype)
    out["beta"] = _to_storage(0.1 * rng.standard_normal(h), w.dtype) if w.has_beta else None
    out["dy"] = _draw(rng, (T, h), w.dtype) if with_dy else None
    return out


def with_hard_rows(inp: Dict, *, loc: float, small: float = 0.003, gamma_range=(8.0, 16.0), dy_scale: float = 8.0,
                   seed: int = 5) -> Dict:
    """A copy of a drawn shard whose first four rows are numerically hard for
    the normalisation, with large gamma and dy so that |y| and |dx| reach well
    above 8.  The rows' z (the residual row, or slab 0's row without a
    residual) are:
      0  constant 1.5 (variance exactly 0);
      1  all zero (RMSNorm: mean square exactly 0);
      2  loc + N(0, 1) (|mean| >> std);
      3  N(0, small^2) (variance of the order of eps).
    With a residual, the rows' slabs are zero except slab 0 = -bias (when
    there is a bias), so the slab sum plus bias is exactly 0 and z equals the
    residual row whatever the dropout mask.  Without a residual the rows go
    into slab 0 and the shard must have neither bias nor dropout.  Only values
    are set here; nothing of the region is computed."""
    w = inp["workload"]
    rng = np.random.default_rng(seed)
    T, h = inp["T"], inp["h"]
    assert T >= 4
    out = dict(inp)
    P = inp["partials"].copy()
    res = inp["residual"].copy() if inp["residual"] is not None else None
    bias = inp["bias"]
    if res is None:
        assert bias is None and w.p_drop == 0.0
    rows = {
        0: np.full(h, 1.5),
        1: np.zeros(h),
        2: loc + rng.standard_normal(h),
        3: small * rng.standard_normal(h),
    }
    zero = _to_storage(np.zeros(h), w.dtype)
    for r, vals in rows.items():
        P[:, r] = zero
        if res is not None:
            res[r] = _to_storage(vals, w.dtype)
            if bias is not None:   # slab 0 = -bias: the sign bit flipped, exact in both dtypes
                P[0, r] = (-bias) if w.dtype == DTYPE_F32 else (bias ^ np.uint16(0x8000))
        else:
            P[0, r] = _to_storage(vals, w.dtype)
    out["partials"], out["residual"] = P, res
    out["gamma"] = _to_storage(rng.uniform(*gamma_range, size=h), w.dtype)
    out["dy"] = _draw(rng, (T, h), w.dtype, scale=dy_scale)
    return out


def as_torch(a: Optional[np.ndarray], device):
    """numpy storage array -> torch tensor on ``device`` (bf16 bits are viewed
    as torch.bfloat16; nothing is converted)."""
    if a is None:
        return None
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def device_normal(shape, *, seed: int, device, scale: float = 1.0, dtype=None):
    """Seeded N(0, scale^2) draws generated on ``device`` (torch's Philox
    generator), stored in ``dtype`` (default bfloat16): the inputs of shards too
    large to draw on the host.  The values are fixed by (seed, shape, device
    type); tests copy back only the rows they check.  Drawn in float32 one
    leading index at a time, so the float32 staging stays one slice."""
    import torch
    dtype = torch.bfloat16 if dtype is None else dtype
    g = torch.Generator(device=device).manual_seed(seed)
    out = torch.empty(shape, dtype=dtype, device=device)
    for i in range(shape[0]):
        out[i] = (torch.randn(shape[1:], generator=g, device=device, dtype=torch.float32) * scale).to(dtype)
    return out
