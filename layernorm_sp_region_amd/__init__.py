"""MI355X-native fused sequence-parallel region: Python binding of libsp_region.so.

The sequence-parallel (non-TP) region of a Megatron TP+SP block on one rank's
shard [s/t][b][h] (hpc.payai.win lesson 7 "Sequence parallelism"):

    forward   z = residual + dropout(sum_k P_k + bias);  y = LayerNorm/RMSNorm(z)
    backward  dx, dgamma, dbeta

This module only marshals arguments: it checks torch tensors (device, dtype,
shape, contiguity), allocates outputs with torch, and calls the C ABI
(include/sp_region.h) on torch's current stream.  Every step of the
computation runs in the library's HIP kernels.  If the library has not been
built the calls raise; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from collections import namedtuple
from typing import Optional, Sequence, Union

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsp_region.so")

SPR_OK, SPR_ERR_INVALID_ARG, SPR_ERR_UNSUPPORTED, SPR_ERR_ALIGNMENT, SPR_ERR_HIP, SPR_ERR_SCRATCH = range(6)
SPR_F32, SPR_BF16 = 0, 1
SPR_LAYERNORM, SPR_RMSNORM = 0, 1
ABI_VERSION = 4
NOALLOC_SCRATCH_BYTES = 32 << 20     # SPR_NOALLOC_SCRATCH_BYTES

# Every symbol include/sp_region.h declares, with its ctypes signature.
_VP, _I64, _I32, _U64, _F32, _SZ = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint64,
                                    ctypes.c_float, ctypes.c_size_t)
SIGNATURES = {
    "sp_region_abi_version": (ctypes.c_int, []),
    "sp_region_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "sp_region_last_hip_error": (ctypes.c_int, []),
    "sp_region_time_next_call": (ctypes.c_int, [_VP, _VP]),
    "sp_region_fwd": (ctypes.c_int, [_I64, _I64, _I64, _I32, _F32, _F32, _VP, _VP, _I32, _I32, _I32, _U64,
                                     _VP, _I64, _VP, _VP, _VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP]),
    "sp_region_partials_stride": (_I64, [_I64, _I64, _I32]),
    "sp_region_fwd_slabs": (ctypes.c_int, [_I64, _I64, _I64, _I32, _F32, _F32, _VP, _VP, _I32, _I32, _I32, _U64,
                                           _VP, _VP, _VP, _VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP]),
    "sp_region_bwd_workspace_bytes": (_SZ, [_I64, _I64]),
    "sp_region_bwd": (ctypes.c_int, [_I64, _I64, _I64, _I32, _VP, _I32, _I32, _VP, _VP, _VP, _VP, _VP,
                                     _VP, _VP, _VP, _VP, _SZ, _VP]),
    "sp_region_bwd_noalloc": (ctypes.c_int, [_I64, _I64, _I64, _I32, _VP, _I32, _I32, _VP, _VP, _VP, _VP, _VP,
                                             _VP, _VP, _VP, _VP]),
    "sp_region_bwd_dropout_workspace_bytes": (_SZ, [_I64, _I64]),
    "sp_region_bwd_dropout": (ctypes.c_int, [_I64, _I64, _I64, _I32, _VP, _I32, _I32, _VP, _VP, _VP, _VP, _VP,
                                             _F32, _I32, _U64, _VP, _I32,
                                             _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "sp_region_bwd_accumulate": (ctypes.c_int, [_I64, _I64, _I64, _I32, _VP, _I32, _I32, _VP, _VP, _VP, _VP, _VP,
                                                _F32, _I32, _U64, _VP, _I32,
                                                _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "sp_region_hbm_copy": (ctypes.c_int, [_VP, _VP, _SZ, _VP]),
    "sp_region_set_bwd_launches": (ctypes.c_int, [_I32]),
    "sp_region_cv_within": (ctypes.c_int, [_VP, _I32, _I32, _VP]),
    "sp_region_bucket_by_tokens": (ctypes.c_int, [_VP, _I32, _I32, _I64, _VP, _VP, _VP]),
    "sp_region_sp_gate": (ctypes.c_int, [_VP, _I32, ctypes.c_double, _I32, ctypes.c_double, _VP]),
    "sp_region_shard_layout": (ctypes.c_int, [_VP, _I32, _I32, _VP, _VP, _VP]),
}

_lib = None


def load_library(reload: bool = False):
    """Load the in-tree libsp_region.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and not reload:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python __graft_entry__.py` "
                          "(the region has no non-HIP implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.sp_region_abi_version() != ABI_VERSION:
        raise ImportError(f"libsp_region ABI {lib.sp_region_abi_version()} != binding ABI {ABI_VERSION}")
    _lib = lib
    return lib


class SpRegionError(RuntimeError):
    def __init__(self, fn: str, status: int):
        lib = load_library()
        msg = lib.sp_region_strerror(status).decode()
        if status == SPR_ERR_HIP:
            msg += f" (hipError_t {lib.sp_region_last_hip_error()})"
        super().__init__(f"{fn}: {msg}")
        self.status = status


def _check(fn: str, status: int):
    if status != SPR_OK:
        raise SpRegionError(fn, status)


FwdOut = namedtuple("FwdOut", "z y mean rstd mask")
BwdOut = namedtuple("BwdOut", "dx dgamma dbeta")


def _norm_code(norm: Union[str, int]) -> int:
    if norm in ("layernorm", SPR_LAYERNORM):
        return SPR_LAYERNORM
    if norm in ("rmsnorm", SPR_RMSNORM):
        return SPR_RMSNORM
    raise ValueError(f"unknown norm {norm!r}")


def _dtype_code(dt) -> int:
    import torch
    if dt == torch.bfloat16:
        return SPR_BF16
    if dt == torch.float32:
        return SPR_F32
    raise TypeError(f"activations must be bfloat16 or float32, got {dt}")


def _current_stream(dev) -> int:
    """The HIP handle of the caller's current stream on device dev (torch's
    raw-stream accessor when present: ~0.1 us against ~1.7 us for building a
    torch.cuda.Stream object on every call)."""
    import torch
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None and dev.index is not None:
        return raw(dev.index)
    return torch.cuda.current_stream(dev).cuda_stream


def _ptr(x) -> Optional[int]:
    return None if x is None else x.data_ptr()


def _require(x, name, device, dtype=None, shape=None):
    if x is None:
        return
    if not x.is_cuda or x.device != device:
        raise ValueError(f"{name} must be on {device}")
    if dtype is not None and x.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {x.dtype}")
    if shape is not None and x.shape != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(x.shape)}")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def local_tokens(b: int, s: int, t: int) -> int:
    return b * s // t


def check_cu_seqlens(cu: Sequence[int], T: int) -> None:
    """Host check of the packed-batch offsets (the kernels trust them)."""
    cu = [int(x) for x in cu]
    if len(cu) < 2 or cu[0] != 0 or cu[-1] != T or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must start at 0, end at T and be non-decreasing")


def fwd(partials, gamma, beta=None, *, bias=None, residual=None, b: int, s: int, t: int, rank: int,
        eps: float, p_drop: float, seed: int, norm: Union[str, int] = "layernorm", cu_seqlens=None,
        return_mask: bool = False, out: Optional[FwdOut] = None) -> FwdOut:
    """Forward of the region.

    partials: [t][T][h] tensor (slab k = partials[k]; each slab row-major; the
    slab stride may exceed T*h), or a list of t separate [T][h] tensors
    (sp_region_fwd_slabs: slab k read through its own pointer, wherever it
    lives).  cu_seqlens: None (uniform shard) or the
    host list / CPU tensor / int32 CUDA tensor of local row offsets of a packed
    batch (b must be 1; a CUDA tensor is trusted as-is).  `out` may supply
    preallocated outputs.  Returns FwdOut(z, y, mean, rstd, mask).
    """
    import torch
    lib = load_library()
    nc = _norm_code(norm)
    slab_list = None
    if isinstance(partials, (list, tuple)):
        slab_list = list(partials)
        if len(slab_list) != t or t < 1:
            raise ValueError(f"expected {t} slab tensors, got {len(slab_list)}")
        first = slab_list[0]
        dev, dt = first.device, first.dtype
        if first.dim() != 2:
            raise ValueError("each slab must be [T][h]")
        T, h = first.shape
        for k, sk in enumerate(slab_list):
            _require(sk, f"slab {k}", dev, dt, (T, h))
    else:
        dev = partials.device
        dt = partials.dtype
        if partials.dim() != 3 or partials.shape[0] != t:
            raise ValueError(f"partials must be [t={t}][T][h], got {tuple(partials.shape)}")
        _, T, h = partials.shape
        if not partials.is_cuda:
            raise ValueError("partials must be a CUDA tensor")
        # Strides of size-0/1 dims carry no layout information (numpy gives an
        # inserted axis stride 0), so only meaningful ones are checked.
        if T > 0 and ((h > 1 and partials.stride(2) != 1) or (T > 1 and partials.stride(1) != h)):
            raise ValueError("each slab of partials must be row-major contiguous")
        slab_stride = partials.stride(0) if t > 1 else T * h
    dcode = _dtype_code(dt)
    if T != local_tokens(b, s, t):
        raise ValueError(f"partials hold {T} rows, expected b*s/t = {local_tokens(b, s, t)}")
    _require(gamma, "gamma", dev, dt, (h,))
    _require(beta, "beta", dev, dt, (h,))
    _require(bias, "bias", dev, dt, (h,))
    _require(residual, "residual", dev, dt, (T, h))
    cu_dev, nseq = _cu_on_device(cu_seqlens, T, dev)
    ln = nc == SPR_LAYERNORM
    if out is None:
        z = torch.empty((T, h), dtype=dt, device=dev)
        y = torch.empty((T, h), dtype=dt, device=dev)
        mean = torch.empty((T,), dtype=torch.float32, device=dev) if ln else None
        rstd = torch.empty((T,), dtype=torch.float32, device=dev)
        mask = torch.empty((T, h), dtype=torch.uint8, device=dev) if return_mask else None
    else:
        z, y, mean, rstd, mask = out
        _require(z, "z", dev, dt, (T, h))
        _require(y, "y", dev, dt, (T, h))
        _require(mean, "mean", dev, torch.float32, (T,))
        _require(rstd, "rstd", dev, torch.float32, (T,))
        _require(mask, "mask", dev, torch.uint8, (T, h))
    stream = _current_stream(dev)
    if slab_list is not None:
        table = (ctypes.c_void_p * t)(*[sk.data_ptr() for sk in slab_list])
        st = lib.sp_region_fwd_slabs(b, s, h, t, float(eps), float(p_drop), _ptr(gamma), _ptr(beta), nc, dcode,
                                     rank, int(seed) & 0xFFFFFFFFFFFFFFFF, table, _ptr(bias), _ptr(residual),
                                     _ptr(cu_dev), nseq, _ptr(z), _ptr(y), _ptr(mean), _ptr(rstd), _ptr(mask),
                                     stream)
        _check("sp_region_fwd_slabs", st)
        return FwdOut(z, y, mean, rstd, mask)
    st = lib.sp_region_fwd(b, s, h, t, float(eps), float(p_drop), _ptr(gamma), _ptr(beta), nc, dcode, rank,
                           int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(partials), slab_stride, _ptr(bias),
                           _ptr(residual), _ptr(cu_dev), nseq, _ptr(z), _ptr(y), _ptr(mean), _ptr(rstd),
                           _ptr(mask), stream)
    _check("sp_region_fwd", st)
    return FwdOut(z, y, mean, rstd, mask)


def time_next_call(start, stop) -> None:
    """The next region call on this thread stamps its first kernel's start
    into `start` and its last kernel's end into `stop` (torch.cuda.Event
    objects with timing enabled, already recorded once so that they exist)."""
    h0 = start.cuda_event if start is not None else None
    h1 = stop.cuda_event if stop is not None else None
    _check("sp_region_time_next_call", load_library().sp_region_time_next_call(h0, h1))


def partials_stride(T: int, h: int, dtype) -> int:
    """Recommended element stride between the t partial slabs (see
    sp_region_partials_stride in include/sp_region.h)."""
    return int(load_library().sp_region_partials_stride(T, h, _dtype_code(dtype)))


def empty_partials(t: int, T: int, h: int, dtype, device):
    """Uninitialised [t][T][h] slabs laid out with the recommended stride."""
    import torch
    stride = partials_stride(T, h, dtype) if T * h > 0 else T * h
    buf = torch.empty(t * stride, dtype=dtype, device=device)
    return buf.as_strided((t, T, h), (stride, h, 1))


def workspace_bytes(T: int, h: int) -> int:
    return int(load_library().sp_region_bwd_workspace_bytes(T, h))


def _cu_on_device(cu_seqlens, T, dev):
    """(device int32 offsets or None, nseq).  Host offsets are checked here
    (the library cannot check a device array without a sync)."""
    import torch
    if cu_seqlens is None:
        return None, 0
    if isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.is_cuda:
        _require(cu_seqlens, "cu_seqlens", dev, torch.int32)
        cu_dev = cu_seqlens
    else:
        cu_list = [int(x) for x in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
        check_cu_seqlens(cu_list, T)
        cu_dev = torch.tensor(cu_list, dtype=torch.int32, device=dev)
    return cu_dev, cu_dev.numel() - 1


def bwd(dy, z, mean, rstd, gamma, *, b: int, s: int, t: int, norm: Union[str, int] = "layernorm",
        dres_in=None, want_dbeta: bool = True, workspace=None, out: Optional[BwdOut] = None,
        accumulate: bool = False) -> BwdOut:
    """Backward of the region's normalisation.  Returns BwdOut(dx, dgamma, dbeta)
    (dbeta None for RMSNorm or when want_dbeta is False).  accumulate=True
    adds the parameter gradients into out's float32 dgamma/dbeta (main-grad
    buffers, sp_region_bwd_accumulate) instead of overwriting them."""
    import torch
    lib = load_library()
    nc = _norm_code(norm)
    dev = z.device
    dt = z.dtype
    dcode = _dtype_code(dt)
    T, h = z.shape
    if T != local_tokens(b, s, t):
        raise ValueError(f"z holds {T} rows, expected b*s/t = {local_tokens(b, s, t)}")
    ln = nc == SPR_LAYERNORM
    _require(z, "z", dev, dt, (T, h))
    _require(dy, "dy", dev, dt, (T, h))
    _require(dres_in, "dres_in", dev, dt, (T, h))
    _require(gamma, "gamma", dev, dt, (h,))
    _require(mean, "mean", dev, torch.float32, (T,))
    _require(rstd, "rstd", dev, torch.float32, (T,))
    if ln and mean is None:
        raise ValueError("LayerNorm backward needs mean")
    need = workspace_bytes(T, h)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    _require(workspace, "workspace", dev, torch.uint8)
    if out is None:
        if accumulate:
            raise ValueError("accumulate=True needs out= holding the main-grad buffers")
        dx = torch.empty((T, h), dtype=dt, device=dev)
        dgamma = torch.empty((h,), dtype=torch.float32, device=dev)
        dbeta = torch.empty((h,), dtype=torch.float32, device=dev) if (ln and want_dbeta) else None
    else:
        dx, dgamma, dbeta = out
        _require(dx, "dx", dev, dt, (T, h))
        _require(dgamma, "dgamma", dev, torch.float32, (h,))
        _require(dbeta, "dbeta", dev, torch.float32, (h,))
    stream = _current_stream(dev)
    if accumulate:
        st = lib.sp_region_bwd_accumulate(b, s, h, t, _ptr(gamma), nc, dcode, _ptr(dy), _ptr(z),
                                          _ptr(mean if ln else None), _ptr(rstd), _ptr(dres_in), 0.0, 0, 0, None, 0,
                                          _ptr(dx), None, _ptr(dgamma), _ptr(dbeta), None, _ptr(workspace),
                                          workspace.numel(), stream)
        _check("sp_region_bwd_accumulate", st)
    else:
        st = lib.sp_region_bwd(b, s, h, t, _ptr(gamma), nc, dcode, _ptr(dy), _ptr(z), _ptr(mean if ln else None),
                               _ptr(rstd), _ptr(dres_in), _ptr(dx), _ptr(dgamma), _ptr(dbeta), _ptr(workspace),
                               workspace.numel(), stream)
        _check("sp_region_bwd", st)
    return BwdOut(dx, dgamma, dbeta)


def bwd_noalloc(dy, z, mean, rstd, gamma, *, b: int, s: int, t: int, out: BwdOut,
                norm: Union[str, int] = "layernorm", dres_in=None) -> BwdOut:
    """sp_region_bwd_noalloc: bwd() with the library's static device scratch as
    its workspace, for callers that cannot allocate.  Allocates nothing, so
    the outputs come in `out` (dx, dgamma, and dbeta or None)."""
    import torch
    lib = load_library()
    nc = _norm_code(norm)
    dev, dt = z.device, z.dtype
    dcode = _dtype_code(dt)
    T, h = z.shape
    if T != local_tokens(b, s, t):
        raise ValueError(f"z holds {T} rows, expected b*s/t = {local_tokens(b, s, t)}")
    ln = nc == SPR_LAYERNORM
    dx, dgamma, dbeta = out
    for x, name, dtype_, shape in ((z, "z", dt, (T, h)), (dy, "dy", dt, (T, h)), (dres_in, "dres_in", dt, (T, h)),
                                   (gamma, "gamma", dt, (h,)), (mean, "mean", torch.float32, (T,)),
                                   (rstd, "rstd", torch.float32, (T,)), (dx, "dx", dt, (T, h)),
                                   (dgamma, "dgamma", torch.float32, (h,)), (dbeta, "dbeta", torch.float32, (h,))):
        _require(x, name, dev, dtype_, shape)
    stream = _current_stream(dev)
    st = lib.sp_region_bwd_noalloc(b, s, h, t, _ptr(gamma), nc, dcode, _ptr(dy), _ptr(z), _ptr(mean if ln else None),
                                   _ptr(rstd), _ptr(dres_in), _ptr(dx), _ptr(dgamma), _ptr(dbeta), stream)
    _check("sp_region_bwd_noalloc", st)
    return out


def dropout_workspace_bytes(T: int, h: int) -> int:
    return int(load_library().sp_region_bwd_dropout_workspace_bytes(T, h))


BwdDropoutOut = namedtuple("BwdDropoutOut", "dx dpartial dgamma dbeta dbias")


def bwd_dropout(dy, z, mean, rstd, gamma, *, b: int, s: int, t: int, rank: int, p_drop: float, seed: int,
                norm: Union[str, int] = "layernorm", cu_seqlens=None, dres_in=None, want_dbeta: bool = True,
                want_dbias: bool = True, workspace=None, out: Optional["BwdDropoutOut"] = None,
                accumulate: bool = False) -> "BwdDropoutOut":
    """Backward of the region through the dropout and the slab sum: BwdOut's
    dx, dgamma, dbeta plus dpartial (the gradient of every slab) and dbias.
    p_drop, rank, seed and cu_seqlens are the forward's.  accumulate=True
    adds dgamma/dbeta/dbias into out's float32 buffers (main gradients)."""
    import torch
    lib = load_library()
    nc = _norm_code(norm)
    dev = z.device
    dt = z.dtype
    dcode = _dtype_code(dt)
    T, h = z.shape
    if T != local_tokens(b, s, t):
        raise ValueError(f"z holds {T} rows, expected b*s/t = {local_tokens(b, s, t)}")
    ln = nc == SPR_LAYERNORM
    _require(z, "z", dev, dt, (T, h))
    _require(dy, "dy", dev, dt, (T, h))
    _require(dres_in, "dres_in", dev, dt, (T, h))
    _require(gamma, "gamma", dev, dt, (h,))
    _require(mean, "mean", dev, torch.float32, (T,))
    _require(rstd, "rstd", dev, torch.float32, (T,))
    if ln and mean is None:
        raise ValueError("LayerNorm backward needs mean")
    cu_dev, nseq = _cu_on_device(cu_seqlens, T, dev)
    need = dropout_workspace_bytes(T, h)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    _require(workspace, "workspace", dev, torch.uint8)
    if out is None:
        if accumulate:
            raise ValueError("accumulate=True needs out= holding the main-grad buffers")
        dx = torch.empty((T, h), dtype=dt, device=dev)
        dpartial = torch.empty((T, h), dtype=dt, device=dev)
        dgamma = torch.empty((h,), dtype=torch.float32, device=dev)
        dbeta = torch.empty((h,), dtype=torch.float32, device=dev) if (ln and want_dbeta) else None
        dbias = torch.empty((h,), dtype=torch.float32, device=dev) if want_dbias else None
    else:
        dx, dpartial, dgamma, dbeta, dbias = out
        _require(dx, "dx", dev, dt, (T, h))
        _require(dpartial, "dpartial", dev, dt, (T, h))
        _require(dgamma, "dgamma", dev, torch.float32, (h,))
        _require(dbeta, "dbeta", dev, torch.float32, (h,))
        _require(dbias, "dbias", dev, torch.float32, (h,))
    stream = _current_stream(dev)
    fn = "sp_region_bwd_accumulate" if accumulate else "sp_region_bwd_dropout"
    st = getattr(lib, fn)(b, s, h, t, _ptr(gamma), nc, dcode, _ptr(dy), _ptr(z),
                          _ptr(mean if ln else None), _ptr(rstd), _ptr(dres_in), float(p_drop), rank,
                          int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(cu_dev), nseq, _ptr(dx), _ptr(dpartial),
                          _ptr(dgamma), _ptr(dbeta), _ptr(dbias), _ptr(workspace), workspace.numel(), stream)
    _check(fn, st)
    return BwdDropoutOut(dx, dpartial, dgamma, dbeta, dbias)


def set_bwd_launches(n: int) -> None:
    """1: small-shard backward in one launch (default); 2: always the partials' two launches."""
    _check("sp_region_set_bwd_launches", load_library().sp_region_set_bwd_launches(n))


def hbm_copy(src, dst) -> None:
    """Calibration copy of src's bytes into dst (same size, 16-byte multiple)."""
    import torch
    lib = load_library()
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("src and dst sizes differ")
    stream = _current_stream(src.device)
    _check("sp_region_hbm_copy", lib.sp_region_hbm_copy(src.data_ptr(), dst.data_ptr(), n, stream))


# ---------------------------------------------------------------------------
# Host-side batch planning (argument marshalling only; the library decides).
# ---------------------------------------------------------------------------
MAX_CV_BP = 1500
GATE_CV_BP = 1800
GATE_RS_WAIT = 0.22


def _lengths_array(lengths):
    import numpy as np
    a = np.ascontiguousarray(np.asarray(lengths, dtype=np.int64))
    if a.ndim != 1:
        raise ValueError("lengths must be one-dimensional")
    if a.size and (a.min() < 0 or a.max() > 2 ** 31 - 1):
        raise ValueError("lengths out of range")
    return np.ascontiguousarray(a.astype(np.int32))


def cv_within(lengths, cv_bp: int) -> bool:
    import numpy as np
    a = _lengths_array(lengths)
    out = np.zeros(1, dtype=np.int32)
    _check("sp_region_cv_within", load_library().sp_region_cv_within(a.ctypes.data, a.size, cv_bp, out.ctypes.data))
    return bool(out[0])


def bucket_by_tokens(lengths, max_cv_bp: int = MAX_CV_BP, max_tokens: int = 0):
    """(order, starts): bucket k is order[starts[k]:starts[k+1]]."""
    import numpy as np
    a = _lengths_array(lengths)
    order = np.zeros(max(a.size, 1), dtype=np.int32)
    starts = np.zeros(a.size + 1, dtype=np.int32)
    nb = np.zeros(1, dtype=np.int32)
    st = load_library().sp_region_bucket_by_tokens(a.ctypes.data, a.size, max_cv_bp, max_tokens, order.ctypes.data,
                                                   starts.ctypes.data, nb.ctypes.data)
    _check("sp_region_bucket_by_tokens", st)
    return order[:a.size].tolist(), starts[:nb[0] + 1].tolist()


def sp_gate(lengths, rs_wait_share: float, max_cv_bp: int = GATE_CV_BP,
            max_rs_wait_share: float = GATE_RS_WAIT) -> bool:
    import numpy as np
    a = _lengths_array(lengths)
    out = np.zeros(1, dtype=np.int32)
    st = load_library().sp_region_sp_gate(a.ctypes.data, a.size, float(rs_wait_share), max_cv_bp,
                                          float(max_rs_wait_share), out.ctypes.data)
    _check("sp_region_sp_gate", st)
    return bool(out[0])


def shard_layout(lengths, t: int):
    """(padded lengths, local cu_seqlens, local token count T)."""
    import numpy as np
    a = _lengths_array(lengths)
    padded = np.zeros(max(a.size, 1), dtype=np.int32)
    cu = np.zeros(a.size + 1, dtype=np.int32)
    T = np.zeros(1, dtype=np.int64)
    st = load_library().sp_region_shard_layout(a.ctypes.data, a.size, t, padded.ctypes.data, cu.ctypes.data,
                                               T.ctypes.data)
    _check("sp_region_shard_layout", st)
    return padded[:a.size].tolist(), cu.tolist(), int(T[0])


# ---------------------------------------------------------------------------
# torch.autograd wiring (argument marshalling around fwd / bwd_dropout).
# ---------------------------------------------------------------------------
def _autograd_function():
    import torch

    class SPRegion(torch.autograd.Function):
        """(gamma, beta, bias, residual, cfg, *slabs) -> (y, z).  The slabs are
        one [t][T][h] tensor, or t separate [T][h] tensors (cfg["slab_list"]).

        Backward: y's gradient is dy, z's gradient (z is also the next
        residual stream) is dres_in; returns the gradients of gamma, beta,
        bias and residual, then of the slabs (the same dpartial for every
        slab)."""

        @staticmethod
        def forward(ctx, gamma, beta, bias, residual, cfg, *slabs):
            fcfg = {k: v for k, v in cfg.items() if k != "slab_list"}
            partials = list(slabs) if cfg["slab_list"] else slabs[0]
            o = fwd(partials, gamma, beta, bias=bias, residual=residual, **fcfg)
            ctx.save_for_backward(o.z, o.mean, o.rstd, gamma)
            ctx.cfg = cfg
            ctx.shapes = [tuple(x.shape) for x in slabs]
            ctx.flags = (beta is not None, bias is not None, residual is not None)
            return o.y, o.z

        @staticmethod
        def backward(ctx, dy, dz):
            z, mean, rstd, gamma = ctx.saved_tensors
            cfg = ctx.cfg
            has_beta, has_bias, has_res = ctx.flags
            dy = torch.zeros_like(z) if dy is None else dy.contiguous()
            g = bwd_dropout(dy, z, mean, rstd, gamma, b=cfg["b"], s=cfg["s"], t=cfg["t"], rank=cfg["rank"],
                            p_drop=cfg["p_drop"], seed=cfg["seed"], norm=cfg.get("norm", "layernorm"),
                            cu_seqlens=cfg.get("cu_seqlens"), dres_in=None if dz is None else dz.contiguous(),
                            want_dbeta=has_beta, want_dbias=has_bias)
            if cfg["slab_list"]:
                dslabs = tuple(g.dpartial for _ in ctx.shapes)
            else:
                dslabs = (g.dpartial.unsqueeze(0).expand(ctx.shapes[0]),)
            return (g.dgamma.to(gamma.dtype), None if g.dbeta is None else g.dbeta.to(gamma.dtype),
                    None if g.dbias is None else g.dbias.to(gamma.dtype), g.dx if has_res else None,
                    None) + dslabs

    return SPRegion


_SPREGION = None


def region(partials, gamma, beta=None, *, bias=None, residual=None, b: int, s: int, t: int, rank: int,
           eps: float, p_drop: float, seed: int, norm: Union[str, int] = "layernorm", cu_seqlens=None):
    """Autograd-aware region: returns (y, z); gradients flow to partials (every
    slab receives dpartial), gamma, beta, bias and residual.  partials is one
    [t][T][h] tensor or a list of t [T][h] tensors (each then receives its
    own gradient).  dgamma, dbeta and dbias are computed in float32 and
    returned in the parameters' dtype."""
    global _SPREGION
    if _SPREGION is None:
        _SPREGION = _autograd_function()
    slab_list = isinstance(partials, (list, tuple))
    slabs = tuple(partials) if slab_list else (partials,)
    cfg = dict(b=b, s=s, t=t, rank=rank, eps=eps, p_drop=p_drop, seed=seed, norm=norm, cu_seqlens=cu_seqlens,
               slab_list=slab_list)
    return _SPREGION.apply(gamma, beta, bias, residual, cfg, *slabs)
