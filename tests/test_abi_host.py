"""The C-ABI library on the host (no GPU needed): it loads, exports every
function include/sp_region.h declares, and rejects invalid arguments with the
documented status before touching the device."""
import ctypes
import os
import re
import subprocess

import pytest

import layernorm_sp_region_amd as spr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sp_region.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sp_region_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(spr.LIB_PATH):
        pytest.skip("library not built (run __graft_entry__.build())")
    return spr.load_library()


def test_header_declares_the_boundary():
    names = declared_functions()
    assert names == sorted(spr.SIGNATURES)
    for required in ("sp_region_fwd", "sp_region_bwd", "sp_region_bwd_workspace_bytes", "sp_region_strerror",
                     "sp_region_abi_version"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", spr.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (sp_region_\w+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported
    for name in declared_functions():
        assert getattr(lib, name) is not None


def test_version_and_strerror(lib):
    assert lib.sp_region_abi_version() == spr.ABI_VERSION == 4
    for st in range(6):
        assert lib.sp_region_strerror(st)
    assert lib.sp_region_strerror(99) == b"unknown status"
    assert lib.sp_region_last_hip_error() == 0


def test_partials_stride_recommendation(lib):
    ps = lib.sp_region_partials_stride
    assert ps(0, 8192, 1) == 0 and ps(10, 0, 1) == 0 and ps(-3, 8, 0) == 0 and ps(10, 8, 7) == 0
    assert ps(2048, 8192, 1) == 2048 * 8192 + 512      # 32 MiB slabs -> 1 KiB apart in residue
    assert ps(2048, 8192, 0) == 2048 * 8192 + 256      # float32: the same 1 KiB
    for T, h, dt in [(1, 8, 1), (3, 520, 1), (5, 4, 0), (2731, 5120, 1), (16384, 8192, 1), (7, 8192, 0)]:
        eb = 2 if dt == 1 else 4
        st = ps(T, h, dt)
        assert st >= T * h
        assert (st * eb) % 2048 == 1024                  # odd multiple of 1 KiB modulo 2 KiB
        assert (st * eb) % 16 == 0                       # a stride the forward accepts
        assert st * eb - T * h * eb < 3072               # the smallest such stride
    import torch
    assert spr.partials_stride(2048, 8192, torch.bfloat16) == ps(2048, 8192, 1)
    assert spr.partials_stride(2048, 8192, torch.float32) == ps(2048, 8192, 0)


def test_workspace_bytes_is_pure(lib):
    ws = lib.sp_region_bwd_workspace_bytes
    assert ws(0, 8192) == 0 and ws(10, 0) == 0 and ws(-1, 8) == 0
    # two slots per block at strides 1 KiB past a multiple of 2 KiB (floats: slot
    # round_up(h, 512) + 256, block round_up(2 * slot, 512) + 256), 256 blocks
    assert ws(2048, 8192) == 256 * (2 * (8192 + 256) + 256) * 4
    # G = min(ceil(T / 4), 256) row blocks: at least 4 rows per block on small shards
    assert ws(64, 512) == 16 * (2 * (512 + 256) + 256) * 4
    assert ws(10, 520) == 3 * (2560 + 256) * 4                   # slot 1024 + 256 floats; 2 slots 2560 -> + 256
    assert ws(1, 8) == 1 * (2 * (512 + 256) + 256) * 4 and ws(1024, 8) == ws(4096, 8) == 256 * 1792 * 4
    assert ws(16384, 8192) == ws(2048, 8192)


# A fake, well-aligned "device" address: validation only looks at its value.
P = 0x10000


def fwd_args(**over):
    a = dict(b=1, s=256, h=512, t=4, eps=1e-5, p=0.1, gamma=P, beta=P, norm=0, dtype=0, rank=0, seed=1,
             partials=P, slab_stride=64 * 512, bias=None, residual=P, cu=None, nseq=0, z=P, y=P, mean=P, rstd=P,
             mask=None, stream=None)
    a.update(over)
    return a


def call_fwd(lib, a):
    return lib.sp_region_fwd(a["b"], a["s"], a["h"], a["t"], a["eps"], a["p"], a["gamma"], a["beta"], a["norm"],
                             a["dtype"], a["rank"], a["seed"], a["partials"], a["slab_stride"], a["bias"],
                             a["residual"], a["cu"], a["nseq"], a["z"], a["y"], a["mean"], a["rstd"], a["mask"],
                             a["stream"])


INVALID, UNSUP, ALIGN = spr.SPR_ERR_INVALID_ARG, spr.SPR_ERR_UNSUPPORTED, spr.SPR_ERR_ALIGNMENT

FWD_CASES = [
    (dict(p=1.0), INVALID), (dict(p=-0.1), INVALID), (dict(p=float("nan")), INVALID),
    (dict(eps=0.0), INVALID), (dict(eps=-1e-5), INVALID), (dict(eps=float("inf")), INVALID),
    (dict(s=258), INVALID),                       # s % t != 0
    (dict(rank=4), INVALID), (dict(rank=-1), INVALID),
    (dict(t=0), INVALID), (dict(t=9, s=252 * 9, rank=0), UNSUP),
    (dict(b=0), INVALID), (dict(h=0), INVALID), (dict(s=-4), INVALID),
    (dict(norm=2), INVALID), (dict(dtype=7), INVALID),
    (dict(h=514), UNSUP),                         # f32 needs h % 4 == 0
    (dict(dtype=1, h=516), UNSUP),                # bf16 needs h % 8 == 0
    (dict(h=8196), UNSUP),                        # above SPR_MAX_H_F32
    (dict(dtype=1, h=16392, slab_stride=64 * 16392), UNSUP),
    (dict(partials=None), INVALID), (dict(gamma=None), INVALID), (dict(z=None), INVALID),
    (dict(y=None), INVALID), (dict(rstd=None), INVALID), (dict(mean=None), INVALID),
    (dict(norm=1, beta=None), INVALID),           # RMSNorm must not get mean
    (dict(norm=1, mean=None), INVALID),           # ... nor beta
    (dict(slab_stride=64 * 512 - 4), INVALID),    # slabs overlap
    (dict(slab_stride=64 * 512 + 2), ALIGN),      # slab starts not 16-byte aligned
    (dict(partials=P + 4), ALIGN), (dict(z=P + 8), ALIGN), (dict(residual=P + 2), ALIGN),
    (dict(mask=P + 1), ALIGN), (dict(mean=P + 4), ALIGN), (dict(bias=P + 4), ALIGN),
    (dict(cu=P, nseq=0), INVALID),                # ragged needs nseq >= 1
    (dict(cu=P, nseq=2, b=2, s=128), INVALID),    # ragged needs b == 1
    (dict(cu=P + 2, nseq=2), ALIGN),
    (dict(nseq=-1), INVALID),
]


@pytest.mark.parametrize("over,status", FWD_CASES, ids=[str(c[0]) for c in FWD_CASES])
def test_fwd_rejects(lib, over, status):
    assert call_fwd(lib, fwd_args(**over)) == status


def call_fwd_slabs(lib, a, slabs):
    table = None if slabs is None else (ctypes.c_void_p * len(slabs))(*slabs)
    return lib.sp_region_fwd_slabs(a["b"], a["s"], a["h"], a["t"], a["eps"], a["p"], a["gamma"], a["beta"],
                                   a["norm"], a["dtype"], a["rank"], a["seed"], table, a["bias"], a["residual"],
                                   a["cu"], a["nseq"], a["z"], a["y"], a["mean"], a["rstd"], a["mask"], a["stream"])


# The strided form's argument checks, except those about the stride itself,
# apply unchanged to the pointer-table form.
SLAB_TABLE_CASES = [c for c in FWD_CASES if not ({"partials", "slab_stride"} & set(c[0]))]


@pytest.mark.parametrize("over,status", SLAB_TABLE_CASES, ids=[str(c[0]) for c in SLAB_TABLE_CASES])
def test_fwd_slabs_rejects(lib, over, status):
    a = fwd_args(**over)
    table = [P + 4096 * k for k in range(max(1, min(a["t"], 8)))]   # t entries (t > 8 is rejected first)
    assert call_fwd_slabs(lib, a, table) == status


def test_fwd_slabs_table_checks(lib):
    four = [P, P + 4096, P + 8192, P + 65536]
    assert call_fwd_slabs(lib, fwd_args(), None) == INVALID
    assert call_fwd_slabs(lib, fwd_args(), [P, None, P, P]) == INVALID
    assert call_fwd_slabs(lib, fwd_args(), [P, P + 8, P, P]) == ALIGN
    assert call_fwd_slabs(lib, fwd_args(s=0), None) == spr.SPR_OK          # T = 0: nothing to read
    assert call_fwd_slabs(lib, fwd_args(p=2.0), four) == INVALID


def test_fwd_empty_shard_is_noop(lib):
    # T == 0: OK without touching any pointer (all NULL).
    a = fwd_args(s=0, partials=None, gamma=None, beta=None, residual=None, z=None, y=None, mean=None, rstd=None)
    assert call_fwd(lib, a) == spr.SPR_OK


# Workspace bytes of the T = 64, h = 512 backward cases: 16 blocks, slots of
# 512 + 256 floats, blocks of round_up(nslots * 768, 512) + 256 floats.
WS2 = 16 * (1536 + 256) * 4
WS3 = 16 * (2560 + 256) * 4


def bwd_args(**over):
    a = dict(b=1, s=256, h=512, t=4, gamma=P, norm=0, dtype=0, dy=P, z=P, mean=P, rstd=P, dres=None, dx=P,
             dgamma=P, dbeta=P, ws=P, ws_bytes=WS2, stream=None)
    a.update(over)
    return a


def call_bwd(lib, a):
    return lib.sp_region_bwd(a["b"], a["s"], a["h"], a["t"], a["gamma"], a["norm"], a["dtype"], a["dy"], a["z"],
                             a["mean"], a["rstd"], a["dres"], a["dx"], a["dgamma"], a["dbeta"], a["ws"],
                             a["ws_bytes"], a["stream"])


BWD_CASES = [
    (dict(ws_bytes=WS2 - 1), INVALID), (dict(ws=None), INVALID),
    (dict(dy=None), INVALID), (dict(z=None), INVALID), (dict(rstd=None), INVALID), (dict(dx=None), INVALID),
    (dict(dgamma=None), INVALID), (dict(gamma=None), INVALID), (dict(mean=None), INVALID),
    (dict(norm=1, dbeta=P, mean=None), INVALID), (dict(norm=1, mean=P, dbeta=None), INVALID),
    (dict(s=257), INVALID), (dict(t=0), INVALID), (dict(h=510), UNSUP), (dict(dtype=2), INVALID),
    (dict(dx=P + 4), ALIGN), (dict(ws=P + 8), ALIGN), (dict(dres=P + 2), ALIGN), (dict(dgamma=P + 4), ALIGN),
]


@pytest.mark.parametrize("over,status", BWD_CASES, ids=[str(c[0]) for c in BWD_CASES])
def test_bwd_rejects(lib, over, status):
    assert call_bwd(lib, bwd_args(**over)) == status


def bwd_dropout_args(**over):
    a = dict(bwd_args(ws_bytes=WS3), p=0.1, rank=1, seed=7, cu=None, nseq=0, dpartial=P, dbias=P)
    a.update(over)
    return a


def call_bwd_dropout(lib, a):
    return lib.sp_region_bwd_dropout(a["b"], a["s"], a["h"], a["t"], a["gamma"], a["norm"], a["dtype"], a["dy"],
                                     a["z"], a["mean"], a["rstd"], a["dres"], a["p"], a["rank"], a["seed"], a["cu"],
                                     a["nseq"], a["dx"], a["dpartial"], a["dgamma"], a["dbeta"], a["dbias"], a["ws"],
                                     a["ws_bytes"], a["stream"])


BWD_DROPOUT_CASES = BWD_CASES[2:] + [
    (dict(ws_bytes=WS3 - 1), INVALID),          # three partial slots per block
    (dict(ws_bytes=WS2), INVALID),
    (dict(ws=None), INVALID),
    (dict(dpartial=None), INVALID),
    (dict(p=1.0), INVALID), (dict(p=-0.1), INVALID), (dict(p=float("nan")), INVALID),
    (dict(rank=4), INVALID), (dict(rank=-1), INVALID),
    (dict(cu=P, nseq=0), INVALID), (dict(cu=P, nseq=2, b=2), INVALID), (dict(nseq=-1), INVALID),
    (dict(cu=P + 2, nseq=1), ALIGN), (dict(dpartial=P + 4), ALIGN), (dict(dbias=P + 8), ALIGN),
]


@pytest.mark.parametrize("over,status", BWD_DROPOUT_CASES, ids=[str(c[0]) for c in BWD_DROPOUT_CASES])
def test_bwd_dropout_rejects(lib, over, status):
    assert call_bwd_dropout(lib, bwd_dropout_args(**over)) == status


def test_bwd_dropout_workspace_bytes(lib):
    ws3, ws2 = lib.sp_region_bwd_dropout_workspace_bytes, lib.sp_region_bwd_workspace_bytes
    assert ws3(0, 64) == 0 and ws3(5, 0) == 0
    for T, h in [(64, 512), (2048, 8192), (100000, 5120), (1, 8)]:
        slot = (h + 511) // 512 * 512 + 256
        blocks = min((T + 3) // 4, 256)
        assert ws2(T, h) == blocks * ((2 * slot + 511) // 512 * 512 + 256) * 4
        assert ws3(T, h) == blocks * ((3 * slot + 511) // 512 * 512 + 256) * 4


def test_bwd_dropout_empty_shard_needs_no_outputs(lib):
    # T = 0: nothing to launch beyond the zero-filled parameter gradients, which
    # need a device; without one only the argument checks can be exercised.
    assert call_bwd_dropout(lib, bwd_dropout_args(s=0, dpartial=None, ws=None, ws_bytes=0, p=2.0)) == INVALID


def call_bwd_accumulate(lib, a):
    return lib.sp_region_bwd_accumulate(a["b"], a["s"], a["h"], a["t"], a["gamma"], a["norm"], a["dtype"], a["dy"],
                                        a["z"], a["mean"], a["rstd"], a["dres"], a["p"], a["rank"], a["seed"],
                                        a["cu"], a["nseq"], a["dx"], a["dpartial"], a["dgamma"], a["dbeta"],
                                        a["dbias"], a["ws"], a["ws_bytes"], a["stream"])


# With dpartial the accumulating call checks what sp_region_bwd_dropout checks;
# without it, the two-slot workspace of sp_region_bwd suffices, dbias must be
# NULL and the dropout arguments are still checked.
BWD_ACCUMULATE_CASES = [c for c in BWD_DROPOUT_CASES if c[0] != dict(dpartial=None)] + [
    (dict(dpartial=None), INVALID),                           # dbias without dpartial
    (dict(dpartial=None, dbias=None, ws_bytes=WS2 - 1), INVALID),
    (dict(dpartial=None, dbias=None, p=1.0), INVALID),
    (dict(dpartial=None, dbias=None, rank=4), INVALID),
    (dict(dpartial=None, dbias=None, dgamma=None), INVALID),
    (dict(dpartial=None, dbias=None, dgamma=P + 4), ALIGN),
]


@pytest.mark.parametrize("over,status", BWD_ACCUMULATE_CASES, ids=[str(c[0]) for c in BWD_ACCUMULATE_CASES])
def test_bwd_accumulate_rejects(lib, over, status):
    assert call_bwd_accumulate(lib, bwd_dropout_args(**over)) == status


def test_bwd_accumulate_empty_shard_launches_nothing(lib):
    # T = 0 adds nothing to the main gradients: OK with no launch at all, so
    # the (host) buffers here are never touched; the arguments are still checked.
    a = bwd_dropout_args(s=0, dy=None, z=None, mean=None, rstd=None, dx=None, ws=None, ws_bytes=0)
    assert call_bwd_accumulate(lib, dict(a, dpartial=None, dbias=None)) == spr.SPR_OK
    assert call_bwd_accumulate(lib, a) == spr.SPR_OK
    assert call_bwd_accumulate(lib, dict(a, p=2.0)) == INVALID


def test_copy_rejects(lib):
    assert lib.sp_region_hbm_copy(P, P, 15, None) == INVALID
    assert lib.sp_region_hbm_copy(None, P, 16, None) == INVALID
    assert lib.sp_region_hbm_copy(P + 4, P, 16, None) == ALIGN
    assert lib.sp_region_hbm_copy(None, None, 0, None) == spr.SPR_OK


def test_python_layer_rejects_host_tensors():
    # The C entry points take raw device pointers and cannot tell host memory
    # from device memory; the binding refuses CPU tensors before any call.
    import torch
    T, h, t = 8, 64, 2
    P = torch.zeros(t, T, h)
    g = torch.ones(h)
    with pytest.raises(ValueError):
        spr.fwd(P, g, g, b=1, s=t * T, t=t, rank=0, eps=1e-5, p_drop=0.0, seed=1)
    with pytest.raises(ValueError):
        spr.fwd([P[0], P[1]], g, g, b=1, s=t * T, t=t, rank=0, eps=1e-5, p_drop=0.0, seed=1)
    z = torch.zeros(T, h)
    st = torch.ones(T)
    with pytest.raises(ValueError):
        spr.bwd(z, z, st, st, g, b=1, s=t * T, t=t)
    with pytest.raises(ValueError):
        spr.bwd_dropout(z, z, st, st, g, b=1, s=t * T, t=t, rank=0, p_drop=0.1, seed=1)


def test_python_layer_checks_cu_seqlens():
    spr.check_cu_seqlens([0, 3, 3, 8], 8)
    for bad, T in (([1, 8], 8), ([0, 5, 4, 8], 8), ([0, 7], 8), ([0], 0)):
        with pytest.raises(ValueError):
            spr.check_cu_seqlens(bad, T)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(spr, "LIB_PATH", str(tmp_path / "absent.so"))
    monkeypatch.setattr(spr, "_lib", None)
    with pytest.raises(ImportError):
        spr.load_library()
