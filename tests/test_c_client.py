"""The library used from plain C (tests/c_client/sp_region_client.c): the
header compiles as strict C99 on its own, the host-only entry points agree
with the oracle's batch planning, and (GPU) a forward + dropout backward run
through the C ABI with the HIP runtime's allocator matches the CPU oracle.

Bars on the GPU case as in the other parity tests: z and the dropped set bit
for bit; bf16 y, dx and dpartial within half a bf16 ulp of the float64 value
plus a float32 slack; dgamma, dbeta and dbias within 1e-4 of their
conditioning scales.
"""
import os
import subprocess

import numpy as np
import pytest
import torch

import layernorm_sp_region_amd as spr
import oracle.batching as ob
import oracle.region as ref
import workloads as W
from test_gpu_parity import assert_out_close

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "tests", "c_client", "sp_region_client")


def client_or_skip():
    if not os.path.exists(CLIENT):
        pytest.skip("C client not built (run __graft_entry__.build())")
    return CLIENT


def test_header_is_strict_c99(tmp_path):
    src = tmp_path / "only_header.c"
    src.write_text('#include "sp_region.h"\nint main(void) { return sp_region_abi_version() == 0; }\n')
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-fsyntax-only",
                        "-I", os.path.join(ROOT, "include"), str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def _host_lines(lengths, t):
    r = subprocess.run([client_or_skip(), "host", str(t)] + [str(x) for x in lengths], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    out = {}
    for line in r.stdout.splitlines():
        key, *vals = line.split()
        out[key] = [int(v) for v in vals]
    return out


@pytest.mark.parametrize("seed,n,t", [(1, 7, 8), (2, 40, 4), (3, 1, 2)])
def test_host_entry_points_match_the_oracle(seed, n, t):
    rng = np.random.default_rng(seed)
    lengths = [int(x) for x in np.maximum(1, rng.lognormal(8.3, 0.4, n)).astype(np.int64)]
    got = _host_lines(lengths, t)
    assert got["abi"] == [spr.ABI_VERSION]
    assert got["stride"] == [spr.partials_stride(2048, 8192, torch.bfloat16)]
    assert got["workspace"] == [spr.workspace_bytes(2048, 8192), spr.dropout_workspace_bytes(2048, 8192)]
    assert got["cv_within"] == [int(ob.cv_within(lengths, ob.MAX_CV_BP))]
    assert got["sp_gate"] == [int(ob.sp_gate(lengths, 0.1))]
    order, starts = ob.bucket_by_tokens(lengths)
    assert got["bucket_order"] == list(order) and got["bucket_starts"] == list(starts)
    padded, cu, T = ob.shard_layout(lengths, t)
    assert got["layout_T"] == [T] and got["layout_padded"] == list(padded) and got["layout_cu"] == list(cu)
    assert got["reject_t0"] == [spr.SPR_ERR_INVALID_ARG]


@pytest.mark.gpu
@pytest.mark.parametrize("w,rank", [
    (W.custom("c_client_ln", h=1032, t=4, s=4 * 45, b=2, p_drop=0.2, seed=31), 3),
    (W.custom("c_client_rms_f32", h=768, t=2, s=2 * 50, dtype="f32", norm="rmsnorm", p_drop=0.3, bias=False,
              seed=32), 1),
], ids=["bf16_layernorm", "f32_rmsnorm"])
def test_c_client_matches_the_oracle(cuda_device, tmp_path, w, rank):
    client = client_or_skip()
    inp = W.make_inputs(w)
    T, h, ln = inp["T"], w.h, w.norm == "layernorm"
    assert inp["seed"] >= 2 ** 32          # the key's high word is exercised too
    params = dict(b=inp["b"], s=inp["s"], h=h, t=w.t, rank=rank, seed=inp["seed"], p_drop=w.p_drop, eps=w.eps,
                  dtype=spr.SPR_BF16 if w.dtype == "bf16" else spr.SPR_F32,
                  norm=spr.SPR_LAYERNORM if ln else spr.SPR_RMSNORM,
                  bias=int(inp["bias"] is not None), residual=int(inp["residual"] is not None))
    (tmp_path / "params.txt").write_text("".join(f"{k} {v!r}\n" for k, v in params.items()))
    for name in ("partials", "gamma", "beta", "bias", "residual", "dy"):
        if inp[name] is not None:
            np.ascontiguousarray(inp[name]).tofile(tmp_path / f"{name}.bin")
    print(f"[c-client] {w.name} rank={rank} T={T} h={h}", flush=True)
    r = subprocess.run([client, "gpu", str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr

    st = np.uint16 if w.dtype == "bf16" else np.float32
    load = lambda n, dt=st, shape=(T, h): np.fromfile(tmp_path / f"{n}.bin", dtype=dt).reshape(shape)
    to64 = lambda a: ref.decode(a, w.dtype).astype(np.float64)

    o = ref.region_forward(inp["partials"], t=w.t, rank=rank, dtype=w.dtype, norm=w.norm, eps=w.eps,
                           p_drop=w.p_drop, seed=inp["seed"], gamma=inp["gamma"], beta=inp["beta"],
                           bias=inp["bias"], residual=inp["residual"])
    obw = ref.region_backward(inp["dy"], o["z"], inp["gamma"], dtype=w.dtype, norm=w.norm, eps=w.eps)
    od = ref.dropout_backward(obw["dx"], t=w.t, rank=rank, p_drop=w.p_drop, seed=inp["seed"])

    z = load("z")
    assert np.array_equal(z.view(np.uint32 if st is np.float32 else np.uint16),
                          o["z"].view(np.uint32 if st is np.float32 else np.uint16)), "z differs from the oracle"
    assert_out_close(to64(load("y")), o["y"], w.dtype, "y", 1e-5)
    rstd = load("rstd", np.float32, (T,)).astype(np.float64)
    assert np.all(np.abs(rstd - o["rstd"]) <= 1e-4 * o["rstd"])
    assert_out_close(to64(load("dx")), obw["dx"], w.dtype, "dx", 3e-5)
    dp = to64(load("dpartial"))
    assert np.all(dp[~od["keep"]] == 0.0), "dpartial nonzero where the forward dropped"
    assert_out_close(dp, od["dpartial"], w.dtype, "dpartial", 4e-5)
    g = lambda n: load(n, np.float32, (h,)).astype(np.float64)
    assert np.all(np.abs(g("dgamma") - obw["dgamma"]) <= 1e-4 * obw["A"])
    assert np.all(np.abs(g("dbias") - od["dbias"]) <= 1e-4 * od["C"])
    if ln:
        assert np.all(np.abs(g("dbeta") - obw["dbeta"]) <= 1e-4 * obw["B"])
