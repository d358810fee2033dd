"""GPU parity on rows that are numerically hard for the normalisation
(hpc.payai.win lesson 7, section 2: mean and population variance over the
full h, eps inside the square root):

  * a constant row: variance exactly 0, so rstd = 1/sqrt(eps), xhat = 0 and
    y = beta (0 for RMSNorm), while dx = rstd*(g - mean(g)) is large;
  * an all-zero row: for RMSNorm the mean square is 0, rstd = 1/sqrt(eps);
  * a row whose mean is large against its spread (|mean| >> std);
  * a row whose variance is of the order of eps;

with gamma in [8, 16] and dy ~ N(0, 64), so |y| and |dx| go well beyond 8 and
the bf16 bar's second clause (half an ulp + 1e-3) is exercised; plus eps =
1e-2.  Bars as in test_gpu_parity, with the float32 slacks of each row scaled
by its conditioning kappa = max(1, |mean|*rstd).
"""
import numpy as np
import pytest

import workloads as W
from test_gpu_parity import compare, log, run_gpu

pytestmark = pytest.mark.gpu

# (name, workload, mean of the large-mean row, rank, return_mask)
CASES = [
    # the benchmark's forward: 16 slots per lane, z in LDS, no mask output
    (W.custom("hard_ln_bf16_h8192", h=8192, t=8, s=8 * 16, p_drop=0.1), 48.0, 0, False),
    (W.custom("hard_ln_bf16_h8192_mask", h=8192, t=8, s=8 * 16, p_drop=0.1), 48.0, 5, True),
    (W.custom("hard_ln_bf16_h4096_eps1e-2", h=4096, t=8, s=8 * 12, eps=1e-2, p_drop=0.1, bias=False), 48.0, 3,
     False),
    (W.custom("hard_rms_bf16_h5120", h=5120, t=8, s=8 * 10, norm="rmsnorm", eps=1e-6, p_drop=0.0, bias=False,
              residual=False), 48.0, 7, False),
    # two waves per row in the forward, 4 vectors per thread in the backward
    (W.custom("hard_ln_bf16_h16384", h=16384, t=4, s=4 * 8, p_drop=0.2), 48.0, 2, False),
    (W.custom("hard_ln_f32_h512", h=512, t=4, s=4 * 16, dtype="f32", p_drop=0.1), 50.0, 1, True),
    (W.custom("hard_rms_f32_h4096_eps1e-2", h=4096, t=2, s=2 * 8, dtype="f32", norm="rmsnorm", eps=1e-2,
              p_drop=0.3), 50.0, 1, False),
    (W.custom("hard_ln_f32_h8192_nobeta", h=8192, t=3, s=3 * 6, dtype="f32", beta=False, p_drop=0.0), 50.0, 0,
     False),
]


@pytest.mark.parametrize("w,loc,rank,mask", CASES, ids=[c[0].name for c in CASES])
def test_hard_rows(cuda_device, w, loc, rank, mask):
    log(f"[hard-rows] {w.name} rank={rank} mask={mask}")
    inp = W.with_hard_rows(W.make_inputs(w), loc=loc)
    gpu = run_gpu(inp, w, rank, cuda_device, return_mask=mask)
    o, ob = compare(w, inp, gpu, rank, conditioned=True)
    eps32 = float(np.float32(w.eps))
    # The constant rows (LayerNorm; with h a power of two the float32 mean of
    # a constant row is exact) and the zero row of RMSNorm: the variance or
    # mean square is exactly 0, so rstd = 1/sqrt(eps) and y = beta (0 when
    # there is no beta) bit for bit.
    exact_rows = ([0, 1] if (w.h & (w.h - 1)) == 0 else []) if w.norm == "layernorm" else [1]
    beta = W.as_torch(inp["beta"], "cpu").double().numpy() if inp["beta"] is not None else np.zeros(w.h)
    for r in exact_rows:
        assert abs(gpu["rstd"][r] * np.sqrt(eps32) - 1.0) <= 1e-6, (r, gpu["rstd"][r])
        assert np.array_equal(gpu["y"][r], beta), r
    # The second clause of the bf16 bar (|ref| >= 8) is reached by y and dx.
    assert np.max(np.abs(o["y"])) >= 8 and np.max(np.abs(ob["dx"])) >= 8
    log(f"  max|y| {np.max(np.abs(o['y'])):.1f}, max|dx| {np.max(np.abs(ob['dx'])):.1f}, "
        f"kappa max {float(np.max(np.abs(o['mean']) * o['rstd'])) if o['mean'] is not None else 1.0:.1f}")
