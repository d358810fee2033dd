"""Oracle of the sequence-parallel region: TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct CPU implementation (NumPy; float32 where the
stored residual stream z is defined by a float32 operation order, float64
everywhere else) of what the fused region computes on one rank's shard.  It
exists to check the HIP path; nothing in the product imports it.  Only the
tests, the package's smoke check and the benchmark's CPU-baseline leg may
import or run it.

Modules:
  bf16     -- bfloat16 storage codec (round to nearest, ties to even)
  philox   -- Philox-4xW-10 counter-based generator (Salmon et al., SC'11)
  region   -- forward (g* partial-slab sum, bias, dropout, residual, norm) and
              backward (dx, dgamma, dbeta) of the region
  analytic -- TP vs TP+SP shape trace, activation-memory formula, ring
              collective volumes (hpc.payai.win lesson 7)

Pins (tests/test_oracle_*.py) tie every function to something other than
itself: values the pages print, closed forms, invariants, library routines
(torch layer_norm / rms_norm / autograd in float64, torch's bf16 cast,
numpy's Philox-4x64), exact error bounds and brute force on tiny inputs.
The Philox-4x32 multipliers are also checked against rocRAND's host
generator, which needs a HIP device and therefore runs among the GPU tests.
"""
from . import analytic, bf16, philox, region  # noqa: F401
