"""CPU fp64 oracle for exact attention (TEST INFRASTRUCTURE).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The library path never calls it, and it shares no code with the
HIP kernels: the two meet only in the seeded input generator (``attn_inputs``).

* ``oracle.attention``: the materialised definition, softmax(scale*Q*K^T)*V,
  in float64 on the exact bf16 inputs, for prefill (MHA/GQA/MQA, causal,
  cross-attention, BSHD/BHSD) and for the paged decode (gather, then the same
  definition).
* ``oracle.online``: a float64 model of the blockwise online softmax and of the
  split-KV merge, used only to pin the oracle to the pages' merge rule.
* ``oracle.backward``: the gradient of the forward (dQ, dK, dV for an upstream
  dO) by the chain rule on the materialised matrices, in float64.
* ``oracle.fp8``: E4M3 decoding and the forward on FP8 inputs with
  per-tensor descales.
* ``oracle.rounding``: the three bf16 rounding rules of the output conversion
  (to nearest with ties to even, to nearest with ties away from zero, toward
  zero) applied to float64 values.
"""
from . import attention, backward, fp8, online, rounding  # noqa: F401
