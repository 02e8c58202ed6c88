"""CPU oracle for the fused LoRA MLP / QKV / O projections and the NF4 format.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this package: only the tests, the smoke check and the CPU-baseline leg of the
benchmark do.  The oracle shares no code with the HIP library (no kernels,
headers, tables or helpers); the two meet only on the seeded inputs drawn by
the ``workload`` package.

The oracle is deliberately plain: numpy array expressions in the order the
pages write the method, with a library matmul as the only building block, in
float32 for parity (the precision the task fixes for the oracle) and float64
for the finite-difference and closed-form checks.

Sources (cited by page title and section):

* "LoRA Optimizations" (Axolotl documentation) -- sections "Custom autograd
  functions", "Triton kernels", "Integration", "Requirements".
* The unsloth compare view ``main...fix/fused-lora-fp32-dtype`` -- the commit
  message "Avoid recomputing LoRA B-projected gradient in fused-LoRA backward"
  and the diff hunks of ``LoRA_MLP``, ``LoRA_QKV``, ``LoRA_W`` and
  ``matmul_lora``.
* "loralei" README -- section "Use" (QLoRA paragraph on NF4 block sizes and the
  fused unpack / double-scale reconstruction).

Parity status of every function is listed in the module docstrings; each
function is pinned by a test in ``tests/test_oracle_*.py``.
"""
from . import lora, nf4  # noqa: F401
