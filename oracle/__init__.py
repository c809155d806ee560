"""CPU oracle for the exact attention forward and its MXFP4 Direct-P variant.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, links or
calls this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
kernels, the C-ABI library or its Python binding; the only common input is
the seeded generator in ``synth/``.

Everything here is plain float64 numpy (or pure Python for the brute-force
check), written from the definitions so that a reader can check it by eye:

* ``exact``  -- O = softmax(scale * Q K^T + mask) V and the row log-sum-exp.
  The FlashAttention series reaches this result exactly (tiling plus
  recomputation avoids the N x N matrix in memory but does not change the
  value; "FlashAttention-4发布：原生支持Blackwell…", section
  "从V1到V4：一部浓缩的注意力优化史", the FlashAttention (2022) entry), so the
  oracle is the plain definition, row chunk by row chunk.
* ``mx``     -- OCP MXFP4 quantisation (E2M1 payload, E8M0 block scale) and a
  step-by-step emulation of Direct-P ("Hardware-Aware FP4 FlashAttention-4",
  section "1. Direct-P para Inferencia Directa").
* ``mxfp8``  -- OCP MXFP8 (E4M3 payload, E8M0 block scale) quantisation and a
  step-by-step emulation of the FP8 forward (P rounded to E4M3 with one
  power-of-two scale per 32 keys; the same page's "Resultados" compares an FP8
  path, and its section "2. Causal Backward Cuantizado" keeps P and V in FP8).
* ``backward`` -- the gradients dQ, dK, dV of the exact forward, with P rebuilt
  from the saved log-sum-exp ("Hardware-Aware FP4 FlashAttention-4", section
  "2. Causal Backward Cuantizado": the forward saves the LSE and the backward
  rebuilds the probabilities from it); also for sampled rows at full sizes.
* ``skipsim`` -- a diagnostic model of how often the thresholded rescale fires
  (the aigc.bar page, section "FlashAttention-4：为Blackwell而生的性能猛兽",
  item 1); not part of the parity definition, since the output does not depend
  on the threshold in exact arithmetic.

Parity status: every function is pinned by tests under ``tests/`` against
brute force, a library routine (torch's CPU attention in float64), closed
forms and invariants; see the test modules ``test_oracle_exact.py``,
``test_oracle_mx.py``, ``test_oracle_mxfp8.py``, ``test_oracle_backward.py`` and
``test_oracle_skipsim.py``.
"""

from .exact import attention, attention_brute, attention_head, attention_rows, kv_head
from . import backward, mx, mxfp8, skipsim

__all__ = ["attention", "attention_brute", "attention_head", "attention_rows", "kv_head", "backward", "mx",
           "mxfp8", "skipsim"]
