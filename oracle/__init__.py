"""CPU oracle for the FP8 fused attention forward pass.  TEST INFRASTRUCTURE ONLY.

This package is the slow, plain reference that the HIP path is checked against.
Only the test suite (``tests/``), ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product package
(``fp8_attention_forward_amd``) never imports, links or calls anything here, and
nothing here imports the product package: the two share no code.  The only
module both sides use is ``workloads`` (seeded synthetic inputs, no arithmetic of
the method).

Everything is numpy/scipy on the CPU.  Floating-point attention is evaluated in
float64; the FP8 pre-processing (rotation, block scaling, e4m3 encoding) is an
encoding, so it is emulated step by step in float32 exactly as specified, so
that the GPU quantiser can be compared bit for bit.

Sources (the pages these functions follow):
  [P1] "FP8 attention that keeps FlashAttention-3 throughput at BF16-level
       accuracy" (distributedagenthub.xyz), sections "What is asked" and
       "How it gets verified".
  [P2] "Fused attention kernel" (wikillm.com), sections "Overview",
       "Variants / 8-bit forward pass (FP8, Hopper)" and "Implementation sketch".
  [P3] "FLAMIA: FLAsh MIcroscaling Attention ..." (paperlayer.ai summary of
       arXiv 2611.03344v1), "4.3 Ablation Study" and "F. System Integration".

Modules
  e4m3       decode / encode of the 8-bit e4m3 float format [P2 8-bit forward pass]
  philox     Philox4x32-10 counter-based generator and the random sign diagonal
             [P2 8-bit forward pass: incoherent processing]
  hadamard   Sylvester Hadamard matrix and its fast transform [same]
  quantize   rotate + per-block scale + e4m3 encode of Q, K, V [P2 8-bit forward pass]
  attention  exact FP64 attention, the running-softmax loop of the sketch,
             brute force, attention of the dequantised FP8 inputs (E1), and
             the block loop with P re-quantised to e4m3 (E2)
             [P2 Overview, Implementation sketch]
  fastexp    Schraudolph's bit-level base-2 exponential (Neural Computation
             11(4), 1999), the option of E2 [P3 4.4 Bit-Level Exponentials]
  varlen     packed variable-length documents: document-local blocks, attention
             inside each document, the work items and their longest-first
             order [P3 Abstract, 4.1 Performance on Packed Documents, 4.3]
  decode     few new queries against an FP8 K/V cache: the E2 loop on key
             ranges merged by their log-sum-exp, grouped query heads
             [P1 Realistic applications]

Every function is pinned by tests in ``tests/test_oracle_*.py`` to something
other than itself (closed forms, an independent library, brute force,
invariants).  Unpinned parts are listed in the functions that have them.
"""

from . import e4m3, philox, hadamard, quantize, attention, fastexp, varlen, decode  # noqa: F401
from .attention import (  # noqa: F401
    attention_fp64,
    reference_attention,
    online_attention_fp64,
    brute_force_attention,
    emulated_fp8_attention,
    emulated_fp8_attention_tiled,
)
from .quantize import quantize_qkv, quantize_tensor, dequantize  # noqa: F401
