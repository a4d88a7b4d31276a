"""CPU oracle for fused attention forward and paged decode -- TEST INFRASTRUCTURE.

This package is the slow, obviously-correct fp64 reference that the HIP kernels are
checked against.  Only the test-suite, the smoke check in ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product path (the C-ABI library
and its Python binding) never imports, calls or links anything here, and this package
imports nothing from the product: the two share no code.

What it computes is the plain definition of attention written out (no tiling, no
fusion, no online softmax), except for the FP8 variant:

* ``attention_ref``     -- materialised three-pass softmax attention (prefill).
* ``paged_decode_ref``  -- one query row per sequence against a KV cache stored in
                           fixed-size physical blocks addressed through a block table.
* ``paged_prefill_ref`` -- the newest Q_b tokens of each sequence (chunked prefill) against the
                           same paged cache, causal with the offset L_b - Q_b.
* ``e4m3_decode``       -- the real values of FP8 (e4m3) codes; the FP8 path's parity oracle
                           is the exact attention (``attention_probs_ref``) of the decoded,
                           descaled tensors.
* ``attention_fp8_ref`` -- a model of rounding the probabilities to e4m3 inside an online
                           softmax over key blocks (not the FP8 parity oracle: tests use it to
                           show that the tolerance derived from the e4m3 format admits such
                           rounding schemes).
* ``attention_bwd_ref`` -- gradients of the prefill definition with respect to Q, K and V
                           (chain rule through the row softmax, full P materialised).

Every function is pinned by ``tests/test_oracle_pins.py`` (backward:
``tests/test_oracle_bwd_pins.py``, FP8: ``tests/test_oracle_fp8_pins.py``) against closed forms,
invariances, a pure-Python brute force and a library routine.
"""

from .attention import attention_ref, attention_probs_ref
from .backward import attention_bwd_ref
from .fp8 import attention_fp8_ref, e4m3_decode, e4m3_round
from .paged import paged_decode_ref, paged_prefill_ref, gather_paged_kv

__all__ = ["attention_ref", "attention_probs_ref", "attention_bwd_ref", "paged_decode_ref",
           "paged_prefill_ref", "gather_paged_kv", "attention_fp8_ref", "e4m3_decode",
           "e4m3_round"]
