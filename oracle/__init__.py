"""Float64 CPU oracle for exact scaled dot-product attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call anything in this package.  The product path (the HIP library
and its Python binding in ``exact_tiled_attention_13_amd``) never imports,
calls or links it, and this package imports nothing from the product.

Contents
--------
``attention``        plain definition, O = softmax(scale*Q K^T + mask) V, with
                     causal (bottom-right), key-padding and GQA semantics.
``attention_rows``   the same definition evaluated one (b, h, i) row at a time,
                     for sampled checks at sizes the dense form cannot reach.
``decode``           one new query per sequence against a contiguous KV cache.
``decode_paged``     the same step with the cache held in pages of a pool and
                     found through a per-sequence block table.
``tiled_attention``  the tile-by-tile online-softmax algorithm (running max and
                     denominator, earlier partials rescaled), step by step.
``attention_backward``  dQ, dK, dV of sum(dO * O) by the chain rule through the
                     definition (softmax Jacobian row by row), float64.
``backward_rows``    dQ of selected rows, for sampled checks at large sizes.
``backward_key_rows`` dK and dV of selected keys from the forward's o and lse.
``e4m3_decode``      value of 8-bit E4M3 codes, from the format's definition.
``attention_fp8``, ``attention_rows_fp8``, ``decode_fp8``, ``decode_paged_fp8``
                     the definitions above on E4M3 inputs with one scale per
                     tensor (values = codes * scale).

Parity status: every function above is pinned by tests/test_oracle_pins.py,
tests/test_oracle_backward_pins.py and tests/test_oracle_fp8_pins.py
(closed forms, invariants, a textbook library routine and brute force on tiny
inputs).  No page prints output values for the seeded workloads, so the
seeded outputs themselves are pinned only through those properties.
"""

from .attention import attention, attention_rows, decode, decode_paged, valid_lengths
from .backward import attention_backward, backward_key_rows, backward_rows
from .fp8 import attention_fp8, attention_rows_fp8, decode_fp8, decode_paged_fp8, e4m3_decode
from .tiled import tiled_attention

__all__ = ["attention", "attention_rows", "attention_backward", "backward_key_rows", "backward_rows", "decode", "decode_paged",
           "valid_lengths", "tiled_attention", "e4m3_decode", "attention_fp8", "attention_rows_fp8", "decode_fp8",
           "decode_paged_fp8"]
