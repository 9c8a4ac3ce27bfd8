"""CPU oracle for blockwise ring attention — TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke entry point and the benchmark's CPU-baseline leg may import this
package.  The product path (the HIP library and its Python binding) never imports, calls or links
anything here, and this package imports nothing from the product path: the two share no code.

What is here, in float64 NumPy:

* :func:`attention_reference` — the plain definition of (causal or full) softmax attention with
  log-sum-exp, written out directly.  The pages state that the ring method reaches exactly this
  result, so it is the oracle for every GPU parity test.
* :func:`attention_rows` — the same definition evaluated only on chosen (batch, head, token) rows,
  for workloads too large for the full O(S^2) computation.
* :func:`ring_replay`, :func:`ring_schedule` — the ring schedule and the online-softmax fold of each
  device's running state, used to check the method's own claims (exactness, arrival-order
  invariance) on the CPU.
* :func:`attention_backward_reference`, :func:`attention_backward_rows`,
  :func:`attention_backward_key_rows` — the gradients dQ, dK, dV of the same definition for an output
  gradient dO (chain rule written out; the pages use the ring for training but do not spell out its
  backward pass), in full, for chosen query rows, or for chosen key rows.
* :func:`ffn_reference`, :func:`gelu`, :func:`relu` — the position-wise feed-forward that the blockwise
  method computes after attention, y = act(x W1 + b1) W2 + b2.
* :mod:`oracle.layout` — contiguous, striped and zigzag token-to-shard assignment.

Every function is pinned by CPU tests to facts outside itself (the pages' demonstration, library
routines, closed forms, brute force); none is "parity unpinned".
"""
from .attention import attention_reference, attention_rows, ring_replay, ring_schedule
from .backward import attention_backward_key_rows, attention_backward_reference, attention_backward_rows
from .ffn import ffn_reference, gelu, relu
from .layout import shard_positions, striped_permutation, contiguous_permutation, zigzag_permutation

__all__ = [
    "attention_reference", "attention_rows", "ring_replay", "ring_schedule",
    "attention_backward_reference", "attention_backward_rows", "attention_backward_key_rows", "ffn_reference", "gelu", "relu",
    "shard_positions", "striped_permutation", "contiguous_permutation", "zigzag_permutation",
]
