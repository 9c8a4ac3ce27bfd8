"""Float64 oracle of the blockwise feed-forward that follows attention — TEST INFRASTRUCTURE ONLY.

The context-parallelism article on cyberairomania.ro (section on Ring Attention, where it cites
"Ring Attention with Blockwise Transformers for Near-Infinite Context") says the method computes both
attention and the feed-forward block by block, with the key/value exchange hidden under compute.
The pages give no formula for the feed-forward.  Reading taken (the plainest that fits): the
transformer's position-wise feed-forward applied to each token's attention output,

    y = act(x W1 + b1) W2 + b2,

with act the exact gelu(z) = z * Phi(z) (Phi the standard normal CDF, Phi(z) = erfc(-z / sqrt 2) / 2:
the erfc form keeps Phi's relative precision in the lower tail, where 1 + erf(z / sqrt 2) cancels) or, as an option, the original transformer's max(z, 0), computed over blocks of tokens, so that only one block's hidden activations [block, d_ff] exist at
a time.  Being position-wise, the result does not depend on the block size; the oracle is the
formula itself, evaluated on all tokens at once.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erfc

__all__ = ["gelu", "relu", "ffn_reference"]


def gelu(z):
    """z * Phi(z) with the exact normal CDF, float64."""
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * erfc(-z / np.sqrt(2.0))


def relu(z):
    """max(z, 0), float64."""
    return np.maximum(np.asarray(z, dtype=np.float64), 0.0)


def ffn_reference(x, w1, b1, w2, b2, activation="gelu"):
    """y [N, d_model] = act(x W1 + b1) W2 + b2 in float64, act = gelu or relu.

    x [N, d_model], w1 [d_model, d_ff], b1 [d_ff], w2 [d_ff, d_model], b2 [d_model].
    """
    act = {"gelu": gelu, "relu": relu}[activation]
    x, w1, b1, w2, b2 = (np.asarray(a, dtype=np.float64) for a in (x, w1, b1, w2, b2))
    if x.ndim != 2 or w1.shape != (x.shape[1], b1.shape[0]) or w2.shape != (b1.shape[0], x.shape[1]) \
            or b2.shape != (x.shape[1],):
        raise ValueError("shapes: x [N, dm], w1 [dm, dff], b1 [dff], w2 [dff, dm], b2 [dm]")
    return act(x @ w1 + b1) @ w2 + b2
