"""Token-to-shard assignment for the ring (oracle side; test infrastructure only).

Contiguous sharding: the sequence is cut into P equal consecutive blocks and shard i owns tokens
[i*n, (i+1)*n) — the layout described on "Sequence Parallelism and Ring Attention"
(aiunderstanding.org, section "Immersione profonda": each GPU owns a contiguous block of tokens).

Striped sharding: tokens are dealt round-robin, token t goes to shard t mod P at local index
t div P.  The Ultralytics glossary page "Ring Attention" (section "Como funciona a atenção em
anel") says only that Striped Attention spreads the sequence's tokens evenly over the devices to
fix causal imbalance; the round-robin deal is the plainest such even spread.
"""
from __future__ import annotations

import numpy as np


def shard_positions(S: int, P: int, layout: str) -> np.ndarray:
    """Global token position of every local row: array [P, S//P], entry [i, r] = position of row r of shard i."""
    if S % P:
        raise ValueError("sequence length must be divisible by the ring size")
    n = S // P
    i = np.arange(P)[:, None]
    r = np.arange(n)[None, :]
    if layout == "contiguous":
        return i * n + r
    if layout == "striped":
        return r * P + i
    raise ValueError(f"unknown layout {layout!r}")


def _perm(S: int, P: int, layout: str) -> np.ndarray:
    return shard_positions(S, P, layout).reshape(-1)


def contiguous_permutation(S: int, P: int) -> np.ndarray:
    """Identity: shard-major order equals token order."""
    return _perm(S, P, "contiguous")


def striped_permutation(S: int, P: int) -> np.ndarray:
    """perm such that x_sharded = x[:, perm] lists shard 0's tokens, then shard 1's, ... (token axis 1)."""
    return _perm(S, P, "striped")
