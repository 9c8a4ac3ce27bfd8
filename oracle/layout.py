"""Token-to-shard assignment for the ring (oracle side; test infrastructure only).

Contiguous sharding: the sequence is cut into P equal consecutive blocks and shard i owns tokens
[i*n, (i+1)*n) — the layout described on "Sequence Parallelism and Ring Attention"
(aiunderstanding.org, section "Immersione profonda": each GPU owns a contiguous block of tokens).

Striped sharding: tokens are dealt round-robin, token t goes to shard t mod P at local index
t div P.  The Ultralytics glossary page "Ring Attention" (section "Como funciona a atenção em
anel") says only that Striped Attention spreads the sequence's tokens evenly over the devices to
fix causal imbalance; the round-robin deal is the plainest such even spread.

Zigzag sharding: the page "Ukulandelana Ukuhambisana Nokunakwa Kwendandatho" (aiunderstanding.org,
section "Ikusasa Lokulandelana Ukufana Nokunakwa Kwendandatho") names it beside striped attention
as a way to rebalance the causal work, without defining it.  Reading taken: the sequence is cut
into 2P equal chunks and shard i holds chunk i followed by chunk 2P-1-i, pairing an early chunk
with a late one so that every shard sees the same number of visible keys.
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
    if layout == "zigzag":
        if n % 2:
            raise ValueError("zigzag sharding needs an even number of tokens per shard")
        c = n // 2
        return np.where(r < c, i * c + r, (2 * P - 1 - i) * c + (r - c))
    raise ValueError(f"unknown layout {layout!r}")


def _perm(S: int, P: int, layout: str) -> np.ndarray:
    return shard_positions(S, P, layout).reshape(-1)


def contiguous_permutation(S: int, P: int) -> np.ndarray:
    """Identity: shard-major order equals token order."""
    return _perm(S, P, "contiguous")


def zigzag_permutation(S: int, P: int) -> np.ndarray:
    """perm such that x_sharded = x[:, perm] lists the zigzag shards in order (token axis 1)."""
    return _perm(S, P, "zigzag")


def striped_permutation(S: int, P: int) -> np.ndarray:
    """perm such that x_sharded = x[:, perm] lists shard 0's tokens, then shard 1's, ... (token axis 1)."""
    return _perm(S, P, "striped")
