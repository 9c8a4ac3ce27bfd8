"""Float64 CPU oracle for blockwise ring attention — TEST INFRASTRUCTURE ONLY (see package docstring).

Sources (the pages are cited by title and section):

* Ultralytics glossary, "Ring Attention", section "Como funciona a atenção em anel": the sequence
  is split into N blocks, one per device; each device keeps its query block and, in each of N
  steps, attends to the key/value block it holds, then passes that block on.  The partial results
  are combined with the accumulated softmax of flash attention: each device keeps a running sum of
  exponentiated scores (denominator) and of score-weighted values (numerator) and divides the two
  at the end.  The demonstration compares this with ``softmax(q k^T / sqrt(dim)) v`` and reports an
  exact match; the same section notes that production kernels subtract a running maximum before
  exponentiating, and names causal masking.
* "Sequence Parallelism and Ring Attention" (aiunderstanding.org), section "Approfondimento
  tecnico": online softmax keeps a running maximum and a running normaliser and rescales the
  earlier partial sums whenever a larger value appears, which makes the result mathematically
  identical to full attention.

Readings where the pages are silent (each is listed in the design notes):

* causal visibility: key position u is visible to query position t iff u <= t;
* grouped-query heads: query head h reads key/value head ``h // (Hq // Hkv)``;
* a row that sees no key at all has output 0 and log-sum-exp -inf;
* log-sum-exp is the natural log of the sum of exp of the *scaled* scores.
"""
from __future__ import annotations

import numpy as np

__all__ = ["attention_reference", "attention_rows", "ring_replay"]


def _attend(qrows, qpos, kh, vh, kpos, scale, causal):
    """Definition of attention for a set of query rows against one key/value head, float64.

    qrows [R, D], kh/vh [Sk, D], qpos [R] and kpos [Sk] global token positions.
    Returns (out [R, D], lse [R]).
    """
    s = (qrows @ kh.T) * scale                      # scaled scores, [R, Sk]
    if causal:
        visible = kpos[None, :] <= qpos[:, None]
        s = np.where(visible, s, -np.inf)
    rowmax = s.max(axis=1, keepdims=True)           # subtracting the row max leaves softmax unchanged
    empty = ~np.isfinite(rowmax[:, 0])
    rowmax = np.where(np.isfinite(rowmax), rowmax, 0.0)
    e = np.exp(s - rowmax)                          # exp(-inf) = 0 for masked keys
    denom = e.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        out = (e @ vh) / denom[:, None]
        lse = rowmax[:, 0] + np.log(denom)
    out[empty] = 0.0
    lse[empty] = -np.inf
    return out, lse


def _prep(q, k, v, scale):
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("expected [B, S, H, D] arrays")
    B, Sq, Hq, D = q.shape
    Bk, Sk, Hkv, Dk = k.shape
    if k.shape != v.shape or Bk != B or Dk != D:
        raise ValueError("q/k/v shapes disagree")
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of key/value heads")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    return q, k, v, float(scale), Hq // Hkv


def attention_reference(q, k, v, *, scale=None, causal=False, q_pos=None, k_pos=None, row_chunk=1024):
    """Full softmax attention by its definition, in float64.

    q: [B, Sq, Hq, D]; k, v: [B, Sk, Hkv, D]; q_pos [Sq] / k_pos [Sk]: global token positions used
    by the causal rule (default 0..S-1).  Returns (out [B, Sq, Hq, D] float64, lse [B, Hq, Sq] float64).
    """
    q, k, v, scale, g = _prep(q, k, v, scale)
    B, Sq, Hq, D = q.shape
    Sk = k.shape[1]
    qpos = np.arange(Sq) if q_pos is None else np.asarray(q_pos)
    kpos = np.arange(Sk) if k_pos is None else np.asarray(k_pos)
    out = np.zeros((B, Sq, Hq, D), dtype=np.float64)
    lse = np.zeros((B, Hq, Sq), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            kh = k[b, :, h // g, :].astype(np.float64)
            vh = v[b, :, h // g, :].astype(np.float64)
            for r0 in range(0, Sq, row_chunk):
                r1 = min(Sq, r0 + row_chunk)
                o, l = _attend(q[b, r0:r1, h, :].astype(np.float64), qpos[r0:r1], kh, vh, kpos, scale, causal)
                out[b, r0:r1, h, :] = o
                lse[b, h, r0:r1] = l
    return out, lse


def attention_rows(q, k, v, rows, *, scale=None, causal=False, q_pos=None, k_pos=None, row_chunk=64):
    """The same definition evaluated only on selected rows.

    rows: int array [R, 3] of (batch, query head, query index into q's token axis).
    Returns (out [R, D] float64, lse [R] float64) in the order of ``rows``.
    """
    q, k, v, scale, g = _prep(q, k, v, scale)
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    D = q.shape[3]
    Sq, Sk = q.shape[1], k.shape[1]
    qpos = np.arange(Sq) if q_pos is None else np.asarray(q_pos)
    kpos = np.arange(Sk) if k_pos is None else np.asarray(k_pos)
    out = np.zeros((len(rows), D), dtype=np.float64)
    lse = np.zeros(len(rows), dtype=np.float64)
    keys = rows[:, 0] * q.shape[2] + rows[:, 1]
    for key in np.unique(keys):
        idx = np.nonzero(keys == key)[0]
        b, h = int(rows[idx[0], 0]), int(rows[idx[0], 1])
        kh = k[b, :, h // g, :].astype(np.float64)
        vh = v[b, :, h // g, :].astype(np.float64)
        for c0 in range(0, len(idx), row_chunk):
            sel = idx[c0:c0 + row_chunk]
            t = rows[sel, 2]
            o, l = _attend(q[b, t, h, :].astype(np.float64), qpos[t], kh, vh, kpos, scale, causal)
            out[sel] = o
            lse[sel] = l
    return out, lse


def ring_replay(q_blocks, k_blocks, v_blocks, *, scale, causal=False, q_pos_blocks=None, k_pos_blocks=None,
                order=None, stabilize=True, dtype=np.float64, trace=None):
    """The ring schedule with the online-softmax fold, one head, on the CPU.

    Device i keeps query block i for the whole computation.  In step ``step`` it holds key/value
    block ``j = (i - step) mod N`` (the block that arrived from the previous device), or
    ``order[i][step]`` when an explicit arrival order is given.  It folds that block into a
    numerator (running sum of exponentiated scores times values) and a denominator (running sum
    of exponentiated scores); after the last step it divides the two.

    With ``stabilize`` the fold keeps a running row maximum m and, when a block raises it, rescales
    the earlier numerator and denominator by exp(m_old - m_new) before adding the new block's
    exp(s - m_new) terms.  Without it the plain exp(s) of the pages' demonstration is summed.

    Causal masking (when enabled) removes key positions greater than the query position.  A row
    whose running maximum is still -inf (nothing visible so far) keeps a zero state: exp of
    (-inf) - (-inf) is never formed.

    Blocks are 2-D arrays [n, D].  Returns (outputs, lses): lists with one [n, D] and one [n]
    array per device, in ``dtype``.  If ``trace`` is a list, the block index held by each device
    at each step is appended to it as ``trace[i][step]``.
    """
    N = len(q_blocks)
    dt = np.dtype(dtype)
    outputs, lses = [], []
    for i in range(N):
        qi = np.asarray(q_blocks[i], dtype=dt)
        n, D = qi.shape
        numerator = np.zeros((n, D), dtype=dt)
        denominator = np.zeros((n, 1), dtype=dt)
        m = np.full((n, 1), -np.inf, dtype=dt)
        held = []
        for step in range(N):
            j = (i - step) % N if order is None else order[i][step]
            held.append(j)
            kj = np.asarray(k_blocks[j], dtype=dt)
            vj = np.asarray(v_blocks[j], dtype=dt)
            s = (qi @ kj.T) * dt.type(scale)
            if causal:
                visible = np.asarray(k_pos_blocks[j])[None, :] <= np.asarray(q_pos_blocks[i])[:, None]
                s = np.where(visible, s, dt.type(-np.inf))
            if stabilize:
                m_new = np.maximum(m, s.max(axis=1, keepdims=True))
                seen = np.isfinite(m_new)                 # rows with at least one visible key so far
                m_ref = np.where(seen, m_new, 0)          # never form (-inf) - (-inf)
                alpha = np.where(seen, np.exp(m - m_ref), 1).astype(dt)
                p = np.where(seen, np.exp(s - m_ref), 0).astype(dt)
                numerator = alpha * numerator + p @ vj
                denominator = alpha * denominator + p.sum(axis=1, keepdims=True)
                m = m_new
            else:
                p = np.exp(s)
                numerator = numerator + p @ vj
                denominator = denominator + p.sum(axis=1, keepdims=True)
        with np.errstate(divide="ignore", invalid="ignore"):
            out = np.where(denominator > 0, numerator / denominator, 0).astype(dt)
            if stabilize:
                lse = np.where(denominator[:, 0] > 0, m[:, 0] + np.log(denominator[:, 0]), -np.inf)
            else:
                lse = np.log(denominator[:, 0])
        outputs.append(out)
        lses.append(lse.astype(dt))
        if trace is not None:
            trace.append(held)
    return outputs, lses
