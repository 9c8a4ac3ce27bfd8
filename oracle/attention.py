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

__all__ = ["attention_reference", "attention_rows", "ring_replay", "ring_schedule"]


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


def ring_schedule(N, order=None):
    """Which key/value block every device holds at every ring step: table[i][step].

    On the ring each device starts with its own block and, after every step, takes over the block
    its predecessor held, so at step s device i holds block (i - s) mod N (Ultralytics glossary,
    "Ring Attention", section "Como funciona a atenção em anel").  An explicit ``order`` (one list
    of N block indices per device) replaces that rotation, for the arrival-order checks.
    """
    if order is not None:
        return [list(map(int, row)) for row in order]
    return [[(i - s) % N for s in range(N)] for i in range(N)]


class _FoldState:
    """Per-device online-softmax state of a query block: reference exponent m (the running row
    maximum of the scores folded so far; -inf before any visible key), normaliser l (sum of
    exp(score - m)) and accumulator acc (sum of exp(score - m) * value)."""

    def __init__(self, n, D, dt):
        self.m = np.full((n, 1), -np.inf, dtype=dt)
        self.l = np.zeros((n, 1), dtype=dt)
        self.acc = np.zeros((n, D), dtype=dt)


def _fold_block(st, s, vj, dt, stabilize):
    """Fold one block's scaled scores s [n, nk] (masked keys at -inf) and values vj into ``st``.

    Stabilised (the running-maximum form of "Sequence Parallelism and Ring Attention", section
    "Approfondimento tecnico"): the reference moves to the larger of the old maximum and the block's
    maximum, the old sums are rescaled by exp(m_old - m_new), and the block's terms enter as
    exp(s - m_new).  A row with no visible key yet keeps the empty state (exp of -inf - -inf is never
    formed).  Unstabilised: plain exp(s) terms are added, as the demonstration on the Ultralytics page
    does; m stays 0.
    """
    if not stabilize:
        w = np.exp(s)
        st.acc = st.acc + w @ vj
        st.l = st.l + w.sum(axis=1, keepdims=True)
        st.m = np.zeros_like(st.m)
        return
    m_new = np.maximum(st.m, s.max(axis=1, keepdims=True))
    live = np.isfinite(m_new)
    ref = np.where(live, m_new, 0)
    rescale = np.where(live, np.exp(st.m - ref), 1).astype(dt)
    w = np.where(live, np.exp(s - ref), 0).astype(dt)
    st.acc = rescale * st.acc + w @ vj
    st.l = rescale * st.l + w.sum(axis=1, keepdims=True)
    st.m = m_new


def ring_replay(q_blocks, k_blocks, v_blocks, *, scale, causal=False, q_pos_blocks=None, k_pos_blocks=None,
                order=None, stabilize=True, dtype=np.float64, trace=None):
    """Ring attention of N emulated devices, one head, on the CPU, step by step.

    The schedule comes first (:func:`ring_schedule`); then all devices advance together, one ring
    step at a time: at each step every device scores its fixed query block against the block it
    holds, masks keys whose position lies after the query's (when causal), and folds the result into
    its own state (:func:`_fold_block`).  Once every step has run, each device divides accumulator by
    normaliser; its log-sum-exp is m + log(l).

    Blocks are 2-D arrays [n, D] (positions per block in q_pos_blocks / k_pos_blocks when causal).
    Returns (outputs, lses): per device one [n, D] and one [n] array in ``dtype``.  If ``trace`` is a
    list, each device's row of the schedule is appended to it.
    """
    N = len(q_blocks)
    dt = np.dtype(dtype)
    table = ring_schedule(N, order)
    qs = [np.asarray(b, dtype=dt) for b in q_blocks]
    states = [_FoldState(qb.shape[0], qb.shape[1], dt) for qb in qs]
    for step in range(N):
        for i in range(N):
            j = table[i][step]
            s = (qs[i] @ np.asarray(k_blocks[j], dtype=dt).T) * dt.type(scale)
            if causal:
                later = np.asarray(k_pos_blocks[j])[None, :] > np.asarray(q_pos_blocks[i])[:, None]
                s = np.where(later, dt.type(-np.inf), s)
            _fold_block(states[i], s, np.asarray(v_blocks[j], dtype=dt), dt, stabilize)
    outputs, lses = [], []
    for st in states:
        with np.errstate(divide="ignore", invalid="ignore"):
            out = np.where(st.l > 0, st.acc / st.l, 0).astype(dt)
            lse = np.where(st.l[:, 0] > 0, st.m[:, 0] + np.log(st.l[:, 0]), -np.inf)
        outputs.append(out)
        lses.append(lse.astype(dt))
    if trace is not None:
        trace.extend(table)
    return outputs, lses
