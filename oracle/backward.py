"""Float64 gradients of attention for the ring backward pass — TEST INFRASTRUCTURE ONLY.

The pages use ring attention to train models on long sequences (Ultralytics glossary, "Ring
Attention": section "Aplicações" — a model trained on million-token contexts with it; section "Como
funciona a atenção em anel" — striped attention raises end-to-end training throughput), but they
never write out the backward pass.  Reading taken: since the ring reaches exactly the attention
output, its backward is exactly the gradient of that output, so the oracle is the gradient of the
definition, written out from the chain rule for one query row t with visible keys u:

    s_u = scale * <q_t, k_u>,  p = softmax(s),  o_t = sum_u p_u v_u,  given dO_t = dL/do_t:
    dp_u  = <dO_t, v_u>                          (dL/dp_u)
    ds_u  = p_u * (dp_u - sum_w p_w dp_w)        (Jacobian of the softmax)
    dq_t  = scale * sum_u ds_u k_u
    dk_u += scale * ds_u q_t                     (summed over every query row that sees u)
    dv_u += p_u dO_t

Grouped-query heads: a key/value head's gradients sum over the query heads that read it.  Masked
keys get p = 0 and contribute nothing; a row that sees no key contributes nothing.
"""
from __future__ import annotations

import numpy as np

__all__ = ["attention_backward_reference", "attention_backward_rows", "attention_backward_key_rows"]


def _row_grads(qrows, qpos, kh, vh, kpos, do_rows, scale, causal):
    """Gradient pieces for a set of query rows against one key/value head, float64.

    Returns (dq [R, D], ds [R, Sk], p [R, Sk]); dk = scale * ds^T q and dv = p^T dO follow.
    """
    s = (qrows @ kh.T) * scale
    if causal:
        s = np.where(kpos[None, :] <= qpos[:, None], s, -np.inf)
    rowmax = s.max(axis=1, keepdims=True)
    seen = np.isfinite(rowmax)
    e = np.exp(s - np.where(seen, rowmax, 0.0))          # 0 for masked keys
    denom = e.sum(axis=1, keepdims=True)
    p = np.where(seen, e / np.where(seen, denom, 1.0), 0.0)
    dp = do_rows @ vh.T                                   # dL/dp_u = <dO_t, v_u>
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq = scale * (ds @ kh)
    return dq, ds, p


def _prep(q, k, v, do, scale):
    q, k, v, do = (np.asarray(x) for x in (q, k, v, do))
    if q.ndim != 4 or k.shape != v.shape or do.shape != q.shape:
        raise ValueError("expected q, dO [B, Sq, Hq, D] and k, v [B, Sk, Hkv, D]")
    if q.shape[0] != k.shape[0] or q.shape[3] != k.shape[3] or q.shape[2] % k.shape[2]:
        raise ValueError("q/k/v shapes disagree")
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[3])
    return q, k, v, do, float(scale), q.shape[2] // k.shape[2]


def attention_backward_reference(q, k, v, do, *, scale=None, causal=False, q_pos=None, k_pos=None, row_chunk=512):
    """dq [B, Sq, Hq, D], dk [B, Sk, Hkv, D], dv [B, Sk, Hkv, D] (float64) for output gradient dO."""
    q, k, v, do, scale, g = _prep(q, k, v, do, scale)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    qpos = np.arange(Sq) if q_pos is None else np.asarray(q_pos)
    kpos = np.arange(Sk) if k_pos is None else np.asarray(k_pos)
    dq = np.zeros((B, Sq, Hq, D))
    dk = np.zeros((B, Sk, Hkv, D))
    dv = np.zeros((B, Sk, Hkv, D))
    for b in range(B):
        for h in range(Hq):
            kh = k[b, :, h // g, :].astype(np.float64)
            vh = v[b, :, h // g, :].astype(np.float64)
            for r0 in range(0, Sq, row_chunk):
                r1 = min(Sq, r0 + row_chunk)
                qr = q[b, r0:r1, h, :].astype(np.float64)
                dor = do[b, r0:r1, h, :].astype(np.float64)
                dqr, ds, p = _row_grads(qr, qpos[r0:r1], kh, vh, kpos, dor, scale, causal)
                dq[b, r0:r1, h, :] = dqr
                dk[b, :, h // g, :] += scale * (ds.T @ qr)
                dv[b, :, h // g, :] += p.T @ dor
    return dq, dk, dv


def attention_backward_rows(q, k, v, do, rows, *, scale=None, causal=False, q_pos=None, k_pos=None, row_chunk=64):
    """dq of selected query rows only: rows int [R, 3] of (batch, query head, query index).

    Returns dq [R, D] float64 in the order of ``rows`` (each row needs only its own scores).
    """
    q, k, v, do, scale, g = _prep(q, k, v, do, scale)
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    Sq, Sk = q.shape[1], k.shape[1]
    qpos = np.arange(Sq) if q_pos is None else np.asarray(q_pos)
    kpos = np.arange(Sk) if k_pos is None else np.asarray(k_pos)
    out = np.zeros((len(rows), q.shape[3]))
    keys = rows[:, 0] * q.shape[2] + rows[:, 1]
    for key in np.unique(keys):
        idx = np.nonzero(keys == key)[0]
        b, h = int(rows[idx[0], 0]), int(rows[idx[0], 1])
        kh = k[b, :, h // g, :].astype(np.float64)
        vh = v[b, :, h // g, :].astype(np.float64)
        for c0 in range(0, len(idx), row_chunk):
            sel = idx[c0:c0 + row_chunk]
            t = rows[sel, 2]
            dq, _, _ = _row_grads(q[b, t, h, :].astype(np.float64), qpos[t], kh, vh, kpos,
                                  do[b, t, h, :].astype(np.float64), scale, causal)
            out[sel] = dq
    return out


def attention_backward_key_rows(q, k, v, do, rows, *, scale=None, causal=False, q_pos=None, k_pos=None, row_chunk=256):
    """dk and dv of selected key rows only: rows int [R, 3] of (batch, key/value head, key index).

    A key's gradients sum over every query row of every query head in its group that sees it, and each
    term needs that query's softmax weight p_tu = exp(s_tu - lse_t) and delta_t = sum_w p_tw dp_tw =
    <dO_t, o_t>; so for each (batch, key/value head) the forward of the definition is evaluated first
    for the query rows that can see a selected key (log-sum-exp and output over all their visible keys),
    then, with ds_tu = p_tu (dp_tu - delta_t) and dp_tu = <dO_t, v_u>:
        dk_u = scale * sum_t ds_tu q_t,   dv_u = sum_t p_tu dO_t.
    Returns (dk [R, D], dv [R, D]) float64 in the order of ``rows``.
    """
    q, k, v, do, scale, g = _prep(q, k, v, do, scale)
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    Sq, Sk, D = q.shape[1], k.shape[1], q.shape[3]
    qpos = np.arange(Sq) if q_pos is None else np.asarray(q_pos)
    kpos = np.arange(Sk) if k_pos is None else np.asarray(k_pos)
    dk = np.zeros((len(rows), D))
    dv = np.zeros((len(rows), D))
    keys = rows[:, 0] * k.shape[2] + rows[:, 1]
    for key in np.unique(keys):
        idx = np.nonzero(keys == key)[0]
        b, kvh = int(rows[idx[0], 0]), int(rows[idx[0], 1])
        kh = k[b, :, kvh, :].astype(np.float64)
        vh = v[b, :, kvh, :].astype(np.float64)
        sel = rows[idx, 2]
        ks, vs, ps = kh[sel], vh[sel], kpos[sel]
        # queries that see at least one selected key (all of them without a mask)
        tq = np.nonzero(qpos >= ps.min())[0] if causal else np.arange(Sq)
        for h in range(kvh * g, (kvh + 1) * g):
            for c0 in range(0, len(tq), row_chunk):
                t = tq[c0:c0 + row_chunk]
                qt = q[b, t, h, :].astype(np.float64)
                dot = do[b, t, h, :].astype(np.float64)
                # forward over every key the rows see: log-sum-exp and output
                s_all = (qt @ kh.T) * scale
                if causal:
                    s_all = np.where(kpos[None, :] <= qpos[t][:, None], s_all, -np.inf)
                mx = s_all.max(axis=1, keepdims=True)
                e = np.exp(s_all - mx)
                den = e.sum(axis=1, keepdims=True)
                lse = mx + np.log(den)
                out = (e @ vh) / den
                delta = (dot * out).sum(axis=1, keepdims=True)
                # the selected keys' terms
                s_sel = (qt @ ks.T) * scale
                if causal:
                    s_sel = np.where(ps[None, :] <= qpos[t][:, None], s_sel, -np.inf)
                p = np.exp(s_sel - lse)                  # 0 where masked
                dp = dot @ vs.T
                ds = p * (dp - delta)
                dk[idx] += scale * (ds.T @ qt)
                dv[idx] += p.T @ dot
    return dk, dv
