"""Pins of the backward oracle (gradients of the attention definition) to facts outside itself.

torch autograd in float64 (a library routine differentiating the plain softmax formula), central
finite differences of the forward oracle (no derivative formula at all), and identities that any
correct gradient satisfies: shifting every key by the same vector leaves each softmax row unchanged
(so the key gradients of a head sum to zero), every softmax row sums to one (so the value gradients
sum to the output gradients of the rows that see a key), constant values make the output independent
of q and k, and zero queries give uniform weights.  A dropped softmax-Jacobian term, a missing scale,
a transposed product or a wrong head map fails at least one of them.  No GPU needed.
"""
import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _torch_grads(q, k, v, do, scale, causal, qpos, kpos):
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    g = q.shape[2] // k.shape[2]
    kk = tk.repeat_interleave(g, dim=2)
    vv = tv.repeat_interleave(g, dim=2)
    s = torch.einsum("bqhd,bkhd->bhqk", tq, kk) * scale
    if causal:
        vis = torch.tensor(kpos[None, :] <= qpos[:, None])
        s = s.masked_fill(~vis, float("-inf"))
    p = torch.softmax(s, dim=-1)
    o = torch.einsum("bhqk,bkhd->bqhd", p, vv)
    o.backward(torch.tensor(do, dtype=torch.float64))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,S,Hq,Hkv,D", [(1, 12, 1, 1, 8), (2, 17, 4, 2, 16), (1, 9, 3, 1, 5)])
def test_backward_matches_torch_autograd(causal, B, S, Hq, Hkv, D):
    q, k, v, do = _rand((B, S, Hq, D), 1), _rand((B, S, Hkv, D), 2), _rand((B, S, Hkv, D), 3), _rand((B, S, Hq, D), 4)
    scale = 1 / np.sqrt(D)
    pos = np.arange(S)
    dq, dk, dv = oracle.attention_backward_reference(q, k, v, do, causal=causal)
    tq, tk, tv = _torch_grads(q, k, v, do, scale, causal, pos, pos)
    assert np.abs(dq - tq).max() < 1e-12 and np.abs(dk - tk).max() < 1e-12 and np.abs(dv - tv).max() < 1e-12


def test_backward_with_positions_matches_autograd():
    # a striped-like query/key position map (keys interleaved) and a few rows that see nothing
    S, D = 10, 6
    q, k, v, do = _rand((1, S, 2, D), 11), _rand((1, S, 1, D), 12), _rand((1, S, 1, D), 13), _rand((1, S, 2, D), 14)
    qpos = np.arange(S) * 2
    kpos = np.arange(S) * 2 + 3
    dq, dk, dv = oracle.attention_backward_reference(q, k, v, do, scale=0.3, causal=True, q_pos=qpos, k_pos=kpos)
    # rows 0 and 1 see no key: their gradients are zero (torch's softmax of an all -inf row is nan)
    assert np.all(dq[:, :2] == 0)
    tq, tk, tv = _torch_grads(q[:, 2:], k, v, do[:, 2:], 0.3, True, qpos[2:], kpos)
    assert np.abs(dq[:, 2:] - tq).max() < 1e-12 and np.abs(dk - tk).max() < 1e-12 and np.abs(dv - tv).max() < 1e-12


def test_backward_matches_finite_differences():
    B, S, Hq, Hkv, D = 1, 5, 2, 1, 3
    q, k, v, do = _rand((B, S, Hq, D), 21), _rand((B, S, Hkv, D), 22), _rand((B, S, Hkv, D), 23), _rand((B, S, Hq, D), 24)
    dq, dk, dv = oracle.attention_backward_reference(q, k, v, do, causal=True)

    def loss(q_, k_, v_):
        o, _ = oracle.attention_reference(q_, k_, v_, causal=True)
        return float((o * do).sum())

    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": (q, k, v), "k": (q, k, v), "v": (q, k, v)}[name]
            ap = [xp if a is x else a for a in args]
            am = [xm if a is x else a for a in args]
            num[idx] = (loss(*ap) - loss(*am)) / (2 * eps)
        assert np.abs(num - g).max() < 1e-7, name


@pytest.mark.parametrize("causal", [False, True])
def test_backward_identities(causal):
    B, S, Hq, Hkv, D = 1, 24, 4, 2, 8
    q, k, v, do = _rand((B, S, Hq, D), 31), _rand((B, S, Hkv, D), 32), _rand((B, S, Hkv, D), 33), _rand((B, S, Hq, D), 34)
    dq, dk, dv = oracle.attention_backward_reference(q, k, v, do, causal=causal)
    # key shift invariance: the key gradients of each head sum to zero
    assert np.abs(dk.sum(axis=1)).max() < 1e-12
    # rows of P sum to one: value gradients of a kv head sum to the output gradients of its query heads
    g = Hq // Hkv
    for h in range(Hkv):
        assert np.abs(dv[:, :, h].sum(axis=1) - do[:, :, h * g:(h + 1) * g].sum(axis=(1, 2))).max() < 1e-12
    # constant values: the output is the constant whatever q and k are
    vc = np.broadcast_to(_rand((1, 1, Hkv, D), 35), v.shape).copy()
    dq0, dk0, dv0 = oracle.attention_backward_reference(q, k, vc, do, causal=causal)
    assert np.abs(dq0).max() < 1e-12 and np.abs(dk0).max() < 1e-12
    # zero queries: uniform weights over the visible keys, so dv_u = sum over rows t seeing u of dO_t / count_t
    dqz, dkz, dvz = oracle.attention_backward_reference(np.zeros_like(q), k, v, do, causal=causal)
    t = np.arange(S)
    count = (t + 1) if causal else np.full(S, S)
    for h in range(Hkv):
        for u in range(S):
            rows = t >= u if causal else np.ones(S, bool)
            expect = (do[0, rows, h * g:(h + 1) * g] / count[rows, None, None]).sum(axis=(0, 1))
            assert np.abs(dvz[0, u, h] - expect).max() < 1e-12


def test_backward_rows_equal_full():
    q, k, v, do = _rand((2, 20, 4, 8), 41), _rand((2, 20, 2, 8), 42), _rand((2, 20, 2, 8), 43), _rand((2, 20, 4, 8), 44)
    dq, _, _ = oracle.attention_backward_reference(q, k, v, do, causal=True)
    rows = np.array([[0, 0, 0], [1, 3, 19], [0, 2, 7], [1, 1, 11]])
    got = oracle.attention_backward_rows(q, k, v, do, rows, causal=True)
    want = np.stack([dq[b, t, h] for b, h, t in rows])
    assert np.abs(got - want).max() < 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_backward_key_rows_match_torch_autograd(causal):
    """dK and dV of chosen key rows (grouped-query heads, two batch elements, positions with an
    interleaved map, rows that see nothing) against torch autograd of the softmax formula."""
    B, S, Hq, Hkv, D = 2, 19, 6, 2, 8
    q, k, v, do = _rand((B, S, Hq, D), 51), _rand((B, S, Hkv, D), 52), _rand((B, S, Hkv, D), 53), _rand((B, S, Hq, D), 54)
    qpos = np.arange(S) * 2 + 1
    kpos = np.arange(S) * 2 + (4 if causal else 0)
    rows = np.array([[b, h, u] for b in range(B) for h in range(Hkv) for u in range(S)])[::3]
    dk, dv = oracle.attention_backward_key_rows(q, k, v, do, rows, scale=0.37, causal=causal, q_pos=qpos, k_pos=kpos)
    if causal:
        # query rows 0 and 1 see no key: leave them out of autograd (their softmax rows are all -inf there)
        _, tk, tv = _torch_grads(q[:, 2:], k, v, do[:, 2:], 0.37, True, qpos[2:], kpos)
    else:
        _, tk, tv = _torch_grads(q, k, v, do, 0.37, False, qpos, kpos)
    want_k = np.stack([tk[b, u, h] for b, h, u in rows])
    want_v = np.stack([tv[b, u, h] for b, h, u in rows])
    assert np.abs(dk - want_k).max() < 1e-12 and np.abs(dv - want_v).max() < 1e-12


def test_backward_key_rows_equal_full_and_catch_a_wrong_head_map():
    q, k, v, do = _rand((1, 24, 4, 8), 61), _rand((1, 24, 2, 8), 62), _rand((1, 24, 2, 8), 63), _rand((1, 24, 4, 8), 64)
    _, dk, dv = oracle.attention_backward_reference(q, k, v, do, causal=True)
    rows = np.array([[0, 0, 0], [0, 1, 23], [0, 1, 5], [0, 0, 17]])
    gk, gv = oracle.attention_backward_key_rows(q, k, v, do, rows, causal=True)
    assert np.abs(gk - np.stack([dk[b, u, h] for b, h, u in rows])).max() < 1e-13
    assert np.abs(gv - np.stack([dv[b, u, h] for b, h, u in rows])).max() < 1e-13
    # swapping the two key/value heads' query groups changes the answer
    q_swapped = q[:, :, [2, 3, 0, 1]]
    bk, _ = oracle.attention_backward_key_rows(q_swapped, k, v, do, rows, causal=True)
    assert np.abs(bk - gk).max() > 1e-3
