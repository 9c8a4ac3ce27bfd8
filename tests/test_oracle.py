"""Pins of the CPU oracle to facts outside itself (no GPU needed).

Each test ties the oracle to something it does not compute itself: the pages' demonstration and
its printed facts, library routines (torch's scaled_dot_product_attention, softmax, logsumexp,
repeat_interleave), brute force in plain Python, closed forms, and the method's own stated
invariants (arrival order does not matter; contiguous and striped sharding give the same result).
A plausible slip in the oracle — a dropped scale, a wrong mask edge, a wrong GQA head, a missing
rescale — fails at least one of them.
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_facts(name):
    facts = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = (x.strip() for x in line.split("=", 1))
            facts[k] = v
    return facts


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------- the pages' demonstration

def test_demo_inputs_follow_the_page_recipe():
    """The shared input generator reproduces the demonstration's global-seed draw bit for bit."""
    torch.manual_seed(0)
    q, k, v = torch.randn(3, 32, 16)
    dq, dk, dv = si.demo_qkv()
    assert np.array_equal(q.numpy(), dq) and np.array_equal(k.numpy(), dk) and np.array_equal(v.numpy(), dv)


def test_demo_replay_matches_printed_facts():
    f = _read_facts("demo_exactness.txt")
    P, block, dim = int(f["n_devices"]), int(f["block"]), int(f["dim"])
    q, k, v = si.demo_qkv()
    qb, kb, vb = np.split(q, P), np.split(k, P), np.split(v, P)
    # largest per-device score block and full matrix sizes
    assert (qb[0] @ kb[0].T).shape == (int(f["score_block_rows"]), int(f["score_block_cols"]))
    assert (q @ k.T).shape == (int(f["full_matrix_rows"]), int(f["full_matrix_cols"]))
    assert block == q.shape[0] // P and dim == q.shape[1]
    # the demo's ring: fp32, plain exp, no running max
    outs, _ = oracle.ring_replay(qb, kb, vb, scale=1.0 / math.sqrt(dim), stabilize=False, dtype=np.float32)
    ring = torch.from_numpy(np.concatenate(outs))
    full = torch.softmax(torch.from_numpy(q) @ torch.from_numpy(k).T / dim ** 0.5, dim=-1) @ torch.from_numpy(v)
    printed = torch.allclose(ring, full, atol=float(f["allclose_atol"]))
    assert str(printed) == f["matches_full_attention"]


def test_demo_reference_and_stabilized_ring_agree_with_library_softmax():
    q, k, v = si.demo_qkv()
    full = (torch.softmax(torch.from_numpy(q).double() @ torch.from_numpy(k).double().T * 0.25, dim=-1)
            @ torch.from_numpy(v).double()).numpy()
    out, lse = oracle.attention_reference(q[None, :, None], k[None, :, None], v[None, :, None])
    assert np.abs(out[0, :, 0] - full).max() < 1e-12
    lse_lib = torch.logsumexp(torch.from_numpy(q).double() @ torch.from_numpy(k).double().T * 0.25, dim=-1)
    assert np.abs(lse[0, 0] - lse_lib.numpy()).max() < 1e-12
    outs, lses = oracle.ring_replay(np.split(q, 4), np.split(k, 4), np.split(v, 4), scale=0.25)
    assert np.abs(np.concatenate(outs) - full).max() < 1e-12
    assert np.abs(np.concatenate(lses) - lse_lib.numpy()).max() < 1e-12


# ---------------------------------------------------------------- library routines and brute force

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,S,Hq,Hkv,D", [(1, 1, 1, 1, 4), (2, 13, 4, 2, 8), (1, 37, 6, 3, 16), (2, 64, 2, 2, 32)])
def test_reference_matches_torch_sdpa(causal, B, S, Hq, Hkv, D):
    q = _rand((B, S, Hq, D), 1)
    k = _rand((B, S, Hkv, D), 2)
    v = _rand((B, S, Hkv, D), 3)
    out, lse = oracle.attention_reference(q, k, v, causal=causal)
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
    assert np.abs(out - ref.permute(0, 2, 1, 3).numpy()).max() < 1e-12
    scores = (tq @ tk.transpose(-1, -2)) / math.sqrt(D)
    if causal:
        scores = scores.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), float("-inf"))
    assert np.abs(lse - torch.logsumexp(scores, dim=-1).numpy()).max() < 1e-12


def test_reference_matches_plain_python_loops():
    rng = np.random.default_rng(7)
    S, D = 6, 3
    for causal in (False, True):
        q, k, v = (rng.standard_normal((S, D)) for _ in range(3))
        out, lse = oracle.attention_reference(q[None, :, None], k[None, :, None], v[None, :, None], scale=0.7,
                                              causal=causal)
        for t in range(S):
            keys = range(t + 1) if causal else range(S)
            w = [math.exp(0.7 * sum(q[t, c] * k[u, c] for c in range(D))) for u in keys]
            z = sum(w)
            for c in range(D):
                assert abs(out[0, t, 0, c] - sum(wi * v[u, c] for wi, u in zip(w, keys)) / z) < 1e-12
            assert abs(lse[0, 0, t] - math.log(z)) < 1e-12


def test_gqa_equals_repeated_kv_heads():
    q = _rand((1, 40, 8, 16), 11)
    k = _rand((1, 40, 2, 16), 12)
    v = _rand((1, 40, 2, 16), 13)
    out, lse = oracle.attention_reference(q, k, v, causal=True)
    kr = torch.from_numpy(k).repeat_interleave(4, dim=2).numpy()
    vr = torch.from_numpy(v).repeat_interleave(4, dim=2).numpy()
    out2, lse2 = oracle.attention_reference(q, kr, vr, causal=True)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    # a wrong head map (h mod Hkv instead of h div group) changes the answer
    kw = np.tile(k, (1, 1, 4, 1))
    vw = np.tile(v, (1, 1, 4, 1))
    out3, _ = oracle.attention_reference(q, kw, vw, causal=True)
    assert np.abs(out3 - out).max() > 1e-3


def test_rows_equal_full_reference():
    q = _rand((2, 50, 4, 8), 21)
    k = _rand((2, 50, 2, 8), 22)
    v = _rand((2, 50, 2, 8), 23)
    out, lse = oracle.attention_reference(q, k, v, causal=True)
    rows = np.array([[b, h, t] for b in range(2) for h in range(4) for t in (0, 1, 17, 49)])
    o2, l2 = oracle.attention_rows(q, k, v, rows, causal=True, row_chunk=3)
    # equal up to the summation order of the BLAS kernel (row-count dependent blocking)
    assert np.abs(o2 - out[rows[:, 0], rows[:, 2], rows[:, 1]]).max() < 1e-13
    assert np.abs(l2 - lse[rows[:, 0], rows[:, 1], rows[:, 2]]).max() < 1e-13


# ---------------------------------------------------------------- closed forms

def test_zero_queries_give_prefix_means():
    S, D = 24, 5
    v = _rand((1, S, 1, D), 31)
    k = _rand((1, S, 1, D), 32)
    q = np.zeros((1, S, 1, D))
    out, lse = oracle.attention_reference(q, k, v, causal=True)
    for t in range(S):
        assert np.allclose(out[0, t, 0], v[0, :t + 1, 0].mean(axis=0), atol=1e-14, rtol=0)
        assert abs(lse[0, 0, t] - math.log(t + 1)) < 1e-14
    out, lse = oracle.attention_reference(q, k, v, causal=False)
    assert np.allclose(out[0, :, 0], v[0, :, 0].mean(axis=0), atol=1e-14, rtol=0)
    assert np.allclose(lse, math.log(S), atol=1e-14, rtol=0)


def test_constant_values_and_first_causal_row():
    q = _rand((1, 16, 2, 8), 41)
    k = _rand((1, 16, 2, 8), 42)
    v = np.full((1, 16, 2, 8), 3.25)
    out, _ = oracle.attention_reference(q, k, v, causal=True)
    assert np.allclose(out, 3.25, atol=1e-14, rtol=0)
    v = _rand((1, 16, 2, 8), 43)
    out, lse = oracle.attention_reference(q, k, v, causal=True, scale=0.3)
    assert np.array_equal(out[0, 0], v[0, 0])
    for h in range(2):
        assert abs(lse[0, h, 0] - 0.3 * float(q[0, 0, h] @ k[0, 0, h])) < 1e-14


def test_one_hot_values_read_out_probabilities():
    S, D = 12, 12
    q = _rand((1, S, 1, D), 51)
    k = _rand((1, S, 1, D), 52)
    v = np.eye(S)[None, :, None, :]
    out, _ = oracle.attention_reference(q, k, v, causal=False)
    probs = torch.softmax(torch.from_numpy(q[0, :, 0] @ k[0, :, 0].T) / math.sqrt(D), dim=-1).numpy()
    assert np.abs(out[0, :, 0] - probs).max() < 1e-14


def test_single_device_ring_is_plain_attention():
    q, k, v = (_rand((9, 4), s) for s in (61, 62, 63))
    outs, lses = oracle.ring_replay([q], [k], [v], scale=0.5)
    out, lse = oracle.attention_reference(q[None, :, None], k[None, :, None], v[None, :, None], scale=0.5)
    assert np.abs(outs[0] - out[0, :, 0]).max() < 1e-14
    assert np.abs(lses[0] - lse[0, 0]).max() < 1e-14


# ---------------------------------------------------------------- the method's invariants

def _blocks(x, P):
    return np.split(x, P)


@pytest.mark.parametrize("P", [1, 2, 4, 7])
def test_ring_schedule_passes_blocks_to_the_next_device(P):
    """Each device starts on its own block; at every later step it holds the block its predecessor
    held one step earlier (it received it from the previous device); over P steps it sees all blocks."""
    x = _rand((P * 2, 3), 75)
    trace = []
    oracle.ring_replay(_blocks(x, P), _blocks(x, P), _blocks(x, P), scale=1.0, trace=trace)
    for i in range(P):
        assert trace[i][0] == i
        assert sorted(trace[i]) == list(range(P))
        for s in range(1, P):
            assert trace[i][s] == trace[(i - 1) % P][s - 1]


@pytest.mark.parametrize("causal", [False, True])
def test_every_arrival_order_gives_full_attention(causal):
    P, n, D = 4, 5, 6
    S = P * n
    q, k, v = (_rand((S, D), s) for s in (71, 72, 73))
    pos = oracle.shard_positions(S, P, "contiguous")
    ref, ref_lse = oracle.attention_reference(q[None, :, None], k[None, :, None], v[None, :, None], causal=causal)
    for perm in itertools.permutations(range(P)):
        order = [list(perm)] * P
        outs, lses = oracle.ring_replay(_blocks(q, P), _blocks(k, P), _blocks(v, P), scale=1 / math.sqrt(D),
                                        causal=causal, q_pos_blocks=pos, k_pos_blocks=pos, order=order)
        assert np.abs(np.concatenate(outs) - ref[0, :, 0]).max() < 1e-12
        assert np.abs(np.concatenate(lses) - ref_lse[0, 0]).max() < 1e-12


def test_random_arrival_orders_p8():
    P, n, D = 8, 3, 4
    S = P * n
    q, k, v = (_rand((S, D), s) for s in (81, 82, 83))
    rng = np.random.default_rng(84)
    for layout in ("contiguous", "striped"):
        pos = oracle.shard_positions(S, P, layout)
        perm = pos.reshape(-1)
        qs, ks, vs = q[perm], k[perm], v[perm]
        ref, _ = oracle.attention_reference(qs[None, :, None], ks[None, :, None], vs[None, :, None], causal=True,
                                            q_pos=perm, k_pos=perm)
        order = [list(rng.permutation(P)) for _ in range(P)]
        outs, _ = oracle.ring_replay(_blocks(qs, P), _blocks(ks, P), _blocks(vs, P), scale=0.5, causal=True,
                                     q_pos_blocks=pos, k_pos_blocks=pos, order=order)
        ref2, _ = oracle.attention_reference(qs[None, :, None], ks[None, :, None], vs[None, :, None], scale=0.5,
                                             causal=True, q_pos=perm, k_pos=perm)
        assert np.abs(np.concatenate(outs) - ref2[0, :, 0]).max() < 1e-12


def test_zigzag_layout_table():
    # written out by hand: 8 chunks of 3 tokens; shard i holds chunk i, then chunk 7 - i
    expected = [[0, 1, 2, 21, 22, 23],
                [3, 4, 5, 18, 19, 20],
                [6, 7, 8, 15, 16, 17],
                [9, 10, 11, 12, 13, 14]]
    assert oracle.shard_positions(24, 4, "zigzag").tolist() == expected
    assert sorted(oracle.zigzag_permutation(24, 4).tolist()) == list(range(24))
    with pytest.raises(ValueError):
        oracle.shard_positions(20, 4, "zigzag")  # 5 tokens per shard cannot be split into two chunks


@pytest.mark.parametrize("layout", ["striped", "zigzag"])
def test_striped_equals_contiguous_after_unpermuting(layout):
    P, n, D, H = 4, 6, 8, 2
    S = P * n
    q = _rand((1, S, H, D), 91)
    k = _rand((1, S, 1, D), 92)
    v = _rand((1, S, 1, D), 93)
    ref, ref_lse = oracle.attention_reference(q, k, v, causal=True)
    perm = oracle.shard_positions(S, P, layout).reshape(-1)
    pos = oracle.shard_positions(S, P, layout)
    for h in range(H):
        outs, lses = oracle.ring_replay(_blocks(q[0, perm, h], P), _blocks(k[0, perm, 0], P), _blocks(v[0, perm, 0], P),
                                        scale=1 / math.sqrt(D), causal=True, q_pos_blocks=pos, k_pos_blocks=pos)
        striped = np.concatenate(outs)
        unperm = np.empty_like(striped)
        unperm[perm] = striped
        assert np.abs(unperm - ref[0, :, h]).max() < 1e-12
        lse_u = np.empty(S)
        lse_u[perm] = np.concatenate(lses)
        assert np.abs(lse_u - ref_lse[0, h]).max() < 1e-12
    # the layout really is a different token order (sanity: not the identity for P > 1)
    assert not np.array_equal(perm, np.arange(S))


def test_running_max_is_what_keeps_large_scores_finite():
    P, n, D = 4, 8, 16
    S = P * n
    q, k, v = (_rand((S, D), s).astype(np.float32) for s in (101, 102, 103))
    q *= 40.0  # scores far above 88.7, where exp overflows in float32
    assert (q @ k.T / 4).max() > 89
    with np.errstate(over="ignore", invalid="ignore"):
        plain, _ = oracle.ring_replay(_blocks(q, P), _blocks(k, P), _blocks(v, P), scale=0.25, stabilize=False,
                                      dtype=np.float32)
    assert not np.isfinite(np.concatenate(plain)).all()
    stable, _ = oracle.ring_replay(_blocks(q, P), _blocks(k, P), _blocks(v, P), scale=0.25, dtype=np.float32)
    ref, _ = oracle.attention_reference(q[None, :, None], k[None, :, None], v[None, :, None], scale=0.25)
    assert np.isfinite(np.concatenate(stable)).all()
    assert np.abs(np.concatenate(stable) - ref[0, :, 0]).max() < 1e-4


def test_fully_masked_rows_give_zero_and_minus_inf():
    q, k, v = (_rand((1, 4, 1, 2), s) for s in (111, 112, 113))
    out, lse = oracle.attention_reference(q, k, v, causal=True, q_pos=np.arange(4), k_pos=np.arange(4) + 2)
    assert np.array_equal(out[0, :2], np.zeros((2, 1, 2))) and np.all(lse[0, 0, :2] == -np.inf)
    assert np.isfinite(out).all() and np.isfinite(lse[0, 0, 2:]).all()
    # the ring replay starts some rows on fully masked blocks; the guard keeps them clean
    pos = [np.array([0, 1]), np.array([2, 3])]
    outs, lses = oracle.ring_replay([q[0, :2, 0], q[0, 2:, 0]], [k[0, :2, 0], k[0, 2:, 0]], [v[0, :2, 0], v[0, 2:, 0]],
                                    scale=0.5, causal=True, q_pos_blocks=pos, k_pos_blocks=pos, order=[[1, 0], [1, 0]])
    ref, _ = oracle.attention_reference(q, k, v, causal=True, scale=0.5)
    assert np.abs(np.concatenate(outs) - ref[0, :, 0]).max() < 1e-12


# ---------------------------------------------------------------- work counts of the two layouts

def _pairs(qpos, kpos):
    return int((kpos[None, :] <= qpos[:, None]).sum())


@pytest.mark.parametrize("P,n", [(4, 8), (8, 16), (8, 5), (32, 4)])
def test_visible_pair_counts_closed_forms(P, n):
    S = P * n
    for layout in ("contiguous", "striped"):
        pos = oracle.shard_positions(S, P, layout)
        per_dev = [sum(_pairs(pos[i], pos[j]) for j in range(P)) for i in range(P)]
        assert sum(per_dev) == S * (S + 1) // 2
        for i in range(P):
            if layout == "contiguous":
                assert per_dev[i] == i * n * n + n * (n + 1) // 2
            else:
                assert per_dev[i] == P * n * (n - 1) // 2 + (i + 1) * n
    # critical path with a barrier after every ring step (sum over steps of the busiest device)
    def crit(layout):
        pos = oracle.shard_positions(S, P, layout)
        return sum(max(_pairs(pos[i], pos[(i - s) % P]) for i in range(P)) for s in range(P))
    assert crit("contiguous") == n * (n + 1) // 2 + (P - 1) * n * n
    assert crit("striped") == P * n * (n + 1) // 2
    if n % 2 == 0:
        # zigzag: shard i's early chunk i sees chunks 0..i, its late chunk 2P-1-i sees 0..2P-1-i;
        # every shard gets (2P-1) c^2 + c (c+1) pairs, and in each step every shard does the same
        # work (c^2 + c (c+1) on its own block, 2 c^2 on any other), so the critical path is that too
        c = n // 2
        pos = oracle.shard_positions(S, P, "zigzag")
        for i in range(P):
            assert sum(_pairs(pos[i], pos[j]) for j in range(P)) == (2 * P - 1) * c * c + c * (c + 1)
            for j in range(P):
                assert _pairs(pos[i], pos[j]) == (c * c + c * (c + 1) if j == i else 2 * c * c)
        assert crit("zigzag") == (2 * P - 1) * c * c + c * (c + 1)


def test_workload_flop_counts():
    w = si.WORKLOADS
    assert w["noncausal_16k"].flops() == 4 * 128 * 8 * 16384 ** 2
    assert w["causal_32k"].flops() == 4 * 128 * 32 * 32768 * 32769 // 2
    assert w["causal_striped_64k"].flops() == 4 * 128 * 32 * 65536 * 65537 // 2
    n = 32768
    assert w["causal_1m_shard"].flops() == 4 * 128 * 8 * (31 * n * n + n * (n + 1) // 2)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e38, 1e-40], dtype=np.float32)
    r = si.bf16_to_f32(si.bf16_bits(x))
    t = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(r, t)
    y = np.random.default_rng(5).standard_normal(100000).astype(np.float32)
    assert np.array_equal(si.bf16_to_f32(si.bf16_bits(y)), torch.from_numpy(y).to(torch.bfloat16).float().numpy())
