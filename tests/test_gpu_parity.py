"""GPU parity of the HIP path against the float64 oracle, through the C ABI (small and ragged shapes).

Tolerances: fp32 inputs, max abs 1e-5; bf16 inputs with fp32 accumulation, output max abs 2e-2 and
log-sum-exp max abs 1e-3.  Shapes span several 128-row query tiles and 64-key tiles plus a ragged
tail, in both layouts, with and without the causal mask, with grouped-query heads.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from ring_harness import (TOL_BF16_LSE, TOL_BF16_O, TOL_F32, max_err, out_to_f64, run_ring_local, shard, to_device,
                          to_float, unshard_lse, unshard_out)

pytestmark = pytest.mark.gpu


def _inputs(B, S, Hq, Hkv, D, seed, dtype, sigma=1.0):
    gen = si.normal_bf16 if dtype == "bf16" else si.normal_f32
    return (gen(seed, (B, S, Hq, D), sigma), gen(seed + 1, (B, S, Hkv, D), sigma), gen(seed + 2, (B, S, Hkv, D), sigma))


def _check_ring(gpu_lib, B, P, n, Hq, Hkv, D, causal, layout, dtype, seed, sigma=1.0, host_kv=False, two_streams=True):
    S = P * n
    q, k, v = _inputs(B, S, Hq, Hkv, D, seed, dtype, sigma)
    o, lse = run_ring_local(q, k, v, P=P, causal=causal, layout=layout, dtype=dtype, host_kv=host_kv,
                            two_streams=two_streams)
    ref_o, ref_lse = oracle.attention_reference(to_float(q, dtype), to_float(k, dtype), to_float(v, dtype),
                                                causal=causal)
    eo = max_err(unshard_out(o, layout), ref_o)
    el = max_err(unshard_lse(lse, layout), ref_lse)
    print(f"[parity] B={B} P={P} n={n} Hq={Hq} Hkv={Hkv} D={D} causal={causal} {layout} {dtype}: "
          f"max|dO|={eo:.3g} max|dLSE|={el:.3g}", flush=True)
    if dtype == "f32":
        assert eo <= TOL_F32 and el <= TOL_F32
    else:
        assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE
    return eo, el


def test_demo_four_devices_fp32(gpu_lib):
    """The pages' demonstration: 4 devices x 8 tokens, d=16, seed 0, fp32, no mask."""
    q, k, v = si.demo_qkv()
    q, k, v = (x.reshape(1, 32, 1, 16) for x in (q, k, v))
    o, lse = run_ring_local(q, k, v, P=4, causal=False, layout="contiguous", dtype="f32", scale=0.25)
    ref_o, ref_lse = oracle.attention_reference(q, k, v, scale=0.25)
    assert max_err(unshard_out(o, "contiguous"), ref_o) <= TOL_F32
    assert max_err(unshard_lse(lse, "contiguous"), ref_lse) <= TOL_F32
    # and against the library softmax the demonstration compares with
    full = torch.softmax(torch.from_numpy(q[0, :, 0]) @ torch.from_numpy(k[0, :, 0]).T / 4.0, dim=-1) @ torch.from_numpy(
        v[0, :, 0])
    assert torch.allclose(torch.from_numpy(unshard_out(o, "contiguous")[0, :, 0]).float(), full, atol=1e-5)


@pytest.mark.parametrize("causal,layout", [(False, "contiguous"), (True, "contiguous"), (True, "striped")])
@pytest.mark.parametrize("D", [16, 40, 64, 128])
def test_fp32_ring(gpu_lib, causal, layout, D):
    _check_ring(gpu_lib, 1, 4, 37, 3, 1, D, causal, layout, "f32", 100 + D)


@pytest.mark.parametrize("causal,layout", [(False, "contiguous"), (True, "contiguous"), (True, "striped")])
@pytest.mark.parametrize("n", [128, 200, 320])
def test_bf16_mfma_ring(gpu_lib, causal, layout, n):
    _check_ring(gpu_lib, 2, 4, n, 4, 2, 128, causal, layout, "bf16", 200 + n)


@pytest.mark.parametrize("steps_per_launch", ["1", "2"])
@pytest.mark.parametrize("P,n,causal,layout", [(5, 200, True, "contiguous"), (4, 320, True, "striped"),
                                               (3, 128, False, "contiguous"), (4, 200, True, "zigzag"),
                                               (7, 130, True, "striped"), (2, 257, True, "contiguous")])
def test_bf16_ring_one_and_two_steps_per_launch(gpu_lib, monkeypatch, steps_per_launch, P, n, causal, layout):
    """The whole local ring folds two ring steps per launch by default (the second block pulled from the
    predecessor's slot, pushed on to the successor's next slot); RING_ATTN_STEPS_PER_LAUNCH=1 keeps one
    step per launch.  Both match the oracle, with odd ring sizes (a last launch of one step) and ragged
    blocks."""
    monkeypatch.setenv("RING_ATTN_STEPS_PER_LAUNCH", steps_per_launch)
    _check_ring(gpu_lib, 1, P, n, 4, 2, 128, causal, layout, "bf16", 270 + P * 10 + n)


@pytest.mark.parametrize("layout", ["contiguous", "striped"])
@pytest.mark.parametrize("n", [65, 257])
def test_bf16_mfma_ring_query_tile_edges(gpu_lib, layout, n):
    """Causal blocks whose last query tile ends one row into a key tile: the rows of that tile reach
    the step kernel's forwarding workgroups only partly, so those blocks travel by copy instead."""
    _check_ring(gpu_lib, 1, 4, n, 2, 1, 128, True, layout, "bf16", 250 + n)


@pytest.mark.parametrize("causal,layout", [(False, "contiguous"), (True, "striped")])
def test_bf16_partly_local_ring(gpu_lib, causal, layout):
    """Devices 2..4 of a 6-device ring run locally: the local devices hand blocks on inside the step
    kernels, and device 2 receives from its remote predecessor by copy."""
    P, n, Hq, Hkv, D, dev0, n_local = 6, 160, 4, 2, 128, 2, 3
    S = P * n
    q, k, v = _inputs(1, S, Hq, Hkv, D, 650 + causal, "bf16")
    pos = oracle.shard_positions(S, P, layout)
    q_local = q[:, pos[dev0:dev0 + n_local].reshape(-1)]
    o, lse = run_ring_local(q_local, k, v, P=P, causal=causal, layout=layout, dtype="bf16", dev0=dev0,
                            n_local=n_local)
    toks = pos[dev0:dev0 + n_local]  # [n_local, n] token of each local row
    rows = np.array([[0, h, int(toks[t, r])] for t in range(n_local) for h in range(Hq) for r in range(n)])
    ref_o, ref_lse = oracle.attention_rows(to_float(q, "bf16"), to_float(k, "bf16"), to_float(v, "bf16"), rows,
                                           causal=causal)
    got_o = np.concatenate([o[t, 0].transpose(1, 0, 2).reshape(-1, D) for t in range(n_local)])
    got_lse = np.concatenate([lse[t, 0].reshape(-1) for t in range(n_local)])
    assert max_err(got_o, ref_o) <= TOL_BF16_O and max_err(got_lse, ref_lse) <= TOL_BF16_LSE


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [40, 128])
def test_fp32_zigzag_ring(gpu_lib, causal, D):
    _check_ring(gpu_lib, 2, 4, 38, 3, 1, D, causal, "zigzag", "f32", 700 + D + causal)


@pytest.mark.parametrize("causal,P,n", [(True, 4, 128), (True, 4, 200), (True, 8, 258), (False, 4, 130)])
def test_bf16_mfma_zigzag_ring(gpu_lib, causal, P, n):
    """Zigzag shards (chunks i and 2P-1-i): each device folds its two chunks as two row windows of
    the step kernel, with ragged chunk lengths (100, 129, 65 rows) and two batch elements."""
    _check_ring(gpu_lib, 2, P, n, 4, 2, 128, causal, "zigzag", "bf16", 720 + n)


def test_bf16_zigzag_partly_local_and_many_devices(gpu_lib):
    """Zigzag for devices 2..4 of a 6-device ring, and a 36-device ring whose 72 chunk units need
    two launches per step."""
    P, n, Hq, Hkv, D, dev0, n_local = 6, 160, 4, 2, 128, 2, 3
    S = P * n
    q, k, v = _inputs(1, S, Hq, Hkv, D, 760, "bf16")
    pos = oracle.shard_positions(S, P, "zigzag")
    q_local = q[:, pos[dev0:dev0 + n_local].reshape(-1)]
    o, lse = run_ring_local(q_local, k, v, P=P, causal=True, layout="zigzag", dtype="bf16", dev0=dev0,
                            n_local=n_local)
    toks = pos[dev0:dev0 + n_local]
    rows = np.array([[0, h, int(toks[t, r])] for t in range(n_local) for h in range(Hq) for r in range(n)])
    ref_o, ref_lse = oracle.attention_rows(to_float(q, "bf16"), to_float(k, "bf16"), to_float(v, "bf16"), rows,
                                           causal=True)
    got_o = np.concatenate([o[t, 0].transpose(1, 0, 2).reshape(-1, D) for t in range(n_local)])
    got_lse = np.concatenate([lse[t, 0].reshape(-1) for t in range(n_local)])
    assert max_err(got_o, ref_o) <= TOL_BF16_O and max_err(got_lse, ref_lse) <= TOL_BF16_LSE
    _check_ring(gpu_lib, 1, 36, 64, 2, 1, 128, True, "zigzag", "bf16", 770)


def test_bf16_mfma_ring_gqa_striped_p8(gpu_lib):
    _check_ring(gpu_lib, 1, 8, 192, 8, 2, 128, True, "striped", "bf16", 300)


def test_bf16_generic_head_dim_64(gpu_lib):
    _check_ring(gpu_lib, 1, 4, 96, 4, 4, 64, True, "contiguous", "bf16", 400)


def test_single_stream_and_host_source(gpu_lib):
    _check_ring(gpu_lib, 1, 4, 160, 4, 1, 128, True, "contiguous", "bf16", 500, two_streams=False)
    _check_ring(gpu_lib, 1, 4, 160, 4, 1, 128, True, "striped", "bf16", 501, host_kv=True)
    _check_ring(gpu_lib, 1, 4, 40, 2, 1, 32, False, "contiguous", "f32", 502, host_kv=True)


def test_one_device_share_of_a_longer_ring(gpu_lib):
    """Only the last device of an 8-way causal ring runs locally (dev0 = 7, n_local = 1)."""
    P, n, Hq, Hkv, D = 8, 192, 4, 4, 128
    S = P * n
    q, k, v = _inputs(1, S, Hq, Hkv, D, 600, "bf16")
    o, lse = run_ring_local(q[:, (P - 1) * n:], k, v, P=P, causal=True, layout="contiguous", dtype="bf16", dev0=P - 1,
                            n_local=1)
    rows = np.array([[0, h, t] for h in range(Hq) for t in range((P - 1) * n, S)])
    ref_o, ref_lse = oracle.attention_rows(to_float(q, "bf16"), to_float(k, "bf16"), to_float(v, "bf16"), rows,
                                           causal=True)
    got_o = o[0, 0].transpose(1, 0, 2).reshape(-1, D)
    got_lse = lse[0, 0].reshape(-1)
    assert max_err(got_o, ref_o) <= TOL_BF16_O and max_err(got_lse, ref_lse) <= TOL_BF16_LSE


def test_large_scores_stay_finite(gpu_lib):
    """Scores far beyond exp's fp32 range (queries scaled by 30, max score > 88.7): the running
    maximum keeps everything finite and the result exact; values stay N(0, 1)."""
    for dtype, D in (("bf16", 128), ("f32", 32)):
        P, n, H = 4, 130, 2
        S = P * n
        q, k, v = _inputs(1, S, H, H, D, 700 + D, dtype)
        qf = to_float(q, dtype) * 30.0
        q = si.bf16_bits(qf) if dtype == "bf16" else qf.astype(np.float32)
        scores = np.einsum("shd,thd->hst", to_float(q, dtype)[0], to_float(k, dtype)[0]) / math.sqrt(D)
        assert scores.max() > 88.7
        o, lse = run_ring_local(q, k, v, P=P, causal=True, layout="contiguous", dtype=dtype)
        ref_o, ref_lse = oracle.attention_reference(to_float(q, dtype), to_float(k, dtype), to_float(v, dtype),
                                                    causal=True)
        assert np.isfinite(o).all() and np.isfinite(lse).all()
        # fp32 bound at these magnitudes: a score near 150 carries fp32 spacing ~1.5e-5 and its D-term
        # dot product about sqrt(D) such roundings, which shifts the weights by that relative amount;
        # the output moves by at most that times max|v|, and the LSE by that plus 2 ulps of |LSE|
        score_err = math.sqrt(D) * 2.0 ** -23 * np.abs(scores).max()
        lse_ulps = 2 * 2.0 ** -23 * np.abs(ref_lse).max()
        vmax = np.abs(to_float(v, dtype)).max()
        tol_o, tol_l = ((TOL_BF16_O, TOL_BF16_LSE) if dtype == "bf16"
                        else (TOL_F32 + score_err * vmax, TOL_F32 + score_err + lse_ulps))
        assert max_err(unshard_out(o, "contiguous"), ref_o) <= tol_o
        assert max_err(unshard_lse(lse, "contiguous"), ref_lse) <= tol_l


# ---------------------------------------------------------------- ring_attn_step used directly

def _state(n_dev, B, Hq, Nq, D):
    return (torch.zeros((n_dev, B, Hq, Nq, D), dtype=torch.float32, device="cuda"),
            torch.zeros((n_dev, B, Hq, Nq), dtype=torch.float32, device="cuda"),
            torch.zeros((n_dev, B, Hq, Nq), dtype=torch.float32, device="cuda"))


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 48)])
def test_arrival_order_does_not_matter(gpu_lib, dtype, D):
    """Each device folds the ring's blocks in a random order (one ring_attn_step per block)."""
    ra = gpu_lib
    P, n, Hq, Hkv = 4, 144, 2, 1
    S = P * n
    q, k, v = _inputs(1, S, Hq, Hkv, D, 800 + D, dtype)
    ref_o, ref_lse = oracle.attention_reference(to_float(q, dtype), to_float(k, dtype), to_float(v, dtype), causal=True)
    layout = "striped"
    qs, ks, vs = shard(q, P, layout), shard(k, P, layout), shard(v, P, layout)
    rng = np.random.default_rng(801)
    o_acc, m, l = _state(P, 1, Hq, n, D)
    tq = to_device(qs, dtype)
    tk = [to_device(np.ascontiguousarray(ks[j:j + 1]), dtype) for j in range(P)]
    tv = [to_device(np.ascontiguousarray(vs[j:j + 1]), dtype) for j in range(P)]
    orders = [rng.permutation(P) for _ in range(P)]
    for i in range(P):
        qi = tq[i:i + 1].contiguous()
        st = [x[i:i + 1].contiguous() for x in (o_acc, m, l)]
        for step, j in enumerate(orders[i]):
            ra.ring_attn_step(qi, tk[j], tv[j], *st, scale=1 / math.sqrt(D), causal=True, q_off=[i], q_stride=P,
                              k_off=[int(j)], k_stride=P, init=(step == 0))
        for x, y in zip((o_acc, m, l), st):
            x[i:i + 1].copy_(y)
    o = torch.empty_like(tq)
    lse = torch.empty((P, 1, Hq, n), dtype=torch.float32, device="cuda")
    ra.ring_attn_finalize(o_acc, m, l, o, lse)
    torch.cuda.synchronize()
    eo = max_err(unshard_out(out_to_f64(o), layout), ref_o)
    el = max_err(unshard_lse(lse.cpu().numpy(), layout), ref_lse)
    tol_o, tol_l = (TOL_BF16_O, TOL_BF16_LSE) if dtype == "bf16" else (TOL_F32, TOL_F32)
    assert eo <= tol_o and el <= tol_l


def test_splitting_a_block_gives_the_same_state(gpu_lib):
    """Folding a block in two parts (a split that is not a tile boundary of the second part) gives
    attention over the whole block: both the one-call and the two-call states finalize to the oracle's
    output and log-sum-exp at the bf16 tolerances, and to each other within the same bounds."""
    ra = gpu_lib
    n, Hq, D = 256, 2, 128
    q, k, v = _inputs(1, n, Hq, Hq, D, 900, "bf16")
    tq, tk, tv = to_device(q[None], "bf16"), to_device(k[None], "bf16"), to_device(v[None], "bf16")
    whole = _state(1, 1, Hq, n, D)
    ra.ring_attn_step(tq, tk, tv, *whole, scale=D ** -0.5, init=True)
    halves = _state(1, 1, Hq, n, D)
    h = n // 2 + 64
    ra.ring_attn_step(tq, tk[:, :, :h].contiguous(), tv[:, :, :h].contiguous(), *halves, scale=D ** -0.5, init=True)
    ra.ring_attn_step(tq, tk[:, :, h:].contiguous(), tv[:, :, h:].contiguous(), *halves, scale=D ** -0.5)
    outs = []
    for st in (whole, halves):
        o = torch.empty_like(tq)
        lse = torch.empty((1, 1, Hq, n), dtype=torch.float32, device="cuda")
        ra.ring_attn_finalize(*st, o, lse)
        outs.append((out_to_f64(o), lse.cpu().numpy()))
    ref_o, ref_lse = oracle.attention_reference(to_float(q, "bf16"), to_float(k, "bf16"), to_float(v, "bf16"))
    for got_o, got_l in outs:
        assert max_err(got_o[0], ref_o) <= TOL_BF16_O
        assert max_err(got_l[0], ref_lse) <= TOL_BF16_LSE
    assert max_err(outs[0][0], outs[1][0]) <= TOL_BF16_O
    assert max_err(outs[0][1], outs[1][1]) <= TOL_BF16_LSE


@pytest.mark.parametrize("dtype,D,qscale", [("bf16", 128, 1.0), ("bf16", 128, 30.0), ("f32", 48, 30.0)])
def test_state_after_steps_keeps_the_documented_bounds(gpu_lib, dtype, D, qscale):
    """The running state read back after two ring_attn_step calls (a fresh fold, then a continuing one
    with a merge) satisfies the bounds the C header states, against the exact row maximum X of
    x = log2(e) * scale * q.k over the visible keys (float64, from the same inputs):
        m <= X <= m + 64,  1 <= l <= N 2^64,  m + log2 l = log2 sum 2^x  (the LSE in base 2),
        o_acc / l = attention output,
    and rows that have seen no key hold m = -inf, l = 0, o_acc = 0.  Queries scaled by 30 give
    score spreads of hundreds of log2 units, so the MFMA kernel's reference exponent lags X by up to
    its limit; the plain kernel (fp32) keeps m = X."""
    ra = gpu_lib
    n_dev, B, Hq, Hkv, Nq, Nk = 2, 1, 4, 2, 300, 200
    q, k, v = _inputs(B, n_dev * Nq, Hq, Hkv, D, 950 + D, dtype)
    _, k2, v2 = _inputs(B, n_dev * Nk, Hq, Hkv, D, 960 + D, dtype)
    k, v = k[:, :n_dev * Nk], v[:, :n_dev * Nk]
    if qscale != 1.0:
        qf = to_float(q, dtype) * qscale
        q = si.bf16_bits(qf) if dtype == "bf16" else qf.astype(np.float32)
    qd = q.reshape(B, n_dev, Nq, Hq, D).transpose(1, 0, 2, 3, 4)
    blocks = [(k.reshape(B, n_dev, Nk, Hkv, D).transpose(1, 0, 2, 3, 4), v.reshape(B, n_dev, Nk, Hkv, D).transpose(1, 0, 2, 3, 4)),
              (k2.reshape(B, n_dev, Nk, Hkv, D).transpose(1, 0, 2, 3, 4), v2.reshape(B, n_dev, Nk, Hkv, D).transpose(1, 0, 2, 3, 4))]
    # positions: device t's queries at 1000 t + 2 r; block 0's keys at 1000 t + 250 + 2 u (query rows
    # below 125 see none of them), block 1's keys at 1000 t + 20 + u (query rows below 10 see none):
    # rows 0..9 end with the empty state, rows 10..124 are first seen by the continuing step
    q_off = [1000 * t for t in range(n_dev)]
    k_offs = [[1000 * t + 250 for t in range(n_dev)], [1000 * t + 20 for t in range(n_dev)]]
    k_strides = [2, 1]
    scale = 1.0 / math.sqrt(D)
    tq = to_device(np.ascontiguousarray(qd), dtype)
    st = _state(n_dev, B, Hq, Nq, D)
    ra.ring_attn_step(tq, to_device(np.ascontiguousarray(blocks[0][0]), dtype),
                      to_device(np.ascontiguousarray(blocks[0][1]), dtype), *st, scale=scale, causal=True, q_off=q_off,
                      q_stride=2, k_off=k_offs[0], k_stride=k_strides[0], init=True)
    ra.ring_attn_step(tq, to_device(np.ascontiguousarray(blocks[1][0]), dtype),
                      to_device(np.ascontiguousarray(blocks[1][1]), dtype), *st, scale=scale, causal=True, q_off=q_off,
                      q_stride=2, k_off=k_offs[1], k_stride=k_strides[1])
    torch.cuda.synchronize()
    o_acc, m, l = (x.cpu().numpy().astype(np.float64) for x in st)
    log2e = 1.0 / math.log(2.0)
    g = Hq // Hkv
    checked_lag = 0.0
    for t in range(n_dev):
        qpos = q_off[t] + 2 * np.arange(Nq)
        kk = np.concatenate([to_float(blocks[b][0][t, 0], dtype) for b in (0, 1)]).astype(np.float64)
        vv = np.concatenate([to_float(blocks[b][1][t, 0], dtype) for b in (0, 1)]).astype(np.float64)
        kpos = np.concatenate([k_offs[b][t] + k_strides[b] * np.arange(Nk) for b in (0, 1)])
        ref_o, ref_lse = oracle.attention_reference(to_float(qd[t], dtype), kk[None], vv[None], causal=True,
                                                    q_pos=qpos, k_pos=kpos)
        for h in range(Hq):
            x = (to_float(qd[t, 0, :, h], dtype).astype(np.float64) @ kk[:, h // g].T) * scale * log2e
            vis = kpos[None, :] <= qpos[:, None]
            n_vis = vis.sum(axis=1)
            X = np.where(vis, x, -np.inf).max(axis=1)
            mh, lh, oh = m[t, 0, h], l[t, 0, h], o_acc[t, 0, h]
            seen = n_vis > 0
            assert (~seen).sum() == 10
            if dtype == "bf16":
                tol_o, tol_l = TOL_BF16_O, TOL_BF16_LSE
            else:  # fp32: each x carries about sqrt(D) roundings of its size (see the large-score test)
                score_err = math.sqrt(D) * 2.0 ** -23 * np.abs(x[vis]).max() / log2e
                tol_o = TOL_F32 + 2 * score_err * np.abs(vv).max()
                tol_l = TOL_F32 + 2 * score_err
            assert np.all(np.isneginf(mh[~seen])) and np.all(lh[~seen] == 0) and np.all(oh[~seen] == 0)
            eps = 1e-3 + 1e-6 * np.abs(X[seen])
            assert np.all(mh[seen] <= X[seen] + eps), "reference exponent above the row maximum"
            assert np.all(X[seen] <= mh[seen] + 64 + eps), "reference exponent lags by more than 64"
            assert np.all(lh[seen] >= 1 - 1e-4) and np.all(lh[seen] <= n_vis[seen] * 2.0 ** 64 * (1 + 1e-6))
            assert max_err(mh[seen] + np.log2(lh[seen]), ref_lse[0, h, seen] * log2e) <= tol_l * log2e
            assert max_err(oh[seen] / lh[seen][:, None], ref_o[0, seen, h]) <= tol_o
            if dtype == "f32":
                assert np.all(np.abs(mh[seen] - X[seen]) <= eps)
            checked_lag = max(checked_lag, float((X[seen] - mh[seen]).max()))
    print(f"[state] {dtype} D={D} q x{qscale}: largest lag X - m = {checked_lag:.3g} (log2 units)", flush=True)


def test_state_snapshot_and_resume(gpu_lib):
    """The (o_acc, m, l) state after k steps is a complete checkpoint of the ring."""
    ra = gpu_lib
    P, n, Hq, D = 4, 128, 2, 128
    S = P * n
    q, k, v = _inputs(1, S, Hq, Hq, D, 1000, "bf16")
    qs, ks, vs = (to_device(shard(x, P, "contiguous"), "bf16") for x in (q, k, v))
    st = _state(P, 1, Hq, n, D)

    def step(s, state):
        # all devices at once: device i holds block (i - s) mod P
        kk = torch.stack([ks[(i - s) % P] for i in range(P)]).contiguous()
        vv = torch.stack([vs[(i - s) % P] for i in range(P)]).contiguous()
        ra.ring_attn_step(qs, kk, vv, *state, scale=D ** -0.5, causal=True, q_off=[i * n for i in range(P)],
                          k_off=[((i - s) % P) * n for i in range(P)], init=(s == 0))

    for s in range(2):
        step(s, st)
    torch.cuda.synchronize()
    saved = [x.cpu() for x in st]
    resumed = [x.cuda() for x in saved]
    for s in range(2, P):
        step(s, st)
        step(s, resumed)
    res = []
    for state in (st, resumed):
        o = torch.empty_like(qs)
        lse = torch.empty((P, 1, Hq, n), dtype=torch.float32, device="cuda")
        ra.ring_attn_finalize(*state, o, lse)
        res.append((out_to_f64(o), lse.cpu().numpy()))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])
    ref_o, ref_lse = oracle.attention_reference(to_float(q, "bf16"), to_float(k, "bf16"), to_float(v, "bf16"),
                                                causal=True)
    assert max_err(unshard_out(res[0][0], "contiguous"), ref_o) <= TOL_BF16_O
    assert max_err(unshard_lse(res[0][1], "contiguous"), ref_lse) <= TOL_BF16_LSE


@pytest.mark.parametrize("D,dtype", [(5, "f32"), (5, "bf16"), (128, "bf16"), (128, "f32"), (12, "bf16"), (64, "bf16"),
                                     (48, "f32")])
def test_finalize_divides_and_writes_lse(gpu_lib, D, dtype):
    """ring_attn_finalize on a random valid state (the four-load kernel for D % 16 == 0, with 8, 4 or 3
    threads per row here; the one-load kernel for other D % 4 == 0; the scalar one otherwise):
    o = o_acc / l in token-major order, lse = (m + log2 l) ln 2, and o = 0, lse = -inf where l = 0;
    checked against the same formulas in float64."""
    ra = gpu_lib
    n_dev, B, Hq, Nq = 3, 2, 5, 37
    rng = np.random.default_rng(1800 + D)
    o_acc = rng.standard_normal((n_dev, B, Hq, Nq, D)).astype(np.float32) * 4
    m = rng.standard_normal((n_dev, B, Hq, Nq)).astype(np.float32) * 10
    l = rng.uniform(1, 100, (n_dev, B, Hq, Nq)).astype(np.float32)
    empty = rng.random((n_dev, B, Hq, Nq)) < 0.1
    l[empty] = 0
    o_acc[empty] = 0
    m[empty] = -np.inf
    t = [torch.from_numpy(x).cuda() for x in (o_acc, m, l)]
    o = torch.empty((n_dev, B, Nq, Hq, D), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda")
    lse = torch.empty((n_dev, B, Hq, Nq), dtype=torch.float32, device="cuda")
    ra.ring_attn_finalize(*t, o, lse)
    torch.cuda.synchronize()
    with np.errstate(divide="ignore", invalid="ignore"):
        want_o = np.where(l[..., None] > 0, o_acc.astype(np.float64) / l[..., None], 0.0).transpose(0, 1, 3, 2, 4)
        want_l = np.where(l > 0, (m.astype(np.float64) + np.log2(l.astype(np.float64))) * math.log(2.0), -np.inf)
    got_o = o.float().cpu().numpy().astype(np.float64)
    tol = 2.0 ** -8 * np.abs(want_o).max() if dtype == "bf16" else 1e-6 * np.abs(want_o).max()
    assert max_err(got_o, want_o) <= tol
    assert max_err(lse.cpu().numpy(), want_l) <= 1e-5 * np.abs(want_l[np.isfinite(want_l)]).max()


def test_empty_and_fully_masked_edges(gpu_lib):
    ra = gpu_lib
    D, Hq = 128, 2
    q, k, v = _inputs(1, 64, Hq, Hq, D, 1100, "bf16")
    tq, tk, tv = to_device(q[None], "bf16"), to_device(k[None], "bf16"), to_device(v[None], "bf16")
    # a block whose keys all lie after every query: skipped; with init the state is the empty state
    st = _state(1, 1, Hq, 64, D)
    st[0].fill_(7.0)
    ra.ring_attn_step(tq, tk, tv, *st, scale=0.1, causal=True, q_off=[0], k_off=[64], init=True)
    o = torch.empty_like(tq)
    lse = torch.empty((1, 1, Hq, 64), dtype=torch.float32, device="cuda")
    ra.ring_attn_finalize(*st, o, lse)
    torch.cuda.synchronize()
    assert torch.all(o.float() == 0) and torch.all(lse == float("-inf"))
    # zero keys: nothing folded; zero queries: nothing to do
    st2 = _state(1, 1, Hq, 64, D)
    ra.ring_attn_step(tq, tk[:, :, :0].contiguous(), tv[:, :, :0].contiguous(), *st2, scale=0.1, init=True)
    empty_state = (st2[0][:, :, :, :0].contiguous(), st2[1][:, :, :, :0].contiguous(), st2[2][:, :, :, :0].contiguous())
    ra.ring_attn_step(tq[:, :, :0].contiguous(), tk, tv, *empty_state, scale=0.1)
    torch.cuda.synchronize()
    # queries that see only part of the block: partially masked rows, first rows see nothing
    st3 = _state(1, 1, Hq, 64, D)
    ra.ring_attn_step(tq, tk, tv, *st3, scale=D ** -0.5, causal=True, q_off=[0], k_off=[10], init=True)
    ra.ring_attn_finalize(*st3, o, lse)
    torch.cuda.synchronize()
    qpos, kpos = np.arange(64), np.arange(64) + 10
    ref_o, ref_lse = oracle.attention_reference(to_float(q, "bf16"), to_float(k, "bf16"), to_float(v, "bf16"),
                                                causal=True, q_pos=qpos, k_pos=kpos)
    assert max_err(out_to_f64(o)[0], ref_o) <= TOL_BF16_O
    assert max_err(lse.cpu().numpy()[0], ref_lse) <= TOL_BF16_LSE
