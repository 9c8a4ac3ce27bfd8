"""GPU parity of the backward ring (bf16 inputs, fp32 gradients) against the float64 gradient oracle.

Each case runs the forward ring (``ring_attn_local``) for O and LSE, then ``ring_attn_bwd_local``
with a seeded output gradient dO, and compares dQ, dK, dV with ``oracle.attention_backward_reference``
on the same bf16 inputs.

Tolerance (derived, the pages fix none for gradients): the kernels recompute P in fp32 from the
forward's log-sum-exp (relative error ~1e-6) and round P and dS to bf16 for the matrix products
(relative error at most 2^-9 per term, unbiased); delta = sum dO * O uses the bf16 output (relative
2^-9 per term).  Each gradient entry is a sum of such terms with fp32 accumulation, so its error is a
few 2^-9 of the magnitude of its terms; bounded here by max |err| <= 2e-2 * max |ref| per tensor and
a relative Frobenius error <= 1e-2.

The other (dtype, head dim) cases run the plain fp32 kernel pair: fp32 inputs keep P, dS and every
product in fp32 (unit roundoff 2^-24), so each gradient entry carries a few 1e-7 of the magnitude of
its terms summed over a few hundred keys or queries; bounded by max |err| <= 1e-4 * max |ref| and a
relative Frobenius error <= 2e-5, hundreds of times below what a dropped term or a wrong mask gives.
bf16 inputs on that path keep the bf16 bounds above.
"""
import math

import numpy as np
import pytest
import torch

import blockwise_ring_attention_step_amd as ra
import oracle
import synth_inputs as si
from ring_harness import shard, to_device, to_float, unshard_out

pytestmark = pytest.mark.gpu

TOL_MAX = 2e-2
TOL_FRO = 1e-2
TOL_F32_MAX = 1e-4
TOL_F32_FRO = 2e-5


def _unshard_kv(x, layout):
    """[P, B, n, H, D] shard order -> [B, S, H, D] token order."""
    return unshard_out(x, layout)


def _errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = max(np.abs(ref).max(), 1e-30)
    emax = np.abs(got - ref).max() / scale
    efro = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    return emax, efro


def _run_bwd(q, k, v, do, *, P, causal, layout, dev0=0, n_local=None, scale=None, two_streams=True, dtype="bf16"):
    """q/dO [B, S, Hq, D] (bf16 bits or fp32 per dtype, token order), k/v [B, S, Hkv, D].  Returns (dq [n_local, B, n, Hq, D],
    dk, dv [P, B, n, Hkv, D]) float64 in shard order, and the local query shards' token positions."""
    B, S, Hkv, D = k.shape
    Hq = q.shape[2]
    n = S // P
    n_local = P if n_local is None else n_local
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    qs = shard(q, P, layout)[dev0:dev0 + n_local]
    dos = shard(do, P, layout)[dev0:dev0 + n_local]
    tq, tdo = to_device(qs, dtype), to_device(dos, dtype)
    tk, tv = to_device(shard(k, P, layout), dtype), to_device(shard(v, P, layout), dtype)
    code = ra.RA_BF16 if dtype == "bf16" else ra.RA_F32
    o = torch.empty_like(tq)
    lse = torch.empty((n_local, B, Hq, n), dtype=torch.float32, device="cuda")
    cs = torch.cuda.current_stream()
    xs = torch.cuda.Stream() if two_streams else None
    ws = torch.empty(ra.ring_attn_local_workspace_bytes(P, n_local, B, Hq, Hkv, n, D, code), dtype=torch.uint8,
                     device="cuda")
    ra.ring_attn_local(tq, tk, tv, o, lse, ws, P=P, dev0=dev0, scale=scale, causal=causal, layout=layout,
                       copy_stream=xs)
    dq = torch.empty(tq.shape, dtype=torch.float32, device="cuda")
    dk = torch.empty(tk.shape, dtype=torch.float32, device="cuda")
    dv = torch.empty(tk.shape, dtype=torch.float32, device="cuda")
    wsb = torch.empty(ra.ring_attn_bwd_local_workspace_bytes(P, n_local, B, Hq, Hkv, n, D, code),
                      dtype=torch.uint8, device="cuda")
    # poison the outputs: every element must be written
    dq.fill_(float("nan"))
    dk.fill_(float("nan"))
    dv.fill_(float("nan"))
    ra.ring_attn_bwd_local(tq, tk, tv, o, tdo, lse, dq, dk, dv, wsb, P=P, dev0=dev0, scale=scale, causal=causal,
                           layout=layout, compute_stream=cs, copy_stream=xs)
    torch.cuda.synchronize()
    f = lambda t: t.cpu().numpy().astype(np.float64)
    return f(dq), f(dk), f(dv)


def _check(B, P, n, Hq, Hkv, causal, layout, seed, dev0=0, n_local=None, dtype="bf16", D=128):
    S = P * n
    gen = si.normal_bf16 if dtype == "bf16" else si.normal_f32
    q = gen(seed, (B, S, Hq, D))
    k = gen(seed + 1, (B, S, Hkv, D))
    v = gen(seed + 2, (B, S, Hkv, D))
    do = gen(seed + 3, (B, S, Hq, D))
    n_local = P if n_local is None else n_local
    dq, dk, dv = _run_bwd(q, k, v, do, P=P, causal=causal, layout=layout, dev0=dev0, n_local=n_local, dtype=dtype)
    qf, kf, vf, dof = (to_float(x, dtype) for x in (q, k, v, do))
    pos = oracle.shard_positions(S, P, layout)
    local_tok = pos[dev0:dev0 + n_local].reshape(-1)
    if n_local < P:  # only the local queries contribute: zero the output gradient of the others
        keep = np.zeros(S, bool)
        keep[local_tok] = True
        dof = np.where(keep[None, :, None, None], dof, 0.0)
    rq, rk, rv = oracle.attention_backward_reference(qf, kf, vf, dof, causal=causal)
    got_q = dq.transpose(1, 0, 2, 3, 4).reshape(B, n_local * n, Hq, D)
    ref_q = rq[:, local_tok]
    got_k, got_v = _unshard_kv(dk, layout), _unshard_kv(dv, layout)
    errs = {"dq": _errors(got_q, ref_q), "dk": _errors(got_k, rk), "dv": _errors(got_v, rv)}
    print(f"[bwd] {dtype} D={D} B={B} P={P} n={n} Hq={Hq} Hkv={Hkv} causal={causal} {layout} dev0={dev0} "
          f"n_local={n_local}: " + " ".join(f"{k_}: max {e[0]:.2e} fro {e[1]:.2e}" for k_, e in errs.items()),
          flush=True)
    tol_max, tol_fro = (TOL_MAX, TOL_FRO) if dtype == "bf16" else (TOL_F32_MAX, TOL_F32_FRO)
    for name, (emax, efro) in errs.items():
        assert np.isfinite(emax) and emax <= tol_max and efro <= tol_fro, name


@pytest.mark.parametrize("causal,layout,n", [(False, "contiguous", 128), (True, "contiguous", 200),
                                             (True, "striped", 160), (False, "contiguous", 72)])
def test_bwd_ring_small(gpu_lib, causal, layout, n):
    _check(2, 4, n, 4, 2, causal, layout, 900 + n)


@pytest.mark.parametrize("steps_per_launch", ["1", "2"])
@pytest.mark.parametrize("P,n,causal,layout", [(3, 200, True, "contiguous"), (5, 96, True, "striped"),
                                               (4, 160, False, "contiguous"), (2, 320, True, "striped"),
                                               (5, 72, True, "contiguous")])
def test_bwd_ring_one_and_two_steps_per_launch(gpu_lib, monkeypatch, steps_per_launch, P, n, causal, layout):
    """With the whole ring local, each query-gradient launch folds two ring steps (the block the device
    holds and its predecessor's, the latter handed on to the successor's next slot from inside the
    kernel); RING_ATTN_STEPS_PER_LAUNCH=1 keeps one step per launch.  Odd P ends on a one-step launch;
    contiguous causal rings pair a visible block with a fully masked one; both paths against the oracle."""
    monkeypatch.setenv("RING_ATTN_STEPS_PER_LAUNCH", steps_per_launch)
    _check(1, P, n, 4, 2, causal, layout, 1700 + 10 * P + n)


@pytest.mark.parametrize("causal,n", [(True, 128), (True, 200), (False, 96)])
def test_bwd_zigzag_ring(gpu_lib, causal, n):
    """Zigzag shards: each device's two chunks are separate units (ragged chunks of 64, 100, 48 rows)."""
    _check(2, 4, n, 4, 2, causal, "zigzag", 990 + n)


def test_bwd_ring_gqa_p8_and_partly_local(gpu_lib):
    _check(1, 8, 96, 8, 2, True, "striped", 950)
    _check(1, 6, 160, 4, 2, True, "contiguous", 960, dev0=2, n_local=3)
    _check(1, 6, 160, 4, 2, True, "zigzag", 970, dev0=2, n_local=3)


def test_bwd_step_accumulates_and_splits(gpu_lib):
    """Two bwd_step calls over the two halves of a key block equal one call over the whole block,
    and RA_BWD_INIT flags overwrite what the buffers held."""
    B, Nq, Nk, Hq, Hkv, D = 1, 160, 192, 4, 2, 128
    rng_seed = 980
    q = to_device(si.normal_bf16(rng_seed, (1, B, Nq, Hq, D)), "bf16")
    k = to_device(si.normal_bf16(rng_seed + 1, (1, B, Nk, Hkv, D)), "bf16")
    v = to_device(si.normal_bf16(rng_seed + 2, (1, B, Nk, Hkv, D)), "bf16")
    do = to_device(si.normal_bf16(rng_seed + 3, (1, B, Nq, Hq, D)), "bf16")
    # forward state of the whole block for lse, then delta and lse2
    oacc = torch.zeros((1, B, Hq, Nq, D), dtype=torch.float32, device="cuda")
    m = torch.zeros((1, B, Hq, Nq), dtype=torch.float32, device="cuda")
    l = torch.zeros_like(m)
    ra.ring_attn_step(q, k, v, oacc, m, l, scale=D ** -0.5, causal=True, q_off=[Nk - Nq], k_off=[0], init=True)
    o = torch.empty_like(q)
    lse = torch.empty_like(m)
    ra.ring_attn_finalize(oacc, m, l, o, lse)
    delta, lse2 = torch.empty_like(m), torch.empty_like(m)
    ra.ring_attn_bwd_prep(o, do, lse, delta, lse2)
    kw = dict(scale=D ** -0.5, causal=True, q_off=[Nk - Nq], k_off=[0])
    dq1 = torch.full((1, B, Nq, Hq, D), 7.0, device="cuda")
    dk1 = torch.full((1, B, Nk, Hkv, D), 7.0, device="cuda")
    dv1 = torch.full_like(dk1, 7.0)
    ra.ring_attn_bwd_step(q, k, v, do, lse2, delta, dq1, dk1, dv1, init_dq=True, init_dkv=True, **kw)
    # the same block in two halves (positions follow the keys)
    h = Nk // 2
    k0, k1 = k[:, :, :h].contiguous(), k[:, :, h:].contiguous()
    v0, v1 = v[:, :, :h].contiguous(), v[:, :, h:].contiguous()
    dq2 = torch.full_like(dq1, 7.0)
    dk2a, dk2b = torch.full((1, B, h, Hkv, D), 7.0, device="cuda"), torch.full((1, B, h, Hkv, D), 7.0, device="cuda")
    dv2a, dv2b = torch.full_like(dk2a, 7.0), torch.full_like(dk2b, 7.0)
    ra.ring_attn_bwd_step(q, k0, v0, do, lse2, delta, dq2, dk2a, dv2a, init_dq=True, init_dkv=True,
                          scale=D ** -0.5, causal=True, q_off=[Nk - Nq], k_off=[0])
    ra.ring_attn_bwd_step(q, k1, v1, do, lse2, delta, dq2, dk2b, dv2b, init_dkv=True,
                          scale=D ** -0.5, causal=True, q_off=[Nk - Nq], k_off=[h])
    torch.cuda.synchronize()
    assert (dq1 - dq2).abs().max().item() <= 1e-4 * max(dq1.abs().max().item(), 1e-6)
    for half, whole in ((torch.cat([dk2a, dk2b], dim=2), dk1), (torch.cat([dv2a, dv2b], dim=2), dv1)):
        assert (half - whole).abs().max().item() <= 1e-5 * max(whole.abs().max().item(), 1e-6)
    # and both agree with the oracle
    qf, kf, vf, dof = (x[0].float().cpu().numpy().astype(np.float64) for x in (q, k, v, do))
    rq, rk, rv = oracle.attention_backward_reference(qf, kf, vf, dof, causal=True, q_pos=np.arange(Nq) + Nk - Nq,
                                                     k_pos=np.arange(Nk))
    for got, ref in ((dq1, rq), (dk1, rk), (dv1, rv)):
        emax, efro = _errors(got[0].cpu().numpy(), ref)
        assert emax <= TOL_MAX and efro <= TOL_FRO


@pytest.mark.parametrize("dtype,D,causal,layout,n,dev0,n_local", [
    ("f32", 64, True, "contiguous", 72, 0, None),
    ("f32", 40, True, "striped", 50, 0, None),
    ("f32", 128, True, "zigzag", 64, 0, None),   # fp32 at D = 128 also takes the plain kernels
    ("f32", 16, False, "contiguous", 33, 1, 2),
    ("bf16", 64, False, "contiguous", 96, 0, None),
    ("bf16", 80, True, "zigzag", 70, 1, 2),
    ("f32", 3, True, "striped", 21, 0, None),     # odd head dim: lanes past D idle
    ("bf16", 1, False, "contiguous", 17, 2, 2),   # head dim 1
])
def test_bwd_ring_generic_kernels(gpu_lib, dtype, D, causal, layout, n, dev0, n_local):
    """Every (dtype, head dim) other than bf16 at 128 runs the plain fp32 kernel pair."""
    _check(2, 4, n, 4, 2, causal, layout, 1100 + D + n, dev0=dev0, n_local=n_local, dtype=dtype, D=D)


def test_bwd_step_generic_accumulates_and_splits(gpu_lib):
    """fp32, head dim 48: two bwd_step calls over the halves of a key block equal one call over the
    whole block (accumulation and both INIT flags on the plain kernels), and match the oracle."""
    B, Nq, Nk, Hq, Hkv, D = 2, 70, 90, 3, 1, 48
    seed = 1200
    q = to_device(si.normal_f32(seed, (1, B, Nq, Hq, D)), "f32")
    k = to_device(si.normal_f32(seed + 1, (1, B, Nk, Hkv, D)), "f32")
    v = to_device(si.normal_f32(seed + 2, (1, B, Nk, Hkv, D)), "f32")
    do = to_device(si.normal_f32(seed + 3, (1, B, Nq, Hq, D)), "f32")
    oacc = torch.zeros((1, B, Hq, Nq, D), dtype=torch.float32, device="cuda")
    m = torch.zeros((1, B, Hq, Nq), dtype=torch.float32, device="cuda")
    l = torch.zeros_like(m)
    kw = dict(scale=D ** -0.5, causal=True, q_off=[Nk - Nq], k_off=[0])
    ra.ring_attn_step(q, k, v, oacc, m, l, init=True, **kw)
    o = torch.empty_like(q)
    lse = torch.empty_like(m)
    ra.ring_attn_finalize(oacc, m, l, o, lse)
    delta, lse2 = torch.empty_like(m), torch.empty_like(m)
    ra.ring_attn_bwd_prep(o, do, lse, delta, lse2)
    dq1 = torch.full((1, B, Nq, Hq, D), 7.0, device="cuda")
    dk1 = torch.full((1, B, Nk, Hkv, D), 7.0, device="cuda")
    dv1 = torch.full_like(dk1, 7.0)
    ra.ring_attn_bwd_step(q, k, v, do, lse2, delta, dq1, dk1, dv1, init_dq=True, init_dkv=True, **kw)
    h = 37
    k0, k1 = k[:, :, :h].contiguous(), k[:, :, h:].contiguous()
    v0, v1 = v[:, :, :h].contiguous(), v[:, :, h:].contiguous()
    dq2 = torch.full_like(dq1, 7.0)
    dk2a, dk2b = torch.full((1, B, h, Hkv, D), 7.0, device="cuda"), torch.full((1, B, Nk - h, Hkv, D), 7.0, device="cuda")
    dv2a, dv2b = torch.full_like(dk2a, 7.0), torch.full_like(dk2b, 7.0)
    ra.ring_attn_bwd_step(q, k0, v0, do, lse2, delta, dq2, dk2a, dv2a, init_dq=True, init_dkv=True, **kw)
    ra.ring_attn_bwd_step(q, k1, v1, do, lse2, delta, dq2, dk2b, dv2b, init_dkv=True, scale=D ** -0.5, causal=True,
                          q_off=[Nk - Nq], k_off=[h])
    torch.cuda.synchronize()
    assert (dq1 - dq2).abs().max().item() <= 1e-5 * max(dq1.abs().max().item(), 1e-6)
    for half, whole in ((torch.cat([dk2a, dk2b], dim=2), dk1), (torch.cat([dv2a, dv2b], dim=2), dv1)):
        assert torch.equal(half, whole)  # the same rows, summed in the same order
    qf, kf, vf, dof = (x[0].cpu().numpy().astype(np.float64) for x in (q, k, v, do))
    rq, rk, rv = oracle.attention_backward_reference(qf, kf, vf, dof, causal=True, q_pos=np.arange(Nq) + Nk - Nq,
                                                     k_pos=np.arange(Nk))
    for name, got, ref in (("dq", dq1, rq), ("dk", dk1, rk), ("dv", dv1, rv)):
        emax, efro = _errors(got[0].cpu().numpy(), ref)
        print(f"[bwd] step fp32 D={D} {name}: max {emax:.2e} fro {efro:.2e}", flush=True)
        assert emax <= TOL_F32_MAX and efro <= TOL_F32_FRO, name
