"""Stress of the ring's double-buffered hop, and the stop-and-resume checkpoint, on the GPU.

The hop that "Ring Attention Là Gì?" (thienlv.com, section "Ring Attention Hoạt Động Thế Nào?")
describes, the next block in flight while the current one is used, is emulated with two receive
slots per device: copies on a second stream, or stores from inside the step kernel (the forward step
kernel, and the backward's query-gradient kernel).  A slot that is
read before its block has landed, or overwritten while still being read, gives wrong results only
under some timings, so the library's test hooks (RING_ATTN_HOP_STRESS, documented in ring_attn.h)
change the timing and make stale data visible:

* poison: every slot range is filled with NaN on the stream about to write it, just before the write;
* jitter-copy / jitter-compute: a bounded sleep kernel before each step's copies / each step kernel.

Under every mode the outputs must equal, bit for bit, those of the unstressed run (the arithmetic is
the same; only the order of independent work changes), which in turn match the oracle.

RING_ATTN_FAIL_AT_STEP=k stops the ring before step k and returns RA_ERR_INJECTED, leaving the
running state of the first k steps in the workspace.  Resuming from it with ring_attn_step for the
remaining steps and ring_attn_finalize must give the oracle's attention (the state is a complete
checkpoint of the fold).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from ring_harness import (TOL_BF16_LSE, TOL_BF16_O, TOL_F32, max_err, run_ring_local, shard, to_device, to_float,
                          unshard_lse, unshard_out)

pytestmark = pytest.mark.gpu

MODES = ["poison", "poison,jitter-copy", "poison,jitter-compute", "jitter-copy,jitter-compute"]


def _inputs(S, Hq, Hkv, D, seed, dtype):
    gen = si.normal_bf16 if dtype == "bf16" else si.normal_f32
    return gen(seed, (1, S, Hq, D)), gen(seed + 1, (1, S, Hkv, D)), gen(seed + 2, (1, S, Hkv, D))


# (P, n, Hq, Hkv, D, causal, layout, dtype, dev0, n_local, host_kv): in-step hops only (the first two),
# copies and in-step hops mixed (partly local ring), copies only (zigzag, fp32), host-to-device copies
CASES = [
    (4, 256, 4, 2, 128, False, "contiguous", "bf16", 0, 4, False),
    (4, 320, 4, 2, 128, True, "striped", "bf16", 0, 4, False),
    (6, 160, 4, 2, 128, True, "contiguous", "bf16", 2, 3, False),
    (4, 200, 4, 2, 128, True, "zigzag", "bf16", 0, 4, False),
    (4, 160, 4, 1, 128, True, "striped", "bf16", 0, 4, True),
    (4, 37, 3, 1, 40, True, "striped", "f32", 0, 4, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"P{c[0]}-n{c[1]}-{c[6]}-{c[7]}-local{c[9]}-host{int(c[10])}")
def test_forward_ring_unchanged_under_hop_stress(gpu_lib, monkeypatch, case):
    P, n, Hq, Hkv, D, causal, layout, dtype, dev0, n_local, host_kv = case
    S = P * n
    q, k, v = _inputs(S, Hq, Hkv, D, 1300 + n + D, dtype)
    pos = oracle.shard_positions(S, P, layout)
    q_in = q if n_local == P else q[:, pos[dev0:dev0 + n_local].reshape(-1)]

    def run():
        return run_ring_local(q_in, k, v, P=P, causal=causal, layout=layout, dtype=dtype, dev0=dev0, n_local=n_local,
                              host_kv=host_kv)

    monkeypatch.delenv("RING_ATTN_HOP_STRESS", raising=False)
    base_o, base_l = run()
    toks = pos[dev0:dev0 + n_local]
    rows = np.array([[0, h, int(toks[t, r])] for t in range(n_local) for h in range(Hq) for r in range(n)])
    ref_o, ref_l = oracle.attention_rows(to_float(q, dtype), to_float(k, dtype), to_float(v, dtype), rows,
                                         causal=causal)
    got_o = np.concatenate([base_o[t, 0].transpose(1, 0, 2).reshape(-1, D) for t in range(n_local)])
    got_l = np.concatenate([base_l[t, 0].reshape(-1) for t in range(n_local)])
    tol_o, tol_l = (TOL_BF16_O, TOL_BF16_LSE) if dtype == "bf16" else (TOL_F32, TOL_F32)
    assert max_err(got_o, ref_o) <= tol_o and max_err(got_l, ref_l) <= tol_l
    for mode in MODES:
        monkeypatch.setenv("RING_ATTN_HOP_STRESS", mode)
        print(f"[hops] forward {case} under {mode}", flush=True)
        o, l = run()
        assert np.isfinite(o).all() and not np.isnan(l).any(), mode
        assert np.array_equal(o, base_o) and np.array_equal(l, base_l), mode
    monkeypatch.delenv("RING_ATTN_HOP_STRESS", raising=False)


@pytest.mark.parametrize("steps_per_launch", ["1", "2"])
@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
def test_backward_ring_unchanged_under_hop_stress(gpu_lib, monkeypatch, layout, steps_per_launch):
    ra = gpu_lib
    monkeypatch.setenv("RING_ATTN_STEPS_PER_LAUNCH", steps_per_launch)
    P, n, Hq, Hkv, D = 4, 256, 4, 2, 128
    S = P * n
    q, k, v = _inputs(S, Hq, Hkv, D, 1400, "bf16")
    do = si.normal_bf16(1403, (1, S, Hq, D))
    tq, tk, tv, tdo = (to_device(shard(x, P, layout), "bf16") for x in (q, k, v, do))
    o = torch.empty_like(tq)
    lse = torch.empty((P, 1, Hq, n), dtype=torch.float32, device="cuda")
    ws = torch.empty(ra.ring_attn_local_workspace_bytes(P, P, 1, Hq, Hkv, n, D, ra.RA_BF16), dtype=torch.uint8,
                     device="cuda")
    monkeypatch.delenv("RING_ATTN_HOP_STRESS", raising=False)
    xs = torch.cuda.Stream()
    ra.ring_attn_local(tq, tk, tv, o, lse, ws, P=P, dev0=0, scale=D ** -0.5, causal=True, layout=layout, copy_stream=xs)
    wsb = torch.empty(ra.ring_attn_bwd_local_workspace_bytes(P, P, 1, Hq, Hkv, n, D, ra.RA_BF16), dtype=torch.uint8,
                      device="cuda")

    def run():
        dq = torch.empty(tq.shape, dtype=torch.float32, device="cuda")
        dk = torch.empty(tk.shape, dtype=torch.float32, device="cuda")
        dv = torch.empty(tk.shape, dtype=torch.float32, device="cuda")
        ra.ring_attn_bwd_local(tq, tk, tv, o, tdo, lse, dq, dk, dv, wsb, P=P, dev0=0, scale=D ** -0.5, causal=True,
                               layout=layout, copy_stream=xs)
        torch.cuda.synchronize()
        return [x.cpu().numpy() for x in (dq, dk, dv)]

    base = run()
    for mode in MODES:
        monkeypatch.setenv("RING_ATTN_HOP_STRESS", mode)
        print(f"[hops] backward {layout} under {mode}", flush=True)
        got = run()
        for g, b in zip(got, base):
            assert np.isfinite(g).all() and np.array_equal(g, b), mode
    monkeypatch.delenv("RING_ATTN_HOP_STRESS", raising=False)


@pytest.mark.parametrize("layout,stop", [("contiguous", 2), ("striped", 1), ("contiguous", 0), ("zigzag", 3)])
def test_stop_after_k_steps_leaves_a_checkpoint(gpu_lib, monkeypatch, layout, stop):
    """ring_attn_local stopped before step `stop` (RA_ERR_INJECTED), then resumed from the workspace
    state with one ring_attn_step per remaining step (every device at once) and finalized."""
    ra = gpu_lib
    P, n, Hq, Hkv, D, B = 4, 192, 4, 2, 128, 1
    S = P * n
    q, k, v = _inputs(S, Hq, Hkv, D, 1500 + stop, "bf16")
    tq, tk, tv = (to_device(shard(x, P, layout), "bf16") for x in (q, k, v))
    o = torch.empty_like(tq)
    lse = torch.empty((P, B, Hq, n), dtype=torch.float32, device="cuda")
    ws = torch.empty(ra.ring_attn_local_workspace_bytes(P, P, B, Hq, Hkv, n, D, ra.RA_BF16), dtype=torch.uint8,
                     device="cuda")
    ws.fill_(0xFF)  # NaN everywhere: a device whose state the stop leaves unwritten would show
    monkeypatch.setenv("RING_ATTN_FAIL_AT_STEP", str(stop))
    with pytest.raises(ra.RingAttnError) as err:
        ra.ring_attn_local(tq, tk, tv, o, lse, ws, P=P, dev0=0, scale=D ** -0.5, causal=True, layout=layout,
                           copy_stream=torch.cuda.Stream())
    monkeypatch.delenv("RING_ATTN_FAIL_AT_STEP")
    assert err.value.code == ra.RA_ERR_INJECTED
    torch.cuda.synchronize()
    # the state, at the offsets the header documents
    R = lambda x: (x + 255) // 256 * 256
    blk = B * n * Hkv * D * 2
    rows = P * B * Hq * n
    off = 4 * R(P * blk)
    o_acc = ws[off:off + rows * D * 4].view(torch.float32).view(P, B, Hq, n, D)
    off += R(rows * D * 4)
    m = ws[off:off + rows * 4].view(torch.float32).view(P, B, Hq, n)
    off += R(rows * 4)
    l = ws[off:off + rows * 4].view(torch.float32).view(P, B, Hq, n)
    state = [x.clone() for x in (o_acc, m, l)]
    assert not any(torch.isnan(x).any().item() for x in state)
    pos = oracle.shard_positions(S, P, layout)
    for s in range(stop, P):
        js = [(i - s) % P for i in range(P)]
        kk = torch.stack([tk[j] for j in js]).contiguous()
        vv = torch.stack([tv[j] for j in js]).contiguous()
        if layout == "zigzag":  # two position runs per shard: one step per chunk of the query rows
            c = n // 2
            for half in range(2):
                qh = tq[:, :, half * c:(half + 1) * c].contiguous()
                sub = [x[:, :, :, half * c:(half + 1) * c].contiguous() for x in state]
                for kh in range(2):  # the key block's two chunks, each one run of positions
                    ra.ring_attn_step(qh, kk[:, :, kh * c:(kh + 1) * c].contiguous(),
                                      vv[:, :, kh * c:(kh + 1) * c].contiguous(), *sub, scale=D ** -0.5, causal=True,
                                      q_off=[int(pos[i, half * c]) for i in range(P)],
                                      k_off=[int(pos[j, kh * c]) for j in js])
                for x, y in zip(state, sub):
                    x[:, :, :, half * c:(half + 1) * c].copy_(y)
        else:
            stride = P if layout == "striped" else 1
            ra.ring_attn_step(tq, kk, vv, *state, scale=D ** -0.5, causal=True, q_off=[int(pos[i, 0]) for i in range(P)],
                              q_stride=stride, k_off=[int(pos[j, 0]) for j in js], k_stride=stride)
    out = torch.empty_like(tq)
    lse2 = torch.empty_like(lse)
    ra.ring_attn_finalize(*state, out, lse2)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attention_reference(to_float(q, "bf16"), to_float(k, "bf16"), to_float(v, "bf16"),
                                              causal=True)
    eo = max_err(unshard_out(out.float().cpu().numpy().astype(np.float64), layout), ref_o)
    el = max_err(unshard_lse(lse2.cpu().numpy().astype(np.float64), layout), ref_l)
    print(f"[hops] stop at {stop} ({layout}) and resume: max|dO|={eo:.3g} max|dLSE|={el:.3g}", flush=True)
    assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE
