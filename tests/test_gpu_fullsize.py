"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

Each workload runs the whole ring through ``ring_attn_local`` (all emulated devices on the GPU, hop
copies on a second stream) on seeded inputs of its real shape.  The float64 oracle is evaluated on
at least 4096 seeded random (head, token) rows plus forced edge rows (token 0, the last token, the
first and last row of every shard), and every sampled row is compared on all D outputs and its
log-sum-exp: output max abs error <= 2e-2, log-sum-exp <= 1e-3 (bf16 inputs, fp32 accumulation).
The contiguous 64k run is checked against the oracle on its own rows, and the striped causal run is
also compared with the contiguous run of the same inputs after un-permuting, on every output element.
The backward rings are checked on sampled query rows (dQ) and sampled key rows (dK, dV).
"""
import math

import numpy as np
import pytest
import torch

import blockwise_ring_attention_step_amd as ra
import oracle
import synth_inputs as si
from ring_harness import TOL_BF16_LSE, TOL_BF16_O, max_err

pytestmark = pytest.mark.gpu

N_SAMPLES = 4096


def _shard_positions(w):
    return oracle.shard_positions(w.S, w.P, w.layout)


def _sample_rows(w, seed, q_tokens):
    """(batch, head, index into q's token axis) rows: random ones plus forced edge rows."""
    rng = np.random.default_rng(seed)
    n_tok = q_tokens
    flat = rng.choice(n_tok * w.Hq, size=min(N_SAMPLES, n_tok * w.Hq), replace=False)
    rows = {(0, int(f % w.Hq), int(f // w.Hq)) for f in flat}
    if w.local_shard is None:
        edges = {0, w.S - 1}
        pos = _shard_positions(w)
        for i in range(w.P):
            edges.add(int(pos[i, 0]))
            edges.add(int(pos[i, -1]))
    else:
        edges = {0, 1, w.n - 1}
    for t in edges:
        for h in range(w.Hq):
            rows.add((0, h, t))
    return np.array(sorted(rows), dtype=np.int64)


def _run(w, q, k, v):
    """Shard, upload, run the ring; returns (o [n_local, B, n, Hq, D] bf16 tensor, lse tensor)."""
    pos = _shard_positions(w)
    perm = pos.reshape(-1)
    B, n = w.B, w.n

    def shard(x):
        return np.ascontiguousarray(x[:, perm].reshape(B, w.P, n, x.shape[2], w.D).transpose(1, 0, 2, 3, 4))

    def up(x):
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()

    if w.local_shard is None:
        tq = up(shard(q))
        dev0, n_local = 0, w.P
    else:
        tq = up(np.ascontiguousarray(q.reshape(B, 1, n, w.Hq, w.D).transpose(1, 0, 2, 3, 4)))
        dev0, n_local = w.local_shard, 1
    tk, tv = up(shard(k)), up(shard(v))
    o = torch.empty_like(tq)
    lse = torch.empty((n_local, B, w.Hq, n), dtype=torch.float32, device="cuda")
    ws = torch.empty(ra.ring_attn_local_workspace_bytes(w.P, n_local, B, w.Hq, w.Hkv, n, w.D, ra.RA_BF16),
                     dtype=torch.uint8, device="cuda")
    ra.ring_attn_local(tq, tk, tv, o, lse, ws, P=w.P, dev0=dev0, scale=1.0 / math.sqrt(w.D), causal=w.causal,
                       layout=w.layout, copy_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    del tk, tv, ws
    return o, lse


def _gather(w, o, lse, rows):
    """GPU outputs of the sampled rows (token-order indices) as float64 arrays."""
    if w.local_shard is None:
        pos = _shard_positions(w)
        shard_of = np.empty(w.S, dtype=np.int64)
        local_of = np.empty(w.S, dtype=np.int64)
        shard_of[pos.reshape(-1)] = np.repeat(np.arange(w.P), w.n)
        local_of[pos.reshape(-1)] = np.tile(np.arange(w.n), w.P)
        i, r = shard_of[rows[:, 2]], local_of[rows[:, 2]]
    else:
        i, r = np.zeros(len(rows), dtype=np.int64), rows[:, 2]
    ti, tb, tr, th = (torch.from_numpy(x).cuda() for x in (i, rows[:, 0], r, rows[:, 1]))
    got_o = o[ti, tb, tr, th].float().cpu().numpy().astype(np.float64)
    got_l = lse[ti, tb, th, tr].cpu().numpy().astype(np.float64)
    return got_o, got_l


def _check(name, seed):
    w = si.WORKLOADS[name]
    print(f"[fullsize] {name}: generating inputs", flush=True)
    q, k, v = si.workload_qkv(w)
    o, lse = _run(w, q, k, v)
    rows = _sample_rows(w, seed, q.shape[1])
    got_o, got_l = _gather(w, o, lse, rows)
    del o, lse
    torch.cuda.empty_cache()
    print(f"[fullsize] {name}: oracle on {len(rows)} rows", flush=True)
    q_pos = None if w.local_shard is None else w.local_shard * w.n + np.arange(w.n)
    ref_o, ref_l = oracle.attention_rows(si.bf16_to_f32(q), si.bf16_to_f32(k), si.bf16_to_f32(v), rows,
                                         causal=w.causal, q_pos=q_pos)
    eo, el = max_err(got_o, ref_o), max_err(got_l, ref_l)
    print(f"[fullsize] {name}: rows={len(rows)} max|dO|={eo:.3g} max|dLSE|={el:.3g}", flush=True)
    assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE


def test_noncausal_16k_eight_devices():
    _check("noncausal_16k", 21)


def test_causal_32k_contiguous():
    _check("causal_32k", 31)


def test_causal_64k_striped_gqa():
    _check("causal_striped_64k", 41)


def test_causal_64k_zigzag_gqa():
    _check("causal_zigzag_64k", 42)


def test_one_device_share_of_1m_ring():
    _check("causal_1m_shard", 51)


def test_causal_64k_contiguous_gqa():
    """The inputs of the striped 64k workload sharded contiguously (the layout the striped one is
    compared with), against the oracle on its own sampled rows."""
    _check("causal_contig_64k", 43)


def test_striped_and_zigzag_match_contiguous_after_unpermuting():
    """The same 64k causal GQA inputs under the three shardings agree on every output element."""
    ws_, wc = si.WORKLOADS["causal_striped_64k"], si.WORKLOADS["causal_contig_64k"]
    wz = si.WORKLOADS["causal_zigzag_64k"]
    q, k, v = si.workload_qkv(ws_)
    outs = {}
    for w in (ws_, wc, wz):
        o, lse = _run(w, q, k, v)
        pos = torch.from_numpy(_shard_positions(w).reshape(-1)).cuda()
        tok_o = torch.empty((w.B, w.S, w.Hq, w.D), dtype=torch.bfloat16, device="cuda")
        tok_o[:, pos] = o.transpose(0, 1).reshape(w.B, w.S, w.Hq, w.D)
        tok_l = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device="cuda")
        tok_l[:, :, pos] = lse.permute(1, 2, 0, 3).reshape(w.B, w.Hq, w.S)
        outs[w.layout] = (tok_o, tok_l)
        del o, lse
        torch.cuda.empty_cache()
    for layout in ("striped", "zigzag"):
        do = (outs[layout][0].float() - outs["contiguous"][0].float()).abs().max().item()
        dl = (outs[layout][1] - outs["contiguous"][1]).abs().max().item()
        print(f"[fullsize] {layout} vs contiguous 64k: max|dO|={do:.3g} max|dLSE|={dl:.3g}", flush=True)
        assert math.isfinite(do) and math.isfinite(dl)
        assert do <= TOL_BF16_O and dl <= TOL_BF16_LSE


def _key_rows(w, seed, kvh=None, min_pos=0, n=N_SAMPLES):
    """(batch, key/value head, key token) rows: random ones (tokens >= min_pos; one head if kvh is
    given) plus every shard's first and last key row among them."""
    rng = np.random.default_rng(seed)
    heads = [kvh] if kvh is not None else list(range(w.Hkv))
    toks = np.arange(min_pos, w.S)
    flat = rng.choice(len(toks) * len(heads), size=min(n, len(toks) * len(heads)), replace=False)
    rows = {(0, heads[int(f % len(heads))], int(toks[f // len(heads)])) for f in flat}
    pos = _shard_positions(w)
    for i in range(w.P):
        for t in (int(pos[i, 0]), int(pos[i, -1])):
            if t >= min_pos:
                for h in heads:
                    rows.add((0, h, t))
    return np.array(sorted(rows), dtype=np.int64)


def _backward_run(w):
    """Forward then backward ring of workload w at full size; returns (q, k, v, do host arrays, dq, dk,
    dv device tensors in shard order)."""
    q, k, v = si.workload_qkv(w)
    do = si.workload_dout(w)
    perm = _shard_positions(w).reshape(-1)
    B, n, P = w.B, w.n, w.P

    def up(x):
        y = np.ascontiguousarray(x[:, perm].reshape(B, P, n, x.shape[2], w.D).transpose(1, 0, 2, 3, 4))
        return torch.from_numpy(y.view(np.int16)).view(torch.bfloat16).cuda()

    tq, tk, tv, tdo = up(q), up(k), up(v), up(do)
    o = torch.empty_like(tq)
    lse = torch.empty((P, B, w.Hq, n), dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(w.D)
    ws = torch.empty(ra.ring_attn_local_workspace_bytes(P, P, B, w.Hq, w.Hkv, n, w.D, ra.RA_BF16), dtype=torch.uint8,
                     device="cuda")
    xs = torch.cuda.Stream()
    ra.ring_attn_local(tq, tk, tv, o, lse, ws, P=P, dev0=0, scale=scale, causal=w.causal, layout=w.layout,
                       copy_stream=xs)
    del ws
    dq = torch.empty(tq.shape, dtype=torch.float32, device="cuda")
    dk = torch.empty(tk.shape, dtype=torch.float32, device="cuda")
    dv = torch.empty(tk.shape, dtype=torch.float32, device="cuda")
    wsb = torch.empty(ra.ring_attn_bwd_local_workspace_bytes(P, P, B, w.Hq, w.Hkv, n, w.D, ra.RA_BF16),
                      dtype=torch.uint8, device="cuda")
    ra.ring_attn_bwd_local(tq, tk, tv, o, tdo, lse, dq, dk, dv, wsb, P=P, dev0=0, scale=scale, causal=w.causal,
                           layout=w.layout, copy_stream=xs)
    torch.cuda.synchronize()
    del tq, tk, tv, tdo, o, lse, wsb
    return q, k, v, do, dq, dk, dv


def _gather_rows(w, t, rows, tok_col=2, head_col=1):
    """Entries of a shard-order tensor [P, B, n, H, D] at token-order rows (batch, head, token)."""
    perm = _shard_positions(w).reshape(-1)
    shard_of = np.empty(w.S, dtype=np.int64)
    local_of = np.empty(w.S, dtype=np.int64)
    shard_of[perm] = np.repeat(np.arange(w.P), w.n)
    local_of[perm] = np.tile(np.arange(w.n), w.P)
    idx = (shard_of[rows[:, tok_col]], rows[:, 0], local_of[rows[:, tok_col]], rows[:, head_col])
    ti, tb, tr, th = (torch.from_numpy(x).cuda() for x in idx)
    return t[ti, tb, tr, th].cpu().numpy().astype(np.float64)


def _rel(got, ref):
    return np.abs(got - ref).max() / np.abs(ref).max(), np.linalg.norm(got - ref) / np.linalg.norm(ref)


def test_backward_noncausal_16k_sampled_rows_and_identities():
    """The backward ring of the non-causal 16k workload at its full size: dQ on >= 4096 sampled query
    rows and dK, dV on >= 4096 sampled key rows (plus every shard's first and last row) against the
    oracle element by element, and dK, dV through identities that hold at any size: each head's key
    gradients sum to zero (softmax rows are invariant to shifting every key) and each key/value head's
    value gradients sum to the output gradients of its query heads (softmax rows sum to one).
    Bound (bf16 inputs, fp32 gradients): max |err| <= 2e-2 max |ref| and relative Frobenius <= 1e-2."""
    w = si.WORKLOADS["bwd_noncausal_16k"]
    print("[fullsize] backward 16k: running the rings", flush=True)
    q, k, v, do, dq, dk, dv = _backward_run(w)
    B = w.B
    g = w.Hq // w.Hkv
    sum_k = dk.double().sum(dim=(0, 2))             # [B, Hkv, D]
    abs_k = dk.double().abs().sum(dim=(0, 2))
    sum_v = dv.double().sum(dim=(0, 2))
    do64 = torch.from_numpy(si.bf16_to_f32(do)).double().reshape(B, w.S, w.Hkv, g, w.D)
    want_v = do64.sum(dim=(1, 3)).cuda()            # [B, Hkv, D]
    ek = (sum_k.abs() / abs_k).max().item()
    ev = ((sum_v - want_v).abs().max() / want_v.abs().max()).item()
    print(f"[fullsize] backward 16k: |sum dK| / sum |dK| <= {ek:.3g}, sum dV vs sum dO rel {ev:.3g}", flush=True)
    assert ek <= 1e-3 and ev <= 1e-3
    qrows = _sample_rows(w, 61, w.S)
    krows = _key_rows(w, 62)
    got_q = _gather_rows(w, dq, qrows)
    got_k, got_v = _gather_rows(w, dk, krows), _gather_rows(w, dv, krows)
    del dq, dk, dv
    torch.cuda.empty_cache()
    qf, kf, vf, dof = (si.bf16_to_f32(x) for x in (q, k, v, do))
    print(f"[fullsize] backward 16k: oracle on {len(qrows)} query rows and {len(krows)} key rows", flush=True)
    ref_q = oracle.attention_backward_rows(qf, kf, vf, dof, qrows, causal=w.causal)
    ref_k, ref_v = oracle.attention_backward_key_rows(qf, kf, vf, dof, krows, causal=w.causal)
    for name, got, ref in (("dQ", got_q, ref_q), ("dK", got_k, ref_k), ("dV", got_v, ref_v)):
        emax, efro = _rel(got, ref)
        print(f"[fullsize] backward 16k: {name} max {emax:.3g} fro {efro:.3g} (relative)", flush=True)
        assert emax <= 2e-2 and efro <= 1e-2, name


def test_backward_causal_striped_64k_late_key_rows():
    """The striped causal GQA backward at its full size (65536 tokens, 32 query / 8 key-value heads):
    dK and dV of >= 4096 sampled key rows of key/value head 3 among the last 8192 token positions
    (spread over every shard's last local rows), and dQ of >= 4096 sampled query rows of that head
    group in the same window, against the oracle element by element.  Those key rows are seen only by
    the last 8192 queries, which keeps the oracle's forward (their log-sum-exp and output over up to
    65536 keys, four heads) to seconds.  Same bound as the non-causal test."""
    w = si.WORKLOADS["bwd_causal_striped_64k"]
    print("[fullsize] backward striped 64k: running the rings", flush=True)
    q, k, v, do, dq, dk, dv = _backward_run(w)
    kvh, g, lo = 3, w.Hq // w.Hkv, w.S - 8192
    krows = _key_rows(w, 71, kvh=kvh, min_pos=lo)
    rng = np.random.default_rng(72)
    qtok = rng.choice(np.arange(lo, w.S), size=N_SAMPLES // g, replace=False)
    qrows = np.array([(0, h, int(t)) for t in qtok for h in range(kvh * g, (kvh + 1) * g)], dtype=np.int64)
    got_q = _gather_rows(w, dq, qrows)
    got_k, got_v = _gather_rows(w, dk, krows), _gather_rows(w, dv, krows)
    del dq, dk, dv
    torch.cuda.empty_cache()
    qf, kf, vf, dof = (si.bf16_to_f32(x) for x in (q, k, v, do))
    print(f"[fullsize] backward striped 64k: oracle on {len(qrows)} query rows and {len(krows)} key rows",
          flush=True)
    ref_q = oracle.attention_backward_rows(qf, kf, vf, dof, qrows, causal=True)
    ref_k, ref_v = oracle.attention_backward_key_rows(qf, kf, vf, dof, krows, causal=True)
    for name, got, ref in (("dQ", got_q, ref_q), ("dK", got_k, ref_k), ("dV", got_v, ref_v)):
        emax, efro = _rel(got, ref)
        print(f"[fullsize] backward striped 64k: {name} max {emax:.3g} fro {efro:.3g} (relative)", flush=True)
        assert emax <= 2e-2 and efro <= 1e-2, name
