"""Helpers shared by the GPU tests: upload seeded inputs, run the ring through the C ABI, and bring
results back in token order for comparison with the oracle.  (No attention arithmetic here.)"""
from __future__ import annotations

import math

import numpy as np
import torch

import blockwise_ring_attention_step_amd as ra
import oracle
import synth_inputs as si

TOL_F32 = 1e-5          # max abs error, fp32 inputs
TOL_BF16_O = 2e-2       # max abs error of the output, bf16 inputs with fp32 accumulation
TOL_BF16_LSE = 1e-3     # max abs error of the log-sum-exp


def to_device(x: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 array or bf16 bit patterns -> GPU tensor."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def to_float(x: np.ndarray, dtype: str) -> np.ndarray:
    return si.bf16_to_f32(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)


def out_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def shard(x: np.ndarray, P: int, layout: str) -> np.ndarray:
    """[B, S, H, D] token order -> [P, B, n, H, D] shard order."""
    B, S, H, D = x.shape
    perm = oracle.shard_positions(S, P, layout).reshape(-1)
    return np.ascontiguousarray(x[:, perm].reshape(B, P, S // P, H, D).transpose(1, 0, 2, 3, 4))


def unshard_out(o: np.ndarray, layout: str) -> np.ndarray:
    """[P, B, n, H, D] shard order -> [B, S, H, D] token order."""
    P, B, n, H, D = o.shape
    perm = oracle.shard_positions(P * n, P, layout).reshape(-1)
    flat = o.transpose(1, 0, 2, 3, 4).reshape(B, P * n, H, D)
    out = np.empty_like(flat)
    out[:, perm] = flat
    return out


def unshard_lse(lse: np.ndarray, layout: str) -> np.ndarray:
    """[P, B, H, n] -> [B, H, S]."""
    P, B, H, n = lse.shape
    perm = oracle.shard_positions(P * n, P, layout).reshape(-1)
    flat = lse.transpose(1, 2, 0, 3).reshape(B, H, P * n)
    out = np.empty_like(flat)
    out[:, :, perm] = flat
    return out


def run_ring_local(q, k, v, *, P, causal, layout, dtype, dev0=0, n_local=None, scale=None, host_kv=False,
                   two_streams=True):
    """q [B, S or n_local*n, Hq, D], k/v [B, S, Hkv, D] (token order; bits for bf16).  A q with S rows
    is in token order and is sharded here; a q with n_local*n < S rows holds the local devices' rows
    already in shard order (so a full local ring takes q in token order).

    Runs ring_attn_local for devices [dev0, dev0+n_local) and returns (o [P_local, B, n, Hq, D] float64
    in shard order, lse [P_local, B, Hq, n])."""
    B, S, Hkv, D = k.shape
    n = S // P
    n_local = P if n_local is None else n_local
    Hq = q.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    qs = shard(q, P, layout)[dev0:dev0 + n_local] if q.shape[1] == S else q.reshape(B, n_local, n, Hq, D).transpose(
        1, 0, 2, 3, 4)
    ks, vs = shard(k, P, layout), shard(v, P, layout)
    tq = to_device(np.ascontiguousarray(qs), dtype)
    if host_kv:
        tk = torch.from_numpy(ks.view(np.int16) if dtype == "bf16" else ks).pin_memory()
        tv = torch.from_numpy(vs.view(np.int16) if dtype == "bf16" else vs).pin_memory()
        if dtype == "bf16":
            tk, tv = tk.view(torch.bfloat16), tv.view(torch.bfloat16)
    else:
        tk, tv = to_device(ks, dtype), to_device(vs, dtype)
    o = torch.empty_like(tq)
    lse = torch.empty((n_local, B, Hq, n), dtype=torch.float32, device="cuda")
    code = ra.RA_BF16 if dtype == "bf16" else ra.RA_F32
    ws = torch.empty(ra.ring_attn_local_workspace_bytes(P, n_local, B, Hq, Hkv, n, D, code), dtype=torch.uint8,
                     device="cuda")
    copy_stream = torch.cuda.Stream() if two_streams else None
    ra.ring_attn_local(tq, tk, tv, o, lse, ws, P=P, dev0=dev0, scale=scale, causal=causal,
                       layout=layout, copy_stream=copy_stream)
    torch.cuda.synchronize()
    return out_to_f64(o), lse.cpu().numpy().astype(np.float64)


def max_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    d = np.where(both_inf, 0.0, np.abs(a - b))
    if np.isnan(d).any():
        return float("inf")
    return float(d.max()) if d.size else 0.0
