"""ring_attn_local_noalloc (no device allocation; the library's fixed scratch) against ring_attn_local
(caller workspace) through the C ABI: the same rings give the same bits, call after call, including a
second call on a smaller input that reuses the scratch the first one left behind, and both match the
oracle at the bf16 / fp32 bounds.  A ring too large for the scratch is refused."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from ring_harness import TOL_BF16_LSE, TOL_BF16_O, TOL_F32, max_err, shard, to_device, to_float, unshard_lse, unshard_out

pytestmark = pytest.mark.gpu


def _ring_pair(ra, P, n, Hq, Hkv, D, causal, layout, dtype, seed, two_streams):
    S = P * n
    gen = si.normal_bf16 if dtype == "bf16" else si.normal_f32
    q, k, v = gen(seed, (1, S, Hq, D)), gen(seed + 1, (1, S, Hkv, D)), gen(seed + 2, (1, S, Hkv, D))
    tq, tk, tv = (to_device(shard(x, P, layout), dtype) for x in (q, k, v))
    code = ra.RA_BF16 if dtype == "bf16" else ra.RA_F32
    assert ra.ring_attn_local_workspace_bytes(P, P, 1, Hq, Hkv, n, D, code) <= ra.ring_attn_noalloc_scratch_bytes()
    cs = torch.cuda.Stream()
    xs = torch.cuda.Stream() if two_streams else None
    outs = []
    for noalloc in (False, True):
        o = torch.empty_like(tq)
        lse = torch.empty((P, 1, Hq, n), dtype=torch.float32, device="cuda")
        if noalloc:
            ra.ring_attn_local_noalloc(tq, tk, tv, o, lse, P=P, dev0=0, scale=1 / math.sqrt(D), causal=causal,
                                       layout=layout, compute_stream=cs, copy_stream=xs)
        else:
            ws = torch.empty(ra.ring_attn_local_workspace_bytes(P, P, 1, Hq, Hkv, n, D, code), dtype=torch.uint8,
                             device="cuda")
            ra.ring_attn_local(tq, tk, tv, o, lse, ws, P=P, dev0=0, scale=1 / math.sqrt(D), causal=causal,
                               layout=layout, compute_stream=cs, copy_stream=xs)
        torch.cuda.synchronize()
        outs.append((o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)))
    ref_o, ref_l = oracle.attention_reference(to_float(q, dtype), to_float(k, dtype), to_float(v, dtype),
                                              causal=causal)
    return outs, ref_o, ref_l


@pytest.mark.parametrize("two_streams_first", [True, False])
def test_noalloc_matches_the_workspace_entry_point(gpu_lib, two_streams_first):
    ra = gpu_lib
    calls = [  # the second and third calls reuse the scratch on smaller rings; one runs on a single stream
        (4, 512, 8, 2, 128, True, "striped", "bf16", 1700, two_streams_first),
        (4, 130, 4, 1, 128, True, "contiguous", "bf16", 1710, not two_streams_first),
        (4, 38, 3, 1, 40, True, "zigzag", "f32", 1720, True),
    ]
    for P, n, Hq, Hkv, D, causal, layout, dtype, seed, two in calls:
        print(f"[noalloc] P={P} n={n} Hq={Hq} Hkv={Hkv} D={D} {layout} {dtype} two_streams={two}", flush=True)
        outs, ref_o, ref_l = _ring_pair(ra, P, n, Hq, Hkv, D, causal, layout, dtype, seed, two)
        (o_ws, l_ws), (o_na, l_na) = outs
        assert np.array_equal(o_na, o_ws) and np.array_equal(l_na, l_ws)
        tol_o, tol_l = (TOL_BF16_O, TOL_BF16_LSE) if dtype == "bf16" else (TOL_F32, TOL_F32)
        assert max_err(unshard_out(o_na, layout), ref_o) <= tol_o
        assert max_err(unshard_lse(l_na, layout), ref_l) <= tol_l


def test_noalloc_refuses_a_ring_larger_than_its_scratch(gpu_lib):
    ra = gpu_lib
    P, n, H, D = 8, 4096, 8, 128
    assert ra.ring_attn_local_workspace_bytes(P, P, 1, H, H, n, D, ra.RA_BF16) > ra.ring_attn_noalloc_scratch_bytes()
    q = torch.zeros((P, 1, n, H, D), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((P, 1, n, H, D), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    with pytest.raises(ra.RingAttnError) as err:
        ra.ring_attn_local_noalloc(q, k, k.clone(), o, None, P=P, dev0=0, scale=D ** -0.5)
    assert err.value.code == ra.RA_ERR_SCRATCH
