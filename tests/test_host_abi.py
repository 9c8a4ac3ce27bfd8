"""Host-side checks of the C ABI library that need no GPU: it loads, exports every declared entry
point, validates arguments before touching the GPU, and its ring planner matches the schedule and
the work counts that follow from the pages (closed forms and brute force over positions)."""
import ctypes
import os
import re

import numpy as np
import pytest

import blockwise_ring_attention_step_amd as ra
import oracle

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "ring_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ring_attn_\w+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    L = ra.lib()
    names = declared_functions()
    assert set(names) == set(ra.EXPORTED_SYMBOLS)
    for name in names:
        assert hasattr(L, name), name


def test_strerror():
    assert ra.ring_attn_strerror(0) == "ok"
    assert "invalid" in ra.ring_attn_strerror(-1)
    assert "unsupported" in ra.ring_attn_strerror(-2)
    assert "workspace" in ra.ring_attn_strerror(-4)
    assert "RING_ATTN_FAIL_AT_STEP" in ra.ring_attn_strerror(-5)
    assert "scratch" in ra.ring_attn_strerror(-6)
    assert ra.ring_attn_strerror(12345) == "unknown status"


# ---------------------------------------------------------------- planner

@pytest.mark.parametrize("P,n", [(1, 16), (4, 8), (8, 2048), (32, 5)])
@pytest.mark.parametrize("causal,striped", [(False, False), (True, False), (True, True)])
def test_plan_follows_the_ring(P, n, causal, striped):
    plan = ra.ring_attn_plan(P, 0, P, n, causal=causal, striped=striped)
    assert plan.shape == (P * P, 5)
    for s, i, j, slot, cls in plan:
        assert j == (i - s) % P and slot == s % 2
        if not causal:
            assert cls == 1
        elif striped:
            # every block pair is partially visible (token-interleaved positions)
            assert cls == (2 if n > 1 else (1 if j <= i else 0))
        else:
            assert cls == (2 if j == i else (1 if j < i else 0))
    # each device sees every block exactly once
    for i in range(P):
        assert sorted(plan[plan[:, 1] == i][:, 2]) == list(range(P))


def test_plan_for_one_device_share():
    P, n = 32, 32768
    plan = ra.ring_attn_plan(P, 31, 1, n, causal=True)
    assert list(plan[:, 2]) == [(31 - s) % P for s in range(P)]
    assert list(plan[:, 4]) == [2] + [1] * 31  # the diagonal block, then 31 fully visible blocks


@pytest.mark.parametrize("P,n", [(4, 8), (8, 16), (8, 5), (32, 4)])
def test_visible_pairs_match_brute_force_and_closed_forms(P, n):
    S = P * n
    for striped in (False, True):
        pos = oracle.shard_positions(S, P, "striped" if striped else "contiguous")
        for i in range(P):
            row = [ra.ring_attn_visible_pairs(P, n, i, j, causal=True, striped=striped) for j in range(P)]
            brute = [int((pos[j][None, :] <= pos[i][:, None]).sum()) for j in range(P)]
            assert row == brute
            if striped:
                assert sum(row) == P * n * (n - 1) // 2 + (i + 1) * n
            else:
                assert sum(row) == i * n * n + n * (n + 1) // 2
        assert ra.ring_attn_visible_pairs(P, n, 0, P - 1, causal=False, striped=striped) == n * n


@pytest.mark.parametrize("P,n", [(1, 2), (4, 8), (8, 16), (32, 4)])
def test_zigzag_plan_and_visible_pairs(P, n):
    S, c = P * n, n // 2
    pos = oracle.shard_positions(S, P, "zigzag")
    plan = ra.ring_attn_plan(P, 0, P, n, causal=True, layout="zigzag")
    for s, i, j, slot, cls in plan:
        assert j == (i - s) % P and slot == s % 2
        assert cls == 2  # each pair mixes visible and masked keys
    for i in range(P):
        row = [ra.ring_attn_visible_pairs(P, n, i, j, causal=True, layout="zigzag") for j in range(P)]
        assert row == [int((pos[j][None, :] <= pos[i][:, None]).sum()) for j in range(P)]
        assert row == [c * c + c * (c + 1) if j == i else 2 * c * c for j in range(P)]
    assert ra.ring_attn_visible_pairs(P, n, 0, P - 1, causal=False, layout="zigzag") == n * n
    L = ra.lib()
    buf = (ctypes.c_int32 * (5 * P * P))()
    assert L.ring_attn_plan(P, 0, P, n + 1, 1, 2, buf) == -1        # zigzag needs n even
    assert L.ring_attn_visible_pairs(P, n + 1, 1, 2, 0, 0) == -1
    assert L.ring_attn_plan(P, 0, P, n, 1, 3, buf) == -1            # unknown layout


def test_causal_critical_path_ratio():
    """Per-step barrier: sum over steps of the busiest device; contiguous/striped -> (2P-1)/P."""
    for P, n in ((8, 4096), (32, 32768)):
        crit = {}
        for striped in (False, True):
            crit[striped] = sum(max(ra.ring_attn_visible_pairs(P, n, i, (i - s) % P, causal=True, striped=striped)
                                    for i in range(P)) for s in range(P))
        ratio = crit[False] / crit[True]
        assert abs(ratio - (2 * P - 1) / P) < 1e-3


# ---------------------------------------------------------------- validation without a GPU

FAKE = 1 << 20  # never dereferenced: every call below fails validation first


def _step(**kw):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, o=FAKE * 4, m=FAKE * 5, l=FAKE * 6, n_dev=1, B=1, Hq=2, Hkv=1, Nq=4,
             Nk=4, D=16, dtype=0, scale=0.25, mask=0, q_off=None, q_stride=1, k_off=None, k_stride=1, flags=0)
    a.update(kw)
    arr = lambda x: None if x is None else (ctypes.c_int64 * len(x))(*x)
    return ra.lib().ring_attn_step(a["q"], a["k"], a["v"], a["o"], a["m"], a["l"], a["n_dev"], a["B"], a["Hq"],
                                   a["Hkv"], a["Nq"], a["Nk"], a["D"], a["dtype"], a["scale"], a["mask"],
                                   arr(a["q_off"]), a["q_stride"], arr(a["k_off"]), a["k_stride"], a["flags"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(o=None), -1), (dict(k=None), -1), (dict(n_dev=0), -1), (dict(n_dev=65), -1),
    (dict(B=0), -1), (dict(Hq=3, Hkv=2), -1), (dict(Nq=-1), -1), (dict(D=0), -1), (dict(D=129), -2),
    (dict(dtype=2), -1), (dict(scale=0.0), -1), (dict(scale=float("nan")), -1), (dict(mask=2), -1),
    (dict(mask=1), -1), (dict(mask=1, q_off=[0], k_off=[0], q_stride=0), -1), (dict(flags=4), -1),
    (dict(o=FAKE), -1),            # state aliases q
    (dict(m=FAKE * 4 + 16), -1),   # m inside o_acc
])
def test_step_rejects_bad_arguments(kw, code):
    assert _step(**kw) == code


def test_finalize_rejects_bad_arguments():
    f = ra.lib().ring_attn_finalize
    assert f(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, None, 0, 1, 1, 4, 16, 0, None) == -1
    assert f(None, FAKE * 2, FAKE * 3, FAKE * 4, None, 1, 1, 1, 4, 16, 0, None) == -1
    assert f(FAKE, FAKE * 2, FAKE * 3, FAKE, None, 1, 1, 1, 4, 16, 0, None) == -1   # o aliases o_acc
    assert f(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, None, 1, 1, 1, 4, 200, 0, None) == -2
    assert f(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, None, 1, 1, 1, 4, 16, 7, None) == -1
    assert f(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, None, 1, 1, 1, 0, 16, 0, None) == 0  # empty: nothing to do


def test_local_rejects_bad_arguments_and_small_workspace():
    L = ra.lib()
    ws = ra.ring_attn_local_workspace_bytes(4, 4, 1, 2, 1, 8, 16, 0)
    blk = 8 * 16 * 4
    rows = 4 * 2 * 8
    assert ws == 4 * ((4 * blk + 255) // 256 * 256) + (rows * 16 * 4 + 255) // 256 * 256 + 2 * ((rows * 4 + 255) // 256 * 256)

    def call(**kw):
        a = dict(q=FAKE, k=FAKE * 8, v=FAKE * 16, host=0, o=FAKE * 24, lse=None, P=4, dev0=0, n_local=4, B=1, Hq=2,
                 Hkv=1, n=8, D=16, dtype=0, scale=0.25, mask=0, layout=0, ws=FAKE * 32, ws_bytes=ws)
        a.update(kw)
        return L.ring_attn_local(a["q"], a["k"], a["v"], a["host"], a["o"], a["lse"], a["P"], a["dev0"], a["n_local"],
                                 a["B"], a["Hq"], a["Hkv"], a["n"], a["D"], a["dtype"], a["scale"], a["mask"],
                                 a["layout"], a["ws"], a["ws_bytes"], None, None, None)

    assert call(ws_bytes=ws - 1) == -4
    assert call(P=0) == -1 and call(P=65, n_local=1) == -1
    assert call(dev0=1) == -1           # dev0 + n_local > P
    assert call(layout=3) == -1 and call(mask=5) == -1
    assert call(o=FAKE) == -1           # output aliases q
    assert call(ws=FAKE * 8) == -1      # workspace aliases k
    assert call(D=256) == -2
    assert call(q=None) == -1
    assert call(n=0) == 0               # nothing to do
    assert ra.ring_attn_local_workspace_bytes(4, 5, 1, 2, 1, 8, 16, 0) == 0


def test_noalloc_scratch_size_and_rejections():
    """ring_attn_local_noalloc's fixed scratch is 64 MiB; a ring whose workspace would not fit is refused
    with RA_ERR_SCRATCH and invalid shapes with RA_ERR_INVALID_ARG, both before any HIP call."""
    L = ra.lib()
    assert ra.ring_attn_noalloc_scratch_bytes() == 64 << 20

    def call(**kw):
        a = dict(q=FAKE, k=FAKE * 8, v=FAKE * 16, host=0, o=FAKE * 24, lse=None, P=4, dev0=0, n_local=4, B=1, Hq=2,
                 Hkv=1, n=8, D=16, dtype=0, scale=0.25, mask=0, layout=0)
        a.update(kw)
        return L.ring_attn_local_noalloc(a["q"], a["k"], a["v"], a["host"], a["o"], a["lse"], a["P"], a["dev0"],
                                         a["n_local"], a["B"], a["Hq"], a["Hkv"], a["n"], a["D"], a["dtype"],
                                         a["scale"], a["mask"], a["layout"], None, None, None)

    # 8 devices of 8192 tokens, 8 heads, D = 128, bf16: 512 MiB of slots alone
    assert ra.ring_attn_local_workspace_bytes(8, 8, 1, 8, 8, 8192, 128, 1) > 64 << 20
    assert call(P=8, n_local=8, Hq=8, Hkv=8, n=8192, D=128, dtype=1) == -6
    assert call(P=0) == -1 and call(n_local=5) == -1 and call(Hq=3, Hkv=2) == -1
    assert call(D=256) == -2            # as ring_attn_local
    assert call(n=0) == 0               # nothing to do


def test_plan_rejects_bad_arguments():
    L = ra.lib()
    buf = (ctypes.c_int32 * 100)()
    assert L.ring_attn_plan(0, 0, 1, 8, 0, 0, buf) == -1
    assert L.ring_attn_plan(4, 2, 3, 8, 0, 0, buf) == -1
    assert L.ring_attn_plan(4, 0, 4, 8, 0, 0, None) == -1
    assert L.ring_attn_visible_pairs(4, 8, 2, 0, 0, 0) == -1
    assert L.ring_attn_visible_pairs(4, 8, 1, 0, 4, 0) == -1


# ---------------------------------------------------------------- backward entry points (validation)

def _bwd_step(**kw):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, do=FAKE * 4, lse2=FAKE * 5, delta=FAKE * 6, dq=FAKE * 7, dk=FAKE * 8,
             dv=FAKE * 9, n_dev=1, B=1, Hq=2, Hkv=1, Nq=4, Nk=4, D=128, dtype=1, scale=0.25, mask=0, q_off=None,
             q_stride=1, k_off=None, k_stride=1, flags=0)
    a.update(kw)
    arr = lambda x: None if x is None else (ctypes.c_int64 * len(x))(*x)
    return ra.lib().ring_attn_bwd_step(a["q"], a["k"], a["v"], a["do"], a["lse2"], a["delta"], a["dq"], a["dk"],
                                       a["dv"], a["n_dev"], a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["D"],
                                       a["dtype"], a["scale"], a["mask"], arr(a["q_off"]), a["q_stride"],
                                       arr(a["k_off"]), a["k_stride"], a["flags"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(dk=None), -1), (dict(n_dev=0), -1), (dict(Hq=3, Hkv=2), -1), (dict(flags=4), -1),
    (dict(scale=-1.0), -1), (dict(mask=1), -1), (dict(dtype=7), -1), (dict(D=129), -2),
    (dict(dq=FAKE), -1),            # dq aliases q
    (dict(dtype=0, dq=FAKE + 2048), -1),  # fp32 q spans 4096 bytes: dq starts inside it
    (dict(dv=FAKE * 8 + 64), -1),   # dv overlaps dk
    (dict(Nq=0, Nk=0), 0),          # nothing to do
])
def test_bwd_step_rejects_bad_arguments(kw, code):
    assert _bwd_step(**kw) == code


def test_bwd_prep_and_local_reject_bad_arguments():
    L = ra.lib()
    p = L.ring_attn_bwd_prep
    assert p(None, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5, 1, 1, 2, 4, 16, 0, None) == -1
    assert p(FAKE, FAKE * 2, FAKE * 3, FAKE, FAKE * 5, 1, 1, 2, 4, 16, 0, None) == -1      # delta aliases o
    assert p(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5, 1, 1, 2, 4, 200, 0, None) == -2
    assert p(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5, 1, 1, 2, 0, 16, 0, None) == 0   # empty
    ws = ra.ring_attn_bwd_local_workspace_bytes(4, 4, 1, 2, 1, 8, 128, 1)
    blk = 8 * 128 * 2
    rows = 4 * 2 * 8
    assert ws == 4 * ((4 * blk + 255) // 256 * 256) + 2 * ((rows * 4 + 255) // 256 * 256)

    def call(**kw):
        a = dict(q=FAKE, k=FAKE * 8, v=FAKE * 16, o=FAKE * 24, do=FAKE * 32, lse=FAKE * 40, dq=FAKE * 48,
                 dk=FAKE * 56, dv=FAKE * 64, P=4, dev0=0, n_local=4, B=1, Hq=2, Hkv=1, n=8, D=128, dtype=1,
                 scale=0.25, mask=1, layout=0, ws=FAKE * 72, ws_bytes=ws)
        a.update(kw)
        return L.ring_attn_bwd_local(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                                     a["P"], a["dev0"], a["n_local"], a["B"], a["Hq"], a["Hkv"], a["n"], a["D"],
                                     a["dtype"], a["scale"], a["mask"], a["layout"], a["ws"], a["ws_bytes"], None, None)
    assert call(ws_bytes=ws - 1) == -4
    assert call(layout=2, n=7) == -1    # zigzag needs n even
    assert call(D=129) == -2 and call(dtype=7) == -1
    assert call(layout=3) == -1 and call(dev0=4) == -1 and call(dk=None) == -1
    assert call(dq=FAKE) == -1          # dq aliases q
    assert call(ws=FAKE * 8) == -1      # workspace aliases k
    assert call(n=0) == 0


def test_ffn_workspace_and_rejects_bad_arguments():
    L = ra.lib()
    assert ra.ring_attn_ffn_workspace_bytes(1000, 128, 512, 256) == 256 * 512 * 2
    assert ra.ring_attn_ffn_workspace_bytes(100, 128, 512, 256) == 100 * 512 * 2   # one block of all tokens
    assert ra.ring_attn_ffn_workspace_bytes(0, 128, 512, 256) == 512 * 2
    for bad in ((10, 96, 512, 4), (10, 128, 500, 4), (10, 128, 512, 0), (-1, 128, 512, 4), (10, 0, 512, 4),
                (10, 128, 65600, 4), (1 << 40, 128, 64, 1 << 40), ((1 << 30) + 1, 64, 64, 1 << 31)):
        assert ra.ring_attn_ffn_workspace_bytes(*bad) == 0, bad
    n, dm, dff, blk = 300, 128, 256, 128
    ws = ra.ring_attn_ffn_workspace_bytes(n, dm, dff, blk)

    def call(**kw):
        a = dict(x=FAKE, w1=FAKE * 8, b1=FAKE * 16, w2=FAKE * 24, b2=FAKE * 32, y=FAKE * 40, n=n, dm=dm, dff=dff,
                 blk=blk, act=0, ws=FAKE * 48, ws_bytes=ws)
        a.update(kw)
        return L.ring_attn_ffn(a["x"], a["w1"], a["b1"], a["w2"], a["b2"], a["y"], a["n"], a["dm"], a["dff"], a["blk"],
                               a["act"], a["ws"], a["ws_bytes"], None)
    assert call(ws_bytes=ws - 1) == -4
    assert call(act=2) == -1 and call(act=-1) == -1
    assert call(dm=96) == -1 and call(dff=100) == -1 and call(blk=0) == -1 and call(n=-5) == -1
    assert call(w1=None) == -1 and call(b2=None) == -1 and call(ws=None) == -1
    assert call(y=FAKE + 2) == -1       # y overlaps x without being x
    assert call(y=FAKE * 8) == -1       # y aliases w1
    assert call(ws=FAKE * 24) == -1     # workspace aliases w2
    assert call(n=0) == 0               # nothing to do


def test_misaligned_pointers_are_rejected():
    L = ra.lib()
    off = (ctypes.c_int64 * 1)(0)
    # ring_attn_step: q 2 bytes off a 16-byte boundary; m 4-byte aligned is fine, 2-byte is not
    step = L.ring_attn_step
    base = dict(q=FAKE, k=FAKE * 8, v=FAKE * 16, o=FAKE * 24, m=FAKE * 40, l=FAKE * 48)

    def call_step(**kw):
        a = dict(base, **kw)
        return step(a["q"], a["k"], a["v"], a["o"], a["m"], a["l"], 1, 1, 2, 1, 8, 8, 128, 1, 0.1, 0, off, 1,
                    off, 1, 0, None)
    assert call_step(q=FAKE + 2) == -1 and call_step(o=FAKE * 24 + 8) == -1 and call_step(m=FAKE * 40 + 2) == -1
    # the feed-forward: biases need 8 bytes, tensors 16
    n, dm, dff, blk = 300, 128, 256, 128
    ws = ra.ring_attn_ffn_workspace_bytes(n, dm, dff, blk)

    def call_ffn(**kw):
        a = dict(x=FAKE, w1=FAKE * 8, b1=FAKE * 16, w2=FAKE * 24, b2=FAKE * 32, y=FAKE * 40, ws=FAKE * 48)
        a.update(kw)
        return L.ring_attn_ffn(a["x"], a["w1"], a["b1"], a["w2"], a["b2"], a["y"], n, dm, dff, blk, 0, a["ws"], ws,
                               None)
    assert call_ffn(w1=FAKE * 8 + 8) == -1 and call_ffn(b1=FAKE * 16 + 4) == -1 and call_ffn(ws=FAKE * 48 + 16 + 4) == -1
    assert L.ring_attn_bwd_prep(FAKE + 4, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5, 1, 1, 2, 4, 16, 0, None) == -1
