"""GPU parity of the blockwise feed-forward (``ring_attn_ffn``) against the float64 oracle.

Both sides take the same bf16 inputs (seeded, ``synth_inputs.ffn_inputs``).  Tolerance (derived; the
pages fix none for the feed-forward): products of bf16 values are exact in fp32 and the sums over
d_model or d_ff keep ~1e-6 relative error; the hidden activations are rounded to bf16 (unit roundoff
2^-9) before the second product, where these independent roundings add up to ~2^-9 of the root
sum of squares of the products, and the output is rounded to bf16 (2^-9 of its magnitude).  The
relative Frobenius error is then ~2e-3, bounded by 5e-3; the largest error by 1e-2 of the largest
output.  A missing bias (0.1 against O(1) outputs), a wrong activation or a dropped k range breaks
both by an order of magnitude.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from ring_harness import to_device

pytestmark = pytest.mark.gpu

TOL_MAX = 1e-2
TOL_FRO = 5e-3


def _upload(seed, tokens, dm, dff):
    x, w1, b1, w2, b2 = si.ffn_inputs(seed, tokens, dm, dff)
    dev = [to_device(a, "bf16") for a in (x, w1, b1, w2, b2)]
    f64 = [si.bf16_to_f32(a).astype(np.float64) for a in (x, w1, b1, w2, b2)]
    return dev, f64


def _run(ra, dev, block_tokens, activation, y=None):
    x, w1, b1, w2, b2 = dev
    y = torch.full_like(x, float("nan")) if y is None else y
    ws = torch.empty(ra.ring_attn_ffn_workspace_bytes(x.shape[0], x.shape[1], w1.shape[0], block_tokens),
                     dtype=torch.uint8, device="cuda")
    ra.ring_attn_ffn(x, w1, b1, w2, b2, y, ws, block_tokens=block_tokens, activation=activation)
    torch.cuda.synchronize()
    return y


def _ref(f64, activation, rows=None):
    x, w1, b1, w2, b2 = f64
    xs = x if rows is None else x[rows]
    return oracle.ffn_reference(xs, w1.T, b1, w2.T, b2, activation=activation)


def _check(got, ref, tag):
    got = got.float().cpu().numpy().astype(np.float64)
    scale = np.abs(ref).max()
    emax = np.abs(got - ref).max() / scale
    efro = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    print(f"[ffn] {tag}: max {emax:.2e} fro {efro:.2e}", flush=True)
    assert np.isfinite(emax) and emax <= TOL_MAX and efro <= TOL_FRO


@pytest.mark.parametrize("activation", ["gelu", "relu"])
@pytest.mark.parametrize("tokens,dm,dff,block", [
    (300, 128, 256, 128),    # three blocks, the last one ragged (44 tokens)
    (600, 192, 320, 512),    # ragged n tiles in both projections (192 and 320 features), blocks 512 + 88
    (1, 64, 64, 7),          # a single token, the smallest sizes
    (777, 256, 512, 777),    # one block of all tokens, 4 m tiles (the last with 9 tokens)
])
def test_ffn_matches_oracle(gpu_lib, tokens, dm, dff, block, activation):
    dev, f64 = _upload(7000 + tokens + dm, tokens, dm, dff)
    y = _run(gpu_lib, dev, block, activation)
    _check(y, _ref(f64, activation), f"tokens={tokens} dm={dm} dff={dff} block={block} {activation}")


def test_ffn_block_size_does_not_change_the_result(gpu_lib):
    """Position-wise: each output row is the same sum in the same order whatever block holds it."""
    dev, f64 = _upload(7100, 1000, 256, 1024)
    ys = [_run(gpu_lib, dev, b, "gelu") for b in (1000, 256, 300, 64)]
    for y in ys[1:]:
        assert torch.equal(y, ys[0])
    _check(ys[0], _ref(f64, "gelu"), "blocks 1000/256/300/64")


def test_ffn_in_place(gpu_lib):
    dev, f64 = _upload(7200, 520, 128, 512)
    x_copy = dev[0].clone()
    y = _run(gpu_lib, dev, 200, "gelu")
    dev[0] = x_copy
    _run(gpu_lib, dev, 200, "gelu", y=dev[0])  # y is x
    assert torch.equal(dev[0], y)


@pytest.mark.parametrize("name", ["ffn_16k", "ffn_32h_4k"])
def test_ffn_fullsize_sampled_rows(gpu_lib, name):
    """The benchmark's workloads at full size and block size; the oracle on seeded sampled rows (1024, or
    256 where d_ff = 16384, to keep the float64 products to seconds)."""
    w = si.FFN_WORKLOADS[name]
    dev, f64 = _upload(w.seed, w.tokens, w.d_model, w.d_ff)
    y = _run(gpu_lib, dev, w.block_tokens, w.activation)
    nrows = 1024 if w.d_ff <= 4096 else 256
    rows = np.sort(np.random.default_rng(w.seed + 9).choice(w.tokens, size=nrows, replace=False))
    _check(y[torch.from_numpy(rows).cuda()], _ref(f64, w.activation, rows), f"{name} ({nrows} sampled rows)")


@pytest.mark.parametrize("activation", ["gelu", "relu"])
def test_ffn_activation_elementwise(gpu_lib, activation):
    """Identity weights and zero biases make y = bf16(act(x)) exactly (each sum has one nonzero term of
    weight 1): the activation itself, element by element, against the oracle's rounded to bf16.  The
    kernel evaluates gelu in fp32 (erfc to a relative 1.2e-7), so a value within that of a bf16
    rounding boundary may land one bf16 step away; everything else is bit-equal down to the
    subnormal range."""
    d = 128
    n = 4096
    vals = np.concatenate([np.linspace(-10, 10, n * d // 2, dtype=np.float32),
                           si.normal_f32(7300, (n * d // 2,), 3.0)]).reshape(n, d)
    vals[0, :8] = [0.0, -0.0, 1e-30, -1e-30, 5.0, -5.0, 0.5, -0.5]
    x = si.bf16_bits(vals)
    eye = si.bf16_bits(np.eye(d, dtype=np.float32))
    zero = si.bf16_bits(np.zeros(d, dtype=np.float32))
    dev = [to_device(a, "bf16") for a in (x, eye, zero, eye, zero)]
    y = _run(gpu_lib, dev, n, activation)
    got = y.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.int32)
    act = oracle.gelu if activation == "gelu" else oracle.relu
    want = si.bf16_bits(act(si.bf16_to_f32(x).astype(np.float64)).astype(np.float32)).astype(np.int32)
    # the same sign, and at most one step apart in the bit pattern (bf16 values of one sign are ordered)
    same_sign = (got >> 15) == (want >> 15)
    diff = np.abs(got - want)
    # zeros and subnormals (exponent field 0: |gelu| < 2^-126, far tail z < -13) count as one class:
    # whether fp32 arithmetic keeps or flushes such values is not part of the definition
    tiny = ((got & 0x7F80) == 0) & ((want & 0x7F80) == 0)
    ok = (same_sign & (diff <= 1)) | tiny
    print(f"[ffn] {activation} elementwise: {np.mean(diff == 0) * 100:.3f}% bit-equal, max step {diff.max()}", flush=True)
    assert ok.all()
    assert np.mean(diff == 0) >= 0.99


def test_ffn_tile_shapes_give_the_same_bits(gpu_lib):
    """Blocks of all 16384 tokens run both projections on 256 x 256 tiles, blocks of 2048 on 128 x 128
    tiles (too few large tiles to fill the CUs): every output is the same k-ordered sum either way."""
    w = si.FFN_WORKLOADS["ffn_16k"]
    dev, _ = _upload(w.seed, w.tokens, w.d_model, w.d_ff)
    big = _run(gpu_lib, dev, 16384, "gelu")
    small = _run(gpu_lib, dev, 2048, "gelu")
    assert torch.equal(big, small)
