"""ctypes binding of libringattn.so: argument marshalling only."""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB_FILE = os.path.join(_PKG_DIR, "libringattn.so")

RA_F32, RA_BF16 = 0, 1
RA_MASK_NONE, RA_MASK_CAUSAL = 0, 1
RA_LAYOUT_CONTIGUOUS, RA_LAYOUT_STRIPED, RA_LAYOUT_ZIGZAG = 0, 1, 2
_LAYOUTS = {"contiguous": RA_LAYOUT_CONTIGUOUS, "striped": RA_LAYOUT_STRIPED, "zigzag": RA_LAYOUT_ZIGZAG}


def _layout_code(layout, striped):
    """Layout name ("contiguous", "striped", "zigzag"); the older striped flag stands for "striped"."""
    if layout is None:
        return RA_LAYOUT_STRIPED if striped else RA_LAYOUT_CONTIGUOUS
    if layout not in _LAYOUTS or (striped and layout != "striped"):
        raise ValueError(f"unknown or conflicting layout {layout!r}")
    return _LAYOUTS[layout]


RA_STEP_INIT = 1
RA_BWD_INIT_DQ, RA_BWD_INIT_DKV = 1, 2
RA_MAX_DEV, RA_MAX_D = 64, 128
RA_FFN_GELU, RA_FFN_RELU = 0, 1
RA_OK, RA_ERR_INVALID_ARG, RA_ERR_UNSUPPORTED, RA_ERR_HIP, RA_ERR_WORKSPACE, RA_ERR_INJECTED = 0, -1, -2, -3, -4, -5
RA_ERR_SCRATCH = -6
_ACTIVATIONS = {"gelu": RA_FFN_GELU, "relu": RA_FFN_RELU}

EXPORTED_SYMBOLS = (
    "ring_attn_step", "ring_attn_finalize", "ring_attn_local", "ring_attn_local_workspace_bytes",
    "ring_attn_plan", "ring_attn_visible_pairs", "ring_attn_strerror",
    "ring_attn_bwd_prep", "ring_attn_bwd_step", "ring_attn_bwd_local", "ring_attn_bwd_local_workspace_bytes",
    "ring_attn_ffn", "ring_attn_ffn_workspace_bytes", "ring_attn_local_noalloc", "ring_attn_noalloc_scratch_bytes",
)

_lib = None


class RingAttnError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed: {code} ({ring_attn_strerror(code)})")
        self.code = code


def lib_path() -> str:
    """The library this process loads: the in-tree build, or the build of the same sources that
    RING_ATTN_LIBRARY names (the host-sanitized build of the CPU tests is loaded that way)."""
    return os.environ.get("RING_ATTN_LIBRARY") or _LIB_FILE


def lib() -> ctypes.CDLL:
    """Load the shared library (built by ``blockwise_ring_attention_step_amd.build``); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m blockwise_ring_attention_step_amd.build`")
    L = ctypes.CDLL(path)
    i32, i64, f32, vp, sz = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
    p64 = ctypes.POINTER(ctypes.c_int64)
    L.ring_attn_step.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, f32, i32, p64, i64,
                                 p64, i64, i32, vp]
    L.ring_attn_step.restype = i32
    L.ring_attn_finalize.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
    L.ring_attn_finalize.restype = i32
    L.ring_attn_local.argtypes = [vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32, f32, i32, i32,
                                  vp, sz, vp, vp, vp]
    L.ring_attn_local.restype = i32
    L.ring_attn_local_noalloc.argtypes = [vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32, f32,
                                          i32, i32, vp, vp, vp]
    L.ring_attn_local_noalloc.restype = i32
    L.ring_attn_noalloc_scratch_bytes.argtypes = []
    L.ring_attn_noalloc_scratch_bytes.restype = sz
    L.ring_attn_local_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32]
    L.ring_attn_local_workspace_bytes.restype = sz
    L.ring_attn_plan.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.POINTER(ctypes.c_int32)]
    L.ring_attn_plan.restype = i32
    L.ring_attn_visible_pairs.argtypes = [i32, i32, i32, i32, i32, i32]
    L.ring_attn_visible_pairs.restype = i64
    L.ring_attn_bwd_prep.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
    L.ring_attn_bwd_prep.restype = i32
    L.ring_attn_bwd_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, f32,
                                     i32, p64, i64, p64, i64, i32, vp]
    L.ring_attn_bwd_step.restype = i32
    L.ring_attn_bwd_local.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                      f32, i32, i32, vp, sz, vp, vp]
    L.ring_attn_bwd_local.restype = i32
    L.ring_attn_bwd_local_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32]
    L.ring_attn_bwd_local_workspace_bytes.restype = sz
    L.ring_attn_ffn.argtypes = [vp, vp, vp, vp, vp, vp, i64, i32, i32, i64, i32, vp, sz, vp]
    L.ring_attn_ffn.restype = i32
    L.ring_attn_ffn_workspace_bytes.argtypes = [i64, i32, i32, i64]
    L.ring_attn_ffn_workspace_bytes.restype = sz
    L.ring_attn_strerror.argtypes = [i32]
    L.ring_attn_strerror.restype = ctypes.c_char_p
    _lib = L
    return L


def ring_attn_strerror(code: int) -> str:
    return lib().ring_attn_strerror(int(code)).decode()


def _check(fn, rc):
    if rc != 0:
        raise RingAttnError(fn, rc)


def _ptr(t):
    """Device pointer of a CUDA tensor (or None)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a GPU tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return RA_BF16
    if t.dtype == torch.float32:
        return RA_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _i64_array(xs):
    if xs is None:
        return None
    arr = (ctypes.c_int64 * len(xs))(*[int(x) for x in xs])
    return arr


def ring_attn_step(q, k, v, o_acc, m, l, *, scale, causal=False, q_off=None, q_stride=1, k_off=None, k_stride=1,
                   init=False, stream=None):
    """Fold the key/value blocks k, v into the state (o_acc, m, l) of the query blocks q.

    q [n_dev, B, Nq, Hq, D], k/v [n_dev, B, Nk, Hkv, D] (bf16 or fp32); o_acc [n_dev, B, Hq, Nq, D],
    m/l [n_dev, B, Hq, Nq] fp32.  q_off/k_off: per-device position offsets (sequences of ints).
    """
    n_dev, B, Nq, Hq, D = q.shape
    Nk, Hkv = k.shape[2], k.shape[3]
    rc = lib().ring_attn_step(_ptr(q), _ptr(k), _ptr(v), _ptr(o_acc), _ptr(m), _ptr(l), n_dev, B, Hq, Hkv, Nq, Nk, D,
                              _dtype_code(q), float(scale), RA_MASK_CAUSAL if causal else RA_MASK_NONE,
                              _i64_array(q_off), int(q_stride), _i64_array(k_off), int(k_stride),
                              RA_STEP_INIT if init else 0, _stream(stream))
    _check("ring_attn_step", rc)


def ring_attn_finalize(o_acc, m, l, o, lse=None, *, stream=None):
    """o = o_acc / l in token-major layout [n_dev, B, Nq, Hq, D]; lse = ln(sum exp(scores)) [n_dev, B, Hq, Nq]."""
    n_dev, B, Hq, Nq, D = o_acc.shape
    rc = lib().ring_attn_finalize(_ptr(o_acc), _ptr(m), _ptr(l), _ptr(o), _ptr(lse), n_dev, B, Hq, Nq, D,
                                  _dtype_code(o), _stream(stream))
    _check("ring_attn_finalize", rc)


def ring_attn_local_workspace_bytes(P, n_local, B, Hq, Hkv, n, D, dtype):
    return int(lib().ring_attn_local_workspace_bytes(P, n_local, B, Hq, Hkv, n, D, dtype))


def ring_attn_local(q_local, k_src, v_src, o, lse, workspace, *, P, dev0, scale, causal=False, striped=False,
                    layout=None, compute_stream=None, copy_stream=None, step_events=None):
    """Run the whole P-step ring for the local devices [dev0, dev0 + n_local).

    q_local [n_local, B, n, Hq, D]; k_src/v_src [P, B, n, Hkv, D] (device tensors, or pinned host
    tensors); o like q_local; lse [n_local, B, Hq, n] fp32 or None; workspace: uint8 device tensor.
    step_events: optional list of 2*P HipEvent objects recorded around each step kernel.
    layout: "contiguous" (default), "striped" (same as striped=True) or "zigzag".
    """
    n_local, B, n, Hq, D = q_local.shape
    Hkv = k_src.shape[3]
    host_src = not k_src.is_cuda
    if host_src and not (k_src.is_pinned() and v_src.is_pinned()):
        raise ValueError("host key/value sources must be pinned")
    kp = k_src.data_ptr() if host_src else _ptr(k_src)
    vp = v_src.data_ptr() if host_src else _ptr(v_src)
    ev = None
    if step_events is not None:
        if len(step_events) != 2 * P:
            raise ValueError("step_events needs 2*P events")
        ev = (ctypes.c_void_p * (2 * P))(*[e.handle for e in step_events])
    cs = _stream(compute_stream)
    xs = _stream(copy_stream) if copy_stream is not None else cs
    rc = lib().ring_attn_local(_ptr(q_local), kp, vp, 1 if host_src else 0, _ptr(o), _ptr(lse), P, dev0, n_local, B,
                               Hq, Hkv, n, D, _dtype_code(q_local), float(scale),
                               RA_MASK_CAUSAL if causal else RA_MASK_NONE,
                               _layout_code(layout, striped), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), cs, xs, ev)
    _check("ring_attn_local", rc)


def ring_attn_noalloc_scratch_bytes() -> int:
    return int(lib().ring_attn_noalloc_scratch_bytes())


def ring_attn_local_noalloc(q_local, k_src, v_src, o, lse, *, P, dev0, scale, causal=False, layout=None,
                            compute_stream=None, copy_stream=None, step_events=None):
    """ring_attn_local working in the library's fixed device scratch instead of a workspace tensor
    (allocates no device memory).  Same arguments as ring_attn_local without ``workspace``."""
    n_local, B, n, Hq, D = q_local.shape
    Hkv = k_src.shape[3]
    host_src = not k_src.is_cuda
    if host_src and not (k_src.is_pinned() and v_src.is_pinned()):
        raise ValueError("host key/value sources must be pinned")
    kp = k_src.data_ptr() if host_src else _ptr(k_src)
    vp = v_src.data_ptr() if host_src else _ptr(v_src)
    ev = None
    if step_events is not None:
        if len(step_events) != 2 * P:
            raise ValueError("step_events needs 2*P events")
        ev = (ctypes.c_void_p * (2 * P))(*[e.handle for e in step_events])
    cs = _stream(compute_stream)
    xs = _stream(copy_stream) if copy_stream is not None else cs
    rc = lib().ring_attn_local_noalloc(_ptr(q_local), kp, vp, 1 if host_src else 0, _ptr(o), _ptr(lse), P, dev0,
                                       n_local, B, Hq, Hkv, n, D, _dtype_code(q_local), float(scale),
                                       RA_MASK_CAUSAL if causal else RA_MASK_NONE, _layout_code(layout, False), cs, xs,
                                       ev)
    _check("ring_attn_local_noalloc", rc)


def ring_attn_plan(P, dev0, n_local, n, *, causal=False, striped=False, layout=None) -> np.ndarray:
    """Schedule table [P * n_local, 5] of (step, device, block, slot, class)."""
    out = np.zeros((P * n_local, 5), dtype=np.int32)
    rc = lib().ring_attn_plan(P, dev0, n_local, n, RA_MASK_CAUSAL if causal else RA_MASK_NONE,
                              _layout_code(layout, striped),
                              out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    _check("ring_attn_plan", rc)
    return out


def ring_attn_visible_pairs(P, n, i, j, *, causal=False, striped=False, layout=None) -> int:
    r = lib().ring_attn_visible_pairs(P, n, RA_MASK_CAUSAL if causal else RA_MASK_NONE,
                                      _layout_code(layout, striped), i, j)
    if r < 0:
        raise RingAttnError("ring_attn_visible_pairs", -1)
    return int(r)


def ring_attn_bwd_prep(o, dout, lse, delta, lse2, *, stream=None):
    """delta = sum_d dout * o and lse2 = log2(e) * lse; o, dout [n_dev, B, Nq, Hq, D], the rest [n_dev, B, Hq, Nq]."""
    n_dev, B, Nq, Hq, D = o.shape
    rc = lib().ring_attn_bwd_prep(_ptr(o), _ptr(dout), _ptr(lse), _ptr(delta), _ptr(lse2), n_dev, B, Hq, Nq, D,
                                  _dtype_code(o), _stream(stream))
    _check("ring_attn_bwd_prep", rc)


def ring_attn_bwd_step(q, k, v, dout, lse2, delta, dq, dk, dv, *, scale, causal=False, q_off=None, q_stride=1,
                       k_off=None, k_stride=1, init_dq=False, init_dkv=False, stream=None):
    """Add the gradient contributions of the pairs (q[t], k[t], v[t]) to dq[t], dk[t], dv[t] (fp32)."""
    n_dev, B, Nq, Hq, D = q.shape
    Nk, Hkv = k.shape[2], k.shape[3]
    flags = (RA_BWD_INIT_DQ if init_dq else 0) | (RA_BWD_INIT_DKV if init_dkv else 0)
    rc = lib().ring_attn_bwd_step(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse2), _ptr(delta), _ptr(dq), _ptr(dk),
                                  _ptr(dv), n_dev, B, Hq, Hkv, Nq, Nk, D, _dtype_code(q), float(scale),
                                  RA_MASK_CAUSAL if causal else RA_MASK_NONE, _i64_array(q_off), int(q_stride),
                                  _i64_array(k_off), int(k_stride), flags, _stream(stream))
    _check("ring_attn_bwd_step", rc)


def ring_attn_bwd_local_workspace_bytes(P, n_local, B, Hq, Hkv, n, D, dtype):
    return int(lib().ring_attn_bwd_local_workspace_bytes(P, n_local, B, Hq, Hkv, n, D, dtype))


def ring_attn_bwd_local(q_local, k_src, v_src, o_local, dout_local, lse_local, dq_local, dk, dv, workspace, *, P,
                        dev0, scale, causal=False, layout=None, striped=False, compute_stream=None, copy_stream=None):
    """Backward ring for the local devices [dev0, dev0 + n_local): dq_local [n_local, B, n, Hq, D] and
    dk, dv [P, B, n, Hkv, D] (fp32), from the forward's inputs, output, log-sum-exp and the output gradient."""
    n_local, B, n, Hq, D = q_local.shape
    Hkv = k_src.shape[3]
    cs = _stream(compute_stream)
    xs = _stream(copy_stream) if copy_stream is not None else cs
    rc = lib().ring_attn_bwd_local(_ptr(q_local), _ptr(k_src), _ptr(v_src), _ptr(o_local), _ptr(dout_local),
                                   _ptr(lse_local), _ptr(dq_local), _ptr(dk), _ptr(dv), P, dev0, n_local, B, Hq, Hkv,
                                   n, D, _dtype_code(q_local), float(scale), RA_MASK_CAUSAL if causal else RA_MASK_NONE,
                                   _layout_code(layout, striped), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), cs, xs)
    _check("ring_attn_bwd_local", rc)


def ring_attn_ffn_workspace_bytes(n_tokens, d_model, d_ff, block_tokens):
    return int(lib().ring_attn_ffn_workspace_bytes(int(n_tokens), int(d_model), int(d_ff), int(block_tokens)))


def ring_attn_ffn(x, w1, b1, w2, b2, y, workspace, *, block_tokens, activation="gelu", stream=None):
    """y = act(x w1^T + b1) w2^T + b2 over the tokens (rows) of x, one block of block_tokens at a time.

    x, y [..., d_model] bf16 (y may be x); w1 [d_ff, d_model], b1 [d_ff], w2 [d_model, d_ff], b2 [d_model] bf16;
    workspace: a device buffer of at least ring_attn_ffn_workspace_bytes(...) bytes."""
    d_ff, d_model = w1.shape
    if x.shape[-1] != d_model or y.shape != x.shape or tuple(w2.shape) != (d_model, d_ff):
        raise ValueError("shapes: x, y [..., d_model], w1 [d_ff, d_model], w2 [d_model, d_ff]")
    if tuple(b1.shape) != (d_ff,) or tuple(b2.shape) != (d_model,):
        raise ValueError("shapes: b1 [d_ff], b2 [d_model]")
    for t in (x, w1, b1, w2, b2, y):
        if _dtype_code(t) != RA_BF16:
            raise ValueError("ring_attn_ffn takes bf16 tensors")
    if activation not in _ACTIVATIONS:
        raise ValueError(f"unknown activation {activation!r}")
    n_tokens = x.numel() // d_model
    rc = lib().ring_attn_ffn(_ptr(x), _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2), _ptr(y), n_tokens, d_model, d_ff,
                             int(block_tokens), _ACTIVATIONS[activation], _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream(stream))
    _check("ring_attn_ffn", rc)


_HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000
_hiprt = None


def _hip_runtime():
    """The HIP runtime already loaded in this process (torch's copy, found by its soname)."""
    global _hiprt
    if _hiprt is None:
        import torch  # noqa: F401  (loads the runtime)
        h = ctypes.CDLL("libamdhip64.so.7")
        h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _hiprt = h
    return _hiprt


class HipEvent:
    """A timing hipEvent_t whose raw handle the library can record between its launches.

    Created without the system-scope fence, so recording it costs no cache flush on the stream it
    times (it orders nothing for the host; the caller synchronizes before reading it)."""

    def __init__(self):
        h = _hip_runtime()
        ev = ctypes.c_void_p()
        rc = h.hipEventCreateWithFlags(ctypes.byref(ev), _HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if rc != 0 or not ev.value:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.handle = ev.value
        self._h = h

    def record(self, stream=None):
        import torch
        st = torch.cuda.current_stream() if stream is None else stream
        rc = self._h.hipEventRecord(self.handle, st.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, end: "HipEvent") -> float:
        ms = ctypes.c_float()
        rc = self._h.hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def __del__(self):
        if getattr(self, "handle", None):
            self._h.hipEventDestroy(self.handle)
            self.handle = None
