"""Nystrom approximate self-attention for MI355X (gfx950).

A thin ctypes binding over libnystrom.so (declared in include/nystrom.h):
it only marshals arguments.  Every step of the computation runs in the HIP
kernels of the library; there is no Python or CPU fallback, and importing
this package fails if the library has not been built
(``python -m efficient_transformer_attention_segment_amd.build``).

torch is used for device memory and streams only: tensors are passed by
``data_ptr()`` and work is enqueued on ``torch.cuda.current_stream()``
unless a stream is given.  The library is loaded on first use.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "NystromError", "nystrom_attention", "nystrom_attention_bf16", "attention", "attention_with_probs", "self_attention", "attention_backward",
    "workspace_bytes", "last_error", "release", "debug_stages", "library_path",
    "profile_enable", "profile_collect", "check_status", "debug_set_rendezvous_spins", "debug_set_workspace_cap",
    "NYS_OK", "NYS_ERR_INVALID", "NYS_ERR_UNSUPPORTED", "NYS_ERR_HIP",
]

NYS_OK, NYS_ERR_INVALID, NYS_ERR_UNSUPPORTED, NYS_ERR_HIP = 0, -1, -2, -3
HEAD_DIM, CONV_TAPS = 64, 65

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libnystrom.so")

_P = ctypes.c_void_p
_I = ctypes.c_int
_lib = None


def _load():
    """Load libnystrom.so once; raise if it has not been built (there is
    no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise ImportError(
            f"{library_path} is missing: build it with "
            "`python -m efficient_transformer_attention_segment_amd.build` (needs hipcc)")
    lib = ctypes.CDLL(library_path)
    lib.nystrom_attention.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P]
    lib.nystrom_attention.restype = _I
    lib.nystrom_attention_bf16.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P]
    lib.nystrom_attention_bf16.restype = _I
    lib.nystrom_attention_conv.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P]
    lib.nystrom_attention_conv.restype = _I
    lib.nystrom_attention_bf16_conv.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P]
    lib.nystrom_attention_bf16_conv.restype = _I
    _L = ctypes.c_longlong
    lib.nystrom_attention_ex.argtypes = [_I, _P, _P, _P, _L, _L, _L, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                                         _P, _L, _L, _L, _P]
    lib.nystrom_attention_ex.restype = _I
    lib.nystrom_attention_noalloc.argtypes = [_I, _P, _P, _P, _L, _L, _L, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                                              _P, _L, _L, _L, _P]
    lib.nystrom_attention_noalloc.restype = _I
    lib.nystrom_attention_probs.argtypes = [_I, _P, _P, _P, _L, _L, _L, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                                            _P, _L, _L, _L, _P, _P]
    lib.nystrom_attention_probs.restype = _I
    lib.nystrom_self_attention.argtypes = [_I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P]
    lib.nystrom_self_attention.restype = _I
    lib.nystrom_attention_backward.argtypes = [_I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P,
                                               _P, _P, _P]
    lib.nystrom_attention_backward.restype = _I
    lib.nystrom_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
    lib.nystrom_workspace_bytes.restype = ctypes.c_size_t
    lib.nystrom_last_error.argtypes = []
    lib.nystrom_last_error.restype = ctypes.c_char_p
    lib.nystrom_release.argtypes = []
    lib.nystrom_release.restype = None
    lib.nystrom_debug_stages.argtypes = [_I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P,
                                         _P, _P, _P, _P, _P, _P, _P, _P]
    lib.nystrom_debug_stages.restype = _I
    lib.nystrom_check_status.argtypes = [_P]
    lib.nystrom_check_status.restype = _I
    lib.nystrom_debug_set_rendezvous_spins.argtypes = [ctypes.c_uint]
    lib.nystrom_debug_set_rendezvous_spins.restype = None
    lib.nystrom_debug_set_workspace_cap.argtypes = [ctypes.c_size_t]
    lib.nystrom_debug_set_workspace_cap.restype = None
    lib.nystrom_profile_enable.argtypes = [_I]
    lib.nystrom_profile_enable.restype = None
    lib.nystrom_profile_collect.argtypes = [ctypes.POINTER(ctypes.c_char_p),
                                            ctypes.POINTER(ctypes.c_double),
                                            ctypes.POINTER(ctypes.c_int), _I]
    lib.nystrom_profile_collect.restype = _I
    _lib = lib
    return lib


class NystromError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"nystrom error {code}: {message}")
        self.code = code


def last_error() -> str:
    return _load().nystrom_last_error().decode()


def _check(rc: int) -> None:
    if rc != NYS_OK:
        raise NystromError(rc, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(getattr(stream, "cuda_stream", stream) or 0)


def _check_io(q, k, v, out, dtype=None):
    """q, k, v (and out when given): 4-D CUDA tensors on one device with one
    dtype, float32 or bfloat16 (``dtype`` when the entry point fixes it).
    Nothing reaches the library before these checks pass: it takes raw
    device pointers and cannot tell a host pointer or a wrong element type
    from a valid one."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t is None:
            continue
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a CUDA (HIP) tensor")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, n, d]")
        if t.dtype != q.dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, q has {q.dtype}")
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"q, k, v must be float32 or bfloat16, not {q.dtype}")
    if dtype is not None and q.dtype != dtype:
        raise ValueError(f"this entry point takes {dtype} tensors, got {q.dtype}")


def _check_aux(ref, B, H, n, key_mask, conv_w):
    """key_mask: uint8 or bool [B, n], dense, on ref's device; conv_w: float32
    [H, K], dense, on ref's device (a Conv2d weight [H, 1, K, 1] must be
    reshaped to [H, K] first)."""
    import torch
    if key_mask is not None:
        if not isinstance(key_mask, torch.Tensor) or key_mask.device != ref.device:
            raise ValueError(f"key_mask must be a tensor on {ref.device}")
        if key_mask.dtype not in (torch.uint8, torch.bool):
            raise ValueError(f"key_mask must be uint8 or bool (1 keeps a key), not {key_mask.dtype}")
        if tuple(key_mask.shape) != (B, n) or not key_mask.is_contiguous():
            raise ValueError(f"key_mask must be a dense [B, n] = [{B}, {n}] tensor, got {tuple(key_mask.shape)}")
    if conv_w is not None:
        if not isinstance(conv_w, torch.Tensor) or conv_w.device != ref.device:
            raise ValueError(f"conv_w must be a tensor on {ref.device}")
        if conv_w.dtype != torch.float32:
            raise ValueError(f"conv_w must be float32, not {conv_w.dtype}")
        if conv_w.dim() != 2 or conv_w.shape[0] != H or not conv_w.is_contiguous():
            raise ValueError(f"conv_w must be a dense [H, K] = [{H}, K] tensor, got {tuple(conv_w.shape)} "
                             "(reshape a Conv2d weight [H, 1, K, 1] to [H, K])")


def _raw_call(fn, q, k, v, key_mask, conv_w, m, n_iter, init_option, out, stream):
    B, H, n, d = q.shape
    return fn(_ptr(q), _ptr(k), _ptr(v), _ptr(key_mask), _ptr(conv_w), B, H, n, d, m, n_iter,
              init_option, _ptr(out), _stream(stream))


def _raw_call_conv(fn, q, k, v, key_mask, conv_w, m, n_iter, init_option, out, stream):
    """The same call with conv_w's kernel size (its last dimension) passed."""
    B, H, n, d = q.shape
    return fn(_ptr(q), _ptr(k), _ptr(v), _ptr(key_mask), _ptr(conv_w), int(conv_w.shape[-1]), B, H, n,
              d, m, n_iter, init_option, _ptr(out), _stream(stream))


def _dense(t) -> bool:
    B, H, n, d = t.shape
    return t.stride() == (H * n * d, n * d, d, 1)


def _call(name, q, k, v, key_mask, conv_w, m, n_iter, init_option, out, stream):
    import torch
    _check_io(q, k, v, out, torch.bfloat16 if name.endswith("bf16") else torch.float32)
    if not (k.shape == v.shape == out.shape == q.shape):
        raise ValueError("q, k, v and out must have one shape [B, H, n, d]")
    _check_aux(q, q.shape[0], q.shape[1], q.shape[2], key_mask, conv_w)
    lib = _load()
    if not all(_dense(t) for t in (q, k, v, out)):
        # strided views of [B, H, n, 64] (channels contiguous): one set of
        # strides for q, k, v and one for out
        if not (q.stride() == k.stride() == v.stride()) or q.stride(-1) != 1 or out.stride(-1) != 1:
            raise ValueError("q, k and v must share strides, with contiguous channels (as must out)")
        B, H, n, d = q.shape
        dtype = 1 if name.endswith("bf16") else 0
        ksize = CONV_TAPS if conv_w is None else int(conv_w.shape[-1])
        return lib.nystrom_attention_ex(dtype, _ptr(q), _ptr(k), _ptr(v), *q.stride()[:3], _ptr(key_mask),
                                        _ptr(conv_w), ksize, B, H, n, d, m, n_iter, init_option, _ptr(out),
                                        *out.stride()[:3], _stream(stream))
    if conv_w is None or conv_w.shape[-1] == CONV_TAPS:
        return _raw_call(getattr(lib, name), q, k, v, key_mask, conv_w, m, n_iter, init_option, out, stream)
    return _raw_call_conv(getattr(lib, name + "_conv"), q, k, v, key_mask, conv_w, m, n_iter, init_option,
                          out, stream)


def nystrom_attention(q, k, v, key_mask=None, conv_w=None, m=64, n_iter=6, init_option=0,
                      out=None, stream=None):
    """float32 [B,H,n,64] CUDA tensors -> out (allocated when None).
    q, k, v (sharing strides) and out may be strided views with contiguous
    channels, e.g. slices of a fused [B, n, 3, H, 64] projection and a
    [B, n, H, 64] output; they then go through nystrom_attention_ex.
    key_mask: uint8 [B,n] (1 keeps a key) or None; conv_w: float32 [H,K]
    (K odd, up to 65; the pages' default is 65) or None.  Enqueued on
    ``stream`` (default: torch's current stream)."""
    import torch
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    _check(_call("nystrom_attention", q, k, v, key_mask, conv_w, m, n_iter, init_option, out, stream))
    return out


def nystrom_attention_bf16(q, k, v, key_mask=None, conv_w=None, m=64, n_iter=6, init_option=0,
                           out=None, stream=None):
    """bfloat16 [B,H,n,64] CUDA tensors (float32 accumulation) -> out."""
    import torch
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    _check(_call("nystrom_attention_bf16", q, k, v, key_mask, conv_w, m, n_iter, init_option, out, stream))
    return out


def attention(q, k, v, key_mask=None, conv_w=None, m=64, n_iter=6, init_option=0, out=None,
              stream=None):
    """Pick the entry point from q's dtype (float32 or bfloat16)."""
    import torch
    fn = nystrom_attention_bf16 if q.dtype == torch.bfloat16 else nystrom_attention
    return fn(q, k, v, key_mask, conv_w, m, n_iter, init_option, out, stream)


def attention_with_probs(q, k, v, key_mask=None, conv_w=None, m=64, n_iter=6, init_option=0, out=None,
                         probs=None, stream=None):
    """The attention output and the attention weights (output_attentions):
    probs [B,H,n,m] = F A^+ when m < n, the exact softmax [B,H,n,n] when
    m == n; both in q's dtype (float32 or bfloat16).  q, k, v (sharing
    strides) and out may be strided views with contiguous channels; probs
    is dense.  Returns (out, probs)."""
    import torch
    _check_io(q, k, v, out)
    if not (k.shape == v.shape == q.shape):
        raise ValueError("q, k and v must have one shape [B, H, n, d]")
    _check_aux(q, q.shape[0], q.shape[1], q.shape[2], key_mask, conv_w)
    if probs is not None and (not probs.is_cuda or probs.device != q.device or probs.dtype != q.dtype):
        raise ValueError("probs must be a CUDA tensor on q's device with q's dtype")
    if q.stride() != k.stride() or k.stride() != v.stride() or q.stride(-1) != 1:
        raise ValueError("q, k and v must share strides, with contiguous channels")
    B, H, n, d = q.shape
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if out.shape != q.shape or out.stride(-1) != 1:
        raise ValueError("out must be [B, H, n, d] with contiguous channels")
    if probs is None:
        probs = torch.empty((B, H, n, m), dtype=q.dtype, device=q.device)
    if probs.shape != (B, H, n, m) or not probs.is_contiguous():
        raise ValueError("probs must be a dense [B, H, n, m] tensor")
    dtype = 1 if q.dtype == torch.bfloat16 else 0
    ksize = CONV_TAPS if conv_w is None else int(conv_w.shape[-1])
    lib = _load()
    _check(lib.nystrom_attention_probs(dtype, _ptr(q), _ptr(k), _ptr(v), *q.stride()[:3], _ptr(key_mask),
                                       _ptr(conv_w), ksize, B, H, n, d, m, n_iter, init_option, _ptr(out),
                                       *out.stride()[:3], _ptr(probs), _stream(stream)))
    return out, probs


def self_attention(x, w_qkv, b_qkv, H, key_mask=None, conv_w=None, m=64, n_iter=6, init_option=0, qkv=None,
                   out=None, stream=None):
    """The self-attention module: x [B, n, hidden] (float32 or bfloat16),
    w_qkv [3 H d, hidden] (query, key, value weights stacked), b_qkv [3 H d]
    or None.  Returns (out [B, n, H d], qkv [B, n, 3, H, d])."""
    import torch
    if not isinstance(x, torch.Tensor) or not x.is_cuda or x.dim() != 3:
        raise ValueError("x must be a CUDA tensor [B, n, hidden]")
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"x must be float32 or bfloat16, not {x.dtype}")
    for name, t in (("w_qkv", w_qkv), ("b_qkv", b_qkv), ("qkv", qkv), ("out", out)):
        if t is not None and (not t.is_cuda or t.device != x.device or t.dtype != x.dtype):
            raise ValueError(f"{name} must be a CUDA tensor on x's device with x's dtype")
    B, n, hidden = x.shape
    if w_qkv.dim() != 2 or w_qkv.shape[1] != hidden or w_qkv.shape[0] % (3 * H) != 0:
        raise ValueError("w_qkv must be [3 H d, hidden]")
    d = w_qkv.shape[0] // (3 * H)
    if b_qkv is not None and tuple(b_qkv.shape) != (3 * H * d,):
        raise ValueError("b_qkv must be [3 H d]")
    _check_aux(x, B, H, n, key_mask, conv_w)
    for t in (x, w_qkv, b_qkv):
        if t is not None and (not t.is_contiguous() or t.dtype != x.dtype):
            raise ValueError("x, w_qkv and b_qkv must be dense and share x's dtype")
    if qkv is None:
        qkv = torch.empty((B, n, 3, H, d), dtype=x.dtype, device=x.device)
    if out is None:
        out = torch.empty((B, n, H * d), dtype=x.dtype, device=x.device)
    if tuple(qkv.shape) != (B, n, 3, H, d) or not qkv.is_contiguous():
        raise ValueError("qkv must be a dense [B, n, 3, H, d] tensor")
    if tuple(out.shape) != (B, n, H * d) or not out.is_contiguous():
        raise ValueError("out must be a dense [B, n, H d] tensor")
    dtype = 1 if x.dtype == torch.bfloat16 else 0
    ksize = CONV_TAPS if conv_w is None else int(conv_w.shape[-1])
    _check(_load().nystrom_self_attention(dtype, _ptr(x), _ptr(w_qkv), _ptr(b_qkv), _ptr(key_mask), _ptr(conv_w),
                                          ksize, B, n, hidden, H, d, m, n_iter, init_option, _ptr(qkv), _ptr(out),
                                          _stream(stream)))
    return out, qkv


def attention_backward(q, k, v, dout, key_mask=None, conv_w=None, m=64, n_iter=6, init_option=0, dq=None,
                       dk=None, dv=None, dconv_w=None, stream=None):
    """Gradients of sum(out * dout) for the call attention(q, k, v, key_mask,
    conv_w, m, n_iter, init_option): returns (dq, dk, dv, dconv_w), the
    first three in q's dtype, dconv_w float32 [H, K] (None without conv_w).
    Dense [B, H, n, d] tensors, d in {32, 64, 128}."""
    import torch
    _check_io(q, k, v, dout)
    for t in (q, k, v, dout):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError("q, k, v and dout must be dense tensors of one shape and dtype")
    B, H, n, d = q.shape
    _check_aux(q, B, H, n, key_mask, conv_w)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if (not t.is_cuda or t.device != q.device or t.shape != q.shape or t.dtype != q.dtype
                or not t.is_contiguous()):
            raise ValueError(f"{name} must be a dense CUDA tensor of q's shape, dtype and device")
    if conv_w is not None and dconv_w is None:
        dconv_w = torch.empty(conv_w.shape, dtype=torch.float32, device=q.device)
    if dconv_w is not None and (conv_w is None or not dconv_w.is_cuda or dconv_w.device != q.device
                                or dconv_w.dtype != torch.float32 or dconv_w.shape != conv_w.shape
                                or not dconv_w.is_contiguous()):
        raise ValueError("dconv_w must be a dense float32 CUDA tensor of conv_w's shape (and needs conv_w)")
    dtype = 1 if q.dtype == torch.bfloat16 else 0
    ksize = CONV_TAPS if conv_w is None else int(conv_w.shape[-1])
    _check(_load().nystrom_attention_backward(dtype, _ptr(q), _ptr(k), _ptr(v), _ptr(key_mask), _ptr(conv_w), ksize,
                                              B, H, n, d, m, n_iter, init_option, _ptr(dout), _ptr(dq), _ptr(dk),
                                              _ptr(dv), _ptr(dconv_w), _stream(stream)))
    return dq, dk, dv, dconv_w


def check_status(stream=None) -> None:
    """Synchronise the stream and raise NystromError if a call on it since
    the last check gave up waiting at the pseudo-inverse rendezvous (its
    output is NaN)."""
    _check(_load().nystrom_check_status(_stream(stream)))


def debug_set_rendezvous_spins(spins: int) -> None:
    """Test hook: bound on the rendezvous polls (default 2**20)."""
    _load().nystrom_debug_set_rendezvous_spins(int(spins))


def debug_set_workspace_cap(nbytes: int) -> None:
    """Test hook: cap the device workspace (0 = no cap)."""
    _load().nystrom_debug_set_workspace_cap(int(nbytes))


def workspace_bytes(B, H, n, d, m) -> int:
    return int(_load().nystrom_workspace_bytes(B, H, n, d, m))


def release() -> None:
    _load().nystrom_release()


def profile_enable(on: bool = True) -> None:
    """Bracket every kernel launch with hipEvents (see profile_collect)."""
    _load().nystrom_profile_enable(1 if on else 0)


def profile_collect() -> dict:
    """{kernel name: (total ms, launches)} for launches since the last collect."""
    lib = _load()
    cap = 16
    names = (ctypes.c_char_p * cap)()
    tot = (ctypes.c_double * cap)()
    cnt = (ctypes.c_int * cap)()
    k = lib.nystrom_profile_collect(names, tot, cnt, cap)
    _check(0 if k >= 0 else k)
    return {names[i].decode(): (float(tot[i]), int(cnt[i])) for i in range(min(k, cap))}


def debug_stages(q, k, v, key_mask=None, conv_w=None, m=64, n_iter=6, init_option=0,
                 stream=None):
    """Run the Nystrom path and return (out, stages) where stages holds the
    float32 intermediates qt, kt, A, c, Z, BV, W as CUDA tensors."""
    import torch
    _check_io(q, k, v, None)
    B, H, n, d = q.shape
    if not (k.shape == v.shape == q.shape) or not all(t.is_contiguous() for t in (q, k, v)):
        raise ValueError("q, k and v must be dense tensors of one shape [B, H, n, d]")
    _check_aux(q, B, H, n, key_mask, conv_w)
    dev = q.device
    f32 = dict(dtype=torch.float32, device=dev)
    st = dict(qt=torch.empty(B, H, m, d, **f32), kt=torch.empty(B, H, m, d, **f32),
              A=torch.empty(B, H, m, m, **f32), c=torch.empty(B * H, **f32),
              Z=torch.empty(B, H, m, m, **f32), BV=torch.empty(B, H, m, d, **f32),
              W=torch.empty(B, H, m, d, **f32))
    out = torch.empty_like(q)
    dtype = 1 if q.dtype == torch.bfloat16 else 0
    rc = _load().nystrom_debug_stages(dtype, _ptr(q), _ptr(k), _ptr(v), _ptr(key_mask), _ptr(conv_w),
                                   B, H, n, d, m, n_iter, init_option, _ptr(out),
                                   _ptr(st["qt"]), _ptr(st["kt"]), _ptr(st["A"]), _ptr(st["c"]),
                                   _ptr(st["Z"]), _ptr(st["BV"]), _ptr(st["W"]), _stream(stream))
    _check(rc)
    return out, st
