"""Seeded synthetic inputs for the Nystrom attention workloads.

This module only draws random numbers and rounds them to the I/O type; it
holds none of the attention arithmetic.  The tests, the benchmark and the
oracle-side checks all take their inputs from here, so both sides of every
comparison see identical arrays.

Workloads (head size d = 64, conv kernel 65, 6 pseudo-inverse iterations):

  1  fp32  B=1 H=2  n=256    m=64   no mask                   init 0
  2  fp32  B=8 H=12 n=512    m=64   valid length U{256..512}  init 0
  3  bf16  B=4 H=12 n=4096   m=64   valid length U{3072..4096} init 0
  4  bf16  B=1 H=8  n=16384  m=128  no mask, inputs x0.5     init 1
  5  bf16  B=1 H=4  n=65536  m=256  valid length 60000        init 0

Generator: ``numpy.random.default_rng(1000 + index)``; draw order q, k, v
(standard normal, float32, times the scale), then the conv weights
(0.02 * standard normal, float32, [H, 65]), then the per-batch valid
lengths.  bf16 workloads round q, k, v to bfloat16 with round-to-nearest-
even; the conv weights stay float32.  Masks are right padding: 1 on
[0, len), 0 on [len, n).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

CONV_TAPS = 65


@dataclass(frozen=True)
class Workload:
    index: int
    dtype: str          # "fp32" or "bf16"
    B: int
    H: int
    n: int
    d: int
    m: int
    scale: float
    mask: tuple | None  # (lo, hi) inclusive valid-length range, or None
    n_iter: int
    init_option: int

    @property
    def name(self):
        return (f"nystrom-{self.dtype}-B{self.B}-H{self.H}-n{self.n}-d{self.d}"
                f"-m{self.m}")

    @property
    def tokens(self):
        return self.B * self.n


WORKLOADS = {
    1: Workload(1, "fp32", 1, 2, 256, 64, 64, 1.0, None, 6, 0),
    2: Workload(2, "fp32", 8, 12, 512, 64, 64, 1.0, (256, 512), 6, 0),
    3: Workload(3, "bf16", 4, 12, 4096, 64, 64, 1.0, (3072, 4096), 6, 0),
    4: Workload(4, "bf16", 1, 8, 16384, 64, 128, 0.5, None, 6, 1),
    5: Workload(5, "bf16", 1, 4, 65536, 64, 256, 1.0, (60000, 60000), 6, 0),
}


def round_bf16(x):
    """Round float32 values to the nearest bfloat16 (ties to even) and
    return them widened back to float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def make_inputs(w: Workload | int, seed_offset: int = 0, qk_scale: float = 1.0):
    """Return dict(q, k, v, key_mask, conv_w, lengths) as numpy arrays.

    q, k, v are float32 [B,H,n,d] (bf16-representable for bf16 workloads);
    key_mask is uint8 [B,n] or None; conv_w is float32 [H,65].
    ``qk_scale`` multiplies q and k after drawing (before rounding); it makes
    the 'peaked' variants whose logits are larger."""
    if isinstance(w, int):
        w = WORKLOADS[w]
    rng = np.random.default_rng(1000 + w.index + seed_offset)
    shp = (w.B, w.H, w.n, w.d)
    q = rng.standard_normal(shp, dtype=np.float32) * np.float32(w.scale)
    k = rng.standard_normal(shp, dtype=np.float32) * np.float32(w.scale)
    v = rng.standard_normal(shp, dtype=np.float32) * np.float32(w.scale)
    conv_w = (np.float32(0.02) * rng.standard_normal((w.H, CONV_TAPS), dtype=np.float32))
    lengths = None
    key_mask = None
    if w.mask is not None:
        lo, hi = w.mask
        lengths = rng.integers(lo, hi + 1, size=w.B)
        key_mask = (np.arange(w.n)[None, :] < lengths[:, None]).astype(np.uint8)
    if qk_scale != 1.0:
        q = q * np.float32(qk_scale)
        k = k * np.float32(qk_scale)
    if w.dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return dict(q=q, k=k, v=v, key_mask=key_mask, conv_w=conv_w, lengths=lengths)


def make_custom(B, H, n, d, seed, dtype="fp32", scale=1.0, lengths=None,
                conv=True, taps=CONV_TAPS):
    """Inputs of an arbitrary shape for edge-case tests, same recipe."""
    rng = np.random.default_rng(seed)
    shp = (B, H, n, d)
    q = rng.standard_normal(shp, dtype=np.float32) * np.float32(scale)
    k = rng.standard_normal(shp, dtype=np.float32) * np.float32(scale)
    v = rng.standard_normal(shp, dtype=np.float32) * np.float32(scale)
    conv_w = (np.float32(0.02) * rng.standard_normal((H, taps), dtype=np.float32)) if conv else None
    key_mask = None
    if lengths is not None:
        lengths = np.asarray(lengths)
        key_mask = (np.arange(n)[None, :] < lengths[:, None]).astype(np.uint8)
    if dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return dict(q=q, k=k, v=v, key_mask=key_mask, conv_w=conv_w, lengths=lengths)


def make_module_inputs(B, n, hidden, H, d, seed, dtype="fp32", lengths=None, bias=True):
    """Inputs of the self-attention module: hidden states x [B, n, hidden]
    (standard normal), stacked q/k/v projection weights [3 H d, hidden]
    (normal with standard deviation hidden^-1/2, so the projections have
    unit scale), biases [3 H d] (0.02 * standard normal) or None, conv
    weights [H, 65] and right-padding masks as above.  bf16 rounds x, the
    weights and the biases; the conv weights stay float32."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, n, hidden), dtype=np.float32)
    w = rng.standard_normal((3 * H * d, hidden), dtype=np.float32) * np.float32(hidden ** -0.5)
    b = (np.float32(0.02) * rng.standard_normal(3 * H * d, dtype=np.float32)) if bias else None
    conv_w = np.float32(0.02) * rng.standard_normal((H, CONV_TAPS), dtype=np.float32)
    key_mask = None
    if lengths is not None:
        lengths = np.asarray(lengths)
        key_mask = (np.arange(n)[None, :] < lengths[:, None]).astype(np.uint8)
    if dtype == "bf16":
        x, w = round_bf16(x), round_bf16(w)
        b = round_bf16(b) if b is not None else None
    return dict(x=x, w_qkv=w, b_qkv=b, conv_w=conv_w, key_mask=key_mask, H=H, lengths=lengths)
