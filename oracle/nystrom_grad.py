"""Float64 CPU oracle for the gradients of Nystrom attention (the backward
pass a training step needs).

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the test suite, the smoke
check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may
import this module.  The HIP library never calls it, and the two share no
code.

The forward is written again with plain torch float64 CPU operations, step
for step as ``nystrom_oracle.nystrom_attention`` (same readings R1-R12), so
that torch's autograd (a library primitive) differentiates it.  Sources, by
page title and section:

[P1] "Nystromformer 源码解析与实战指南" (blog.gitcode.com): 2.1 exact branch,
     2.2 the d^-1/4 scale on each of Q and K, 2.3 segment means, 2.4 the
     three softmax kernels and the product chain, 2.5 the iterative inverse
     and its initial scale, 2.6 the depthwise convolution; section 3.3 and
     the model-class section mention training (gradient checkpointing, the
     Trainer), which is what the gradients are for.
[P2] Hugging Face Transformers docs (zh), Nystromformer model page
     (attention_mask: 1 keeps a key, 0 masks it).

Reading (R19): the initial scale c = (max column sum) * (max row sum) is
differentiated as written, through the maxima (the gradient of a maximum
goes to its argmax).  The row-sum factor contributes nothing: every row of
a softmax sums to 1, so a gradient that is constant along a row vanishes in
the softmax's backward.  For init option 0 the column-sum maximum runs over
every (batch, head), so its gradient reaches one head only.
"""

from __future__ import annotations

import numpy as np
import torch

INIT_ORIGINAL = 0
INIT_EXACT = 1


def _t(x):
    return None if x is None else torch.as_tensor(np.asarray(x, dtype=np.float64))


def softmax_masked(s, valid=None):
    """[P1 2.4] Row softmax; columns where ``valid`` is False get weight 0
    (R5) and a row with no valid column is all zeros (R6)."""
    if valid is None:
        return torch.softmax(s, dim=-1)
    valid = valid.expand_as(s)
    any_valid = valid.any(dim=-1, keepdim=True)
    s2 = torch.where(valid, s, torch.full_like(s, float("-inf")))
    s2 = torch.where(any_valid, s2, torch.zeros_like(s))  # finite rows; zeroed below
    p = torch.softmax(s2, dim=-1)
    return torch.where(valid & any_valid, p, torch.zeros_like(p))


def depthwise_conv_same(v, w):
    """[P1 2.6] out[t] = sum_j w[h, j] v[t + j - K//2], zero outside [0, n)
    (R11), as a sum of shifted copies."""
    K = w.shape[-1]
    n = v.shape[-2]
    half = K // 2
    out = torch.zeros_like(v)
    for j in range(K):
        off = j - half
        wj = w[:, j][None, :, None, None]
        if off >= 0 and off < n:
            out = out + wj * torch.nn.functional.pad(v[..., off:, :], (0, 0, 0, off))
        elif off < 0 and -off < n:
            out = out + wj * torch.nn.functional.pad(v[..., : n + off, :], (0, 0, -off, 0))
    return out


def forward(q, k, v, key_mask=None, conv_w=None, m=64, n_iter=6, init_option=INIT_ORIGINAL):
    """The forward of ``nystrom_oracle.nystrom_attention`` in torch float64
    (differentiable).  q, k, v: [B,H,n,d] tensors; key_mask [B,n] or None;
    conv_w [H,K] tensor or None."""
    B, H, n, d = q.shape
    s = d ** -0.25                                            # [P1 2.2]
    qs, ks = q * s, k * s
    valid = None
    if key_mask is not None:
        valid = torch.as_tensor(np.asarray(key_mask) != 0)[:, None, None, :]
    if m == n:                                                # [P1 2.1], R2
        attn = softmax_masked(qs @ ks.transpose(-1, -2), valid) @ v
    else:
        L = n // m
        qt = qs.reshape(B, H, m, L, d).mean(dim=-2)           # [P1 2.3]
        kt = ks.reshape(B, H, m, L, d).mean(dim=-2)
        F = torch.softmax(qs @ kt.transpose(-1, -2), dim=-1)  # [P1 2.4]
        A = torch.softmax(qt @ kt.transpose(-1, -2), dim=-1)
        Bm = softmax_masked(qt @ ks.transpose(-1, -2), valid)
        colsum, rowsum = A.sum(dim=-2), A.sum(dim=-1)         # [P1 2.5], R8, R9
        if init_option == INIT_ORIGINAL:
            c = (colsum.max() * rowsum.max()).reshape(1, 1, 1, 1)
        elif init_option == INIT_EXACT:
            c = (colsum.max(dim=-1).values * rowsum.max(dim=-1).values)[..., None, None]
        else:
            raise ValueError("init_option must be 0 or 1")
        I = torch.eye(m, dtype=A.dtype)
        Z = A.transpose(-1, -2) / c
        for _ in range(n_iter):
            X = A @ Z
            Z = 0.25 * Z @ (13.0 * I - X @ (15.0 * I - X @ (7.0 * I - X)))
        attn = F @ (Z @ (Bm @ v))                             # R10
    if conv_w is not None:
        attn = attn + depthwise_conv_same(v, conv_w)          # R4
    return attn


def gradients(q, k, v, dout, key_mask=None, conv_w=None, m=64, n_iter=6, init_option=INIT_ORIGINAL):
    """Gradients of sum(out * dout) with respect to q, k, v and conv_w
    (float64 numpy; dconv_w is None without a convolution)."""
    q, k, v = (_t(x).requires_grad_(True) for x in (q, k, v))
    w = _t(conv_w)
    if w is not None:
        w.requires_grad_(True)
    out = forward(q, k, v, key_mask, w, m, n_iter, init_option)
    ins = [q, k, v] + ([w] if w is not None else [])
    g = torch.autograd.grad(out, ins, grad_outputs=_t(dout))
    res = [x.detach().numpy() for x in g]
    return res[0], res[1], res[2], (res[3] if w is not None else None)
