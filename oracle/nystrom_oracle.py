"""Float64 CPU oracle for Nystrom approximate self-attention.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the test suite, the smoke
check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may
import this module.  The HIP library never calls it, and the two share no
code: no kernels, helpers, constants or pre/post-processing.

It is deliberately plain: every step is the textbook definition or the
pages' algorithm, written in numpy float64 with no blocking, fusion or
reordering, so that a reader can check it against the pages by eye.

Sources, cited by page title and section (no line numbers):

[P1] "Nystromformer 源码解析与实战指南：基于 Nystrom 采样的 O(n) 自注意力近似与
     Transformers 实现" (blog.gitcode.com):
       2.1  exact-attention fallback ("path A") versus the Nystrom path;
       2.2  the 1/sqrt(d) scale split as d^-1/4 on each of Q and K;
       2.3  segment-means landmarks;
       2.4  the three softmax kernels and the product chain;
       2.5  the iterative Moore-Penrose inverse and its two initialisations;
       2.6  the depthwise convolution skip on V;
       3.1  the Nystrom configuration fields and their defaults.
[P2] Hugging Face Transformers documentation (zh), Nystromformer model page:
       NystromformerModel.forward, the ``attention_mask`` argument
       (values in {0, 1}; 1 keeps a token, 0 masks it).

Readings taken where the pages are silent, garbled or disagree (each is
repeated at the function that applies it):

R1  segment length is the run-time n/m (P1 2.3 uses a config length);
R2  the exact branch runs when m == n (P1 2.1 ties it to two config fields);
R3  the key mask is applied in the exact branch too, to Q K^T;
R4  the convolution is added in both branches;
R5  masked keys are excluded exactly (weight 0, the -inf reading of the
    additive mask of P1 2.4);
R6  a batch row with no valid key gets an all-zero B row (so B V = 0 and
    the output is the convolution alone) instead of NaN;
R7  the mask enters kernel_3 (B) only; padded tokens still enter the
    landmarks, F, A and the convolution;
R8  init option 0 ("original") takes its maxima over every (batch, head)
    of the call; option 1 (exact coefficient) takes them per (batch, head);
R9  the initial scale is (max column sum) * (max row sum) of A;
R10 product order F (Z (B V)) (P1 2.4 groups it (F Z)(B V); equal in exact
    arithmetic);
R11 the convolution is a cross-correlation (tap j multiplies V at offset
    j - K//2), zero outside [0, n), one filter per head shared by all d
    columns;
R12 n_iter = 0 is allowed and returns Z_0;
R18 the self-attention module (P1 2.2, 2.7): q, k, v are x W^T + b for
    the stacked query, key and value weights [3 H d, hidden], split into
    heads as (batch, heads, seq, head_dim); the context goes back to
    (batch, seq, H d) with head h in columns [h d, (h + 1) d);
R17 the weights returned on request (output_attentions, P1 2.7 and 5.3)
    are the matrix P1 2.4 calls attention_probs, F Z (n x m, whose rows
    are the approximate attention weights; 2.7 and 5.3 name its size
    "m x n" loosely), and the full softmax(Qs Ks^T + mask) (n x n) when
    the exact branch runs.
"""

from __future__ import annotations

import math

import numpy as np

INIT_ORIGINAL = 0
INIT_EXACT = 1


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def scale_qk(q, k):
    """[P1 2.2] Divide Q and K each by the fourth root of the head size d,
    so that Q K^T carries the usual 1/sqrt(d) factor."""
    d = q.shape[-1]
    s = 1.0 / math.sqrt(math.sqrt(d))
    return q * s, k * s


def segment_means(x, m):
    """[P1 2.3] Landmarks: cut the n tokens into m contiguous segments of
    L = n/m tokens (R1) and average each segment.  x: [..., n, d]."""
    n, d = x.shape[-2], x.shape[-1]
    if n % m != 0:
        raise ValueError("n must be a multiple of m")
    L = n // m
    return x.reshape(*x.shape[:-2], m, L, d).mean(axis=-2)


def softmax_rows(s, valid=None):
    """Row softmax over the last axis, max-subtracted.

    ``valid`` (bool, broadcastable to s) marks the columns that take part;
    the others get weight exactly 0 (R5).  A row with no valid column
    returns all zeros (R6)."""
    s = np.asarray(s, dtype=np.float64)
    if valid is None:
        mx = s.max(axis=-1, keepdims=True)
        e = np.exp(s - mx)
        return e / e.sum(axis=-1, keepdims=True)
    valid = np.broadcast_to(valid, s.shape)
    sm = np.where(valid, s, -np.inf)
    mx = sm.max(axis=-1, keepdims=True)
    mx = np.where(np.isfinite(mx), mx, 0.0)
    e = np.where(valid, np.exp(sm - mx), 0.0)
    tot = e.sum(axis=-1, keepdims=True)
    return np.where(tot > 0, e / np.where(tot > 0, tot, 1.0), 0.0)


def nystrom_kernels(qs, ks, qt, kt, key_valid=None):
    """[P1 2.4] The three softmax kernels.

    F = softmax(Qs Kt^T)  (n x m), A = softmax(Qt Kt^T)  (m x m),
    B = softmax(Qt Ks^T + mask)  (m x n).  The mask enters B only (R7)."""
    F = softmax_rows(qs @ np.swapaxes(kt, -1, -2))
    A = softmax_rows(qt @ np.swapaxes(kt, -1, -2))
    Bm = softmax_rows(qt @ np.swapaxes(ks, -1, -2), key_valid)
    return F, A, Bm


def init_scale(A, init_option):
    """[P1 2.5] Scale c of the initial iterate Z_0 = A^T / c.

    c = (max column sum of A) * (max row sum of A)  (R9).  With option 0
    ("original", the default of P1 3.1 / P2) both maxima run over every
    (batch, head) in A, giving one scalar; with option 1 (exact
    coefficient) they run per (batch, head) (R8).  A: [..., m, m].
    Returns c broadcastable against A."""
    colsum = A.sum(axis=-2)  # [..., m]: sum over rows i of A[i, j]
    rowsum = A.sum(axis=-1)  # [..., m]: sum over columns j of A[i, j]
    if init_option == INIT_ORIGINAL:
        c = colsum.max() * rowsum.max()
        return np.full(A.shape[:-2] + (1, 1), c)
    if init_option == INIT_EXACT:
        c = colsum.max(axis=-1) * rowsum.max(axis=-1)
        return c[..., None, None]
    raise ValueError("init_option must be 0 or 1")


def newton_schulz_pinv(A, c, n_iter):
    """[P1 2.5] Iterative Moore-Penrose inverse of A.

    Z_0 = A^T / c; then n_iter times: X = A Z and
    Z <- (1/4) Z (13 I - X (15 I - X (7 I - X))).  n_iter = 0 returns Z_0
    (R12)."""
    m = A.shape[-1]
    I = np.eye(m)
    Z = np.swapaxes(A, -1, -2) / c
    for _ in range(n_iter):
        X = A @ Z
        Z = 0.25 * Z @ (13.0 * I - X @ (15.0 * I - X @ (7.0 * I - X)))
    return Z


def depthwise_conv_same(v, w):
    """[P1 2.6] Per-head depthwise convolution along the sequence, 'same'
    padding: out[b,h,t,:] = sum_j w[h,j] * v[b,h,t+j-K//2,:], with v taken
    as zero outside [0, n) (R11).  v: [B,H,n,d], w: [H,K] with K odd.
    Written as the direct sum over taps."""
    w = np.asarray(w, dtype=np.float64)
    Hh, K = w.shape
    if K % 2 != 1:
        raise ValueError("kernel size must be odd")
    n = v.shape[-2]
    half = K // 2
    out = np.zeros_like(v)
    for j in range(K):
        off = j - half
        wj = w[:, j][None, :, None, None]
        if off >= 0:
            if off < n:
                out[..., : n - off, :] += wj * v[..., off:, :]
        else:
            if -off < n:
                out[..., -off:, :] += wj * v[..., : n + off, :]
    return out


def exact_attention(qs, ks, v, key_valid=None):
    """[P1 2.1] Exact softmax attention softmax(Qs Ks^T + mask) V, used when
    m == n (R2), with the key mask applied to the scores (R3)."""
    P = softmax_rows(qs @ np.swapaxes(ks, -1, -2), key_valid)
    return P @ v


def self_attention(x, w_qkv, b_qkv, H, key_mask=None, conv_w=None, m=64, n_iter=6,
                   init_option=INIT_ORIGINAL, return_qkv=False):
    """[P1 2.2, 2.7] The self-attention module around the core (R18).

    x: [B, n, hidden]; w_qkv: [3 H d, hidden], the query, key and value
    projection weights stacked in that order (each nn.Linear's [out, in]);
    b_qkv: [3 H d] or None.  q, k, v = x W^T + b per projection, each split
    into H heads of d columns -> [B, H, n, d]; the attention output
    [B, H, n, d] goes back to [B, n, H d].  With ``return_qkv`` also
    returns the projection [B, n, 3, H, d]."""
    x = _f64(x)
    w = _f64(w_qkv)
    B, n, hidden = x.shape
    if w.ndim != 2 or w.shape[1] != hidden or w.shape[0] % (3 * H) != 0:
        raise ValueError("w_qkv must be [3 H d, hidden]")
    d = w.shape[0] // (3 * H)
    y = x @ w.T
    if b_qkv is not None:
        y = y + _f64(b_qkv)
    qkv = y.reshape(B, n, 3, H, d)
    q, k, v = (np.transpose(qkv[:, :, i], (0, 2, 1, 3)) for i in range(3))
    ctx = nystrom_attention(q, k, v, key_mask, conv_w, m, n_iter, init_option)
    out = np.transpose(ctx, (0, 2, 1, 3)).reshape(B, n, H * d)
    return (out, qkv) if return_qkv else out


def attention_probs(q, k, key_mask=None, m=64, n_iter=6, init_option=INIT_ORIGINAL):
    """[P1 2.4, 2.7, 5.3] The attention weights handed back on request
    (output_attentions), R17.

    Nystrom path: F Z, kernel_1 times the iterative inverse of kernel_2,
    [B,H,n,m] (the mask does not enter F or A, R7).  When m == n (R2): the
    exact branch's softmax(Qs Ks^T + mask), [B,H,n,n] (R3, R5, R6).
    q, k: raw projections [B,H,n,d]."""
    q, k = _f64(q), _f64(k)
    B, H, n, d = q.shape
    if k.shape != q.shape:
        raise ValueError("q and k must share one shape")
    if m <= 0 or m > n or n % m != 0:
        raise ValueError("need 0 < m <= n and n % m == 0")
    if n_iter < 0:
        raise ValueError("n_iter must be >= 0")
    valid = _key_valid(key_mask, B, n)
    qs, ks = scale_qk(q, k)
    if m == n:
        return softmax_rows(qs @ np.swapaxes(ks, -1, -2), valid)
    qt = segment_means(qs, m)
    kt = segment_means(ks, m)
    F, A, _ = nystrom_kernels(qs, ks, qt, kt, valid)
    Z = newton_schulz_pinv(A, init_scale(A, init_option), n_iter)
    return F @ Z


def _key_valid(key_mask, B, n):
    if key_mask is None:
        return None
    km = np.asarray(key_mask)
    if km.shape != (B, n):
        raise ValueError("key_mask must be [B, n]")
    return (km != 0)[:, None, None, :]  # broadcast over heads and rows


def nystrom_attention(q, k, v, key_mask=None, conv_w=None, m=64, n_iter=6,
                      init_option=INIT_ORIGINAL, force_nystrom=False,
                      return_stages=False):
    """Nystrom approximate self-attention, [B,H,n,d] -> [B,H,n,d] float64.

    q, k: raw projections (the d^-1/4 scale is applied here, [P1 2.2]);
    v: values; key_mask: [B,n], nonzero = keep ([P2] attention_mask);
    conv_w: [H,K] depthwise filter or None to disable it ([P1 2.6]);
    m: landmarks; n_iter: pseudo-inverse iterations; init_option: 0 or 1.

    When m == n the exact branch runs ([P1 2.1], R2) unless
    ``force_nystrom`` asks for the approximate formula at L = 1 (a test
    hook that ties the two branches together).  Output:
    F (Z (B V)) (R10) plus the convolution (R4)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, n, d = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one shape")
    if m <= 0 or m > n or n % m != 0:
        raise ValueError("need 0 < m <= n and n % m == 0")
    if n_iter < 0:
        raise ValueError("n_iter must be >= 0")
    valid = _key_valid(key_mask, B, n)
    qs, ks = scale_qk(q, k)
    st = {}
    if m == n and not force_nystrom:
        attn = exact_attention(qs, ks, v, valid)
    else:
        qt = segment_means(qs, m)
        kt = segment_means(ks, m)
        F, A, Bm = nystrom_kernels(qs, ks, qt, kt, valid)
        c = init_scale(A, init_option)
        Z = newton_schulz_pinv(A, c, n_iter)
        BV = Bm @ v
        W = Z @ BV
        attn = F @ W
        st.update(qt=qt, kt=kt, F=F, A=A, B=Bm, c=c, Z=Z, BV=BV, W=W)
    conv = depthwise_conv_same(v, conv_w) if conv_w is not None else np.zeros_like(v)
    out = attn + conv
    if return_stages:
        st.update(attn=attn, conv=conv, out=out)
        return out, st
    return out
