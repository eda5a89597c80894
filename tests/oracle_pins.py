"""Pins for the float64 oracle: checks against things other than the oracle
itself (closed forms, library routines, brute force, exact invariants).

Each ``pin_*`` takes the oracle module and returns a non-negative error;
the oracle is pinned when every error is below its tolerance.  The same
functions are run against deliberately broken copies of oracle functions
(test_oracle_mutations.py) to show that each plausible mistake is caught.

Citations are to the pages by title and section:
[P1] "Nystromformer 源码解析与实战指南" (blog.gitcode.com), sections 2.1-2.7;
[P2] Hugging Face Transformers docs (zh), Nystromformer model page,
     NystromformerModel.forward ``attention_mask``.
"""

from __future__ import annotations

import math

import numpy as np
import scipy.special
import torch

RNG = np.random.default_rng


def _rel(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def _rand_rowstochastic(rng, shape_lead, m, logit_std):
    """A softmax-of-random-logits matrix, the shape A takes on the path."""
    s = rng.standard_normal(shape_lead + (m, m)) * logit_std
    e = np.exp(s - s.max(-1, keepdims=True))
    return e / e.sum(-1, keepdims=True)


# --------------------------------------------------------------- scaling ---
def pin_scale(O):
    """[P1 2.2] Splitting 1/sqrt(d) as d^-1/4 on each side must give
    Qs Ks^T = Q K^T / sqrt(d) exactly (up to rounding), and for d = 64 the
    factor is 2^-1.5."""
    rng = RNG(1)
    q = rng.standard_normal((2, 3, 5, 64))
    k = rng.standard_normal((2, 3, 5, 64))
    qs, ks = O.scale_qk(q, k)
    e1 = _rel(qs @ np.swapaxes(ks, -1, -2), (q @ np.swapaxes(k, -1, -2)) / 8.0)
    e2 = abs(qs[0, 0, 0, 0] / q[0, 0, 0, 0] - 2.0 ** -1.5)
    e3 = _rel(qs / q, ks / k)  # same factor on both sides
    return max(e1, e2, e3)


# --------------------------------------------------------- segment means ---
def pin_segment_means_direct(O):
    """[P1 2.3] Landmark i is the plain average of tokens [iL, (i+1)L),
    computed here by explicit Python loops."""
    rng = RNG(2)
    B, H, n, d, m = 2, 2, 12, 3, 4
    x = rng.standard_normal((B, H, n, d))
    got = O.segment_means(x, m)
    L = n // m
    ref = np.zeros((B, H, m, d))
    for b in range(B):
        for h in range(H):
            for i in range(m):
                for c in range(d):
                    acc = 0.0
                    for t in range(i * L, (i + 1) * L):
                        acc += x[b, h, t, c]
                    ref[b, h, i, c] = acc / L
    return _rel(got, ref)


def pin_segment_means_invariants(O):
    """Permuting tokens inside a segment leaves the landmarks unchanged;
    a segment filled with one vector averages to that vector."""
    rng = RNG(3)
    n, d, m = 32, 5, 8
    L = n // m
    x = rng.standard_normal((1, 1, n, d))
    perm = np.concatenate([rng.permutation(L) + i * L for i in range(m)])
    e1 = _rel(O.segment_means(x[:, :, perm], m), O.segment_means(x, m))
    c = rng.standard_normal((m, d))
    y = np.repeat(c, L, axis=0)[None, None]
    e2 = _rel(O.segment_means(y, m)[0, 0], c)
    # moving one token across a segment boundary must change two landmarks
    z = x.copy()
    z[0, 0, [L - 1, L]] = z[0, 0, [L, L - 1]]
    diff = np.abs(O.segment_means(z, m) - O.segment_means(x, m)).sum(-1)[0, 0]
    e3 = 0.0 if (diff[0] > 1e-9 and diff[1] > 1e-9 and diff[2:].max() < 1e-12) else 1.0
    return max(e1, e2, e3)


# --------------------------------------------------------------- softmax ---
def pin_softmax_library(O):
    """Row softmax equals scipy.special.softmax; masked columns get exactly
    0 and the rest equals scipy's softmax over the kept columns ([P2] mask
    polarity, 1 = keep); a row with no kept column is all zeros."""
    rng = RNG(4)
    s = rng.standard_normal((3, 7, 11)) * 5
    e1 = _rel(O.softmax_rows(s), scipy.special.softmax(s, axis=-1))
    valid = rng.random((3, 1, 11)) < 0.6
    valid[0, 0, :] = False
    valid[1, 0, 3] = True
    got = O.softmax_rows(s, valid)
    err = 0.0
    for b in range(3):
        keep = valid[b, 0]
        if not keep.any():
            err = max(err, float(np.abs(got[b]).max()))
            continue
        ref = scipy.special.softmax(s[b][:, keep], axis=-1)
        err = max(err, _rel(got[b][:, keep], ref), float(np.abs(got[b][:, ~keep]).max()))
    e3 = abs(float(O.softmax_rows(s).sum(-1).max()) - 1.0)
    return max(e1, err, e3)


def pin_softmax_rows_axis(O):
    """The softmax runs along the last axis (over keys / landmarks), and a
    constant added to a row changes nothing."""
    rng = RNG(5)
    s = rng.standard_normal((4, 6))
    p = O.softmax_rows(s)
    e1 = float(np.abs(p.sum(-1) - 1).max())
    e2 = _rel(O.softmax_rows(s + rng.standard_normal((4, 1)) * 30), p)
    return max(e1, e2)


# ---------------------------------------------------------- exact branch ---
def pin_exact_bruteforce(O):
    """[P1 2.1] With m == n the output is exact softmax attention
    softmax(Q K^T / sqrt(d) + mask) V; here by explicit loops, per query."""
    rng = RNG(6)
    B, H, n, d = 2, 2, 8, 4
    q = rng.standard_normal((B, H, n, d))
    k = rng.standard_normal((B, H, n, d))
    v = rng.standard_normal((B, H, n, d))
    mask = np.ones((B, n), np.uint8)
    mask[1, 5:] = 0
    got = O.nystrom_attention(q, k, v, mask, None, m=n)
    ref = np.zeros_like(got)
    for b in range(B):
        for h in range(H):
            for t in range(n):
                sc = []
                for j in range(n):
                    dot = sum(q[b, h, t, c] * k[b, h, j, c] for c in range(d))
                    sc.append(dot / math.sqrt(d))
                keep = [j for j in range(n) if mask[b, j]]
                mx = max(sc[j] for j in keep)
                wts = {j: math.exp(sc[j] - mx) for j in keep}
                tot = sum(wts.values())
                for c in range(d):
                    ref[b, h, t, c] = sum(wts[j] / tot * v[b, h, j, c] for j in keep)
    return _rel(got, ref)


def pin_exact_sdpa(O):
    """The exact branch equals torch's scaled_dot_product_attention in
    float64 with a boolean key mask (True = attend), a library routine."""
    rng = RNG(7)
    B, H, n, d = 2, 3, 64, 64
    q = rng.standard_normal((B, H, n, d))
    k = rng.standard_normal((B, H, n, d))
    v = rng.standard_normal((B, H, n, d))
    lens = np.array([64, 40])
    mask = (np.arange(n)[None] < lens[:, None]).astype(np.uint8)
    got = O.nystrom_attention(q, k, v, mask, None, m=n)
    am = torch.from_numpy(mask.astype(bool))[:, None, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=am).numpy()
    return _rel(got, ref)


# ----------------------------------------------------------------- pinv ---
def _spectral_Z(A, c, n_iter):
    """Closed form of the iteration: with A = U S V^T, every iterate is
    Z_t = V diag(z_t) U^T with z_0 = s/c and
    z_{t+1} = z_t (13 - 15x + 7x^2 - x^3)/4, x = s z_t."""
    U, S, Vt = np.linalg.svd(A)
    z = S / c
    for _ in range(n_iter):
        x = S * z
        z = z * (13 - 15 * x + 7 * x ** 2 - x ** 3) / 4
    return Vt.T @ np.diag(z) @ U.T


def pin_pinv_spectral(O):
    """[P1 2.5] The iteration from Z_0 = A^T / c against its spectral closed
    form, for several iteration counts, both init scales and sizes 4-16."""
    rng = RNG(8)
    err = 0.0
    for m, std in ((4, 0.5), (8, 1.0), (16, 2.0)):
        A = _rand_rowstochastic(rng, (), m, std)
        for c in (A.sum(0).max() * A.sum(1).max(), 1.7):
            for n_iter in (0, 1, 2, 6, 12):
                got = O.newton_schulz_pinv(A, c, n_iter)
                err = max(err, _rel(got, _spectral_Z(A, c, n_iter)))
    return err


def pin_pinv_limit(O):
    """As the iteration count grows on a well-conditioned A, Z approaches
    numpy's SVD pseudo-inverse and the Penrose identities hold."""
    rng = RNG(9)
    err = 0.0
    for m in (4, 8):
        A = _rand_rowstochastic(rng, (), m, 2.0)
        c = A.sum(0).max() * A.sum(1).max()
        Z = O.newton_schulz_pinv(A, c, 40)
        err = max(err, _rel(Z, np.linalg.pinv(A)), _rel(A @ Z @ A, A), _rel(Z @ A @ Z, Z),
                  _rel((A @ Z).T, A @ Z), _rel((Z @ A).T, Z @ A))
    return err


def pin_pinv_residual_law(O):
    """With E_t = I - A Z_t the update obeys E_{t+1} = (3 E_t^3 + E_t^4)/4
    exactly (a polynomial identity of the (7, 15, 13)/4 step)."""
    rng = RNG(10)
    m = 6
    A = _rand_rowstochastic(rng, (), m, 1.0)
    c = A.sum(0).max() * A.sum(1).max()
    I = np.eye(m)
    err = 0.0
    for t in range(0, 5):
        E0 = I - A @ O.newton_schulz_pinv(A, c, t)
        E1 = I - A @ O.newton_schulz_pinv(A, c, t + 1)
        pred = 0.75 * np.linalg.matrix_power(E0, 3) + 0.25 * np.linalg.matrix_power(E0, 4)
        err = max(err, float(np.abs(E1 - pred).max()) / max(1.0, float(np.abs(E0).max())))
    return err


def pin_pinv_uniform_fixed_point(O):
    """A = J/m (all logits equal) gives c = 1 and Z_0 = J/m, which the step
    maps to itself."""
    err = 0.0
    for m in (4, 16):
        A = np.full((m, m), 1.0 / m)
        c = O.init_scale(A[None, None], 0)
        err = max(err, abs(float(np.asarray(c).ravel()[0]) - 1.0))
        for n_iter in (0, 1, 6):
            err = max(err, _rel(O.newton_schulz_pinv(A, 1.0, n_iter), A))
    return err


def pin_init_scale(O):
    """[P1 2.5] Hand-worked scales.  A1 = [[.5,.5],[.25,.75]] has column sums
    (.75, 1.25) and row sums (1, 1): c = 1.25.  A2 = [[.9,.1],[.2,.8]] has
    column sums (1.1, .9): c = 1.1.  Option 1 is per head (1.25, 1.1);
    option 0 takes both maxima over the whole batch (1.25, 1.25).  A
    non-stochastic A3 = [[1, 2], [0, 1]] (column sums 1, 3; row sums 3, 1)
    gives c = 9, which separates column sums from row sums."""
    A1 = np.array([[0.5, 0.5], [0.25, 0.75]])
    A2 = np.array([[0.9, 0.1], [0.2, 0.8]])
    A = np.stack([A1, A2])[None]  # [1, 2, 2, 2]
    c1 = np.asarray(O.init_scale(A, 1)).ravel()
    c0 = np.broadcast_to(np.asarray(O.init_scale(A, 0)), (1, 2, 1, 1)).ravel()
    A3 = np.array([[1.0, 2.0], [0.0, 1.0]])[None, None]
    c3 = float(np.asarray(O.init_scale(A3, 1)).ravel()[0])
    # and Z_0 = A^T / c: one step from n_iter = 0
    z0 = O.newton_schulz_pinv(A1, 1.25, 0)
    return max(float(np.abs(c1 - [1.25, 1.1]).max()), float(np.abs(c0 - [1.25, 1.25]).max()),
               abs(c3 - 9.0), _rel(z0, A1.T / 1.25))


def pin_pinv_diag_worked(O):
    """[P1 2.5] Worked by hand: A = diag(1, 1/2) has column and row sums
    (1, 1/2), so c = 1 and Z_0 = diag(1, 1/2); then x = (1, 1/4) and the
    step multiplies by (13 - 15x + 7x^2 - x^3)/4 = (1, 619/256), giving
    Z_1 = diag(1, 619/512)."""
    A = np.diag([1.0, 0.5])
    c = float(np.asarray(O.init_scale(A[None, None], 1)).ravel()[0])
    Z1 = O.newton_schulz_pinv(A, c, 1)
    return max(abs(c - 1.0), float(np.abs(Z1 - np.diag([1.0, 619.0 / 512.0])).max()))


# ------------------------------------------------------------------ conv ---
def pin_conv_direct(O):
    """[P1 2.6] Depthwise 'same' convolution as a per-output direct sum with
    explicit bounds."""
    rng = RNG(11)
    B, H, n, d, K = 1, 2, 40, 3, 9
    v = rng.standard_normal((B, H, n, d))
    w = rng.standard_normal((H, K))
    got = O.depthwise_conv_same(v, w)
    ref = np.zeros_like(v)
    for h in range(H):
        for t in range(n):
            for c in range(d):
                acc = 0.0
                for j in range(K):
                    s = t + j - K // 2
                    if 0 <= s < n:
                        acc += w[h, j] * v[0, h, s, c]
                ref[0, h, t, c] = acc
    return _rel(got, ref)


def pin_conv_library(O):
    """The same convolution through torch.nn.functional.conv1d (groups = H,
    padding = K//2, float64), a library routine with Conv2d's (K,1) semantics
    along the sequence; at the default 65 taps and at other odd kernel sizes
    (the conv_kernel_size field, [P1] 3.1)."""
    rng = RNG(12)
    B, H, n, d = 2, 3, 100, 4
    err = 0.0
    for K in (65, 1, 3, 31):
        v = rng.standard_normal((B, H, n, d))
        w = rng.standard_normal((H, K))
        got = O.depthwise_conv_same(v, w)
        x = torch.from_numpy(v).permute(0, 3, 1, 2).reshape(B * d, H, n)
        y = torch.nn.functional.conv1d(x, torch.from_numpy(w)[:, None, :], padding=K // 2, groups=H)
        ref = y.reshape(B, d, H, n).permute(0, 2, 3, 1).numpy()
        err = max(err, _rel(got, ref))
    return err


def pin_conv_delta(O):
    """Delta filters: tap K//2 alone is the identity; tap K//2 + s alone
    shifts by s (out[t] = v[t + s]) with zero fill."""
    rng = RNG(13)
    n, d, K = 50, 2, 65
    v = rng.standard_normal((1, 1, n, d))
    err = 0.0
    for s in (0, 1, -3, 32, -32):
        w = np.zeros((1, K))
        w[0, K // 2 + s] = 1.0
        ref = np.zeros_like(v)
        for t in range(n):
            if 0 <= t + s < n:
                ref[0, 0, t] = v[0, 0, t + s]
        err = max(err, _rel(O.depthwise_conv_same(v, w), ref))
    return err


# ------------------------------------------------------------ whole path ---
def pin_path_q_zero(O):
    """[P1 2.4] With Q = 0 every kernel is uniform (B over the kept keys), A
    is J/m with c = 1, and the attention output is exactly the mean of the
    kept V rows on every token, for any iteration count and either init."""
    rng = RNG(14)
    B, H, n, d, m = 2, 2, 32, 8, 8
    q = np.zeros((B, H, n, d))
    k = rng.standard_normal((B, H, n, d))
    v = rng.standard_normal((B, H, n, d))
    lens = np.array([32, 19])
    mask = (np.arange(n)[None] < lens[:, None]).astype(np.uint8)
    err = 0.0
    for n_iter in (0, 3, 6):
        for init in (0, 1):
            got = O.nystrom_attention(q, k, v, mask, None, m=m, n_iter=n_iter, init_option=init)
            for b in range(B):
                vbar = v[b, :, : lens[b]].mean(axis=1, keepdims=True)
                err = max(err, _rel(got[b], np.broadcast_to(vbar, got[b].shape)))
    return err


def pin_path_nystrom_to_exact(O):
    """With m = n forced onto the Nystrom formula (L = 1) the landmarks are
    the tokens, so F = A; as the iteration count grows F A^+ -> I and the
    output tends to masked exact attention (ties the two branches)."""
    rng = RNG(15)
    B, H, n, d = 1, 2, 8, 16
    q = rng.standard_normal((B, H, n, d)) * 1.5
    k = rng.standard_normal((B, H, n, d)) * 1.5
    v = rng.standard_normal((B, H, n, d))
    mask = np.ones((B, n), np.uint8)
    mask[0, 6:] = 0
    got = O.nystrom_attention(q, k, v, mask, None, m=n, n_iter=60, force_nystrom=True)
    ref = O.nystrom_attention(q, k, v, mask, None, m=n)
    return _rel(got, ref)


def pin_path_mask_semantics(O):
    """[P1 2.4] The mask enters B only.  With the conv off, V at masked
    positions has no effect; K at masked positions still does (through the
    key landmarks)."""
    rng = RNG(16)
    B, H, n, d, m = 1, 2, 32, 8, 8
    q = rng.standard_normal((B, H, n, d))
    k = rng.standard_normal((B, H, n, d))
    v = rng.standard_normal((B, H, n, d))
    mask = np.ones((B, n), np.uint8)
    mask[0, 20:] = 0
    base = O.nystrom_attention(q, k, v, mask, None, m=m)
    v2 = v.copy()
    v2[:, :, 20:] += 100.0
    e1 = _rel(O.nystrom_attention(q, k, v2, mask, None, m=m), base)
    k2 = k.copy()
    k2[:, :, 20:] += 1.0
    changed = _rel(O.nystrom_attention(q, k2, v, mask, None, m=m), base)
    e2 = 0.0 if changed > 1e-6 else 1.0
    # and with no mask at all, the V change must show
    nomask = O.nystrom_attention(q, k, v, None, None, m=m)
    e3 = 0.0 if _rel(O.nystrom_attention(q, k, v2, None, None, m=m), nomask) > 1e-3 else 1.0
    return max(e1, e2, e3)


def pin_path_zero_valid(O):
    """A batch row with no kept key: B V = 0, so the output is the
    convolution of V alone, with no NaN."""
    rng = RNG(17)
    B, H, n, d, m, K = 2, 2, 32, 8, 8, 65
    q = rng.standard_normal((B, H, n, d))
    k = rng.standard_normal((B, H, n, d))
    v = rng.standard_normal((B, H, n, d))
    w = rng.standard_normal((H, K)) * 0.02
    mask = np.ones((B, n), np.uint8)
    mask[1, :] = 0
    got = O.nystrom_attention(q, k, v, mask, w, m=m)
    if not np.isfinite(got).all():
        return float("inf")
    conv = O.depthwise_conv_same(v, w)
    return _rel(got[1], conv[1])


def pin_path_composition(O):
    """Stage outputs compose as the pages' product chain: attention =
    F (Z (B V)), with F, A, B rows summing to 1 and B zero on masked keys."""
    rng = RNG(18)
    B, H, n, d, m = 2, 2, 64, 16, 16
    q = rng.standard_normal((B, H, n, d))
    k = rng.standard_normal((B, H, n, d))
    v = rng.standard_normal((B, H, n, d))
    lens = np.array([64, 50])
    mask = (np.arange(n)[None] < lens[:, None]).astype(np.uint8)
    out, st = O.nystrom_attention(q, k, v, mask, None, m=m, return_stages=True)
    e1 = _rel(st["F"] @ (st["Z"] @ (st["B"] @ v)), out)
    e2 = max(float(np.abs(st[x].sum(-1) - 1).max()) for x in ("F", "A", "B"))
    e3 = float(np.abs(st["B"][1][..., 50:]).max())
    # F is n x m, A is m x m, B is m x n
    e4 = 0.0 if (st["F"].shape[-2:] == (n, m) and st["A"].shape[-2:] == (m, m)
                 and st["B"].shape[-2:] == (m, n)) else 1.0
    return max(e1, e2, e3, e4)


# ------------------------------------------------ attention weights ---

def pin_probs_exact_bruteforce(O):
    """[P1 2.1, 2.7] m == n: the returned weights are softmax(q k^T / sqrt(d))
    over the kept keys, written out element by element; a batch row with no
    kept key gives zero rows."""
    rng = RNG(31)
    B, H, n, d = 2, 2, 6, 4
    q = rng.standard_normal((B, H, n, d))
    k = rng.standard_normal((B, H, n, d))
    mask = np.ones((B, n), np.uint8)
    mask[0, [1, 4]] = 0
    mask[1, :] = 0
    got = O.attention_probs(q, k, mask, m=n)
    ref = np.zeros((B, H, n, n))
    for b in range(B):
        for h in range(H):
            for i in range(n):
                keep = [j for j in range(n) if mask[b, j]]
                if not keep:
                    continue
                s = {j: sum(q[b, h, i, c] * k[b, h, j, c] for c in range(d)) / math.sqrt(d) for j in keep}
                top = max(s.values())
                tot = sum(math.exp(s[j] - top) for j in keep)
                for j in keep:
                    ref[b, h, i, j] = math.exp(s[j] - top) / tot
    if got.shape != ref.shape:
        return float("inf")
    return float(np.abs(got - ref).max())


def _landmark_kernels_lib(q, k, m):
    """F and A from library softmax and reshaped means, d^-1/4 on each side."""
    d = q.shape[-1]
    qs, ks = q * d ** -0.25, k * d ** -0.25
    lead, n = q.shape[:-2], q.shape[-2]
    qt = qs.reshape(*lead, m, n // m, d).mean(-2)
    kt = ks.reshape(*lead, m, n // m, d).mean(-2)
    F = scipy.special.softmax(qs @ np.swapaxes(kt, -1, -2), axis=-1)
    A = scipy.special.softmax(qt @ np.swapaxes(kt, -1, -2), axis=-1)
    return F, A, ks, qt


def pin_probs_converged_inverse(O):
    """[P1 2.4, 2.5] With the iteration run to convergence the weights are
    F A^-1 (LAPACK inverse), and their rows sum to 1 (A 1 = 1, so
    A^-1 1 = 1, and F 1 = 1)."""
    rng = RNG(32)
    B, H, n, d, m = 1, 3, 48, 8, 12
    q = rng.standard_normal((B, H, n, d))
    k = rng.standard_normal((B, H, n, d))
    got = O.attention_probs(q, k, None, m=m, n_iter=40, init_option=1)
    F, A, _, _ = _landmark_kernels_lib(q, k, m)
    ref = F @ np.linalg.inv(A)
    if got.shape != (B, H, n, m):
        return float("inf")
    return max(_rel(got, ref), float(np.abs(got.sum(-1) - 1).max()))


def pin_probs_output_consistency(O):
    """[P1 2.4] The weights times B V, plus the convolution, give the output:
    B formed here with the library softmax over kept keys, a partial mask,
    six iterations, both initialisations."""
    rng = RNG(33)
    B, H, n, d, m = 2, 2, 64, 16, 16
    q = rng.standard_normal((B, H, n, d))
    k = rng.standard_normal((B, H, n, d))
    v = rng.standard_normal((B, H, n, d))
    w = rng.standard_normal((H, 65)) * 0.02
    lens = np.array([64, 41])
    mask = (np.arange(n)[None] < lens[:, None]).astype(np.uint8)
    _, _, ks, qt = _landmark_kernels_lib(q, k, m)
    s = qt @ np.swapaxes(ks, -1, -2)
    s = np.where(mask[:, None, None, :] != 0, s, -np.inf)
    Bm = scipy.special.softmax(s, axis=-1)
    err = 0.0
    for opt in (0, 1):
        P = O.attention_probs(q, k, mask, m=m, n_iter=6, init_option=opt)
        out = O.nystrom_attention(q, k, v, mask, w, m=m, n_iter=6, init_option=opt)
        err = max(err, _rel(P @ (Bm @ v) + O.depthwise_conv_same(v, w), out))
    return err


# ---------------------------------------------------------------- module ---

def pin_module_identity_projection(O):
    """[P1 2.2, 2.7] With hidden = 3 H d, W = I and b = 0, x is q, k, v laid
    side by side per token: the module must equal the core on those q, k, v
    (head h of q in columns [h d, (h + 1) d) of the first third), with the
    context's head h back in columns [h d, (h + 1) d)."""
    rng = RNG(41)
    B, H, n, d, m = 2, 3, 32, 8, 8
    q, k, v = (rng.standard_normal((B, H, n, d)) for _ in range(3))
    w = rng.standard_normal((H, 65)) * 0.02
    mask = (np.arange(n)[None] < np.array([32, 20])[:, None]).astype(np.uint8)
    x = np.zeros((B, n, 3 * H * d))
    for i, t in enumerate((q, k, v)):
        for h in range(H):
            x[:, :, (i * H + h) * d:(i * H + h + 1) * d] = t[:, h]
    got = O.self_attention(x, np.eye(3 * H * d), None, H, mask, w, m=m)
    core = O.nystrom_attention(q, k, v, mask, w, m=m)
    ref = np.zeros((B, n, H * d))
    for h in range(H):
        ref[:, :, h * d:(h + 1) * d] = core[:, h]
    return _rel(got, ref)


def pin_module_projection_library(O):
    """[P1 2.2] The projection is torch's linear layer (x W^T + b), in
    float64."""
    rng = RNG(42)
    B, H, n, d, hidden = 2, 2, 16, 8, 24
    x = rng.standard_normal((B, n, hidden))
    wq = rng.standard_normal((3 * H * d, hidden)) * 0.2
    bq = rng.standard_normal(3 * H * d)
    _, qkv = O.self_attention(x, wq, bq, H, m=4, return_qkv=True)
    ref = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(wq), torch.from_numpy(bq)).numpy()
    return _rel(qkv.reshape(B, n, -1), ref)


# --------------------------------------------------------------- gradients ---

def _fd_case(seed, B, H, n, d, m, K, lens, n_iter, init):
    rng = RNG(seed)
    q, k, v = (rng.standard_normal((B, H, n, d)) for _ in range(3))
    w = rng.standard_normal((H, K)) * 0.3 if K else None
    mask = None if lens is None else (np.arange(n)[None] < np.asarray(lens)[:, None]).astype(np.uint8)
    dout = rng.standard_normal((B, H, n, d))
    return q, k, v, w, mask, dout


GRAD_CASES = [
    # seed, B, H, n, d, m, K, valid lengths, n_iter, init
    (51, 1, 2, 8, 4, 4, 3, [6], 3, 1),
    (52, 2, 1, 8, 4, 4, 5, [8, 5], 2, 0),
    (53, 1, 2, 6, 4, 6, 3, [4], 6, 0),       # exact branch (m == n)
    (54, 1, 1, 12, 3, 3, None, None, 4, 0),
]


def pin_grad_forward(O):
    """The differentiable forward equals the numpy oracle's output."""
    from oracle import nystrom_grad as G
    err = 0.0
    for seed, B, H, n, d, m, K, lens, it, init in GRAD_CASES:
        q, k, v, w, mask, _ = _fd_case(seed, B, H, n, d, m, K, lens, it, init)
        ref = O.nystrom_attention(q, k, v, mask, w, m=m, n_iter=it, init_option=init)
        got = G.forward(*(torch.from_numpy(x) for x in (q, k, v)), mask,
                        None if w is None else torch.from_numpy(w), m, it, init).numpy()
        err = max(err, _rel(got, ref))
    return err


def pin_grad_finite_differences(O):
    """[P1 2.2-2.6] Every gradient entry against central differences of the
    numpy oracle (step 1e-6 in float64), on tiny inputs covering both
    initialisations, a partial mask, the convolution and the exact branch;
    the derivative of sum(out * dout) is independent of autograd here."""
    from oracle import nystrom_grad as G
    err = 0.0
    h = 1e-6
    for seed, B, H, n, d, m, K, lens, it, init in GRAD_CASES:
        q, k, v, w, mask, dout = _fd_case(seed, B, H, n, d, m, K, lens, it, init)
        got = G.gradients(q, k, v, dout, mask, w, m, it, init)

        def loss(qq, kk, vv, ww):
            return float((O.nystrom_attention(qq, kk, vv, mask, ww, m=m, n_iter=it, init_option=init) * dout).sum())

        args = [q, k, v, w]
        for idx in range(4):
            if args[idx] is None:
                continue
            fd = np.zeros_like(args[idx])
            for pos in np.ndindex(*args[idx].shape):
                up = [a.copy() if (a is not None and j == idx) else a for j, a in enumerate(args)]
                dn = [a.copy() if (a is not None and j == idx) else a for j, a in enumerate(args)]
                up[idx][pos] += h
                dn[idx][pos] -= h
                fd[pos] = (loss(*up) - loss(*dn)) / (2 * h)
            err = max(err, _rel(got[idx], fd))
    return err


ALL_PINS = {
    "scale": (pin_scale, 1e-12),
    "segment_means_direct": (pin_segment_means_direct, 1e-12),
    "segment_means_invariants": (pin_segment_means_invariants, 1e-12),
    "softmax_library": (pin_softmax_library, 1e-12),
    "softmax_rows_axis": (pin_softmax_rows_axis, 1e-12),
    "exact_bruteforce": (pin_exact_bruteforce, 1e-12),
    "exact_sdpa": (pin_exact_sdpa, 1e-12),
    "pinv_spectral": (pin_pinv_spectral, 1e-9),
    "pinv_limit": (pin_pinv_limit, 1e-9),
    "pinv_residual_law": (pin_pinv_residual_law, 1e-10),
    "pinv_uniform_fixed_point": (pin_pinv_uniform_fixed_point, 1e-12),
    "init_scale": (pin_init_scale, 1e-12),
    "pinv_diag_worked": (pin_pinv_diag_worked, 1e-15),
    "conv_direct": (pin_conv_direct, 1e-12),
    "conv_library": (pin_conv_library, 1e-12),
    "conv_delta": (pin_conv_delta, 1e-15),
    "path_q_zero": (pin_path_q_zero, 1e-12),
    "path_nystrom_to_exact": (pin_path_nystrom_to_exact, 1e-8),
    "path_mask_semantics": (pin_path_mask_semantics, 1e-12),
    "path_zero_valid": (pin_path_zero_valid, 1e-12),
    "path_composition": (pin_path_composition, 1e-12),
    "probs_exact_bruteforce": (pin_probs_exact_bruteforce, 1e-12),
    "probs_converged_inverse": (pin_probs_converged_inverse, 1e-9),
    "probs_output_consistency": (pin_probs_output_consistency, 1e-12),
    "module_identity_projection": (pin_module_identity_projection, 1e-13),
    "module_projection_library": (pin_module_projection_library, 1e-13),
    "grad_forward": (pin_grad_forward, 1e-12),
    "grad_finite_differences": (pin_grad_finite_differences, 1e-6),
}
