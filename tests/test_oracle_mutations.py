"""Plant plausible mistakes in the oracle (on the CPU) and check that its
pins catch each one.  A pin set that lets a mutant through is not a pin."""
import math

import numpy as np
import pytest

import oracle_pins as P
from oracle import nystrom_oracle as O

_orig = {name: getattr(O, name) for name in dir(O) if callable(getattr(O, name))}


def _scale_double(q, k):
    s = 1.0 / math.sqrt(q.shape[-1])
    return q * s, k * s


def _scale_q_only(q, k):
    return q / math.sqrt(q.shape[-1]), k


def _segments_interleaved(x, m):
    n, d = x.shape[-2:]
    return x.reshape(*x.shape[:-2], n // m, m, d).mean(axis=-3)


def _softmax_wrong_axis(s, valid=None):
    s = np.asarray(s, np.float64)
    e = np.exp(s - s.max(axis=-2, keepdims=True))
    if valid is not None:
        e = np.where(np.broadcast_to(valid, s.shape), e, 0.0)
    return e / e.sum(axis=-2, keepdims=True)


def _softmax_mask_inverted(s, valid=None):
    return _orig["softmax_rows"](s, None if valid is None else ~np.asarray(valid))


def _softmax_no_guard(s, valid=None):
    s = np.asarray(s, np.float64)
    if valid is None:
        return _orig["softmax_rows"](s)
    sm = np.where(np.broadcast_to(valid, s.shape), s, -np.inf)
    e = np.exp(sm - sm.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def _kernels_no_mask(qs, ks, qt, kt, key_valid=None):
    return _orig["nystrom_kernels"](qs, ks, qt, kt, None)


def _ns_factory(z0_transpose=True, c13=13.0, c15=15.0, c7=7.0, right=True, quarter=0.25):
    def ns(A, c, n_iter):
        m = A.shape[-1]
        I = np.eye(m)
        Z = (np.swapaxes(A, -1, -2) if z0_transpose else A) / c
        for _ in range(n_iter):
            X = A @ Z
            T = c13 * I - X @ (c15 * I - X @ (c7 * I - X))
            Z = quarter * (Z @ T if right else T @ Z)
        return Z
    return ns


def _init_factory(mode):
    def init(A, init_option):
        colsum = A.sum(axis=-2)
        rowsum = A.sum(axis=-1)
        if mode == "rows_twice":
            return _plain(rowsum, rowsum, init_option, A)
        if mode == "no_rowsum":
            rowsum = np.ones_like(rowsum)
            return _plain(colsum, rowsum, init_option, A)
        if mode == "orig_per_head":
            return _plain(colsum, rowsum, 1, A)
        if mode == "exact_global":
            return _plain(colsum, rowsum, 0, A)
        raise AssertionError(mode)
    return init


def _plain(colsum, rowsum, opt, A):
    if opt == 0:
        return np.full(A.shape[:-2] + (1, 1), colsum.max() * rowsum.max())
    return (colsum.max(-1) * rowsum.max(-1))[..., None, None]


def _conv_flipped(v, w):
    return _orig["depthwise_conv_same"](v, np.asarray(w)[:, ::-1])


def _conv_off_by_one(v, w):
    out = _orig["depthwise_conv_same"](v, w)
    return np.concatenate([out[..., 1:, :], np.zeros_like(out[..., :1, :])], axis=-2)


def _probs_factory(mode):
    real = O.attention_probs

    def probs(q, k, key_mask=None, m=64, n_iter=6, init_option=0):
        if mode == "exact_no_mask" and m == q.shape[-2]:
            return real(q, k, None, m, n_iter, init_option)
        if m == q.shape[-2]:
            return real(q, k, key_mask, m, n_iter, init_option)
        qs, ks = O.scale_qk(np.asarray(q, np.float64), np.asarray(k, np.float64))
        qt, kt = O.segment_means(qs, m), O.segment_means(ks, m)
        valid = None if key_mask is None else (np.asarray(key_mask) != 0)[:, None, None, :]
        F, A, _ = O.nystrom_kernels(qs, ks, qt, kt, None)
        Z = O.newton_schulz_pinv(A, O.init_scale(A, init_option), n_iter)
        if mode == "z_transposed":
            return F @ np.swapaxes(Z, -1, -2)
        if mode == "f_only":
            return F
        if mode == "full_fzb":
            Bm = O.softmax_rows(qt @ np.swapaxes(ks, -1, -2), valid)
            return F @ Z @ Bm
        if mode == "a_not_inverted":
            return F @ A
        return F @ Z
    return probs


def _module_factory(mode):
    def module(x, w_qkv, b_qkv, H, key_mask=None, conv_w=None, m=64, n_iter=6, init_option=0, return_qkv=False):
        x = np.asarray(x, np.float64)
        w = np.asarray(w_qkv, np.float64)
        B, n, _ = x.shape
        d = w.shape[0] // (3 * H)
        y = x @ w.T + (0 if b_qkv is None else np.asarray(b_qkv, np.float64))
        if mode == "heads_outer":
            qkv = y.reshape(B, n, H, 3, d).transpose(0, 1, 3, 2, 4)
        else:
            qkv = y.reshape(B, n, 3, H, d)
        q, k, v = (np.transpose(qkv[:, :, i], (0, 2, 1, 3)) for i in range(3))
        if mode == "k_v_swapped":
            k, v = v, k
        ctx = O.nystrom_attention(q, k, v, key_mask, conv_w, m, n_iter, init_option)
        if mode == "context_heads_inner":
            out = np.transpose(ctx, (0, 2, 3, 1)).reshape(B, n, H * d)
        else:
            out = np.transpose(ctx, (0, 2, 1, 3)).reshape(B, n, H * d)
        return (out, qkv) if return_qkv else out
    return module


MUTANTS = {
    "scale_double": ({"scale_qk": _scale_double}, ["scale", "exact_sdpa"]),
    "scale_q_only": ({"scale_qk": _scale_q_only}, ["scale"]),
    "segments_interleaved": ({"segment_means": _segments_interleaved}, ["segment_means_direct"]),
    "softmax_wrong_axis": ({"softmax_rows": _softmax_wrong_axis}, ["softmax_library"]),
    "mask_inverted": ({"softmax_rows": _softmax_mask_inverted}, ["softmax_library", "exact_sdpa"]),
    "zero_valid_nan": ({"softmax_rows": _softmax_no_guard}, ["path_zero_valid"]),
    "mask_ignored": ({"nystrom_kernels": _kernels_no_mask}, ["path_mask_semantics"]),
    "z0_no_transpose": ({"newton_schulz_pinv": _ns_factory(z0_transpose=False)}, ["pinv_spectral"]),
    "coef13_is_12": ({"newton_schulz_pinv": _ns_factory(c13=12.0)}, ["pinv_spectral", "pinv_residual_law", "pinv_diag_worked"]),
    "coef15_is_14": ({"newton_schulz_pinv": _ns_factory(c15=14.0)}, ["pinv_spectral"]),
    "coef7_is_6": ({"newton_schulz_pinv": _ns_factory(c7=6.0)}, ["pinv_spectral"]),
    "left_multiply": ({"newton_schulz_pinv": _ns_factory(right=False)}, ["pinv_spectral"]),
    "no_quarter": ({"newton_schulz_pinv": _ns_factory(quarter=1.0 / 3.0)}, ["pinv_spectral"]),
    "init_rows_twice": ({"init_scale": _init_factory("rows_twice")}, ["init_scale"]),
    "init_no_rowsum": ({"init_scale": _init_factory("no_rowsum")}, ["init_scale"]),
    "init_original_per_head": ({"init_scale": _init_factory("orig_per_head")}, ["init_scale"]),
    "init_exact_global": ({"init_scale": _init_factory("exact_global")}, ["init_scale"]),
    "conv_flipped": ({"depthwise_conv_same": _conv_flipped}, ["conv_library", "conv_delta"]),
    "conv_off_by_one": ({"depthwise_conv_same": _conv_off_by_one}, ["conv_delta", "conv_direct"]),
    "probs_z_transposed": ({"attention_probs": _probs_factory("z_transposed")}, ["probs_converged_inverse"]),
    "probs_f_only": ({"attention_probs": _probs_factory("f_only")},
                     ["probs_converged_inverse", "probs_output_consistency"]),
    "probs_full_fzb": ({"attention_probs": _probs_factory("full_fzb")},
                       ["probs_converged_inverse", "probs_output_consistency"]),
    "probs_a_not_inverted": ({"attention_probs": _probs_factory("a_not_inverted")},
                             ["probs_converged_inverse", "probs_output_consistency"]),
    "probs_exact_no_mask": ({"attention_probs": _probs_factory("exact_no_mask")}, ["probs_exact_bruteforce"]),
    "module_heads_outer": ({"self_attention": _module_factory("heads_outer")}, ["module_identity_projection"]),
    "module_k_v_swapped": ({"self_attention": _module_factory("k_v_swapped")}, ["module_identity_projection"]),
    "module_context_heads_inner": ({"self_attention": _module_factory("context_heads_inner")},
                                   ["module_identity_projection"]),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_mutant_is_caught(mutant, monkeypatch):
    patches, pins = MUTANTS[mutant]
    for name, fn in patches.items():
        monkeypatch.setattr(O, name, fn)
    caught = []
    for pin in pins:
        fn, tol = P.ALL_PINS[pin]
        with np.errstate(all="ignore"):
            try:
                err = fn(O)
            except Exception:  # a crash also counts as caught
                err = float("inf")
        if not (err < tol):
            caught.append(pin)
    assert caught, f"mutant {mutant} passed every pin in {pins}"


# ------------------------------------------------------ gradient oracle ---
def _grad_forward_c_detached(q, k, v, key_mask=None, conv_w=None, m=64, n_iter=6, init_option=0):
    """The differentiable forward with the initial scale c treated as a
    constant (a plausible slip: c comes from maxima)."""
    import torch

    from oracle import nystrom_grad as G
    B, H, n, d = q.shape
    s = d ** -0.25
    qs, ks = q * s, k * s
    valid = None if key_mask is None else torch.as_tensor(np.asarray(key_mask) != 0)[:, None, None, :]
    if m == n:
        attn = G.softmax_masked(qs @ ks.transpose(-1, -2), valid) @ v
    else:
        L = n // m
        qt = qs.reshape(B, H, m, L, d).mean(dim=-2)
        kt = ks.reshape(B, H, m, L, d).mean(dim=-2)
        F = torch.softmax(qs @ kt.transpose(-1, -2), dim=-1)
        A = torch.softmax(qt @ kt.transpose(-1, -2), dim=-1)
        Bm = G.softmax_masked(qt @ ks.transpose(-1, -2), valid)
        colsum, rowsum = A.sum(dim=-2), A.sum(dim=-1)
        if init_option == 0:
            c = (colsum.max() * rowsum.max()).reshape(1, 1, 1, 1)
        else:
            c = (colsum.max(dim=-1).values * rowsum.max(dim=-1).values)[..., None, None]
        c = c.detach()
        I = torch.eye(m, dtype=A.dtype)
        Z = A.transpose(-1, -2) / c
        for _ in range(n_iter):
            X = A @ Z
            Z = 0.25 * Z @ (13.0 * I - X @ (15.0 * I - X @ (7.0 * I - X)))
        attn = F @ (Z @ (Bm @ v))
    if conv_w is not None:
        attn = attn + G.depthwise_conv_same(v, conv_w)
    return attn


def _grad_softmax_no_mask(s, valid=None):
    import torch
    return torch.softmax(s, dim=-1)


def _grad_conv_flipped(v, w):
    from oracle import nystrom_grad as G
    return _REAL_GRAD_CONV(v, w.flip(-1))


_REAL_GRAD_CONV = None

GRAD_MUTANTS = {
    "grad_c_detached": ({"forward": _grad_forward_c_detached}, ["grad_finite_differences"]),
    "grad_mask_ignored": ({"softmax_masked": _grad_softmax_no_mask}, ["grad_forward", "grad_finite_differences"]),
    "grad_conv_flipped": ({"depthwise_conv_same": _grad_conv_flipped}, ["grad_forward"]),
}


@pytest.mark.parametrize("mutant", sorted(GRAD_MUTANTS))
def test_grad_mutant_is_caught(mutant, monkeypatch):
    global _REAL_GRAD_CONV
    from oracle import nystrom_grad as G
    _REAL_GRAD_CONV = G.depthwise_conv_same
    patches, pins = GRAD_MUTANTS[mutant]
    for name, fn in patches.items():
        monkeypatch.setattr(G, name, fn)
    caught = []
    for pin in pins:
        fn, tol = P.ALL_PINS[pin]
        with np.errstate(all="ignore"):
            try:
                err = fn(O)
            except Exception:  # a crash also counts as caught
                err = float("inf")
        if not (err < tol):
            caught.append(pin)
    assert caught, f"mutant {mutant} passed every pin in {pins}"
