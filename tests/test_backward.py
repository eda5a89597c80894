"""GPU parity of the backward pass (nystrom_attention_backward) against the
float64 autograd oracle (oracle/nystrom_grad.py, itself pinned by central
finite differences): dq, dk, dv per (batch, head) slice and dconv_w per
head, relative Frobenius error.

Tolerance: the gradients pass through the iteration run backwards, which
multiplies rounding errors by up to the conditioning of A, so they are
held to 1e-3 for float32 I/O (ten times the forward's bound) and 3e-2 for
bf16 I/O (whose forward products already round to bf16)."""
import numpy as np
import pytest

from efficient_transformer_attention_segment_amd.workloads import make_custom, round_bf16
from gpu_util import announce, to_dev

pytestmark = pytest.mark.gpu

GTOL = {"fp32": 1e-3, "bf16": 3e-2}


def rel_frob_floor(got, ref):
    """Max over (b, h) of ||got - ref||_F / ||ref||_F per [n, d] slice, with
    the denominator floored at 1e-6 of the largest slice norm: a slice whose
    exact gradient is zero up to float64 noise (a batch row with no kept key
    whose head gets no share of c) is compared in absolute terms."""
    num = np.sqrt(((got - ref) ** 2).sum(axis=(-1, -2)))
    den = np.sqrt((ref ** 2).sum(axis=(-1, -2)))
    return float((num / np.maximum(den, 1e-6 * den.max())).max())


def _dout(shape, seed, dtype):
    d = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    return round_bf16(d) if dtype == "bf16" else d


def _check(name, x, dtype, m, n_iter, init, conv=True, seed=0, zero_qk=False):
    """zero_qk: dq and dk are exactly zero (a single key: the softmax is the
    constant 1); they are then held to a small absolute bound instead."""
    import torch

    import efficient_transformer_attention_segment_amd as nys
    from oracle import nystrom_grad as G
    dout = _dout(x["q"].shape, 970 + seed, dtype)
    cw = x["conv_w"] if conv else None
    announce(f"backward {name} dtype={dtype} shape={x['q'].shape} m={m} n_iter={n_iter} init={init} conv={conv}")
    q, k, v, do = (to_dev(a, dtype) for a in (x["q"], x["k"], x["v"], dout))
    km = to_dev(x["key_mask"], None) if x.get("key_mask") is not None else None
    cwd = to_dev(cw, None) if cw is not None else None
    dq, dk, dv, dw = nys.attention_backward(q, k, v, do, km, cwd, m=m, n_iter=n_iter, init_option=init)
    torch.cuda.synchronize()
    got = [t.float().cpu().double().numpy() for t in (dq, dk, dv)]
    ref = G.gradients(x["q"], x["k"], x["v"], dout, x["key_mask"], cw, m, n_iter, init)
    errs = []
    for nm, g_, r_ in zip(("dq", "dk", "dv"), got, ref[:3]):
        assert np.isfinite(g_).all(), f"{name}: non-finite {nm}"
        if zero_qk and nm in ("dq", "dk"):
            assert np.abs(r_).max() < 1e-12 and np.abs(g_).max() < 1e-3, f"{name}: {nm} not ~0"
            continue
        errs.append((nm, rel_frob_floor(g_, r_)))
    if cw is not None:
        gw = dw.cpu().double().numpy()
        rw = ref[3]
        errs.append(("dconv_w", float(np.max(np.linalg.norm(gw - rw, axis=-1) / np.linalg.norm(rw, axis=-1)))))
    announce(f"backward {name}: " + ", ".join(f"{nm} {e:.3e}" for nm, e in errs))
    for nm, e in errs:
        assert e < GTOL[dtype], f"{name}: {nm} {e:.3e} >= {GTOL[dtype]:.0e}"


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("m,n", [(64, 256), (64, 1024), (50, 400), (128, 512), (32, 96), (96, 960),
                                 (256, 1024), (160, 640), (200, 600)])
def test_backward(dtype, m, n):
    """Both initialisations (option 0: the maximum column sum over every
    head), partial masks, the convolution, padded landmark counts, ragged
    tiles."""
    x = make_custom(2, 2, n, 64, seed=980 + m + n, dtype=dtype, lengths=[n, n - n // 3])
    _check(f"m{m}-n{n}", x, dtype, m, 6, 0, seed=1)
    _check(f"m{m}-n{n}-init1-noconv", x, dtype, m, 6, 1, conv=False, seed=2)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("n_iter", [0, 1, 12])
def test_backward_iterations(dtype, n_iter):
    x = make_custom(1, 3, 512, 64, seed=990 + n_iter, dtype=dtype, lengths=[400])
    _check(f"iter{n_iter}", x, dtype, 64, n_iter, 1, seed=3)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("n_iter", [0, 12])
def test_backward_iterations_many_landmarks(dtype, n_iter):
    """The launch-chain pseudo-inverse backward (above 64 landmarks) with no
    iteration and with twelve."""
    x = make_custom(1, 3, 1024, 64, seed=993 + n_iter, dtype=dtype, lengths=[900])
    _check(f"m128-iter{n_iter}", x, dtype, 128, n_iter, 0, seed=3)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_backward_many_heads_many_landmarks(dtype):
    """96 heads above 64 landmarks: every launch of the chain covers all
    heads, and init option 0 takes its maximum over all of them."""
    x = make_custom(8, 12, 512, 64, seed=1030, dtype=dtype, lengths=[512 - 37 * j for j in range(8)])
    _check("B8-H12-m128", x, dtype, 128, 6, 0, seed=9)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_backward_conv_sizes_and_empty_row(dtype):
    """Conv kernel sizes 1 and 33, and a batch row with no kept key."""
    for K in (1, 33):
        x = make_custom(2, 2, 256, 64, seed=995 + K, dtype=dtype, lengths=[256, 0], taps=K)
        _check(f"conv{K}-emptyrow", x, dtype, 64, 6, 0, seed=4)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("n", [64, 200, 512, 1])
def test_backward_exact_branch(dtype, n):
    """m == n (the pages' default configuration takes this branch): the
    softmax attention's gradients, with a partial mask, a batch row with no
    kept key and the convolution."""
    x = make_custom(2, 2, n, 64, seed=1000 + n, dtype=dtype, lengths=[max(1, n - n // 3), 0])
    _check(f"exact-n{n}", x, dtype, n, 6, 0, seed=5, zero_qk=n == 1)
    y = make_custom(1, 2, n, 64, seed=1001 + n, dtype=dtype, lengths=None)
    _check(f"exact-n{n}-nomask-noconv", y, dtype, n, 6, 0, conv=False, seed=6, zero_qk=n == 1)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("d,m,n", [(32, 64, 512), (32, 128, 512), (32, 50, 400), (32, 200, 200),
                                   (32, 256, 512), (32, 176, 528),
                                   (128, 64, 512), (128, 32, 96), (128, 50, 400), (128, 200, 200)])
def test_backward_head_sizes(dtype, d, m, n):
    """Head sizes 32 and 128: the Nystrom path (up to 256 landmarks at
    d = 32, up to 64 at d = 128; padded landmark counts) and the exact
    branch (m == n), with a partial mask and the convolution."""
    x = make_custom(2, 2, n, d, seed=1010 + d + m, dtype=dtype, lengths=[n, n - n // 3])
    _check(f"d{d}-m{m}-n{n}", x, dtype, m, 6, 0, seed=7)
    _check(f"d{d}-m{m}-n{n}-init1-noconv", x, dtype, m, 6, 1, conv=False, seed=8)


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_backward_workload(idx):
    """The workloads at their full sizes (workload 5: 256 landmarks over
    65536 tokens, the pages' long-sequence setting)."""
    from efficient_transformer_attention_segment_amd.workloads import WORKLOADS, make_inputs
    w = WORKLOADS[idx]
    x = make_inputs(w)
    _check(f"workload{idx}", x, w.dtype, w.m, w.n_iter, w.init_option, seed=10 + idx)


@pytest.mark.parametrize("m", [64, 128, 256])
def test_backward_deterministic(m):
    """Repeated calls give identical gradients (fixed reduction orders; above
    64 landmarks the launch chain, the side stream and, above 128, the key
    pass's first-half buffer)."""
    import torch

    import efficient_transformer_attention_segment_amd as nys
    n = max(512, 4 * m)
    x = make_custom(2, 2, n, 64, seed=999 + m, dtype="bf16", lengths=[n, (3 * n) // 5])
    do = to_dev(_dout(x["q"].shape, 5, "bf16"), "bf16")
    args = [to_dev(x[n_], "bf16") for n_ in ("q", "k", "v")]
    announce(f"backward deterministic m{m} n{n}")
    outs = [nys.attention_backward(*args, do, to_dev(x["key_mask"], None), to_dev(x["conv_w"], None), m=m)
            for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        for a_, b_ in zip(o, outs[0]):
            assert torch.equal(a_, b_)


@pytest.mark.parametrize("m", [64, 256])
def test_backward_user_streams(m):
    """Calls on two user streams (each with its own workspace; the library's
    side stream forks from and joins back into the calling stream) give the
    default stream's results bit for bit, with the calls of both streams in
    flight together."""
    import torch

    import efficient_transformer_attention_segment_amd as nys
    n = max(512, 4 * m)
    x = make_custom(2, 3, n, 64, seed=1020 + m, dtype="bf16", lengths=[n, (2 * n) // 3])
    do = to_dev(_dout(x["q"].shape, 6, "bf16"), "bf16")
    args = [to_dev(x[n_], "bf16") for n_ in ("q", "k", "v")]
    km, cw = to_dev(x["key_mask"], None), to_dev(x["conv_w"], None)
    announce(f"backward user streams m{m} n{n}")
    ref = nys.attention_backward(*args, do, km, cw, m=m)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for i in range(4):
        s = s1 if i % 2 == 0 else s2
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            outs.append(nys.attention_backward(*args, do, km, cw, m=m, stream=s))
    torch.cuda.synchronize()
    for o in outs:
        for a_, b_ in zip(o, ref):
            assert torch.equal(a_, b_)
