"""GPU parity: the HIP path against the float64 oracle on the same seeded
inputs, element by element (max relative Frobenius error per (batch, head)
slice).  Tolerances: 1e-4 for float32 I/O, 2e-2 for bf16 I/O with float32
accumulation.

Beyond the headline metric, every workload is also checked with the
convolution off (the attention term alone: in the long workloads the
convolution dominates the output norm and would hide a broken attention
path) and with 'peaked' inputs (q, k times 4, so the softmaxes are far from
uniform), at the same tolerances."""
import numpy as np
import pytest

from efficient_transformer_attention_segment_amd.workloads import WORKLOADS, make_inputs, make_custom
from gpu_util import TOL, announce, oracle_out, rel_frob_slices, run_gpu

pytestmark = pytest.mark.gpu


def _check(name, x, dtype, m, n_iter, init, conv=True, mask=True, tol=None, **okw):
    announce(f"{name} dtype={dtype} shape={x['q'].shape} m={m} n_iter={n_iter} init={init} conv={conv} mask={mask}")
    got = run_gpu(x, dtype, m, n_iter, init, conv=conv, mask=mask)
    assert np.isfinite(got).all(), f"{name}: non-finite output"
    ref = oracle_out(x, m, n_iter, init, conv=conv, mask=mask, **okw)
    per, whole = rel_frob_slices(got, ref)
    tol = TOL[dtype] if tol is None else tol
    announce(f"{name}: max rel Frobenius {per:.3e} (whole {whole:.3e}, tol {tol:.0e})")
    assert per < tol, f"{name}: {per:.3e} >= {tol:.0e}"
    return per


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_workload(idx):
    w = WORKLOADS[idx]
    x = make_inputs(w)
    _check(f"workload{idx}", x, w.dtype, w.m, w.n_iter, w.init_option)


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_workload_attention_only(idx):
    w = WORKLOADS[idx]
    x = make_inputs(w)
    _check(f"workload{idx}-noconv", x, w.dtype, w.m, w.n_iter, w.init_option, conv=False)


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_workload_peaked(idx):
    w = WORKLOADS[idx]
    x = make_inputs(w, qk_scale=4.0)
    _check(f"workload{idx}-peaked", x, w.dtype, w.m, w.n_iter, w.init_option, conv=False)


# Centred attention error: the attention term minus 1 vbar^T, vbar the mean
# of the batch row's kept V rows, i.e. what separates the computed attention
# from a uniform average.  In workloads 3-5 the softmaxes are nearly uniform
# (logit std 0.125, 0.022, 0.0625), so the attention-only output is mostly
# 1 vbar^T (the centred term is 1.8e-2, 1.9e-3 and 3.8e-3 of its norm) and
# its relative error alone would not see a wrong deviation from uniform.
# The bf16 output's own rounding (2^-9 of |out|) is already of the size of
# the centred term, so the gate is on what the kernels add beyond it: per
# (b, h) slice, with e the centred error of the GPU output and r that of
# the oracle output rounded to bf16 (RNE), the excess sqrt(max(e^2 - r^2, 0))
# estimates the centred error before the final rounding.  The gate is 5x the
# excess measured on MI355X with these kernels; an attention path with the
# wrong deviation from uniform has an excess near 1.
CENTRED_EXCESS_MEASURED = {3: 2.83e-2, 4: 1.82e-1, 5: 9.49e-2}


def _centred(o, x, mask):
    v = x["v"].astype(np.float64)
    if mask and x.get("key_mask") is not None:
        keep = x["key_mask"].astype(np.float64)[:, None, :, None]
    else:
        keep = np.ones(v.shape[:1] + (1,) + v.shape[2:3] + (1,))
    vbar = (v * keep).sum(axis=2, keepdims=True) / keep.sum(axis=2, keepdims=True)
    return o - vbar


def _slice_rel(a, b):
    num = np.sqrt(((a - b) ** 2).sum(axis=(-1, -2)))
    return num / np.sqrt((b ** 2).sum(axis=(-1, -2)))


@pytest.mark.parametrize("idx", [3, 4, 5])
def test_workload_centred_attention(idx):
    import torch
    w = WORKLOADS[idx]
    x = make_inputs(w)
    announce(f"workload{idx}-centred dtype={w.dtype}")
    got = run_gpu(x, w.dtype, w.m, w.n_iter, w.init_option, conv=False)
    ref = oracle_out(x, w.m, w.n_iter, w.init_option, conv=False)
    rounded = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
    cref = _centred(ref, x, True)
    e = _slice_rel(_centred(got, x, True), cref)
    r = _slice_rel(_centred(rounded, x, True), cref)
    excess = float(np.sqrt(np.maximum(e ** 2 - r ** 2, 0.0)).max())
    gate = 5.0 * CENTRED_EXCESS_MEASURED[idx]
    announce(f"workload{idx}-centred: max error {e.max():.3e}, rounding floor {r.max():.3e}, "
             f"excess {excess:.3e} (gate {gate:.2e})")
    assert excess < gate


# ------------------------------------------------------------- edge cases ---
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("n", [256, 100, 1, 33])
def test_exact_branch(dtype, n):
    """m == n: exact softmax attention (+ conv), including ragged n."""
    lengths = [n, max(1, n // 2)]
    x = make_custom(2, 3, n, 64, seed=500 + n, dtype=dtype, lengths=lengths)
    _check(f"exact-n{n}", x, dtype, n, 6, 0)
    _check(f"exact-n{n}-noconv", x, dtype, n, 6, 0, conv=False)


@pytest.mark.parametrize("dtype,m,n", [
    ("fp32", 32, 64), ("fp32", 32, 160), ("fp32", 96, 192), ("fp32", 128, 512),
    ("bf16", 32, 64), ("bf16", 96, 480), ("bf16", 128, 384), ("bf16", 160, 320),
    ("bf16", 192, 768), ("bf16", 224, 448), ("bf16", 256, 1024),
])
def test_landmark_counts(dtype, m, n):
    """Every landmark count built, short segments (L = 2 .. 5), ragged
    output tiles (n not a multiple of 128)."""
    x = make_custom(2, 2, n, 64, seed=700 + m + n, dtype=dtype, lengths=[n, n - n // 4])
    _check(f"m{m}-n{n}", x, dtype, m, 6, 0)
    _check(f"m{m}-n{n}-init1-noconv", x, dtype, m, 6, 1, conv=False)


@pytest.mark.parametrize("dtype,m,n", [
    ("fp32", 16, 256), ("fp32", 7, 224), ("fp32", 100, 400), ("fp32", 1, 64), ("fp32", 5, 200),
    ("fp32", 160, 640), ("fp32", 200, 800), ("fp32", 256, 1024), ("fp32", 150, 450),
    ("bf16", 48, 480), ("bf16", 50, 400), ("bf16", 144, 576), ("bf16", 200, 1000), ("bf16", 3, 96),
    ("bf16", 11, 440),
])
def test_unpadded_landmark_counts(dtype, m, n):
    """Landmark counts that are not multiples of 32 (padded inside to the
    next one with landmarks that take no weight): multiples of 16, odd
    counts, a single landmark; and with them sequence lengths that are not
    multiples of 32 or 16 (a ragged last key tile and output tile)."""
    x = make_custom(2, 2, n, 64, seed=720 + m + n, dtype=dtype, lengths=[n, n - n // 4])
    _check(f"m{m}-n{n}", x, dtype, m, 6, 0)
    _check(f"m{m}-n{n}-init1-noconv", x, dtype, m, 6, 1, conv=False)
    y = make_custom(1, 3, n, 64, seed=721 + m + n, dtype=dtype, scale=4.0, lengths=None)
    _check(f"m{m}-n{n}-peaked", y, dtype, m, 6, 0, conv=False)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("ksize", [1, 3, 7, 33, 63])
def test_conv_kernel_sizes(dtype, ksize):
    """The conv_kernel_size argument (odd, up to 65) on both branches: the
    Nystrom path (output kernels) and the exact branch."""
    x = make_custom(2, 2, 512, 64, seed=740 + ksize, dtype=dtype, lengths=[512, 300], taps=ksize)
    assert x["conv_w"].shape == (2, ksize)
    _check(f"conv{ksize}", x, dtype, 64, 6, 0)
    y = make_custom(1, 2, 200, 64, seed=741 + ksize, dtype=dtype, lengths=[150], taps=ksize)
    _check(f"conv{ksize}-exact", y, dtype, 200, 6, 0)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("d", [32, 128])
@pytest.mark.parametrize("m,n", [(64, 1024), (50, 400), (128, 512), (200, 1000), (256, 2048), (100, 100),
                                 (32, 96)])
def test_head_sizes(dtype, d, m, n):
    """Head sizes 32 and 128 (the d = 64 instances are tuned separately):
    padded and unpadded landmark counts, both pseudo-inverse paths (up to
    128 landmarks fused, above in separate launches), ragged tiles, the
    exact branch; both initialisations, with and without the convolution."""
    x = make_custom(2, 3, n, d, seed=760 + d + m + n, dtype=dtype, lengths=[n, n - n // 3])
    _check(f"d{d}-m{m}-n{n}", x, dtype, m, 6, 0)
    _check(f"d{d}-m{m}-n{n}-init1-noconv", x, dtype, m, 6, 1, conv=False)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("d", [32, 128])
def test_head_sizes_peaked(dtype, d):
    """Larger logits at both head sizes, and 12 iterations."""
    x = make_custom(1, 2, 1024, d, seed=790 + d, dtype=dtype, scale=3.0)
    _check(f"d{d}-peaked", x, dtype, 64, 12, 1, conv=False)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("m,n", [(64, 512), (50, 400), (200, 200), (20, 100)])
def test_strided_layouts(dtype, d, m, n):
    """q, k, v read straight out of a fused [B, n, 3, H, d] projection and
    out written as [B, n, H, d] (the module's layouts), through strided
    views: the same result as the dense call."""
    import torch

    import efficient_transformer_attention_segment_amd as nys
    from gpu_util import to_dev
    B, H = 2, 3
    x = make_custom(B, H, n, d, seed=750 + m + n + d, dtype=dtype, lengths=[n, n - n // 3])
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    qkv = torch.empty(B, n, 3, H, d, dtype=tdt, device="cuda")
    for i, name in enumerate(("q", "k", "v")):
        qkv[:, :, i] = torch.from_numpy(x[name]).to("cuda").to(tdt).permute(0, 2, 1, 3)
    q, k, v = (qkv[:, :, i].permute(0, 2, 1, 3) for i in range(3))
    out_buf = torch.full((B, n, H * d), float("nan"), dtype=tdt, device="cuda")
    out = out_buf.view(B, n, H, d).permute(0, 2, 1, 3)
    announce(f"strided dtype={dtype} d={d} m={m} n={n} q.stride={q.stride()} out.stride={out.stride()}")
    nys.attention(q, k, v, to_dev(x["key_mask"], None), to_dev(x["conv_w"], None), m=m, n_iter=6, init_option=0,
                  out=out)
    torch.cuda.synchronize()
    got = out.float().cpu().double().numpy()
    assert np.isfinite(got).all()
    per, _ = rel_frob_slices(got, oracle_out(x, m, 6, 0))
    announce(f"strided: max rel Frobenius {per:.3e}")
    assert per < TOL[dtype]
    dense = run_gpu(x, dtype, m, 6, 0)
    assert np.array_equal(got, dense), "strided and dense calls differ"


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_many_heads(dtype):
    """More (batch, head) pairs than the fused Gram rendezvous allows (the
    original init then takes the separate Gram launch), ragged masks, both
    inits."""
    x = make_custom(3, 48, 128, 64, seed=760, dtype=dtype, lengths=[128, 70, 1])
    _check("heads144-init0", x, dtype, 32, 6, 0)
    _check("heads144-init1", x, dtype, 32, 6, 1)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("n_iter", [0, 1, 2, 12])
def test_iteration_counts(dtype, n_iter):
    x = make_custom(2, 2, 512, 64, seed=800 + n_iter, dtype=dtype, lengths=[512, 300])
    for init in (0, 1):
        _check(f"niter{n_iter}-init{init}", x, dtype, 64, n_iter, init, conv=False)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("m", [128, 256])
@pytest.mark.parametrize("n_iter", [0, 1, 8, 9])
def test_iteration_counts_many_landmarks(dtype, m, n_iter):
    """Every pseudo-inverse path at 128 and 256 landmarks: at bf16 I/O the
    fp16 iteration up to 8 steps and the split-bf16 one from 9 (in LDS at
    m = 128, the launch chains above 128), at float32 I/O the float32 ones,
    and n_iter = 0 (Z = A^T / c) on each; the original init with a ragged
    mask."""
    x = make_custom(1, 2, 4 * m, 64, seed=810 + m + n_iter, dtype=dtype, lengths=[4 * m - 100])
    _check(f"niter{n_iter}-m{m}", x, dtype, m, n_iter, 0, conv=False)


@pytest.mark.parametrize("B,H,m,n", [(1, 1, 256, 1024), (1, 3, 160, 640), (2, 3, 192, 768), (3, 3, 224, 448)])
def test_head_counts_many_landmarks(B, H, m, n):
    """Above 128 landmarks (bf16, d = 64) the B V launch forms A by row
    blocks in its first workgroups and the chain places a head's tiles on
    one XCD, or on two with at most four heads: one head, three, six and
    nine (two groups of eight XCDs), an odd row-block count (m = 160, 224)."""
    x = make_custom(B, H, n, 64, seed=830 + B * H + m, dtype="bf16", lengths=[n - 7 * b for b in range(B)])
    _check(f"B{B}H{H}-m{m}", x, "bf16", m, 6, 0)
    _check(f"B{B}H{H}-m{m}-init1", x, "bf16", m, 6, 1, conv=False)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_zero_valid_keys(dtype):
    """A batch row with every key masked: B V = 0, output = conv(V), no NaN."""
    x = make_custom(2, 2, 256, 64, seed=901, dtype=dtype, lengths=[256, 0])
    _check("zero-valid", x, dtype, 64, 6, 0)
    from oracle import nystrom_oracle as O
    got = run_gpu(x, dtype, 64, 6, 0)
    conv = O.depthwise_conv_same(np.float64(x["v"]), x["conv_w"])
    per, _ = rel_frob_slices(got[1:], conv[1:])
    assert per < TOL[dtype]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_no_mask_no_conv(dtype):
    x = make_custom(3, 2, 512, 64, seed=902, dtype=dtype, lengths=None, conv=False)
    _check("plain", x, dtype, 64, 6, 0, conv=False, mask=False)


def test_init_scope_matters():
    """The default init takes its maxima over every head of the call: a head
    whose A differs from the others changes the result of the other heads
    (and both readings are distinguishable at the float32 tolerance)."""
    x = make_custom(2, 2, 256, 64, seed=903, dtype="fp32", lengths=None, conv=False)
    x["q"][0, 0] *= 6.0
    x["k"][0, 0] *= 6.0
    got = run_gpu(x, "fp32", 64, 6, 0, conv=False)
    ref0 = oracle_out(x, 64, 6, 0, conv=False)
    ref1 = oracle_out(x, 64, 6, 1, conv=False)
    e0, _ = rel_frob_slices(got, ref0)
    e1, _ = rel_frob_slices(got, ref1)
    assert e0 < 1e-4 and e1 > 1e-3


def test_deterministic():
    """Repeated calls give bit-identical results (no float atomics)."""
    w = WORKLOADS[2]
    x = make_inputs(w)
    a = run_gpu(x, w.dtype, w.m, w.n_iter, w.init_option)
    for _ in range(3):
        b = run_gpu(x, w.dtype, w.m, w.n_iter, w.init_option)
        assert np.array_equal(a, b)


def test_shape_changes_reuse_workspace():
    """Calls of different shapes back to back on one stream stay correct
    (the cached workspace grows and the arrival counters stay consistent)."""
    cases = [(1, 2, 256, 64), (4, 6, 1024, 128), (1, 2, 256, 64), (2, 3, 512, 32)]
    for i, (B, H, n, m) in enumerate(cases):
        x = make_custom(B, H, n, 64, seed=950 + i, dtype="fp32", lengths=[n] * B)
        _check(f"reuse{i}", x, "fp32", m, 6, i % 2)


def test_side_stream_and_error_leaves_out_untouched():
    import torch

    import efficient_transformer_attention_segment_amd as nys
    from gpu_util import to_dev
    x = make_custom(1, 2, 256, 64, seed=960, dtype="fp32", lengths=[200])
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        got = run_gpu(x, "fp32", 64, 6, 0, stream=s)
    ref = oracle_out(x, 64, 6, 0)
    assert rel_frob_slices(got, ref)[0] < 1e-4
    q, k, v = (to_dev(x[n], "fp32") for n in ("q", "k", "v"))
    out = torch.full_like(q, 7.0)
    with pytest.raises(nys.NystromError) as ei:
        nys.nystrom_attention(q, k, v, None, None, m=48, out=out)   # n % m != 0
    assert ei.value.code == nys.NYS_ERR_INVALID
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
