"""GPU parity of the self-attention module (nystrom_self_attention: the
stacked q/k/v projection as one library GEMM, then the attention reading
q, k, v in place from its [B, n, 3, H, d] output and writing [B, n, H d])
against the float64 oracle's module.

For bf16 with d = 64, a landmark count that is a multiple of 32 and
segments of L = n / m tokens with L dividing 64, the projection also forms
the landmarks in its epilogue and the landmark pass is skipped.  Those sums
are the same bf16 values added in another float32 order, so there the module
is compared with the core on its own projection to FOLD_TOL instead of bit
for bit: a last-place difference in a landmark can flip one bf16 rounding
of an operand (2^-9 relative), far below the oracle tolerance."""
import numpy as np
import pytest

from efficient_transformer_attention_segment_amd.workloads import make_module_inputs
from gpu_util import TOL, announce, rel_frob_slices, to_dev

pytestmark = pytest.mark.gpu


FOLD_TOL = 2e-3  # module against the core on the same projection, when the landmarks are folded


def _folds(dtype, n, d, m):
    """Whether the module forms the landmarks in the projection's epilogue."""
    L = n // m
    return dtype == "bf16" and d == 64 and m != n and m % 32 == 0 and n % m == 0 and L >= 2 and 64 % L == 0


def _run(inp, dtype, m, n_iter, init, conv=True):
    import torch

    import efficient_transformer_attention_segment_amd as nys
    x, w = to_dev(inp["x"], dtype), to_dev(inp["w_qkv"], dtype)
    b = to_dev(inp["b_qkv"], dtype) if inp["b_qkv"] is not None else None
    km = to_dev(inp["key_mask"], None) if inp["key_mask"] is not None else None
    cw = to_dev(inp["conv_w"], None) if conv else None
    out, qkv = nys.self_attention(x, w, b, inp["H"], km, cw, m=m, n_iter=n_iter, init_option=init)
    # the core called on views of the same projection: the module adds no arithmetic of its own
    q, k, v = (qkv[:, :, i].permute(0, 2, 1, 3) for i in range(3))
    ref_core = nys.attention(q, k, v, km, cw, m=m, n_iter=n_iter, init_option=init)
    torch.cuda.synchronize()
    core = ref_core.permute(0, 2, 1, 3).reshape(out.shape)
    B, n = out.shape[:2]
    if _folds(dtype, n, q.shape[-1], m):
        per, _ = rel_frob_slices(out.float().cpu().double().numpy().reshape(B, n, inp["H"], -1),
                                 core.float().cpu().double().numpy().reshape(B, n, inp["H"], -1))
        announce(f"module (landmarks in the projection) against the core: {per:.3e}")
        assert per < FOLD_TOL, f"module differs from the core on its own projection: {per:.3e}"
    else:
        assert torch.equal(out, core), "module output differs from the core on its own projection"
    return out.float().cpu().double().numpy(), qkv.float().cpu().double().numpy()


def _check(name, inp, dtype, m, n_iter=6, init=0, conv=True):
    from oracle import nystrom_oracle as O
    announce(f"module {name} dtype={dtype} x={inp['x'].shape} H={inp['H']} m={m} init={init}")
    out, qkv = _run(inp, dtype, m, n_iter, init, conv)
    assert np.isfinite(out).all()
    ref, ref_qkv = O.self_attention(inp["x"], inp["w_qkv"], inp["b_qkv"], inp["H"], inp["key_mask"],
                                    inp["conv_w"] if conv else None, m, n_iter, init, return_qkv=True)
    B, n = out.shape[:2]
    # per (batch, head) slices of the context and of each projection
    per, whole = rel_frob_slices(out.reshape(B, n, inp["H"], -1).transpose(0, 2, 1, 3),
                                 ref.reshape(B, n, inp["H"], -1).transpose(0, 2, 1, 3))
    pq, _ = rel_frob_slices(qkv.reshape(B, n, -1, qkv.shape[-1]).transpose(0, 2, 1, 3),
                            ref_qkv.reshape(B, n, -1, qkv.shape[-1]).transpose(0, 2, 1, 3))
    announce(f"module {name}: out {per:.3e} (whole {whole:.3e}), projection {pq:.3e}")
    assert pq < TOL[dtype] / 4, f"{name}: projection {pq:.3e}"
    assert per < TOL[dtype], f"{name}: {per:.3e} >= {TOL[dtype]:.0e}"


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("B,n,hidden,H,d,m", [(2, 512, 768, 12, 64, 64), (1, 1024, 256, 4, 64, 128),
                                              (2, 400, 96, 2, 64, 50), (1, 200, 128, 2, 64, 200),
                                              (3, 96, 64, 1, 64, 32), (2, 512, 256, 8, 32, 64),
                                              (1, 512, 512, 4, 128, 64), (1, 256, 256, 2, 128, 256)])
def test_module(dtype, B, n, hidden, H, d, m):
    """The pages' module shape (hidden 768, 12 heads), other widths and head
    counts, head sizes 32 and 128, a landmark count that pads, and the exact
    branch (m == n)."""
    lengths = [n - (n // 4) * (i % 2) for i in range(B)]
    inp = make_module_inputs(B, n, hidden, H, d, seed=900 + n + hidden + d, dtype=dtype, lengths=lengths)
    _check(f"B{B}-n{n}-h{hidden}-H{H}-d{d}-m{m}", inp, dtype, m)
    nob = make_module_inputs(B, n, hidden, H, d, seed=901 + n + d, dtype=dtype, lengths=None, bias=False)
    _check(f"B{B}-n{n}-h{hidden}-H{H}-d{d}-m{m}-nobias-init1", nob, dtype, m, init=1, conv=False)


@pytest.mark.parametrize("init", [0, 1])
@pytest.mark.parametrize("L,B,m,H,hidden", [(2, 2, 32, 3, 96), (4, 1, 64, 2, 128), (8, 2, 32, 3, 192),
                                             (16, 1, 32, 5, 64), (32, 2, 32, 2, 256), (64, 1, 64, 3, 128),
                                             (64, 2, 32, 1, 64)])
def test_module_landmark_fold(L, B, m, H, hidden, init):
    """bf16 shapes where the projection forms the landmarks, at every
    segment length it takes (2 .. 64), odd head counts (a 128-column tile
    holding the last q head and the first k head), a padded key mask, and
    both inits (init 0's meeting slots are cleared by the projection)."""
    n = m * L
    lengths = [n - (n // 4) * (i % 2) for i in range(B)]
    inp = make_module_inputs(B, n, hidden, H, 64, seed=960 + L + m + H, dtype="bf16", lengths=lengths)
    assert _folds("bf16", n, 64, m)
    _check(f"fold-L{L}-B{B}-n{n}-h{hidden}-H{H}-m{m}", inp, "bf16", m, init=init)


def test_module_headline_size():
    """bf16, B 4, n 4096, hidden 768, 12 heads, 64 landmarks: the headline
    attention shape behind its projection."""
    inp = make_module_inputs(4, 4096, 768, 12, 64, seed=950, dtype="bf16", lengths=[3072, 4096, 3500, 4000])
    _check("headline", inp, "bf16", 64)


def test_module_rejects_overlap():
    """A qkv buffer overlapping x is rejected before the GEMM is enqueued."""
    import torch

    import efficient_transformer_attention_segment_amd as nys
    B, n, hidden, H = 1, 256, 64, 1
    buf = torch.randn(B * n * max(hidden, 3 * H * 64) * 2, device="cuda")
    x = buf[: B * n * hidden].view(B, n, hidden)
    w = torch.randn(3 * H * 64, hidden, device="cuda")
    qkv = buf[: B * n * 3 * H * 64].view(B, n, 3, H, 64)
    before = buf.clone()
    with pytest.raises(nys.NystromError):
        nys.self_attention(x, w, None, H, m=64, qkv=qkv)
    torch.cuda.synchronize()
    assert torch.equal(buf, before)
