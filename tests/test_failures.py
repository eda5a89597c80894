"""Failure handling: the bounded rendezvous of the original init reports a
timeout to the host, a workspace that cannot be had fails the call before
anything is enqueued, and NaN inputs give NaN outputs without a hang.

Each failure is forced from the host (a poll bound of 0, a workspace cap),
so every kernel still exits normally."""
import numpy as np
import pytest

from gpu_util import announce, to_dev

pytestmark = pytest.mark.gpu


def _inputs(dtype="fp32", B=1, H=2, n=256, seed=5):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((B, H, n, 64), dtype=np.float32) for _ in range(3))
    w = (0.02 * rng.standard_normal((H, 65))).astype(np.float32)
    return [to_dev(x, dtype) for x in (q, k, v)] + [to_dev(w, None)]


def test_rendezvous_timeout_is_reported():
    """With the poll bound at 0 every pseudo-inverse block of the original
    init gives up at once: the output is NaN, the call itself returns OK
    (it is asynchronous), and the status check raises; a second check is
    clean, and with the default bound the same call is correct again."""
    import torch

    import efficient_transformer_attention_segment_amd as nys
    announce("failures: rendezvous timeout B1 H2 n256 m64 init 0")
    q, k, v, w = _inputs()
    good = nys.attention(q, k, v, None, w, m=64, n_iter=6, init_option=0)
    nys.check_status()
    try:
        nys.debug_set_rendezvous_spins(0)
        bad = nys.attention(q, k, v, None, w, m=64, n_iter=6, init_option=0)
        with pytest.raises(nys.NystromError) as e:
            nys.check_status()
        assert e.value.code == nys.NYS_ERR_HIP
        assert "rendezvous" in str(e.value)
        assert torch.isnan(bad).all()
        nys.check_status()  # the record was cleared by the check
        # the exact-coefficient init has no rendezvous: unaffected
        ok1 = nys.attention(q, k, v, None, w, m=64, n_iter=6, init_option=1)
        nys.check_status()
        assert torch.isfinite(ok1).all()
    finally:
        nys.debug_set_rendezvous_spins(1 << 20)
    again = nys.attention(q, k, v, None, w, m=64, n_iter=6, init_option=0)
    nys.check_status()
    torch.cuda.synchronize()
    assert torch.equal(again, good)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_workspace_cap_fails_before_launch(dtype):
    """A call whose workspace exceeds the cap returns NYS_ERR_HIP and leaves
    out untouched; without the cap the same call succeeds."""
    import torch

    import efficient_transformer_attention_segment_amd as nys
    announce(f"failures: workspace cap {dtype}")
    q, k, v, w = _inputs(dtype)
    side = torch.cuda.Stream()
    out = torch.full_like(q, 7.0)
    try:
        nys.debug_set_workspace_cap(4096)
        with pytest.raises(nys.NystromError) as e:
            nys.attention(q, k, v, None, w, m=64, out=out, stream=side)
        assert e.value.code == nys.NYS_ERR_HIP and "cap" in str(e.value)
        # the backward pass has the same guard
        with pytest.raises(nys.NystromError):
            nys.attention_backward(q, k, v, q, None, w, m=64, stream=side)
    finally:
        nys.debug_set_workspace_cap(0)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    nys.attention(q, k, v, None, w, m=64, out=out, stream=side)
    side.synchronize()
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("m", [64, 256])
def test_nan_input_gives_nan_output(dtype, m):
    """A NaN in one head's q reaches that head's output (every token: the
    landmark it enters feeds F, A and B) and no other head's (exact-coefficient
    init, so heads share nothing); the call returns and the stream drains."""
    import torch

    import efficient_transformer_attention_segment_amd as nys
    announce(f"failures: NaN input {dtype} m{m}")
    q, k, v, w = _inputs(dtype, B=1, H=3, n=1024)
    clean = nys.attention(q, k, v, None, w, m=m, init_option=1)
    qn = q.clone()
    qn[0, 1, 100, 5] = float("nan")
    got = nys.attention(qn, k, v, None, w, m=m, init_option=1)
    nys.check_status()
    torch.cuda.synchronize()
    assert torch.isnan(got[0, 1]).any()
    assert torch.equal(got[0, 0], clean[0, 0]) and torch.equal(got[0, 2], clean[0, 2])
