"""The float64 oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle_pins as P
from oracle import nystrom_oracle as O


@pytest.mark.parametrize("name", sorted(P.ALL_PINS))
def test_pin(name):
    fn, tol = P.ALL_PINS[name]
    err = fn(O)
    assert err < tol, f"{name}: error {err:.3e} >= {tol:.0e}"


def test_rejects_bad_shapes():
    q = np.zeros((1, 1, 10, 4))
    with pytest.raises(ValueError):
        O.nystrom_attention(q, q, q, None, None, m=3)   # n % m != 0
    with pytest.raises(ValueError):
        O.nystrom_attention(q, q, q, None, None, m=20)  # m > n
    with pytest.raises(ValueError):
        O.nystrom_attention(q, q, q, None, None, m=5, n_iter=-1)
    with pytest.raises(ValueError):
        O.nystrom_attention(q, q, q, None, None, m=5, init_option=2)


def test_workload_stats_small():
    """The small fp32 workload runs and is finite; its logit spreads follow
    the iid-normal estimates (std sigma^2/sqrt(L) for F and B, sigma^2/L
    for A)."""
    from efficient_transformer_attention_segment_amd.workloads import make_inputs, WORKLOADS
    w = WORKLOADS[1]
    x = make_inputs(w)
    out, st = O.nystrom_attention(x["q"], x["k"], x["v"], x["key_mask"], x["conv_w"],
                                  w.m, w.n_iter, w.init_option, return_stages=True)
    assert np.isfinite(out).all()
    qs, ks = O.scale_qk(np.float64(x["q"]), np.float64(x["k"]))
    la = st["qt"] @ np.swapaxes(st["kt"], -1, -2)
    lf = qs @ np.swapaxes(st["kt"], -1, -2)
    L = w.n // w.m
    assert 0.7 < la.std() * L < 1.4
    assert 0.7 < lf.std() * np.sqrt(L) < 1.4


def test_oracle_regression_fixture():
    """The oracle still reproduces its stored outputs (tests/golden)."""
    import json, os
    from efficient_transformer_attention_segment_amd.workloads import make_custom
    path = os.path.join(os.path.dirname(__file__), "golden", "oracle_regression.json")
    data = json.load(open(path))
    for c in data["cases"]:
        x = make_custom(c["B"], c["H"], c["n"], c["d"], c["seed"], lengths=c["lengths"])
        o = O.nystrom_attention(x["q"], x["k"], x["v"], x["key_mask"], x["conv_w"],
                                c["m"], c["n_iter"], c["init_option"])
        for idx, val in c["samples"]:
            assert abs(o[tuple(idx)] - val) <= 1e-12 * max(1.0, abs(val))
        fro = [np.linalg.norm(o[b, h]) for b in range(c["B"]) for h in range(c["H"])]
        np.testing.assert_allclose(fro, c["fro"], rtol=1e-12)
