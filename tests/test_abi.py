"""The C ABI: the library loads, exports what include/nystrom.h declares,
and rejects bad arguments on the host before anything is launched (so these
run without a GPU: no call here reaches a kernel)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nystrom.h")


@pytest.fixture(scope="module")
def lib():
    import efficient_transformer_attention_segment_amd as nys
    if not os.path.exists(nys.library_path):
        from efficient_transformer_attention_segment_amd import build
        build.build()
    return nys._load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nystrom_\w+)\s*\(", text)))


def test_header_declares_entry_points():
    names = declared_functions()
    for n in ("nystrom_attention", "nystrom_attention_bf16", "nystrom_workspace_bytes",
              "nystrom_last_error", "nystrom_release", "nystrom_debug_stages"):
        assert n in names


def test_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in nystrom.h but not exported"


def test_dynamic_symbols_are_c_names():
    """The entry points are exported unmangled (extern "C")."""
    import subprocess
    import efficient_transformer_attention_segment_amd as nys
    out = subprocess.run(["nm", "-D", "--defined-only", nys.library_path], capture_output=True,
                         text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported


FAKE = ctypes.c_void_p(0x100000)   # never dereferenced: validation fails first
FAKE2 = ctypes.c_void_p(0x900000)
NULL = None


def call(lib, fn="nystrom_attention", q=FAKE, k=FAKE, v=FAKE, out=FAKE2, B=1, H=2, n=256, d=64,
         m=64, n_iter=6, init=0):
    f = getattr(lib, fn)
    return f(q, k, v, NULL, NULL, B, H, n, d, m, n_iter, init, out, NULL)


@pytest.mark.parametrize("fn", ["nystrom_attention", "nystrom_attention_bf16"])
@pytest.mark.parametrize("kw,code", [
    (dict(q=NULL), -1), (dict(k=NULL), -1), (dict(v=NULL), -1), (dict(out=NULL), -1),
    (dict(B=0), -1), (dict(H=-1), -1), (dict(n=0), -1), (dict(d=0), -1), (dict(m=0), -1),
    (dict(n=250), -1),                 # n % m != 0
    (dict(m=512), -1),                 # m > n
    (dict(n_iter=-1), -1),
    (dict(init=2), -1),
    (dict(out=FAKE), -1),              # out aliases q, k, v
    (dict(d=48, n=256), -2),           # head sizes 32, 64, 128 are built
    (dict(d=256, n=256), -2),
    (dict(m=512, n=1024), -2),         # m above 256 (and not n)
    (dict(B=300, H=300), -2),          # B*H above the grid limit
])
def test_invalid_arguments(lib, fn, kw, code):
    rc = call(lib, fn, **kw)
    assert rc == code
    assert lib.nystrom_last_error().decode() != ""


@pytest.mark.parametrize("fn", ["nystrom_attention_conv", "nystrom_attention_bf16_conv"])
@pytest.mark.parametrize("ksize,code", [(4, -1), (0, -1), (-3, -1), (67, -2), (129, -2)])
def test_conv_kernel_size_validation(lib, fn, ksize, code):
    """Odd kernel sizes 1 .. 65 only; checked on the host before any launch
    (every other argument here is valid, so only this check can fail)."""
    f = getattr(lib, fn)
    rc = f(FAKE, FAKE, FAKE, NULL, FAKE, ksize, 1, 2, 256, 64, 64, 6, 0, FAKE2, NULL)
    assert rc == code
    assert "conv_kernel_size" in lib.nystrom_last_error().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), -1),
    (dict(ist=60), -1),                  # bf16 token rows of 120 bytes: not 16-byte aligned
    (dict(ost=32), -1),                  # out rows overlap
    (dict(ob=0, oh=0), -1),              # every (batch, head) writes the same rows
    (dict(out=FAKE), -1),                # out is q
    (dict(q=ctypes.c_void_p(0x100008)), -1),   # misaligned pointer
])
def test_strided_validation(lib, kw, code):
    """nystrom_attention_ex rejects unaligned or self-overlapping layouts
    on the host (everything else valid, so nothing is launched)."""
    B, H, n = 1, 2, 256
    a = dict(dtype=1, q=FAKE, k=FAKE, v=FAKE, ib=H * n * 64, ih=n * 64, ist=64, out=FAKE2,
             ob=H * n * 64, oh=n * 64, ost=64)
    a.update(kw)
    rc = lib.nystrom_attention_ex(a["dtype"], a["q"], a["k"], a["v"], a["ib"], a["ih"], a["ist"], NULL, NULL, 65,
                                  B, H, n, 64, 64, 6, 0, a["out"], a["ob"], a["oh"], a["ost"], NULL)
    assert rc == code
    assert lib.nystrom_last_error().decode() != ""


@pytest.mark.parametrize("probs", [None, FAKE, FAKE2, ctypes.c_void_p(0x500008), ctypes.c_void_p(0x11fff0)])
def test_probs_validation(lib, probs):
    """nystrom_attention_probs rejects a NULL, misaligned or overlapping
    weights buffer (q, k, v at FAKE, out at FAKE2) before any launch."""
    B, H, n = 1, 2, 256
    rc = lib.nystrom_attention_probs(0, FAKE, FAKE, FAKE, H * n * 64, n * 64, 64, NULL, NULL, 65, B, H, n, 64, 64,
                                     6, 0, FAKE2, H * n * 64, n * 64, 64, probs, NULL)
    assert rc == -1
    assert "probs" in lib.nystrom_last_error().decode()


FAKE3 = ctypes.c_void_p(0x1100000)
FAKE4 = ctypes.c_void_p(0x1900000)
FAKE5 = ctypes.c_void_p(0x2100000)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), -1),
    (dict(dq=None), -1),
    (dict(dv=None), -1),
    (dict(dq=FAKE), -1),                      # dq is q
    (dict(dk=FAKE3), -1),                     # dk is dq
    (dict(dv=ctypes.c_void_p(0x2100008)), -1),  # misaligned
    (dict(d=48), -2),                         # head size not built
    (dict(d=128, m=128), -2),                 # more than 64 landmarks at d = 128
    (dict(d=128, m=80, n=480), -2),           # 80 landmarks pad to 96 > 64 at d = 128
    (dict(m=512, n=1024), -2),                # more than 256 landmarks
    (dict(d=32, m=300, n=600), -2),           # the same at d = 32
])
def test_backward_validation(lib, kw, code):
    """nystrom_attention_backward rejects bad arguments before any launch
    (q, k, v, dout at FAKE/FAKE2 ranges; dq, dk, dv at FAKE3..FAKE5)."""
    a = dict(dtype=0, d=64, m=64, n=256, dq=FAKE3, dk=FAKE4, dv=FAKE5)
    a.update(kw)
    rc = lib.nystrom_attention_backward(a["dtype"], FAKE, FAKE, FAKE, NULL, NULL, 65, 1, 2, a["n"], a["d"], a["m"], 6,
                                        0, FAKE2, a["dq"], a["dk"], a["dv"], NULL, NULL)
    assert rc == code
    assert lib.nystrom_last_error().decode() != ""


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), -1),
    (dict(x=None), -1),
    (dict(qkv=None), -1),
    (dict(hidden=6), -1),                     # 24-byte rows: not 16-byte multiples
    (dict(qkv=FAKE), -1),                     # qkv overlaps x
    (dict(d=48), -2),                         # head size not built
    (dict(m=48), -1),                         # n % m != 0 (n = 256)
])
def test_module_validation(lib, kw, code):
    """nystrom_self_attention checks everything before the projection GEMM
    is enqueued (x at FAKE, weights at FAKE2, qkv at FAKE3, out at FAKE4)."""
    a = dict(dtype=0, x=FAKE, w=FAKE2, qkv=FAKE3, out=FAKE4, hidden=64, d=64, m=64)
    a.update(kw)
    H = 1
    rc = lib.nystrom_self_attention(a["dtype"], a["x"], a["w"], NULL, NULL, NULL, 65, 1, 256, a["hidden"], H,
                                    a["d"], a["m"], 6, 0, a["qkv"], a["out"], NULL)
    assert rc == code
    assert lib.nystrom_last_error().decode() != ""


@pytest.mark.parametrize("fn", ["nystrom_attention", "nystrom_attention_bf16"])
def test_landmarks_above_256_unsupported(lib, fn):
    assert call(lib, fn, n=600, m=300) == -2


def test_debug_stages_rejects_exact_branch_and_bad_dtype(lib):
    f = lib.nystrom_debug_stages
    args = [FAKE, FAKE, FAKE, NULL, NULL, 1, 2, 64, 64, 64, 6, 0, FAKE2] + [NULL] * 7 + [NULL]
    assert f(0, *args) == -1          # m == n has no stages
    args[9] = 32
    assert f(7, *args) == -1          # dtype must be 0 or 1


def test_workspace_bytes(lib):
    w = lib.nystrom_workspace_bytes
    assert w(1, 2, 256, 64, 64) > 0
    assert w(2, 2, 256, 64, 64) > w(1, 2, 256, 64, 64)
    assert w(1, 2, 256, 48, 64) == 0      # unsupported d
    # head sizes 32 and 128: the per-landmark buffers scale with d
    assert 0 < w(1, 2, 256, 32, 64) < w(1, 2, 256, 64, 64) < w(1, 2, 256, 128, 64)
    assert w(1, 2, 250, 64, 64) == 0      # n % m
    assert w(1, 2, 256, 64, 256) == 0     # exact branch needs no workspace
    # any landmark count up to 256 (padded to a multiple of 32 inside)
    assert w(1, 2, 480, 64, 48) > 0 and w(1, 2, 400, 64, 50) > 0 and w(1, 2, 64, 64, 1) > 0
    assert w(1, 2, 1200, 64, 300) == 0    # above 256 landmarks
    # fits easily on one GPU at the largest workload
    assert w(1, 4, 65536, 64, 256) < 64 << 20


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    """No fallback: with the library missing the binding raises."""
    import efficient_transformer_attention_segment_amd as nys
    monkeypatch.setattr(nys, "_lib", None)
    monkeypatch.setattr(nys, "library_path", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        nys.workspace_bytes(1, 1, 64, 64, 32)
