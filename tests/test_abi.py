"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/x3conv.h, and rejects invalid arguments with the
documented status before enqueuing anything."""
import ctypes
import os
import re
import subprocess

import pytest

import x3_conv2d_epilogue_amd as x3

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "x3conv.h")

OK, EINVAL, ESHAPE, EUNSUP, EWS, EHIP = range(6)
P = ctypes.c_void_p


def fake(addr):
    """A non-null pointer value that validation accepts but never follows."""
    return P(addr)


X, W_, B_, O, M = fake(0x10000000), fake(0x20000000), fake(0x30000000), fake(0x40000000), \
    fake(0x50000000)


def header_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(x3_[a-z0-9_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def lib():
    return x3.load_library()


def test_header_declares_expected_api():
    assert header_functions() == sorted(x3.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", x3.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (x3_\w+)", out))
    for name in header_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None
    # nothing else leaks out of the library under the x3_ prefix
    assert exported == set(header_functions())


def test_status_strings_and_version(lib):
    for s in range(6):
        assert lib.x3_status_str(s)
    assert lib.x3_status_str(99) == b"unknown status"
    assert b"gfx950" in lib.x3_version()
    assert x3.version().startswith("x3conv")


def _min(lib, *args):
    return lib.x3_conv3x3_min_tanh2_f32(*args)


def test_min_tanh2_validation(lib):
    s = P(0)
    assert _min(lib, X, W_, B_, O, -1, 16, 32, 32, 64, s) == EINVAL
    assert b"positive" in lib.x3_last_error()
    assert _min(lib, X, W_, B_, O, 2, 0, 32, 32, 64, s) == EINVAL
    assert _min(lib, X, W_, B_, O, 2, 16, 2, 32, 64, s) == ESHAPE
    assert _min(lib, X, W_, B_, O, 2, 16, 32, 2, 64, s) == ESHAPE
    assert _min(lib, X, W_, B_, O, 2, 16, 32, 32, 1025, s) == EUNSUP
    assert b"Cout=1025" in lib.x3_last_error()
    assert _min(lib, None, W_, B_, O, 2, 16, 32, 32, 64, s) == EINVAL
    assert _min(lib, X, None, B_, O, 2, 16, 32, 32, 64, s) == EINVAL
    assert _min(lib, X, W_, None, O, 2, 16, 32, 32, 64, s) == EINVAL
    assert _min(lib, X, W_, B_, None, 2, 16, 32, 32, 64, s) == EINVAL
    # out aliasing x
    assert _min(lib, X, W_, B_, X, 2, 16, 32, 32, 64, s) == EINVAL
    assert b"overlaps" in lib.x3_last_error()
    # a sample of x of 2 GiB or more
    assert _min(lib, X, W_, B_, O, 1, 8192, 256, 256, 64, s) == EUNSUP
    # empty batch: valid, nothing enqueued (null x/out allowed)
    assert _min(lib, None, W_, B_, None, 0, 16, 32, 32, 64, s) == OK


def test_mul_lrelu_gelu_validation(lib):
    f = lib.x3_conv3x3_mul_lrelu_gelu_f32
    s = P(0)
    assert f(X, W_, B_, None, 0.01, O, 2, 16, 32, 32, 64, s) == EINVAL
    assert f(X, W_, B_, M, float("nan"), O, 2, 16, 32, 32, 64, s) == EINVAL
    assert f(X, W_, B_, M, float("inf"), O, 2, 16, 32, 32, 64, s) == EINVAL
    assert f(X, W_, B_, M, 0.01, O, 2, 16, 32, 32, 1100, s) == EUNSUP
    # a sample of out (padded to whole 128-channel blocks) of 2 GiB or more
    assert f(X, W_, B_, M, 0.01, O, 1, 4, 4098, 1026, 127, s) == EUNSUP
    assert f(X, W_, B_, M, 0.01, M, 2, 16, 32, 32, 64, s) == EINVAL  # out == mult
    assert f(None, W_, B_, M, 0.01, None, 0, 16, 32, 32, 64, s) == OK


def test_scale_min_validation(lib):
    f = lib.x3_conv3x3_scale_min_f32
    s = P(0)
    assert f(X, W_, B_, float("nan"), O, 2, 64, 32, 32, 128, s) == EINVAL
    assert f(X, W_, B_, 2.0, O, 2, 64, 1, 32, 128, s) == ESHAPE
    assert f(X, W_, B_, 2.0, O, 2, 64, 32, 32, 2000, s) == EUNSUP
    assert f(X, W_, B_, 2.0, B_, 2, 64, 32, 32, 128, s) == EINVAL  # out == bias


def test_gn_workspace_bytes(lib):
    f = lib.x3_conv3x3_gn_workspace_bytes
    # [128,8,128,128] -> conv 126x126; Cin <= 8 and Cout <= 64: tiles of 4 rows
    # x 128 columns, 4 waves: 32 row tiles * 1 column tile * 4 = 128 partial
    # slots per (n, g) of 16 B
    assert f(128, 8, 128, 128, 64, 16, 4) == 128 * 16 * 128 * 16
    # Cout 128: 64-channel blocks, tiles of 8 rows x 128 columns, 8 waves:
    # 16 * 1 * 8 = 128 slots
    assert f(2, 8, 128, 128, 128, 32, 4) == 2 * 32 * 128 * 16
    # Cin 16 (two K chunks): the same 8-wave tiles
    assert f(2, 16, 128, 128, 64, 16, 4) == 2 * 16 * 128 * 16
    assert f(0, 8, 128, 128, 64, 16, 4) == 0
    assert f(2, 8, 128, 128, 64, 15, 4) == 0   # 64 % 15
    # 8 channels per group: per-channel partials, 8 per group and slot
    assert f(2, 8, 128, 128, 64, 8, 4) == 2 * 8 * 8 * 128 * 16
    # one group of all 64 channels
    assert f(2, 8, 128, 128, 64, 1, 4) == 2 * 1 * 64 * 128 * 16
    # windows 1..16 other than 4 run fused too, on tiles of 16 x 64 outputs
    # trimmed to whole windows (NCHW columns to a multiple of lcm(k, 4)),
    # 8 waves.  k = 2: 16 x 64 tiles, 8 * 2 * 8 = 128 slots per group of 4
    assert f(2, 8, 128, 128, 64, 16, 2) == 2 * 16 * 128 * 16
    # k = 3: 15 x 60 tiles, 9 * 3 * 8 = 216 slots, partials per channel
    # (4 per group) for windows of 3 and more
    assert f(2, 8, 128, 128, 64, 16, 3) == 2 * 16 * 4 * 216 * 16
    # k = 7: 14 x 56 tiles -> 9 * 3 * 8 = 216 slots
    assert f(2, 8, 128, 128, 64, 16, 7) == 2 * 16 * 4 * 216 * 16
    # k = 16: 16 x 64 tiles -> 128 slots
    assert f(2, 8, 128, 128, 64, 16, 16) == 2 * 16 * 4 * 128 * 16
    # k = 1 (no pooling): 128 slots per group of 4
    assert f(2, 8, 128, 128, 64, 16, 1) == 2 * 16 * 128 * 16
    # larger windows take the split path: the workspace holds the conv
    # output, [2, 64, 126, 126] floats, then 2 * 64 plane partials of 16 B at
    # the next 256-byte boundary
    y_bytes = (2 * 64 * 126 * 126 * 4 + 255) // 256 * 256
    assert f(2, 8, 128, 128, 64, 16, 17) == y_bytes + 2 * 64 * 16
    assert f(2, 8, 128, 128, 64, 16, 0) == 0   # pool 0: invalid
    assert f(2, 8, 5, 5, 64, 16, 4) == 0       # 3x3 conv output < pool window
    assert f(2, 8, 128, 128, 1028, 257, 4) == 0  # Cout above 1024


def test_gn_validation(lib):
    f = lib.x3_conv3x3_gn_scale_pool_clamp_f32
    s = P(0)
    ws = fake(0x60000000)
    need = lib.x3_conv3x3_gn_workspace_bytes(2, 8, 34, 34, 64, 16, 4)
    assert need > 0

    def call(**kw):
        a = dict(x=X, w=W_, b=B_, g=M, be=fake(0x51000000), sc=fake(0x52000000), groups=16,
                 eps=1e-5, k=4, lo=0.0, hi=1.0, out=O, ws=ws, wsb=need, B=2, Cin=8, H=34, W=34,
                 Cout=64)
        a.update(kw)
        return f(a["x"], a["w"], a["b"], a["g"], a["be"], a["sc"], a["groups"], a["eps"], a["k"],
                 a["lo"], a["hi"], a["out"], a["ws"], a["wsb"], a["B"], a["Cin"], a["H"], a["W"],
                 a["Cout"], s)

    assert call(groups=0) == EINVAL
    assert call(k=0) == EINVAL
    assert call(groups=5) == ESHAPE
    assert call(H=5) == ESHAPE
    assert call(groups=8) == EWS  # supported; needs per-channel partials
    assert call(k=2) == EWS   # window 2: 16 partial slots per group, more than k=4's 8
    assert call(k=20) == EWS  # split path: the workspace must hold the conv output
    assert call(Cout=1028, groups=257) == EUNSUP
    # Cout 128 is supported, but needs a workspace for 32 groups
    assert call(Cout=128, groups=32) == EWS
    assert call(eps=0.0) == EINVAL
    assert call(eps=float("nan")) == EINVAL
    assert call(lo=1.0, hi=0.0) == EINVAL
    assert call(hi=float("inf")) == EINVAL
    assert call(g=None) == EINVAL
    assert call(ws=None) == EWS
    assert call(wsb=need - 1) == EWS
    assert b"workspace" in lib.x3_last_error()
    assert call(ws=fake(0x60000004)) == EINVAL  # misaligned workspace
    assert call(out=X) == EINVAL
    assert call(ws=O) == EINVAL  # workspace overlaps out
    # the workspace overlapping any parameter vector is refused too (the
    # kernels write partials while other workgroups still read them)
    for name, ptr in (("b", B_), ("g", M), ("be", fake(0x51000000)), ("sc", fake(0x52000000))):
        assert call(ws=fake(ptr.value - 16)) == EINVAL, name
        assert b"overlaps" in lib.x3_last_error()
    assert call(B=0, x=None, out=None) == OK


def test_python_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 16, 8, 8)
    w = torch.zeros(64, 16, 3, 3)
    b = torch.zeros(64)
    with pytest.raises(ValueError):
        x3.conv3x3_min_tanh2(x, w, b)
    with pytest.raises(TypeError):
        x3.conv3x3_scale_min(x.double(), w, b)


def test_conv_bias_and_tanh_gelu_validation(lib):
    s = P(0)
    f = lib.x3_conv3x3_bias_f32
    assert f(X, W_, B_, O, -1, 16, 32, 32, 64, s) == EINVAL
    assert f(X, W_, B_, O, 2, 16, 2, 32, 64, s) == ESHAPE
    assert f(X, W_, B_, O, 2, 16, 32, 32, 1025, s) == EUNSUP
    assert f(X, W_, B_, X, 2, 16, 32, 32, 64, s) == EINVAL   # y aliases x
    assert f(None, W_, B_, None, 0, 16, 32, 32, 64, s) == OK
    g = lib.x3_conv3x3_mul_lrelu_gelu_tanh_f32
    assert g(X, W_, B_, None, 0.01, O, 2, 16, 32, 32, 64, s) == EINVAL
    assert g(X, W_, B_, M, float("nan"), O, 2, 16, 32, 32, 64, s) == EINVAL
    assert g(None, W_, B_, M, 0.01, None, 0, 16, 32, 32, 64, s) == OK


def test_standalone_epilogue_validation(lib):
    s = P(0)
    Y = fake(0x10000000)
    assert lib.x3_epi_min_tanh2_f32(Y, O, -1, 4, 8, 8, s) == EINVAL
    assert lib.x3_epi_min_tanh2_f32(Y, O, 2, 0, 8, 8, s) == EINVAL
    assert lib.x3_epi_min_tanh2_f32(None, O, 2, 4, 8, 8, s) == EINVAL
    assert lib.x3_epi_min_tanh2_f32(Y, Y, 2, 4, 8, 8, s) == EINVAL   # out overlaps y
    assert lib.x3_epi_min_tanh2_f32(None, None, 0, 4, 8, 8, s) == OK
    assert lib.x3_epi_scale_min_f32(Y, float("inf"), O, 2, 4, 8, 8, s) == EINVAL
    for name in ("x3_epi_mul_lrelu_gelu_f32", "x3_epi_mul_lrelu_gelu_tanh_f32"):
        f = getattr(lib, name)
        assert f(Y, None, 0.01, O, 2, 4, 8, 8, s) == EINVAL
        assert f(Y, M, float("nan"), O, 2, 4, 8, 8, s) == EINVAL
        # partial overlap of out and y is refused
        assert f(Y, M, 0.01, fake(0x10000010), 2, 4, 8, 8, s) == EINVAL
        assert f(None, M, 0.01, None, 0, 4, 8, 8, s) == OK
    f = lib.x3_epi_gn_scale_pool_clamp_f32
    G_, BE, SC, WS = M, fake(0x51000000), fake(0x52000000), fake(0x60000000)
    assert lib.x3_epi_gn_workspace_bytes(2, 16) == 2 * 16 * 16
    assert lib.x3_epi_gn_workspace_bytes(2, 0) == 0

    def call(**kw):
        a = dict(y=Y, g=G_, be=BE, sc=SC, groups=4, eps=1e-5, k=4, lo=0.0, hi=1.0, out=O,
                 ws=WS, wsb=2 * 16 * 16, B=2, C=16, H=32, W=32)
        a.update(kw)
        return f(a["y"], a["g"], a["be"], a["sc"], a["groups"], a["eps"], a["k"], a["lo"],
                 a["hi"], a["out"], a["ws"], a["wsb"], a["B"], a["C"], a["H"], a["W"], s)

    assert call(groups=0) == EINVAL
    assert call(k=0) == EINVAL
    assert call(groups=3) == ESHAPE
    assert call(H=3) == ESHAPE          # smaller than the window
    assert call(eps=0.0) == EINVAL
    assert call(lo=2.0) == EINVAL
    assert call(sc=None) == EINVAL
    assert call(out=Y) == EINVAL
    assert call(ws=None) == EWS
    assert call(wsb=2 * 16 * 16 - 1) == EWS
    assert call(ws=fake(0x60000008)) == EINVAL   # misaligned workspace
    assert call(ws=O) == EINVAL                  # workspace overlaps out
    assert call(B=0, y=None, out=None) == OK


def test_nhwc_entry_validation(lib):
    s = P(0)
    assert lib.x3_conv3x3_min_tanh2_nhwc_f32(X, W_, B_, O, -1, 16, 32, 32, 64, s) == EINVAL
    assert lib.x3_conv3x3_min_tanh2_nhwc_f32(X, W_, B_, O, 2, 16, 32, 32, 1025, s) == EUNSUP
    assert lib.x3_conv3x3_scale_min_nhwc_f32(X, W_, B_, float("nan"), O, 2, 16, 32, 32, 64,
                                             s) == EINVAL
    assert lib.x3_conv3x3_mul_lrelu_gelu_nhwc_f32(X, W_, B_, None, 0.01, O, 2, 16, 32, 32, 64,
                                                  s) == EINVAL
    assert lib.x3_conv3x3_min_tanh2_nhwc_f32(None, W_, B_, None, 0, 16, 32, 32, 64, s) == OK
    # the NHWC GroupNorm form pools windows 1..16 (no split path)
    f = lib.x3_conv3x3_gn_nhwc_workspace_bytes
    assert f(2, 8, 34, 34, 64, 16, 4) > 0
    # k = 3, NHWC: 15 x 63 tiles -> 3 * 1 * 8 = 24 slots, 4 per group
    assert f(2, 8, 34, 34, 64, 16, 3) == 2 * 16 * 4 * 24 * 16
    assert f(2, 8, 40, 40, 64, 16, 17) == 0
    # [2,8,34,34] -> 32x32, Cin <= 8 and Cout <= 64: resident-weight tiles
    # of 16 rows x 32 columns, 4 waves -> 2 * 1 * 4 = 8 slots
    assert f(2, 8, 34, 34, 64, 16, 4) == 2 * 16 * 8 * 16
    # Cin 16: 8-wave tiles of 32 rows x 32 columns -> 8 slots
    assert f(2, 16, 34, 34, 64, 16, 4) == 2 * 16 * 8 * 16
    # [*, 8, 128, 128] -> 126x126 resident: 16 row tiles x 2 column tiles x 4
    assert f(1, 8, 128, 128, 64, 16, 4) == 16 * 16 * 2 * 4 * 16
    g = lib.x3_conv3x3_gn_scale_pool_clamp_nhwc_f32
    ws = fake(0x60000000)
    assert g(X, W_, B_, M, fake(0x51000000), fake(0x52000000), 16, 1e-5, 17, 0.0, 1.0, O, ws,
             1 << 20, 2, 8, 40, 40, 64, s) == EUNSUP
    assert g(X, W_, B_, M, fake(0x51000000), fake(0x52000000), 16, 1e-5, 4, 0.0, 1.0, O, ws,
             16, 2, 8, 34, 34, 64, s) == EWS


def test_noalloc_gn_validation(lib):
    """The allocation-free GroupNorm entry point validates like the
    workspace form and refuses a shape whose partial statistics exceed its
    static scratch, all before touching the device."""
    f = lib.x3_conv3x3_gn_scale_pool_clamp_noalloc_f32
    s = P(0)
    BE, SC = fake(0x51000000), fake(0x52000000)

    def call(**kw):
        a = dict(x=X, w=W_, b=B_, g=M, be=BE, sc=SC, groups=16, eps=1e-5, k=4, lo=0.0, hi=1.0,
                 out=O, B=2, Cin=8, H=34, W=34, Cout=64)
        a.update(kw)
        return f(a["x"], a["w"], a["b"], a["g"], a["be"], a["sc"], a["groups"], a["eps"], a["k"],
                 a["lo"], a["hi"], a["out"], a["B"], a["Cin"], a["H"], a["W"], a["Cout"], s)

    assert call(groups=0) == EINVAL
    assert call(groups=5) == ESHAPE
    assert call(eps=0.0) == EINVAL
    assert call(lo=2.0) == EINVAL
    assert call(g=None) == EINVAL
    assert call(out=X) == EINVAL
    assert call(B=0, x=None, out=None) == OK
    # 1024 samples of [8,128,128] -> 64 channels: 1024*16*128 partials of
    # 16 B = 32 MiB > the 16 MiB scratch
    assert lib.x3_conv3x3_gn_workspace_bytes(1024, 8, 128, 128, 64, 16, 4) > x3.NOALLOC_SCRATCH_BYTES
    assert call(B=1024, H=128, W=128) == EWS
    assert b"static scratch" in lib.x3_last_error()


def test_probe_mfma_validation():
    """The MFMA-loop probe rejects a null output, an output length that is
    not a positive multiple of 256, and an iteration count outside
    1..65535, before launching anything."""
    lib = x3.load_library()
    f = lib.x3_probe_mfma_f32
    s = P(0)
    assert f(None, 256, 10, s) == EINVAL
    for n in (0, -256, 100, 257):
        assert f(O, n, 10, s) == EINVAL
    for it in (0, -1, 65536):
        assert f(O, 256, it, s) == EINVAL
    assert b"iters" in lib.x3_last_error()
    assert x3.probe_mfma_flop(256, 10) == 4 * 10 * 8 * 4096
