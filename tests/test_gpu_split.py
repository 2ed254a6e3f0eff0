"""GPU parity of the split path and the tanh-approximation GELU.

The standalone epilogues take a stored conv output y.  Their expected
values come from the oracle's fused functions applied to a convolution that
reproduces y exactly: x is y with a 1-pixel border, the weights are the
identity on the centre tap (w[c][c][1][1] = 1, everything else 0) and the
bias is 0, so the oracle's double-precision conv returns y unchanged.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import x3_conv2d_epilogue_amd as x3
from x3_conv2d_epilogue_amd.synthetic import random_case

pytestmark = pytest.mark.gpu

TOL = 2e-4
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def assert_close(got, ref, tol=TOL, what=""):
    got = got.detach().cpu().numpy().astype(np.float64) if torch.is_tensor(got) else got
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = np.abs(got - ref)
    mx = float(err.max()) if err.size else 0.0
    say(f"  {what}: max_abs_err={mx:.3e}")
    assert np.all(np.isfinite(got)), what
    assert mx <= tol, f"{what}: max-abs {mx:.3e} > {tol}"


def identity_case(B, C, H, W, seed):
    g = torch.Generator().manual_seed(seed)
    y = torch.randn(B, C, H, W, generator=g)
    x = torch.randn(B, C, H + 2, W + 2, generator=g)
    x[:, :, 1:-1, 1:-1] = y
    w = torch.zeros(C, C, 3, 3)
    w[torch.arange(C), torch.arange(C), 1, 1] = 1.0
    b = torch.zeros(C)
    return y, x.numpy(), w.numpy(), b.numpy()


EPI_SHAPES = [  # (B, C, H, W) of y
    (2, 16, 30, 30),    # H*W % 4 == 0: 16-byte path
    (1, 5, 13, 17),     # odd plane: scalar path
    (2, 64, 31, 31),
    (1, 3, 4, 260),
]


@pytest.mark.parametrize("shape", EPI_SHAPES)
def test_epi_channel_extremum(shape):
    say(f"epi min/scale {shape}")
    y, x, w, b = identity_case(*shape, seed=sum(shape))
    yd = y.to(DEV)
    assert_close(x3.epi_min_tanh2(yd), oracle.min_tanh2(x, w, b), what="min_tanh2")
    for s in (2.0, -1.5):
        assert_close(x3.epi_scale_min(yd, s), oracle.scale_min(x, w, b, s), what=f"scale {s}")


@pytest.mark.parametrize("shape", EPI_SHAPES)
def test_epi_mul_lrelu_gelu_both_forms(shape):
    say(f"epi gelu {shape}")
    y, x, w, b = identity_case(*shape, seed=100 + sum(shape))
    g = torch.Generator().manual_seed(7)
    m = (1.0 + 0.3 * torch.randn(shape[1], generator=g)).float()
    yd, md = y.to(DEV), m.to(DEV)
    mn = m.numpy()
    assert_close(x3.epi_mul_lrelu_gelu(yd, md, 0.01), oracle.mul_lrelu_gelu(x, w, b, mn, 0.01),
                 what="erf")
    assert_close(x3.epi_mul_lrelu_gelu_tanh(yd, md, 0.2),
                 oracle.mul_lrelu_gelu_tanh(x, w, b, mn, 0.2), what="tanh")
    # in place
    y2 = yd.clone()
    x3.epi_mul_lrelu_gelu(y2, md, 0.01, out=y2)
    assert_close(y2, oracle.mul_lrelu_gelu(x, w, b, mn, 0.01), what="erf in place")


@pytest.mark.parametrize("shape", [(2, 6, 64, 66), (1, 3, 128, 128)])
def test_epi_mul_lrelu_gelu_flat_blocks(shape):
    """Planes of at least 1024 float4 take the flat form: whole 16 KB blocks
    over the tensor, a block meeting two planes (P/4 = 1056) or exactly
    aligned to them (P/4 = 4096)."""
    say(f"epi gelu flat {shape}")
    y, x, w, b = identity_case(*shape, seed=400 + sum(shape))
    g = torch.Generator().manual_seed(8)
    m = (1.0 + 0.3 * torch.randn(shape[1], generator=g)).float()
    yd, md = y.to(DEV), m.to(DEV)
    mn = m.numpy()
    assert_close(x3.epi_mul_lrelu_gelu(yd, md, 0.01), oracle.mul_lrelu_gelu(x, w, b, mn, 0.01),
                 what="erf")
    assert_close(x3.epi_mul_lrelu_gelu_tanh(yd, md, -0.3),
                 oracle.mul_lrelu_gelu_tanh(x, w, b, mn, -0.3), what="tanh")
    assert_close(x3.epi_mul_lrelu_gelu(yd, md, -0.3), oracle.mul_lrelu_gelu(x, w, b, mn, -0.3),
                 what="erf, negative slope")
    y2 = yd.clone()
    x3.epi_mul_lrelu_gelu(y2, md, 0.01, out=y2)
    assert_close(y2, oracle.mul_lrelu_gelu(x, w, b, mn, 0.01), what="erf in place")


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 7])
@pytest.mark.parametrize("cg", [(16, 4), (12, 3), (8, 8), (6, 1)])
@pytest.mark.parametrize("hw", [(23, 29), (22, 30), (23, 30), (13, 260), (20, 32), (26, 126),
                                (18, 128)])
def test_epi_gn_any_pool(k, cg, hw):
    """Odd and even row lengths (even rows with 4x4 windows take the
    one-kernel group form with 8-byte row spans; rows of 4m and 4m+2
    floats, the latter the benchmark's 126), planes of a multiple of 4
    floats or not, one and several 128-column spans, remainder rows and
    columns outside the last window."""
    C, groups = cg
    shape = (2, C) + hw
    say(f"epi gn {shape} groups={groups} k={k}")
    y, x, w, b = identity_case(*shape, seed=200 + k + C)
    g = torch.Generator().manual_seed(k)
    gamma = (1.0 + 0.2 * torch.randn(C, generator=g)).float()
    gamma[::3] *= -1.0
    beta = (0.1 * torch.randn(C, generator=g)).float()
    scale = (1.0 + 0.2 * torch.randn(C, generator=g)).float()
    got = x3.epi_gn_scale_pool_clamp(y.to(DEV), gamma.to(DEV), beta.to(DEV), scale.to(DEV),
                                     groups, 1e-5, k, -2.0, 2.0)
    ref = oracle.gn_scale_pool_clamp(x, w, b, gamma.numpy(), beta.numpy(), scale.numpy(),
                                     groups, 1e-5, k, -2.0, 2.0)
    assert_close(got, ref, what=f"k={k}")


@pytest.mark.parametrize("hw", [(10, 14), (22, 30), (19, 128)])
@pytest.mark.parametrize("offset", [0, 1])
def test_epi_gn_many_groups_unaligned_out(hw, offset):
    """Groups of 4 planes of at most 128 columns, 2400 (sample, group)
    workgroups: one window row per plane pair (10 x 14), an odd number of
    window rows (22 x 30), a full 128-column row with 3 remainder rows
    (19 x 128); out 16-byte aligned (16-byte stores) and, offset by one
    float, not (4-byte stores).  Nothing is written outside out."""
    B, C, groups = 1200, 8, 2
    shape = (B, C) + hw
    say(f"epi gn {shape} groups={groups} k=4 out offset={offset}")
    y, x, w, b = identity_case(*shape, seed=700 + hw[0] + offset)
    g = torch.Generator().manual_seed(70 + offset)
    gamma = (1.0 + 0.2 * torch.randn(C, generator=g)).float()
    gamma[::3] *= -1.0
    beta = (0.1 * torch.randn(C, generator=g)).float()
    scale = (1.0 + 0.2 * torch.randn(C, generator=g)).float()
    ph, pw = hw[0] // 4, hw[1] // 4
    buf = torch.full((B * C * ph * pw + 1,), float("nan"), device=DEV)
    out = buf[offset:offset + B * C * ph * pw].view(B, C, ph, pw)
    x3.epi_gn_scale_pool_clamp(y.to(DEV), gamma.to(DEV), beta.to(DEV), scale.to(DEV),
                               groups, 1e-5, 4, -2.0, 2.0, out=out)
    ref = oracle.gn_scale_pool_clamp(x, w, b, gamma.numpy(), beta.numpy(), scale.numpy(),
                                     groups, 1e-5, 4, -2.0, 2.0)
    assert_close(out, ref, what=f"{hw} offset {offset}")
    rest = buf[B * C * ph * pw:] if offset == 0 else buf[:1]
    assert torch.isnan(rest).all(), "a store left the output"


@pytest.mark.parametrize("groups", [1, 4])
def test_epi_gn_pooled_block_beyond_lds(groups):
    """4x4 windows on even rows: a group whose pooled block fits the LDS
    budget (groups=4: one 64x64 pooled plane) runs in the one-kernel group
    form; a group of 4 such planes (groups=1) does not, and takes the plane
    kernel plus the finalize."""
    shape = (1, 4, 258, 256)
    say(f"epi gn {shape} groups={groups} k=4")
    y, x, w, b = identity_case(*shape, seed=300 + groups)
    g = torch.Generator().manual_seed(30 + groups)
    gamma = (1.0 + 0.2 * torch.randn(4, generator=g)).float()
    gamma[1] *= -1.0
    beta = (0.1 * torch.randn(4, generator=g)).float()
    scale = (1.0 + 0.2 * torch.randn(4, generator=g)).float()
    got = x3.epi_gn_scale_pool_clamp(y.to(DEV), gamma.to(DEV), beta.to(DEV), scale.to(DEV),
                                     groups, 1e-5, 4, -2.0, 2.0)
    ref = oracle.gn_scale_pool_clamp(x, w, b, gamma.numpy(), beta.numpy(), scale.numpy(),
                                     groups, 1e-5, 4, -2.0, 2.0)
    assert_close(got, ref, what=f"groups={groups}")


SHAPES = [(2, 16, 32, 32), (1, 12, 20, 67), (1, 16, 11, 131), (1, 20, 7, 300),
          (20, 8, 34, 70), (10, 5, 30, 132)]  # (the last two: past the one-row-tile size)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("Cout", [17, 64, 128, 200])
def test_conv3x3_bias(shape, Cout):
    B, Cin, H, W = shape
    say(f"conv3x3_bias {shape} Cout={Cout}")
    d = random_case("min_tanh2", B, Cin, H, W, Cout, seed=300 + Cout)
    g = {k: v.to(DEV) for k, v in d.items()}
    got = x3.conv3x3_bias(g["x"], g["weight"], g["bias"])
    assert_close(got, oracle.conv3x3_bias(d["x"].numpy(), d["weight"].numpy(),
                                          d["bias"].numpy()), what="conv")


def test_conv3x3_bias_integer_bit_exact():
    d = random_case("min_tanh2", 2, 9, 13, 130, 96, seed=310, dist="int")
    g = {k: v.to(DEV) for k, v in d.items()}
    got = x3.conv3x3_bias(g["x"], g["weight"], g["bias"]).cpu().numpy().astype(np.float64)
    ref = oracle.conv3x3_bias(d["x"].numpy(), d["weight"].numpy(), d["bias"].numpy())
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("Cout", [40, 64, 128])
def test_conv3x3_mul_lrelu_gelu_tanh(shape, Cout):
    B, Cin, H, W = shape
    say(f"gelu tanh {shape} Cout={Cout}")
    d = random_case("mul_lrelu_gelu", B, Cin, H, W, Cout, seed=400 + Cout)
    g = {k: v.to(DEV) for k, v in d.items()}
    got = x3.conv3x3_mul_lrelu_gelu_tanh(g["x"], g["weight"], g["bias"], g["multiplier"], 0.01)
    n = {k: v.numpy() for k, v in d.items()}
    assert_close(got, oracle.mul_lrelu_gelu_tanh(n["x"], n["weight"], n["bias"],
                                                 n["multiplier"], 0.01), what="gelu tanh")


@pytest.mark.parametrize("k", [1, 2, 3, 5, 17, 20])
@pytest.mark.parametrize("cg", [(64, 16), (48, 6)])
def test_fused_entry_other_pool_sizes(k, cg):
    """x3_conv3x3_gn_scale_pool_clamp_f32 with windows other than 4 (fused
    window-k kernels; windows above 16 take the split path, below)."""
    Cout, groups = cg
    B, Cin, H, W = 2, 8, 26, 37 + (20 if k > 16 else 0)
    say(f"fused gn entry k={k} Cout={Cout} groups={groups}")
    d = random_case("gn_scale_pool_clamp", B, Cin, H, W, Cout, seed=500 + k)
    g = {k_: v.to(DEV) for k_, v in d.items()}
    got = x3.conv3x3_gn_scale_pool_clamp(g["x"], g["weight"], g["bias"], g["gamma"], g["beta"],
                                         g["scale"], groups, 1e-5, k, 0.0, 1.0)
    n = {k_: v.numpy() for k_, v in d.items()}
    ref = oracle.gn_scale_pool_clamp(n["x"], n["weight"], n["bias"], n["gamma"], n["beta"],
                                     n["scale"], groups, 1e-5, k, 0.0, 1.0)
    assert_close(got, ref, what=f"k={k}")


def test_split_composition_matches_fused():
    """conv3x3_bias followed by each standalone epilogue equals the fused
    entry point (to the parity bar) on one shape."""
    d = random_case("mul_lrelu_gelu", 2, 16, 34, 70, 64, seed=600)
    g = {k: v.to(DEV) for k, v in d.items()}
    y = x3.conv3x3_bias(g["x"], g["weight"], g["bias"])
    pairs = [
        (x3.epi_min_tanh2(y), x3.conv3x3_min_tanh2(g["x"], g["weight"], g["bias"])),
        (x3.epi_scale_min(y, 2.0), x3.conv3x3_scale_min(g["x"], g["weight"], g["bias"], 2.0)),
        (x3.epi_mul_lrelu_gelu(y, g["multiplier"]),
         x3.conv3x3_mul_lrelu_gelu(g["x"], g["weight"], g["bias"], g["multiplier"])),
    ]
    for a, b in pairs:
        assert_close(a, b.detach().cpu().numpy().astype(np.float64), tol=1e-5, what="split vs fused")
