"""GPU parity of the NHWC (channels_last) input path against the oracle.

The oracle works on NCHW arrays; the GPU call gets the same values in
channels_last memory format and its outputs are compared by logical index.
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


def dev_cl(d):
    g = {k: v.to(DEV) for k, v in d.items()}
    g["x"] = g["x"].contiguous(memory_format=torch.channels_last)
    assert x3.is_nhwc(g["x"])
    return g


def close(got, ref, what, tol=TOL):
    got = got.detach().cpu().numpy().astype(np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = float(np.abs(got - ref).max()) if got.size else 0.0
    say(f"  {what}: max_abs_err={err:.3e}")
    assert np.all(np.isfinite(got)) and err <= tol, f"{what}: {err:.3e}"


# widths on each side of the tile-width switches (32, 64 output columns),
# ragged rows and columns, Cin below / at / above / not a multiple of the
# 8-channel K chunk
SHAPES = [  # (B, Cin, H, W)
    (2, 8, 21, 30),     # Wo=28: one 32-column strip
    (1, 3, 35, 35),     # Wo=33: two strips, Cin=3
    (2, 16, 13, 66),    # Wo=64
    (1, 12, 20, 67),    # Wo=65: 128-column tiles, ragged
    (1, 20, 9, 300),    # Wo=298: three column tiles, ragged
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("Cout", [40, 64, 96, 128, 200])
def test_nhwc_scale_min_integer_bit_exact(shape, Cout):
    B, Cin, H, W = shape
    say(f"nhwc scale_min int-exact {shape} Cout={Cout}")
    d = random_case("scale_min", B, Cin, H, W, Cout, seed=1500 + Cout, dist="int")
    g = dev_cl(d)
    for s in (2.0, -1.0):
        got = x3.conv3x3_scale_min(g["x"], g["weight"], g["bias"], s).cpu().numpy()
        ref = oracle.scale_min(d["x"].numpy(), d["weight"].numpy(), d["bias"].numpy(), s)
        assert np.array_equal(got.astype(np.float64), ref), f"scale {s}"


@pytest.mark.parametrize("Cin", [233016, 233020])
def test_nhwc_weight_offsets_near_the_16_byte_bound(Cin):
    """The 16-byte NHWC kernels that stage permuted weight rows keep a flag
    in bit 30 of each weight offset, so Cin >= 233,017 takes the 4-byte
    kernels.  One output pixel on each side of that bound, integer inputs
    (every fp32 partial sum exact), bit-exact against the oracle."""
    say(f"nhwc scale_min int-exact Cin={Cin}")
    d = random_case("scale_min", 1, Cin, 3, 3, 64, seed=1600, dist="int")
    g = dev_cl(d)
    got = x3.conv3x3_scale_min(g["x"], g["weight"], g["bias"], 2.0).cpu().numpy()
    ref = oracle.scale_min(d["x"].numpy(), d["weight"].numpy(), d["bias"].numpy(), 2.0)
    assert np.array_equal(got.astype(np.float64), ref)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("Cout", [64, 128])
def test_nhwc_min_tanh2(shape, Cout):
    B, Cin, H, W = shape
    say(f"nhwc min_tanh2 {shape} Cout={Cout}")
    d = random_case("min_tanh2", B, Cin, H, W, Cout, seed=1600 + W)
    g = dev_cl(d)
    close(x3.conv3x3_min_tanh2(g["x"], g["weight"], g["bias"]),
          oracle.min_tanh2(d["x"].numpy(), d["weight"].numpy(), d["bias"].numpy()), "min_tanh2")


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("Cout", [17, 64, 128, 200])
def test_nhwc_mul_lrelu_gelu(shape, Cout):
    B, Cin, H, W = shape
    say(f"nhwc gelu {shape} Cout={Cout}")
    d = random_case("mul_lrelu_gelu", B, Cin, H, W, Cout, seed=1700 + Cout)
    g = dev_cl(d)
    out = x3.conv3x3_mul_lrelu_gelu(g["x"], g["weight"], g["bias"], g["multiplier"], 0.01)
    assert Cout == 1 or out.is_contiguous(memory_format=torch.channels_last)
    n = {k: v.numpy() for k, v in d.items()}
    close(out, oracle.mul_lrelu_gelu(n["x"], n["weight"], n["bias"], n["multiplier"], 0.01),
          "gelu")


@pytest.mark.parametrize("shape", [(2, 8, 34, 34), (1, 3, 22, 39), (1, 16, 18, 131)])
@pytest.mark.parametrize("cg", [(64, 16), (64, 8), (128, 32), (36, 9)])
def test_nhwc_gn_pool(shape, cg):
    Cout, groups = cg
    B, Cin, H, W = shape
    say(f"nhwc gn {shape} Cout={Cout} groups={groups}")
    d = random_case("gn_scale_pool_clamp", B, Cin, H, W, Cout, seed=1800 + Cout + groups)
    d["gamma"][::3] *= -1.0
    g = dev_cl(d)
    out = x3.conv3x3_gn_scale_pool_clamp(g["x"], g["weight"], g["bias"], g["gamma"], g["beta"],
                                         g["scale"], groups, 1e-5, 4, -50.0, 50.0)
    assert out.is_contiguous(memory_format=torch.channels_last)
    n = {k: v.numpy() for k, v in d.items()}
    close(out, oracle.gn_scale_pool_clamp(n["x"], n["weight"], n["bias"], n["gamma"], n["beta"],
                                          n["scale"], groups, 1e-5, 4, -50.0, 50.0), "gn")


@pytest.mark.parametrize("case", [
    ((1, 8, 200, 130), 64, 16),   # 200 partials per group: the finalize's looped merge
    ((2, 8, 34, 34), 30, 10),     # 30 channels: the finalize's 4-byte accesses
    ((1, 16, 12, 40), 128, 128),  # 128 groups of one channel
    ((1, 8, 130, 130), 36, 9),    # 36 channels: a thread's float4 walk across channels
])
def test_nhwc_gn_pool_finalize_paths(case):
    (B, Cin, H, W), Cout, groups = case
    say(f"nhwc gn finalize {case}")
    d = random_case("gn_scale_pool_clamp", B, Cin, H, W, Cout, seed=1900 + Cout + groups)
    d["gamma"][1::4] *= -1.0
    g = dev_cl(d)
    out = x3.conv3x3_gn_scale_pool_clamp(g["x"], g["weight"], g["bias"], g["gamma"], g["beta"],
                                         g["scale"], groups, 1e-5, 4, -50.0, 50.0)
    n = {k: v.numpy() for k, v in d.items()}
    close(out, oracle.gn_scale_pool_clamp(n["x"], n["weight"], n["bias"], n["gamma"], n["beta"],
                                          n["scale"], groups, 1e-5, 4, -50.0, 50.0), "gn")


def test_nhwc_matches_nchw_on_full_width_shape():
    """One larger shape through both layouts: identical inputs, results
    within fp32 rounding of each other (the two layouts sum the K terms in
    different orders), and both within the parity bar of the oracle."""
    d = random_case("mul_lrelu_gelu", 2, 16, 40, 258, 64, seed=1900)
    g = {k: v.to(DEV) for k, v in d.items()}
    gc = dev_cl(d)
    a = x3.conv3x3_min_tanh2(g["x"], g["weight"], g["bias"])
    b = x3.conv3x3_min_tanh2(gc["x"], gc["weight"], gc["bias"])
    assert (a - b).abs().max().item() <= 2e-6
    a = x3.conv3x3_mul_lrelu_gelu(g["x"], g["weight"], g["bias"], g["multiplier"])
    b = x3.conv3x3_mul_lrelu_gelu(gc["x"], gc["weight"], gc["bias"], gc["multiplier"])
    assert (a - b.contiguous()).abs().max().item() <= 2e-6
    n = {k: v.numpy() for k, v in d.items()}
    close(b, oracle.mul_lrelu_gelu(n["x"], n["weight"], n["bias"], n["multiplier"], 0.01),
          "gelu 258")


@pytest.mark.parametrize("layout", ["nchw", "nhwc"])
def test_nonfinite_input_stays_local(layout):
    """An infinite input element reaches only the outputs whose 3x3 window
    contains it.  Cin = 12 leaves the last K chunk with 4 real channels, so
    the staging must read the missing ones as zeros rather than as the
    following data (the next pixel in NHWC, the next sample in NCHW)."""
    B, Cin, H, W, Cout = 2, 12, 20, 67, 64
    d = random_case("mul_lrelu_gelu", B, Cin, H, W, Cout, seed=1950)
    hits = [(1, 5, 0), (0, 7, 0), (1, 0, 0)]  # (n, row, col): channels 0-3 infinite
    for n, r, c in hits:
        d["x"][n, 0:4, r, c] = float("inf")
    g = dev_cl(d) if layout == "nhwc" else {k: v.to(DEV) for k, v in d.items()}
    Ho, Wo = H - 2, W - 2
    clean = np.ones((B, Ho, Wo), dtype=bool)
    for n, r, c in hits:
        clean[n, max(r - 2, 0):r + 1, max(c - 2, 0):c + 1] = False
    n_ = {k: v.numpy() for k, v in d.items()}
    for name, got, ref in [
        ("min_tanh2", x3.conv3x3_min_tanh2(g["x"], g["weight"], g["bias"]),
         oracle.min_tanh2(n_["x"], n_["weight"], n_["bias"])),
        ("gelu", x3.conv3x3_mul_lrelu_gelu(g["x"], g["weight"], g["bias"], g["multiplier"]),
         oracle.mul_lrelu_gelu(n_["x"], n_["weight"], n_["bias"], n_["multiplier"], 0.01)),
    ]:
        got = got.detach().cpu().numpy().astype(np.float64)
        m = np.broadcast_to(clean[:, None], got.shape)
        assert np.all(np.isfinite(got[m])), name
        err = float(np.abs(got[m] - ref[m]).max())
        say(f"  {layout} {name}: max_abs_err on clean outputs={err:.3e}")
        assert err <= TOL, (name, err)


def _pixels(B, Ho, Wo, n, seed):
    """Edge pixels of the first and last sample plus n random ones."""
    rng = np.random.default_rng(seed)
    fixed = [(b, r, c) for b in (0, B - 1) for r in (0, Ho // 2, Ho - 1)
             for c in (0, 31, 32, 127, 128, Wo - 1) if c < Wo]
    rand = np.stack([rng.integers(0, B, n), rng.integers(0, Ho, n), rng.integers(0, Wo, n)], 1)
    return np.concatenate([np.array(fixed), rand]).astype(np.int64)


@pytest.mark.parametrize("name", ["min_tanh2", "mul_lrelu_gelu", "scale_min", "gn_pool"])
def test_nhwc_workloads_full_size(name):
    """The NHWC form of each benchmark workload at its full size: every
    output against the NCHW kernel's (whose sampled parity with the oracle
    is tested separately), and sampled outputs against the oracle."""
    from x3_conv2d_epilogue_amd.synthetic import WORKLOADS, make_inputs
    wl = WORKLOADS[name]
    say("generating", wl.about)
    d = make_inputs(wl)
    g = {k: v.to(DEV) for k, v in d.items()}
    xc = g["x"].contiguous(memory_format=torch.channels_last)
    n = {k: v.numpy() for k, v in d.items() if k != "x"}
    x = d["x"].numpy()
    if name == "min_tanh2":
        a, b = (x3.conv3x3_min_tanh2(xx, g["weight"], g["bias"]) for xx in (g["x"], xc))
    elif name == "scale_min":
        a, b = (x3.conv3x3_scale_min(xx, g["weight"], g["bias"], 2.0) for xx in (g["x"], xc))
    elif name == "mul_lrelu_gelu":
        a, b = (x3.conv3x3_mul_lrelu_gelu(xx, g["weight"], g["bias"], g["multiplier"], 0.01)
                for xx in (g["x"], xc))
    else:
        p = wl.params
        a, b = (x3.conv3x3_gn_scale_pool_clamp(xx, g["weight"], g["bias"], g["gamma"], g["beta"],
                                               g["scale"], p["groups"], p["eps"], p["pool_k"],
                                               -1e3, 1e3) for xx in (g["x"], xc))
    torch.cuda.synchronize()
    assert a.shape == b.shape
    diff = (a - b).abs().max().item()
    say(f"  {name}: NHWC vs NCHW max_abs_diff={diff:.3e}")
    assert diff <= 2e-5, diff
    if name == "gn_pool":
        sub = {k: (v[:1] if k == "x" else v) for k, v in d.items()}
        s = {k: v.numpy() for k, v in sub.items()}
        p = wl.params
        ref = oracle.gn_scale_pool_clamp(s["x"], s["weight"], s["bias"], s["gamma"], s["beta"],
                                         s["scale"], p["groups"], p["eps"], p["pool_k"], -1e3, 1e3)
        close(b[:1], ref, "gn sample 0 (NHWC)")
        return
    pix = _pixels(wl.B, wl.Ho, wl.Wo, 3000, 11)
    got = b.detach().cpu()
    if name == "mul_lrelu_gelu":
        co = np.random.default_rng(12).integers(0, wl.Cout, pix.shape[0])
        el = np.stack([pix[:, 0], co, pix[:, 1], pix[:, 2]], 1)
        ref = oracle.mul_lrelu_gelu_at(x, n["weight"], n["bias"], n["multiplier"], el, 0.01)
        sel = got[el[:, 0], el[:, 1], el[:, 2], el[:, 3]]
    else:
        ref = (oracle.min_tanh2_at(x, n["weight"], n["bias"], pix) if name == "min_tanh2"
               else oracle.scale_min_at(x, n["weight"], n["bias"], pix, 2.0))
        sel = got[pix[:, 0], 0, pix[:, 1], pix[:, 2]]
    close(sel, ref, f"{name} sampled (NHWC)")


@pytest.mark.parametrize("k", [1, 2, 3, 5, 7, 16])
@pytest.mark.parametrize("case", [((2, 8, 26, 37), 64, 16), ((1, 16, 35, 131), 48, 6),
                                  ((1, 4, 20, 80), 128, 32)])
def test_nhwc_gn_pool_other_windows(k, case):
    """Windows other than 4 with channels-last x and output (the 16-byte
    channel-half staging: Cin % 4 == 0)."""
    shape, Cout, groups = case
    B, Cin, H, W = shape
    if H - 2 < k or W - 2 < k:
        pytest.skip("window larger than the conv output")
    say(f"nhwc gn k={k} {shape} Cout={Cout} groups={groups}")
    d = random_case("gn_scale_pool_clamp", B, Cin, H, W, Cout, seed=1900 + k + Cout)
    d["gamma"][1::4] *= -1.0
    g = dev_cl(d)
    out = x3.conv3x3_gn_scale_pool_clamp(g["x"], g["weight"], g["bias"], g["gamma"], g["beta"],
                                         g["scale"], groups, 1e-5, k, -50.0, 50.0)
    assert Cout == 1 or out.is_contiguous(memory_format=torch.channels_last)
    n = {k_: v.numpy() for k_, v in d.items()}
    close(out, oracle.gn_scale_pool_clamp(n["x"], n["weight"], n["bias"], n["gamma"], n["beta"],
                                          n["scale"], groups, 1e-5, k, -50.0, 50.0), f"gn k={k}")


def test_nhwc_gn_pool_other_windows_need_cin_multiple_of_4():
    d = random_case("gn_scale_pool_clamp", 1, 3, 22, 39, 64, seed=1950)
    g = dev_cl(d)
    with pytest.raises(x3.X3Error) as e:
        x3.conv3x3_gn_scale_pool_clamp(g["x"], g["weight"], g["bias"], g["gamma"], g["beta"],
                                       g["scale"], 16, 1e-5, 3, 0.0, 1.0)
    assert e.value.status_name == "X3_EUNSUPPORTED"
