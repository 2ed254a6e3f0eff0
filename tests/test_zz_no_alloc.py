"""The allocation-free GroupNorm entry point
(x3_conv3x3_gn_scale_pool_clamp_noalloc_f32, partial statistics in the
library's static device scratch) against the entry point that takes a
caller workspace, through the C ABI: identical results on two calls in a
row, the second with a smaller input, and both within the parity bar of the
oracle."""
import sys

import numpy as np
import pytest
import torch

import oracle
import x3_conv2d_epilogue_amd as x3
from x3_conv2d_epilogue_amd.synthetic import random_case

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 2e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _both(d, **kw):
    g = {k: v.to(DEV) for k, v in d.items()}
    args = (g["x"], g["weight"], g["bias"], g["gamma"], g["beta"], g["scale"])
    ref = x3.conv3x3_gn_scale_pool_clamp(*args, **kw)
    got = x3.conv3x3_gn_scale_pool_clamp_noalloc(*args, **kw)
    torch.cuda.synchronize()
    return got.cpu().numpy(), ref.cpu().numpy()


def _oracle(d, **kw):
    n = {k: v.numpy() for k, v in d.items()}
    return oracle.gn_scale_pool_clamp(n["x"], n["weight"], n["bias"], n["gamma"], n["beta"],
                                      n["scale"], kw.get("groups", 16), kw.get("eps", 1e-5),
                                      kw.get("pool_k", 4), kw.get("lo", 0.0), kw.get("hi", 1.0))


def test_noalloc_matches_workspace_entry_two_calls():
    kw = dict(groups=16, eps=1e-5, pool_k=4, lo=-50.0, hi=50.0)
    # first call: 16 samples of the benchmark's sample shape (one fourth of
    # the scratch); second call: a smaller, ragged input
    for i, shape in enumerate([(16, 8, 128, 128), (2, 8, 30, 46)]):
        say(f"noalloc call {i}: x {shape}")
        d = random_case("gn_scale_pool_clamp", *shape, 64, seed=1500 + i)
        got, ref = _both(d, **kw)
        assert got.shape == ref.shape
        assert np.array_equal(got, ref), np.abs(got - ref).max()
        err = float(np.abs(got.astype(np.float64) - _oracle(d, **kw)).max())
        say(f"  max_abs_err vs oracle {err:.3e}")
        assert err <= TOL


def test_noalloc_other_group_size_then_smaller():
    """Per-channel partials (8 channels per group), then a smaller call of
    the default grouping: stale partials of the first call never leak."""
    d = random_case("gn_scale_pool_clamp", 4, 16, 66, 70, 64, seed=1510)
    got, ref = _both(d, groups=8, lo=-50.0, hi=50.0)
    assert np.array_equal(got, ref)
    d = random_case("gn_scale_pool_clamp", 1, 8, 20, 20, 64, seed=1511)
    got, ref = _both(d, lo=-50.0, hi=50.0)
    assert np.array_equal(got, ref)
    assert float(np.abs(got.astype(np.float64) - _oracle(d, lo=-50.0, hi=50.0)).max()) <= TOL


def test_noalloc_rejects_shapes_beyond_the_scratch():
    d = {k: v.to(DEV) for k, v in
         random_case("gn_scale_pool_clamp", 1, 8, 10, 10, 64, seed=1520).items()}
    # a batch whose partial statistics exceed the static scratch: refused
    # before anything is enqueued (the input is never read)
    need = x3.gn_workspace_bytes(1024, 8, 128, 128, 64, 16, 4)
    assert need > x3.NOALLOC_SCRATCH_BYTES
    x = torch.empty((1024, 8, 128, 128), device=DEV)
    with pytest.raises(x3.X3Error) as e:
        x3.conv3x3_gn_scale_pool_clamp_noalloc(x, d["weight"], d["bias"], d["gamma"],
                                               d["beta"], d["scale"])
    assert e.value.status_name == "X3_EWORKSPACE"
