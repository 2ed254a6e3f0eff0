"""Seeded synthetic inputs for the five workloads the pages discuss.

This module holds the workload shapes and the random draws only -- none of
the method's arithmetic -- and is shared by the tests, the smoke check and
the benchmark.  Inputs are drawn on the CPU with a fresh
``torch.Generator('cpu').manual_seed(seed)`` per workload, in a fixed order:
x ~ N(0, 1); weight ~ U(-a, a) and bias ~ U(-a, a) with a = 1/sqrt(Cin*9)
(PyTorch's default Conv2d init range); then the epilogue parameters in the
order of the op's signature.

Shapes follow the pages (POPCORNBENCH level-2 problems 25, 54, 32 and 85 as
worked through in the Kimi-K2.6 transcripts); the value distributions of the
epilogue parameters (multiplier, gamma, beta, scale) are random rather than
PyTorch's constant initial values so that a channel-indexing mistake shows up.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    op: str            # min_tanh2 | mul_lrelu_gelu | scale_min | gn_scale_pool_clamp
    B: int
    Cin: int
    H: int
    W: int
    Cout: int
    params: dict = field(default_factory=dict)
    about: str = ""

    @property
    def Ho(self) -> int:
        return self.H - 2

    @property
    def Wo(self) -> int:
        return self.W - 2

    def conv_flops(self) -> int:
        """2 * B * Cout * Ho * Wo * Cin * 9 (multiply + add per tap)."""
        return 2 * self.B * self.Cout * self.Ho * self.Wo * self.Cin * 9

    def with_batch(self, B: int) -> "Workload":
        return Workload(self.name, self.op, B, self.Cin, self.H, self.W, self.Cout,
                        dict(self.params), self.about)


WORKLOADS = {
    "tiny_min_tanh2": Workload(
        "tiny_min_tanh2", "min_tanh2", 2, 16, 32, 32, 64, {},
        "conv 16->64 on [2,16,32,32] -> channel-min -> tanh -> tanh"),
    "min_tanh2": Workload(
        "min_tanh2", "min_tanh2", 128, 16, 256, 256, 64, {},
        "conv 16->64 on [128,16,256,256] -> channel-min -> tanh -> tanh"),
    "mul_lrelu_gelu": Workload(
        "mul_lrelu_gelu", "mul_lrelu_gelu", 64, 64, 256, 256, 64, {"neg_slope": 0.01},
        "conv 64->64 on [64,64,256,256] -> x multiplier[64] -> LeakyReLU(0.01) -> erf GELU"),
    "scale_min": Workload(
        "scale_min", "scale_min", 64, 64, 256, 256, 128, {"scale": 2.0},
        "conv 64->128 on [64,64,256,256] -> x 2.0 -> channel-min"),
    "gn_pool": Workload(
        "gn_pool", "gn_scale_pool_clamp", 128, 8, 128, 128, 64,
        {"groups": 16, "eps": 1e-5, "pool_k": 4, "lo": 0.0, "hi": 1.0},
        "conv 8->64 on [128,8,128,128] -> GroupNorm(16) -> x scale[64] -> "
        "MaxPool2d(4) -> clamp[0,1]"),
}

# The order the workloads are listed in the benchmark configuration.
WORKLOAD_ORDER = ["tiny_min_tanh2", "min_tanh2", "mul_lrelu_gelu", "scale_min", "gn_pool"]


def make_inputs(wl: Workload, seed: int = 0) -> dict:
    """CPU float32 tensors for one workload: x, weight, bias and the
    epilogue's parameter tensors (names as in the op signatures)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn((wl.B, wl.Cin, wl.H, wl.W), generator=g, dtype=torch.float32)
    a = 1.0 / math.sqrt(wl.Cin * 9)
    w = torch.empty((wl.Cout, wl.Cin, 3, 3), dtype=torch.float32).uniform_(-a, a, generator=g)
    b = torch.empty((wl.Cout,), dtype=torch.float32).uniform_(-a, a, generator=g)
    d = {"x": x, "weight": w, "bias": b}
    if wl.op == "mul_lrelu_gelu":
        d["multiplier"] = 1.0 + 0.1 * torch.randn((wl.Cout,), generator=g, dtype=torch.float32)
    elif wl.op == "gn_scale_pool_clamp":
        d["gamma"] = 1.0 + 0.1 * torch.randn((wl.Cout,), generator=g, dtype=torch.float32)
        d["beta"] = 0.1 * torch.randn((wl.Cout,), generator=g, dtype=torch.float32)
        d["scale"] = 1.0 + 0.1 * torch.randn((wl.Cout,), generator=g, dtype=torch.float32)
    return d


def random_case(op: str, B: int, Cin: int, H: int, W: int, Cout: int, seed: int,
                dist: str = "normal") -> dict:
    """A small seeded case of any shape.  dist='int' draws small integers
    (x, w in {-2..2}, bias in {-3..3}) so that fp32 sums are exact."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    if dist == "int":
        x = torch.randint(-2, 3, (B, Cin, H, W), generator=g).float()
        w = torch.randint(-2, 3, (Cout, Cin, 3, 3), generator=g).float()
        b = torch.randint(-3, 4, (Cout,), generator=g).float()
    else:
        x = torch.randn((B, Cin, H, W), generator=g)
        a = 1.0 / math.sqrt(Cin * 9)
        w = torch.empty((Cout, Cin, 3, 3)).uniform_(-a, a, generator=g)
        b = torch.empty((Cout,)).uniform_(-a, a, generator=g)
    d = {"x": x, "weight": w, "bias": b}
    if op == "mul_lrelu_gelu":
        d["multiplier"] = 1.0 + 0.1 * torch.randn((Cout,), generator=g)
    elif op == "gn_scale_pool_clamp":
        d["gamma"] = 1.0 + 0.1 * torch.randn((Cout,), generator=g)
        d["beta"] = 0.1 * torch.randn((Cout,), generator=g)
        d["scale"] = 1.0 + 0.1 * torch.randn((Cout,), generator=g)
    return d
