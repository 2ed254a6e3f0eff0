"""x3_conv2d_epilogue_amd -- fused 3x3 conv + epilogue kernels for MI355X.

A thin ctypes binding over ``libx3conv.so`` (see ``include/x3conv.h``).  It
only marshals arguments: it checks dtype/device/contiguity/shape of torch
tensors, allocates outputs (and the GroupNorm workspace) with torch, and
passes raw device pointers plus the current HIP stream to the C ABI.  Every
step of the computation runs in the library's HIP kernels; there is no CPU or
PyTorch fallback -- if the library is missing, every call raises.

The fused ops follow x's memory format: a channels_last x selects the NHWC
kernels, and per-channel outputs are then allocated channels_last too.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "conv3x3_min_tanh2", "conv3x3_mul_lrelu_gelu", "conv3x3_mul_lrelu_gelu_tanh",
    "conv3x3_scale_min", "conv3x3_gn_scale_pool_clamp", "gn_workspace_bytes",
    "conv3x3_gn_scale_pool_clamp_noalloc", "NOALLOC_SCRATCH_BYTES",
    "conv3x3_bias", "epi_min_tanh2", "epi_scale_min", "epi_mul_lrelu_gelu",
    "epi_mul_lrelu_gelu_tanh", "epi_gn_scale_pool_clamp",
    "library_path", "version", "X3Error", "load_library", "EXPORTED_SYMBOLS",
    "probe_mfma", "probe_mfma_flop",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libx3conv.so")
_lib = None

EXPORTED_SYMBOLS = (
    "x3_conv3x3_min_tanh2_f32", "x3_conv3x3_mul_lrelu_gelu_f32",
    "x3_conv3x3_mul_lrelu_gelu_tanh_f32", "x3_conv3x3_bias_f32",
    "x3_conv3x3_scale_min_f32", "x3_conv3x3_gn_workspace_bytes",
    "x3_conv3x3_gn_scale_pool_clamp_f32", "x3_conv3x3_gn_scale_pool_clamp_noalloc_f32",
    "x3_conv3x3_min_tanh2_nhwc_f32", "x3_conv3x3_mul_lrelu_gelu_nhwc_f32",
    "x3_conv3x3_scale_min_nhwc_f32", "x3_conv3x3_gn_nhwc_workspace_bytes",
    "x3_conv3x3_gn_scale_pool_clamp_nhwc_f32",
    "x3_epi_min_tanh2_f32", "x3_epi_scale_min_f32", "x3_epi_mul_lrelu_gelu_f32",
    "x3_epi_mul_lrelu_gelu_tanh_f32", "x3_epi_gn_workspace_bytes",
    "x3_epi_gn_scale_pool_clamp_f32",
    "x3_status_str", "x3_last_error", "x3_version", "x3_probe_mfma_f32",
)

STATUS_NAMES = {0: "X3_OK", 1: "X3_EINVAL", 2: "X3_ESHAPE", 3: "X3_EUNSUPPORTED",
                4: "X3_EWORKSPACE", 5: "X3_EHIP"}


class X3Error(RuntimeError):
    """A libx3conv call returned a non-zero status."""

    def __init__(self, fn: str, status: int, detail: str):
        self.status = status
        self.status_name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{fn}: {self.status_name}: {detail}")


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libx3conv.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with `python -c \"import "
            f"__graft_entry__ as g; g.build()\"` (there is no fallback path)")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, f, i, sz = ctypes.c_void_p, ctypes.c_float, ctypes.c_int, ctypes.c_size_t
    lib.x3_conv3x3_min_tanh2_f32.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp]
    lib.x3_conv3x3_mul_lrelu_gelu_f32.argtypes = [vp, vp, vp, vp, f, vp, i, i, i, i, i, vp]
    lib.x3_conv3x3_mul_lrelu_gelu_tanh_f32.argtypes = [vp, vp, vp, vp, f, vp, i, i, i, i, i, vp]
    lib.x3_conv3x3_bias_f32.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp]
    lib.x3_conv3x3_min_tanh2_nhwc_f32.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp]
    lib.x3_conv3x3_mul_lrelu_gelu_nhwc_f32.argtypes = [vp, vp, vp, vp, f, vp, i, i, i, i, i,
                                                       vp]
    lib.x3_conv3x3_scale_min_nhwc_f32.argtypes = [vp, vp, vp, f, vp, i, i, i, i, i, vp]
    lib.x3_conv3x3_gn_nhwc_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.x3_conv3x3_gn_nhwc_workspace_bytes.restype = sz
    lib.x3_conv3x3_gn_scale_pool_clamp_nhwc_f32.argtypes = [
        vp, vp, vp, vp, vp, vp, i, f, i, f, f, vp, vp, sz, i, i, i, i, i, vp]
    lib.x3_epi_min_tanh2_f32.argtypes = [vp, vp, i, i, i, i, vp]
    lib.x3_epi_scale_min_f32.argtypes = [vp, f, vp, i, i, i, i, vp]
    lib.x3_epi_mul_lrelu_gelu_f32.argtypes = [vp, vp, f, vp, i, i, i, i, vp]
    lib.x3_epi_mul_lrelu_gelu_tanh_f32.argtypes = [vp, vp, f, vp, i, i, i, i, vp]
    lib.x3_epi_gn_workspace_bytes.argtypes = [i, i]
    lib.x3_epi_gn_workspace_bytes.restype = sz
    lib.x3_epi_gn_scale_pool_clamp_f32.argtypes = [
        vp, vp, vp, vp, i, f, i, f, f, vp, vp, sz, i, i, i, i, vp]
    lib.x3_conv3x3_scale_min_f32.argtypes = [vp, vp, vp, f, vp, i, i, i, i, i, vp]
    lib.x3_conv3x3_gn_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.x3_conv3x3_gn_workspace_bytes.restype = sz
    lib.x3_conv3x3_gn_scale_pool_clamp_f32.argtypes = [
        vp, vp, vp, vp, vp, vp, i, f, i, f, f, vp, vp, sz, i, i, i, i, i, vp]
    lib.x3_conv3x3_gn_scale_pool_clamp_noalloc_f32.argtypes = [
        vp, vp, vp, vp, vp, vp, i, f, i, f, f, vp, i, i, i, i, i, vp]
    for name in EXPORTED_SYMBOLS:
        if name.endswith("_f32"):
            getattr(lib, name).restype = i
    lib.x3_status_str.argtypes = [i]
    lib.x3_status_str.restype = ctypes.c_char_p
    lib.x3_last_error.argtypes = []
    lib.x3_last_error.restype = ctypes.c_char_p
    lib.x3_version.argtypes = []
    lib.x3_version.restype = ctypes.c_char_p
    lib.x3_probe_mfma_f32.argtypes = [vp, i, i, vp]
    _lib = lib
    return lib


def version() -> str:
    return load_library().x3_version().decode()


def _check(fn: str, status: int):
    if status != 0:
        detail = load_library().x3_last_error().decode()
        raise X3Error(fn, status, detail)


def _tensor(t: torch.Tensor, name: str, ndim: int, channels_last: bool = False) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device (cuda/hip) tensor")
    if channels_last:
        if not t.is_contiguous(memory_format=torch.channels_last):
            raise ValueError(f"{name} must be contiguous in channels_last memory format")
    elif not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return t


def _vec(t: torch.Tensor, name: str, n: int) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.numel() != n:
        raise ValueError(f"{name} must have {n} elements, got {tuple(t.shape)}")
    t = _tensor(t.reshape(-1), name, 1)
    return t


def is_nhwc(x: torch.Tensor) -> bool:
    """True for a 4-D tensor stored channels-last (and not also plain
    contiguous, as tensors with one channel or a 1x1 plane are)."""
    return (isinstance(x, torch.Tensor) and x.dim() == 4 and not x.is_contiguous()
            and x.is_contiguous(memory_format=torch.channels_last))


def _conv_inputs(x, w, b):
    x = _tensor(x, "x", 4, channels_last=is_nhwc(x))
    w = _tensor(w, "weight", 4)
    B, Cin, H, W = x.shape
    Cout = w.shape[0]
    if tuple(w.shape[1:]) != (Cin, 3, 3):
        raise ValueError(f"weight must be [Cout, {Cin}, 3, 3], got {tuple(w.shape)}")
    b = _vec(b, "bias", Cout)
    for t, nm in ((w, "weight"), (b, "bias")):
        if t.device != x.device:
            raise ValueError(f"{nm} is on {t.device}, x on {x.device}")
    return x, w, b, B, Cin, H, W, Cout


def _out(out, shape, like, channels_last=False):
    if out is None:
        if channels_last:
            return torch.empty(shape, dtype=torch.float32, device=like.device,
                               memory_format=torch.channels_last)
        return torch.empty(shape, dtype=torch.float32, device=like.device)
    # (a channels-last output of one channel is also plain contiguous)
    out = _tensor(out, "out", len(shape), channels_last=channels_last and shape[1] > 1)
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"out must be {tuple(shape)}, got {tuple(out.shape)}")
    if out.device != like.device:
        raise ValueError("out is on another device")
    return out


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def conv3x3_min_tanh2(x, weight, bias, out=None) -> torch.Tensor:
    """tanh(tanh(min over output channels of conv3x3(x) + bias)), [B,1,H-2,W-2]."""
    lib = load_library()
    x, w, b, B, Cin, H, W, Cout = _conv_inputs(x, weight, bias)
    out = _out(out, (B, 1, max(H - 2, 0), max(W - 2, 0)), x)
    name = "x3_conv3x3_min_tanh2_nhwc_f32" if is_nhwc(x) else "x3_conv3x3_min_tanh2_f32"
    _check(name, getattr(lib, name)(
        _ptr(x), _ptr(w), _ptr(b), _ptr(out), B, Cin, H, W, Cout, _stream(x.device)))
    return out


def conv3x3_mul_lrelu_gelu(x, weight, bias, multiplier, neg_slope=0.01,
                           out=None) -> torch.Tensor:
    """gelu_erf(leaky_relu((conv3x3(x) + bias) * multiplier[c])), [B,Cout,H-2,W-2]."""
    lib = load_library()
    x, w, b, B, Cin, H, W, Cout = _conv_inputs(x, weight, bias)
    m = _vec(multiplier, "multiplier", Cout)
    nhwc = is_nhwc(x)
    out = _out(out, (B, Cout, max(H - 2, 0), max(W - 2, 0)), x, channels_last=nhwc)
    name = "x3_conv3x3_mul_lrelu_gelu_nhwc_f32" if nhwc else "x3_conv3x3_mul_lrelu_gelu_f32"
    _check(name, getattr(lib, name)(
        _ptr(x), _ptr(w), _ptr(b), _ptr(m), float(neg_slope), _ptr(out),
        B, Cin, H, W, Cout, _stream(x.device)))
    return out


def conv3x3_mul_lrelu_gelu_tanh(x, weight, bias, multiplier, neg_slope=0.01,
                                out=None) -> torch.Tensor:
    """gelu_tanh(leaky_relu((conv3x3(x) + bias) * multiplier[c])), [B,Cout,H-2,W-2]."""
    lib = load_library()
    x, w, b, B, Cin, H, W, Cout = _conv_inputs(x, weight, bias)
    m = _vec(multiplier, "multiplier", Cout)
    out = _out(out, (B, Cout, max(H - 2, 0), max(W - 2, 0)), x)
    _check("x3_conv3x3_mul_lrelu_gelu_tanh_f32", lib.x3_conv3x3_mul_lrelu_gelu_tanh_f32(
        _ptr(x), _ptr(w), _ptr(b), _ptr(m), float(neg_slope), _ptr(out),
        B, Cin, H, W, Cout, _stream(x.device)))
    return out


def conv3x3_bias(x, weight, bias, out=None) -> torch.Tensor:
    """conv3x3(x) + bias (valid, stride 1), [B,Cout,H-2,W-2]."""
    lib = load_library()
    x, w, b, B, Cin, H, W, Cout = _conv_inputs(x, weight, bias)
    out = _out(out, (B, Cout, max(H - 2, 0), max(W - 2, 0)), x)
    _check("x3_conv3x3_bias_f32", lib.x3_conv3x3_bias_f32(
        _ptr(x), _ptr(w), _ptr(b), _ptr(out), B, Cin, H, W, Cout, _stream(x.device)))
    return out


def conv3x3_scale_min(x, weight, bias, scale=2.0, out=None) -> torch.Tensor:
    """min over output channels of (scale * (conv3x3(x) + bias)), [B,1,H-2,W-2]."""
    lib = load_library()
    x, w, b, B, Cin, H, W, Cout = _conv_inputs(x, weight, bias)
    out = _out(out, (B, 1, max(H - 2, 0), max(W - 2, 0)), x)
    name = "x3_conv3x3_scale_min_nhwc_f32" if is_nhwc(x) else "x3_conv3x3_scale_min_f32"
    _check(name, getattr(lib, name)(
        _ptr(x), _ptr(w), _ptr(b), float(scale), _ptr(out), B, Cin, H, W, Cout,
        _stream(x.device)))
    return out


def gn_workspace_bytes(B, Cin, H, W, Cout, groups=16, pool_k=4, nhwc=False) -> int:
    lib = load_library()
    fn = lib.x3_conv3x3_gn_nhwc_workspace_bytes if nhwc else lib.x3_conv3x3_gn_workspace_bytes
    return int(fn(B, Cin, H, W, Cout, groups, pool_k))


def conv3x3_gn_scale_pool_clamp(x, weight, bias, gamma, beta, scale, groups=16,
                                eps=1e-5, pool_k=4, lo=0.0, hi=1.0, out=None,
                                workspace=None) -> torch.Tensor:
    """clamp(maxpool_k(GroupNorm(conv3x3(x) + bias) * scale[c]), lo, hi)."""
    lib = load_library()
    x, w, b, B, Cin, H, W, Cout = _conv_inputs(x, weight, bias)
    g = _vec(gamma, "gamma", Cout)
    be = _vec(beta, "beta", Cout)
    s = _vec(scale, "scale", Cout)
    Ho, Wo = H - 2, W - 2
    k = int(pool_k)
    Ph = (Ho - k) // k + 1 if (k > 0 and Ho >= k) else 0
    Pw = (Wo - k) // k + 1 if (k > 0 and Wo >= k) else 0
    nhwc = is_nhwc(x)
    out = _out(out, (B, Cout, Ph, Pw), x, channels_last=nhwc)
    need = gn_workspace_bytes(B, Cin, H, W, Cout, groups, k, nhwc)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    if workspace.device != x.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on x's device")
    ws_bytes = workspace.numel() * workspace.element_size()
    name = ("x3_conv3x3_gn_scale_pool_clamp_nhwc_f32" if nhwc
            else "x3_conv3x3_gn_scale_pool_clamp_f32")
    _check(name, getattr(lib, name)(
        _ptr(x), _ptr(w), _ptr(b), _ptr(g), _ptr(be), _ptr(s), int(groups), float(eps), k,
        float(lo), float(hi), _ptr(out), _ptr(workspace), ws_bytes, B, Cin, H, W, Cout,
        _stream(x.device)))
    return out


# Size of the library's static device scratch (X3_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 16 << 20


def conv3x3_gn_scale_pool_clamp_noalloc(x, weight, bias, gamma, beta, scale, groups=16,
                                        eps=1e-5, pool_k=4, lo=0.0, hi=1.0,
                                        out=None) -> torch.Tensor:
    """conv3x3_gn_scale_pool_clamp through the allocation-free entry point:
    the partial statistics live in the library's static device scratch, so
    the library allocates nothing (pass `out` to allocate nothing at all).
    NCHW x only; calls on one GPU must not overlap in time."""
    lib = load_library()
    x, w, b, B, Cin, H, W, Cout = _conv_inputs(x, weight, bias)
    if is_nhwc(x):
        raise ValueError("the allocation-free GroupNorm entry point takes NCHW x")
    g = _vec(gamma, "gamma", Cout)
    be = _vec(beta, "beta", Cout)
    s = _vec(scale, "scale", Cout)
    k = int(pool_k)
    Ph = (H - 2 - k) // k + 1 if (k > 0 and H - 2 >= k) else 0
    Pw = (W - 2 - k) // k + 1 if (k > 0 and W - 2 >= k) else 0
    out = _out(out, (B, Cout, Ph, Pw), x)
    _check("x3_conv3x3_gn_scale_pool_clamp_noalloc_f32",
           lib.x3_conv3x3_gn_scale_pool_clamp_noalloc_f32(
               _ptr(x), _ptr(w), _ptr(b), _ptr(g), _ptr(be), _ptr(s), int(groups), float(eps),
               k, float(lo), float(hi), _ptr(out), B, Cin, H, W, Cout, _stream(x.device)))
    return out


# ---------------------------------------------------------------------------
# Standalone epilogues over a stored conv output y [B, C, H, W]


def _y(y):
    y = _tensor(y, "y", 4)
    return (y, *y.shape)


def epi_min_tanh2(y, out=None) -> torch.Tensor:
    """tanh(tanh(min over channels of y)), [B,1,H,W]."""
    lib = load_library()
    y, B, C, H, W = _y(y)
    out = _out(out, (B, 1, H, W), y)
    _check("x3_epi_min_tanh2_f32", lib.x3_epi_min_tanh2_f32(
        _ptr(y), _ptr(out), B, C, H, W, _stream(y.device)))
    return out


def epi_scale_min(y, scale=2.0, out=None) -> torch.Tensor:
    """min over channels of (scale * y), [B,1,H,W]."""
    lib = load_library()
    y, B, C, H, W = _y(y)
    out = _out(out, (B, 1, H, W), y)
    _check("x3_epi_scale_min_f32", lib.x3_epi_scale_min_f32(
        _ptr(y), float(scale), _ptr(out), B, C, H, W, _stream(y.device)))
    return out


def _epi_gelu(name, y, multiplier, neg_slope, out):
    lib = load_library()
    y, B, C, H, W = _y(y)
    m = _vec(multiplier, "multiplier", C)
    out = _out(out, (B, C, H, W), y)
    _check(name, getattr(lib, name)(_ptr(y), _ptr(m), float(neg_slope), _ptr(out),
                                    B, C, H, W, _stream(y.device)))
    return out


def epi_mul_lrelu_gelu(y, multiplier, neg_slope=0.01, out=None) -> torch.Tensor:
    """gelu_erf(leaky_relu(y * multiplier[c])); out may be y (in place)."""
    return _epi_gelu("x3_epi_mul_lrelu_gelu_f32", y, multiplier, neg_slope, out)


def epi_mul_lrelu_gelu_tanh(y, multiplier, neg_slope=0.01, out=None) -> torch.Tensor:
    """gelu_tanh(leaky_relu(y * multiplier[c])); out may be y (in place)."""
    return _epi_gelu("x3_epi_mul_lrelu_gelu_tanh_f32", y, multiplier, neg_slope, out)


def epi_gn_scale_pool_clamp(y, gamma, beta, scale, groups=16, eps=1e-5, pool_k=4,
                            lo=0.0, hi=1.0, out=None, workspace=None) -> torch.Tensor:
    """clamp(maxpool_k(GroupNorm(y) * scale[c]), lo, hi), [B,C,Ph,Pw]."""
    lib = load_library()
    y, B, C, H, W = _y(y)
    g = _vec(gamma, "gamma", C)
    be = _vec(beta, "beta", C)
    s = _vec(scale, "scale", C)
    k = int(pool_k)
    Ph = (H - k) // k + 1 if (k > 0 and H >= k) else 0
    Pw = (W - k) // k + 1 if (k > 0 and W >= k) else 0
    out = _out(out, (B, C, Ph, Pw), y)
    need = int(lib.x3_epi_gn_workspace_bytes(B, C))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=y.device)
    if workspace.device != y.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on y's device")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("x3_epi_gn_scale_pool_clamp_f32", lib.x3_epi_gn_scale_pool_clamp_f32(
        _ptr(y), _ptr(g), _ptr(be), _ptr(s), int(groups), float(eps), k, float(lo),
        float(hi), _ptr(out), _ptr(workspace), ws_bytes, B, C, H, W, _stream(y.device)))
    return out


def probe_mfma_flop(n_out: int, iters: int) -> int:
    """Matrix FLOP of one x3_probe_mfma_f32 call."""
    return (n_out // 64) * iters * 8 * 2 * 32 * 32 * 2


def probe_mfma(out: torch.Tensor, iters: int) -> torch.Tensor:
    """The fp32 MFMA-loop probe (a measurement aid, not part of the method):
    len(out)/256 workgroups, every wavefront `iters` rounds of 8 independent
    32x32x2 fp32 MFMAs on constant operands; every element of out becomes
    exactly 256 * iters.  Asynchronous on the current stream."""
    lib = load_library()
    out = _tensor(out, "out", 1)
    _check("x3_probe_mfma_f32",
           lib.x3_probe_mfma_f32(_ptr(out), out.numel(), int(iters), _stream(out.device)))
    return out
