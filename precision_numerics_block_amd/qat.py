"""Autograd wrappers for quantization-aware training with rollout guidance.

The forward pass is the library's fake-quant kernel (guided, full-code or
plain RTN).  The pages describe that rounding ("Alibaba Qwen Proposes TRACE
for 5.4x Faster FP4 RL Rollouts", section "TRACE Core Concept": the training
side fake-quantises, rounding toward the rollout's code) and say nothing
about gradients.  The backward pass is the straight-through estimator,
clipped at the quantiser's range by default (``ste="clipped"``): the incoming
gradient passes where the normalised value |v| = |x * inv| is at most 6, the
largest E2M1 magnitude, and is zero where the forward saturated (there its
output stays at +-6 s g as x moves).  The mask is computed on the GPU by
trace_fakequant_ste_grad from x and the scales the forward used.
``ste="identity"`` passes the gradient everywhere.

Plain QAT with the tensor's own scales (``own_scale_fake_quant``) runs one of
two kernel paths, chosen by the caller:
  "two_kernel"  trace_amax, then trace_fakequant_rtn (reads x twice; needs no
                more of the GPU than any streaming kernel; the default);
  "onepass"     trace_fakequant_rtn_onepass (reads x once where a group fits
                on chip; its grid barrier needs a workgroup resident on every
                compute unit at once, so work on other streams can make it time
                out).  It passes a status word and reads it back (one device
                synchronisation per call); after TRACE_E_BARRIER it warns and
                recomputes through the two-kernel path (the one-pass call
                leaves its work buffer zeroed either way), and a non-finite
                input raises.
No arithmetic happens here: every value comes from the HIP kernels.
"""
import warnings

import torch

from . import trace_quant as tq

__all__ = ["guided_fake_quant", "fullcode_fake_quant", "rtn_fake_quant", "own_scale_fake_quant", "PATHS",
           "STE_MODES"]

PATHS = ("two_kernel", "onepass")
STE_MODES = ("clipped", "identity")
E_NONFINITE, E_BARRIER = -7, -10


def _ste_mode(ste):
    if ste not in STE_MODES:
        raise ValueError(f"ste must be one of {STE_MODES}, got {ste!r}")
    return ste == "clipped"


def _grad(ctx, gy):
    """The backward of every wrapper: gy unchanged, or the clipped mask."""
    if not ctx.clipped:
        return gy
    x, g, scales = ctx.saved_tensors
    return tq.fakequant_ste_grad(x, g, scales, gy.contiguous(), ctx.G)


class _GuidedFakeQuant(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, g, guidance, k, G, clipped):
        x = x.contiguous()
        y, _ = tq.fakequant_guided(x, g, guidance, k, G)
        ctx.G, ctx.clipped = G, clipped
        if clipped:
            ctx.save_for_backward(x, g, guidance)      # the stream's first n/16 bytes: the scale plane
        return y

    @staticmethod
    def backward(ctx, gy):
        return _grad(ctx, gy), None, None, None, None, None


class _FullcodeFakeQuant(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, g, guidance, G, clipped):
        x = x.contiguous()
        y, _ = tq.fakequant_fullcode(x, g, guidance, G)
        ctx.G, ctx.clipped = G, clipped
        if clipped:
            ctx.save_for_backward(x, g, guidance)
        return y

    @staticmethod
    def backward(ctx, gy):
        return _grad(ctx, gy), None, None, None, None


class _RtnFakeQuant(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, g, scales, G, clipped):
        x = x.contiguous()
        y, _, used = tq.fakequant_rtn(x, g, scales, G, scales_out=scales is None and clipped)
        ctx.G, ctx.clipped = G, clipped
        if clipped:
            ctx.save_for_backward(x, g, scales if scales is not None else used)
        return y

    @staticmethod
    def backward(ctx, gy):
        return _grad(ctx, gy), None, None, None, None


def _own_scale_two_kernel(x, G):
    g = tq.amax(x, G)
    y, _, scales = tq.fakequant_rtn(x, g, None, G, scales_out=True)
    return g, y, scales


def _own_scale_onepass(x, G, work):
    st = torch.zeros(4, dtype=torch.int32, device=x.device)
    g, y, _, scales = tq.fakequant_rtn_onepass(x, G, scales_out=True, work=work, status=st)
    status = int(st[0].item())
    if status == E_NONFINITE:
        raise tq.TraceError("trace_fakequant_rtn_onepass", status)
    if status == E_BARRIER:
        warnings.warn("one-pass plain QAT: the grid barrier timed out (other work held compute units); "
                      "recomputed with the two-kernel path", RuntimeWarning, stacklevel=4)
        return _own_scale_two_kernel(x, G)
    if status != 0:
        raise tq.TraceError("trace_fakequant_rtn_onepass", status)
    return g, y, scales


class _OwnScaleFakeQuant(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, G, work, path, clipped):
        x = x.contiguous()
        g, y, scales = _own_scale_onepass(x, G, work) if path == "onepass" else _own_scale_two_kernel(x, G)
        ctx.G, ctx.clipped = G, clipped
        if clipped:
            ctx.save_for_backward(x, g, scales)
        return y

    @staticmethod
    def backward(ctx, gy):
        return _grad(ctx, gy), None, None, None, None


def guided_fake_quant(x, g, guidance, k=2, G=1, ste="clipped"):
    """Rollout-guided FP4 fake-quant of bf16 `x` (GPU) with the rollout's
    global scales `g` and k-bit guidance stream; straight-through gradient
    (clipped where |v| > 6 unless ste="identity")."""
    return _GuidedFakeQuant.apply(x, g, guidance, k, G, _ste_mode(ste))


def fullcode_fake_quant(x, g, guidance, G=1, ste="clipped"):
    """Full-code variant (k = 4 guidance stream); straight-through gradient."""
    return _FullcodeFakeQuant.apply(x, g, guidance, G, _ste_mode(ste))


def rtn_fake_quant(x, g, scales=None, G=1, ste="clipped"):
    """Plain RTN fake-quant (own block scales when `scales` is None; then `g`
    should be x's own global scales, from trace_amax on x); straight-through
    gradient."""
    return _RtnFakeQuant.apply(x, g, scales, G, _ste_mode(ste))


def own_scale_fake_quant(x, G=1, work=None, path="two_kernel", ste="clipped"):
    """Plain QAT fake-quant with the tensor's own scales (its global scale per
    group and its block scales, as the rollout would compute them);
    straight-through gradient.  `path`: "two_kernel" (default) or "onepass"
    (see the module notes).  `work`: the one-pass work buffer (uint8,
    onepass_work_bytes(G) bytes, zero-filled before its first use and left
    zeroed by every call); None allocates one."""
    if path not in PATHS:
        raise ValueError(f"path must be one of {PATHS}, got {path!r}")
    return _OwnScaleFakeQuant.apply(x, G, work, path, _ste_mode(ste))
