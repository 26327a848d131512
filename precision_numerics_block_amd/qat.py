"""Autograd wrappers for quantization-aware training with rollout guidance.

The forward pass is the library's fake-quant kernel (guided, full-code or
plain RTN); the backward pass is the straight-through estimator: the incoming
gradient passes unchanged to x.  The pages describe the forward rounding
("Alibaba Qwen Proposes TRACE for 5.4x Faster FP4 RL Rollouts", section
"TRACE Core Concept": fake quantisation on the training side that rounds
toward the rollout's code) and say nothing about gradients, so the plainest
reading, the usual QAT estimator, is taken.  No arithmetic happens here: the
forward calls the HIP kernels through the binding, the backward returns the
gradient tensor itself.
"""
import torch

from . import trace_quant as tq

__all__ = ["guided_fake_quant", "fullcode_fake_quant", "rtn_fake_quant", "own_scale_fake_quant"]


class _GuidedFakeQuant(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, g, guidance, k, G):
        y, _ = tq.fakequant_guided(x.contiguous(), g, guidance, k, G)
        return y

    @staticmethod
    def backward(ctx, gy):
        return gy, None, None, None, None


class _FullcodeFakeQuant(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, g, guidance, G):
        y, _ = tq.fakequant_fullcode(x.contiguous(), g, guidance, G)
        return y

    @staticmethod
    def backward(ctx, gy):
        return gy, None, None, None


class _RtnFakeQuant(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, g, scales, G):
        y, _, _ = tq.fakequant_rtn(x.contiguous(), g, scales, G)
        return y

    @staticmethod
    def backward(ctx, gy):
        return gy, None, None, None


class _OwnScaleFakeQuant(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, G, work):
        _, y, _, _ = tq.fakequant_rtn_onepass(x.contiguous(), G, work=work)
        return y

    @staticmethod
    def backward(ctx, gy):
        return gy, None, None


def guided_fake_quant(x, g, guidance, k=2, G=1):
    """Rollout-guided FP4 fake-quant of bf16 `x` (GPU) with the rollout's
    global scales `g` and k-bit guidance stream; straight-through gradient."""
    return _GuidedFakeQuant.apply(x, g, guidance, k, G)


def fullcode_fake_quant(x, g, guidance, G=1):
    """Full-code variant (k = 4 guidance stream); straight-through gradient."""
    return _FullcodeFakeQuant.apply(x, g, guidance, G)


def rtn_fake_quant(x, g, scales=None, G=1):
    """Plain RTN fake-quant (own block scales when `scales` is None; then `g`
    should be x's own global scales, from trace_amax on x); straight-through
    gradient."""
    return _RtnFakeQuant.apply(x, g, scales, G)


def own_scale_fake_quant(x, G=1, work=None):
    """Plain QAT fake-quant with the tensor's own scales (its global scale per
    group and its block scales, as the rollout would compute them), from one
    read of x where a group fits on chip; straight-through gradient.  `work`:
    the one-pass work buffer (uint8, onepass_work_bytes(G) bytes, zero-filled
    before its first use and left zeroed by every call); None allocates one."""
    return _OwnScaleFakeQuant.apply(x, G, work)
