"""Seeded synthetic inputs for the rollout-guided FP4 path.

This module holds no quantisation arithmetic: it only draws random tensors
with the shapes and value distributions of the workloads below and rounds
them to bf16.  Both the HIP path (tests, benchmark) and the CPU oracle are fed
from it.

Workloads (shapes and distributions; the pages' own RL runs on Qwen MoE
models are not reproducible here, so these stand in for their routed-expert
activations and KV states, "Alibaba Qwen Proposes TRACE for 5.4x Faster FP4
RL Rollouts", section "TRACE Core Concept"):

  1  single tensor 256x2048: X ~ N(0,1) with 0.5% of entries x20;
     rollout Y = bf16(X + 0.005 |X| Z)
  2  routed-expert activations 64 experts x 512 tokens x 2048 hidden,
     X ~ Student-t(nu=4), relative noise 0.01
  3  KV states, K and V each 32768 tokens x 8 heads x 128, X = s[h,d] * N(0,1)
     with s ~ LogNormal(0, 0.5) per channel, relative noise 0.005
  4  long-trajectory KV, K and V each 131072 x 4 x 128, as 3 plus 1% of
     token rows x10 (the same rows in K and V)
  5  batched MoE step: activations 128 x 1024 x 4096 Student-t(nu=3) plus K, V
     each 65536 x 8 x 128 (as 3), relative noise 0.01

Weights (the rollout's FP4 weights; not guided, so no rollout copy):
  W  expert weight matrices E x out x in (64 x 1024 x 2048), blocks along in:
     W[e] = sigma_e * N(0,1) with sigma_e = 0.02 * exp(0.3 * z_e), z_e ~ N(0,1),
     and 0.1% of entries x8 (outlier weights); seeds 9000 + role.

"Relative noise r" means Y = bf16(float(X) + r * |float(X)| * Z), Z ~ N(0,1).
Seeds: one torch.Generator per (workload, tensor, role), seeded with
1000 * workload + 10 * tensor index + role (0 = X, 1 = noise, 2 = extra).
"""
from dataclasses import dataclass, field

import torch

__all__ = ["Workload", "WORKLOADS", "WEIGHT_SHAPE", "make_pair", "make_weights", "make_workload", "tensor_specs"]

WEIGHT_SHAPE = (64, 1024, 2048)     # experts x out x in


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    tensors: tuple          # ((name, shape), ...)
    dist: str               # normal_outliers | student_t4 | student_t3 | kv | kv_outliers | moe_step
    rel_noise: float
    ks: tuple               # guidance widths exercised (1, 2 or 4 = full code)
    notes: str = field(default="")


WORKLOADS = {
    1: Workload(1, "single tensor 256x2048", (("x", (256, 2048)),), "normal_outliers", 0.005, (2,)),
    2: Workload(2, "routed-expert activations 64x512x2048", (("act", (64, 512, 2048)),),
                "student_t4", 0.01, (2,)),
    3: Workload(3, "KV states 32768x8x128 (K, V)", (("k", (32768, 8, 128)), ("v", (32768, 8, 128))),
                "kv", 0.005, (1, 2)),
    4: Workload(4, "long-trajectory KV 131072x4x128 (K, V)",
                (("k", (131072, 4, 128)), ("v", (131072, 4, 128))), "kv_outliers", 0.005, (2, 4)),
    5: Workload(5, "batched MoE step: act 128x1024x4096 + KV 65536x8x128",
                (("act", (128, 1024, 4096)), ("k", (65536, 8, 128)), ("v", (65536, 8, 128))),
                "moe_step", 0.01, (2,)),
}


def tensor_specs(index, rows=None):
    """(name, shape) list of a workload; ``rows`` shrinks the leading dim
    (tokens / experts) for small test cases, keeping every other dim."""
    w = WORKLOADS[index]
    out = []
    for name, shape in w.tensors:
        if rows is not None:
            shape = (min(rows, shape[0]),) + tuple(shape[1:])
        out.append((name, shape))
    return out


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(shape, device, seed):
    return torch.randn(shape, generator=_gen(device, seed), device=device, dtype=torch.float32)


def _student_t(shape, nu, device, seed):
    """Student-t with integer nu: Z / sqrt(chi2_nu / nu), chi2 as a sum of nu
    squared normals (separate generator)."""
    gz = _gen(device, seed)
    z = torch.randn(shape, generator=gz, device=device, dtype=torch.float32)
    gc = _gen(device, seed + 5)
    chi2 = torch.zeros(shape, device=device, dtype=torch.float32)
    for _ in range(nu):
        e = torch.randn(shape, generator=gc, device=device, dtype=torch.float32)
        chi2.addcmul_(e, e)
    return z / torch.sqrt(chi2 / nu)


def _kv(shape, device, seed, row_mask=None):
    T, H, D = shape
    s = torch.exp(0.5 * _normal((H, D), device, seed + 2))
    x = _normal(shape, device, seed) * s
    if row_mask is not None:
        x = x * torch.where(row_mask, 10.0, 1.0).view(T, 1, 1)
    return x


def _rollout_copy(x_bf16, rel, device, seed):
    xf = x_bf16.float()
    z = _normal(xf.shape, device, seed)
    return (xf + rel * xf.abs() * z).to(torch.bfloat16)


def make_pair(index, tensor_pos, shape, device="cpu"):
    """Training tensor X and rollout tensor Y (both bf16) for tensor number
    ``tensor_pos`` of workload ``index``, at ``shape``."""
    w = WORKLOADS[index]
    base = 1000 * index + 10 * tensor_pos
    dist = w.dist
    if dist == "moe_step":
        dist = "student_t3" if tensor_pos == 0 else "kv"
    if dist == "normal_outliers":
        x = _normal(shape, device, base)
        u = torch.rand(shape, generator=_gen(device, base + 2), device=device)
        x = torch.where(u < 0.005, x * 20.0, x)
    elif dist == "student_t4":
        x = _student_t(shape, 4, device, base)
    elif dist == "student_t3":
        x = _student_t(shape, 3, device, base)
    elif dist == "kv":
        x = _kv(shape, device, base)
    elif dist == "kv_outliers":
        # one token mask for K and V: drawn from the workload's own seed
        u = torch.rand(shape[0], generator=_gen(device, 1000 * index + 7), device=device)
        x = _kv(shape, device, base, row_mask=u < 0.01)
    else:
        raise ValueError(dist)
    xb = x.to(torch.bfloat16)
    yb = _rollout_copy(xb, w.rel_noise, device, base + 1)
    return xb, yb


def make_workload(index, device="cpu", rows=None):
    """{name: (X, Y)} for every tensor of the workload."""
    return {name: make_pair(index, pos, shape, device)
            for pos, (name, shape) in enumerate(tensor_specs(index, rows))}


def make_weights(shape=WEIGHT_SHAPE, device="cpu"):
    """bf16 expert weights E x out x in (workload W above)."""
    E = shape[0]
    sigma = 0.02 * torch.exp(0.3 * _normal((E,), device, 9002))
    w = _normal(shape, device, 9000) * sigma.view(E, *([1] * (len(shape) - 1)))
    u = torch.rand(shape, generator=_gen(device, 9001), device=device)
    return torch.where(u < 0.001, w * 8.0, w).to(torch.bfloat16)
