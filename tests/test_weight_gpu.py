"""GPU parity of FP4 weight quantisation (trace_quant_weight: global scale
per matrix, RTN codes and E4M3 block scales along the contiguous dimension,
no guidance) against the CPU oracle's amax and RTN quantiser: g, codes and
scale bytes bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from precision_numerics_block_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from precision_numerics_block_amd import trace_quant

    return trace_quant


@pytest.fixture(autouse=True)
def announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", flush=True)
    yield


def h16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)


def h8(t):
    return t.contiguous().cpu().numpy().reshape(-1)


def eq(got, want, what):
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if not np.array_equal(got, want):
        i = np.flatnonzero(got != want)
        raise AssertionError(f"{what}: {i.size} of {got.size} differ; first at {i[0]}: got {got[i[0]]} want {want[i[0]]}")


def check(tq, W, G, what):
    g, codes, scales = tq.quant_weight(W, G)
    torch.cuda.synchronize()
    og, st = oracle.amax(h16(W), G)
    assert st == 0
    oc, os_, _ = oracle.quant_rollout(h16(W), og, 2, G, guidance=False)
    eq(g.cpu().numpy().view(np.uint32), og.view(np.uint32), f"{what}: g")
    eq(h8(codes), oc, f"{what}: codes")
    eq(h8(scales), os_, f"{what}: scales")


@pytest.mark.parametrize("shape", [(8, 128, 256), (3, 48, 512), (16, 1, 16)])
def test_weight_small_full(tq, shape):
    W = synth.make_weights(shape, DEV)
    check(tq, W, shape[0], f"weights {shape}")


def test_weight_degenerate_matrices(tq):
    """Matrices of zeros, of bf16 subnormals, near the largest bf16, and a
    matrix whose only non-zero is one element: each its own group."""
    W = synth.make_weights((6, 32, 64), DEV).float()
    W[0] = 0.0
    W[1] = W[1] * 1e-38                                   # bf16 subnormals
    W[2] = torch.sign(W[2]) * 3.0e38
    W[3] = 0.0
    W[3, 5, 7] = -1.5
    W[4] = W[4] * 1e-30                                   # tiny group amax
    check(tq, W.to(torch.bfloat16), 6, "degenerate")


def test_weight_full_size_sampled(tq):
    """64 x 1024 x 2048 expert weights, G = 64: every g, and codes and scales
    of experts 0, 31 and 63 (each matrix is its own group, so the oracle on
    one matrix with G = 1 gives that matrix's slice)."""
    shape = synth.WEIGHT_SHAPE
    W = synth.make_weights(shape, DEV)
    E = shape[0]
    g, codes, scales = tq.quant_weight(W, E)
    torch.cuda.synchronize()
    og, st = oracle.amax(h16(W), E)
    assert st == 0
    eq(g.cpu().numpy().view(np.uint32), og.view(np.uint32), "g")
    per = W.numel() // E
    for e in (0, 31, 63):
        oc, os_, _ = oracle.quant_rollout(h16(W[e]), og[e:e + 1].copy(), 2, 1, guidance=False)
        eq(h8(codes[e * per // 2:(e + 1) * per // 2]), oc, f"codes of expert {e}")
        eq(h8(scales[e * per // 16:(e + 1) * per // 16]), os_, f"scales of expert {e}")


@pytest.mark.parametrize("shape,cap", [((64, 64, 256), 1), ((8, 128, 256), 0)])
def test_weight_onepass_small(tq, shape, cap):
    """Weights through the one-pass rollout without guidance: with a cap of
    one workgroup (33 tiles on chip) the 64 two-tile matrices take four
    launches of 16 matrices; uncapped, one launch.  Every byte against the
    oracle; the outputs start as a canary."""
    W = synth.make_weights(shape, DEV)
    G, n = shape[0], W.numel()
    g = torch.full((G,), -1.0, device=DEV)
    codes = torch.full((n // 2,), 0xA5, dtype=torch.uint8, device=DEV)
    scales = torch.full((n // 16,), 0xA5, dtype=torch.uint8, device=DEV)
    tq.quant_rollout_onepass(W, 2, G, g=g, guidance=False, codes=codes, scales=scales, max_workgroups=cap)
    torch.cuda.synchronize()
    og, st = oracle.amax(h16(W), G)
    assert st == 0
    oc, os_, _ = oracle.quant_rollout(h16(W), og, 2, G, guidance=False)
    eq(g.cpu().numpy().view(np.uint32), og.view(np.uint32), "g")
    eq(h8(codes), oc, "codes")
    eq(h8(scales), os_, "scales")


def test_weight_onepass_full_size(tq):
    """64 x 1024 x 2048 expert weights, G = 64, through the one-pass rollout
    without guidance, as the benchmark times it (two launches of 32 matrices
    on one MI355X): g, codes and scales equal trace_quant_weight's bit for
    bit, and the oracle's for experts 0, 31, 32 and 63."""
    shape = synth.WEIGHT_SHAPE
    W = synth.make_weights(shape, DEV)
    E, n = shape[0], W.numel()
    g0, c0, s0 = tq.quant_weight(W, E)
    g = torch.full((E,), -1.0, device=DEV)
    codes = torch.full((n // 2,), 0xA5, dtype=torch.uint8, device=DEV)
    scales = torch.full((n // 16,), 0xA5, dtype=torch.uint8, device=DEV)
    tq.quant_rollout_onepass(W, 2, E, g=g, guidance=False, codes=codes, scales=scales)
    torch.cuda.synchronize()
    assert torch.equal(g.view(torch.int32), g0.view(torch.int32))
    assert torch.equal(codes, c0) and torch.equal(scales, s0)
    og, st = oracle.amax(h16(W), E)
    assert st == 0
    eq(g.cpu().numpy().view(np.uint32), og.view(np.uint32), "g")
    per = n // E
    for e in (0, 31, 32, 63):
        oc, os_, _ = oracle.quant_rollout(h16(W[e]), og[e:e + 1].copy(), 2, 1, guidance=False)
        eq(h8(codes[e * per // 2:(e + 1) * per // 2]), oc, f"codes of expert {e}")
        eq(h8(scales[e * per // 16:(e + 1) * per // 16]), os_, f"scales of expert {e}")


def test_weight_writes_only_its_outputs(tq):
    """Outputs inside larger buffers: the guard bytes around codes and
    scales keep their sentinel (nothing like a guidance stream is written)."""
    W = synth.make_weights((4, 64, 128), DEV)
    n = W.numel()
    cbuf = torch.full((n // 2 + 512,), 0xA5, dtype=torch.uint8, device=DEV)
    sbuf = torch.full((n // 16 + 512,), 0x5A, dtype=torch.uint8, device=DEV)
    g = torch.empty(4, dtype=torch.float32, device=DEV)
    tq.quant_weight(W, 4, g=g, codes=cbuf[256:256 + n // 2], scales=sbuf[256:256 + n // 16])
    torch.cuda.synchronize()
    og, _ = oracle.amax(h16(W), 4)
    oc, os_, _ = oracle.quant_rollout(h16(W), og, 2, 4, guidance=False)
    eq(h8(cbuf[256:256 + n // 2]), oc, "codes")
    eq(h8(sbuf[256:256 + n // 16]), os_, "scales")
    assert bool((cbuf[:256] == 0xA5).all() and (cbuf[256 + n // 2:] == 0xA5).all()), "code guard bytes"
    assert bool((sbuf[:256] == 0x5A).all() and (sbuf[256 + n // 16:] == 0x5A).all()), "scale guard bytes"


def test_weight_nonfinite_flag(tq):
    W = synth.make_weights((4, 32, 64), DEV).float()
    W[2, 3, 4] = float("inf")
    W = W.to(torch.bfloat16)
    st = torch.zeros(4, dtype=torch.int32, device=DEV)
    g, _, _ = tq.quant_weight(W, 4, status=st)
    torch.cuda.synchronize()
    assert int(st[0]) == -7
    og, ost = oracle.amax(h16(W), 4)
    assert ost == -7
    eq(g.cpu().numpy().view(np.uint32), og.view(np.uint32), "g")
