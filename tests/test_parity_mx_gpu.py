"""GPU parity of the MXFP4 variant (32-element blocks, E8M0 scales, no global
scale) against the CPU oracle: codes, scale bytes and guidance bytes
bit-exact, bf16 outputs bit-exact, fp32 outputs within a relative 1e-6
(expected exact: every product is by a power of two), chosen codes exact."""
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


def to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def eq(got, want, what):
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if not np.array_equal(got, want):
        i = np.flatnonzero(got != want)
        raise AssertionError(f"{what}: {i.size} of {got.size} differ; first at {i[0]}: got {got[i[0]]} want {want[i[0]]}")


def close_f32(got, want, what):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: finite positions differ"
    assert np.array_equal(got[~fin], want[~fin], equal_nan=True), f"{what}: overflow values differ"
    bad = np.abs(got[fin] - want[fin]) > 1e-6 * np.abs(want[fin])
    assert not bad.any(), f"{what}: {bad.sum()} outside rel 1e-6"
    assert np.array_equal(np.signbit(got), np.signbit(want)), f"{what}: sign bits"


def check_all(tq, X, Y, k, out_f32, windows=None):
    """Every MX entry point on the GPU against the oracle (whole tensor, or
    windows of 32-element blocks)."""
    n = X.numel()
    nb = n // 32
    od = tq.OUT_F32 if out_f32 else tq.OUT_BF16
    codes, scales, gd = tq.mx_quant_rollout(Y, k)
    yg, cg = tq.mx_fakequant_guided(X, gd, k, od, codes_out=True)
    yr, cr, _ = tq.mx_fakequant_rtn(X, scales, od, codes_out=True)
    yo, co, so = tq.mx_fakequant_rtn(X, None, od, codes_out=True, scales_out=True)
    torch.cuda.synchronize()
    Xh, Yh = h16(X), h16(Y)
    full = windows is None
    windows = [(0, nb)] if full else windows
    oc = np.zeros(n // 2, np.uint8)
    osc = np.zeros(nb, np.uint8)
    ogd = np.zeros(oracle.mx_guidance_bytes(n, k), np.uint8)
    for b0, b1 in windows:
        oracle.mx_quant_rollout(Yh, k, b0, b1, out=(oc, osc, ogd))
    off = oracle.mx_bitplane_offset(n)
    for b0, b1 in windows:
        e0, e1 = 32 * b0, 32 * b1
        eq(h8(codes[e0 // 2:e1 // 2]), oc[e0 // 2:e1 // 2], f"codes {b0}:{b1}")
        eq(h8(scales[b0:b1]), osc[b0:b1], f"scales {b0}:{b1}")
        eq(h8(gd[b0:b1]), ogd[b0:b1], f"guidance scales {b0}:{b1}")
        eq(h8(gd[off + b0 * 4 * k: off + b1 * 4 * k]), ogd[off + b0 * 4 * k: off + b1 * 4 * k], f"bits {b0}:{b1}")
    if full:
        eq(h8(gd), ogd, "whole guidance stream")
    for b0, b1 in windows:
        e0, e1 = 32 * b0, 32 * b1
        wyg, wcg = oracle.mx_fakequant_guided(Xh, ogd, k, out_f32, b0, b1)
        wyr, wcr, _ = oracle.mx_fakequant_rtn(Xh, osc, out_f32, b0, b1)
        wyo, wco, wso = oracle.mx_fakequant_rtn(Xh, None, out_f32, b0, b1)
        for nm, got, want in (("guided", yg, wyg), ("rtn shared", yr, wyr), ("rtn own", yo, wyo)):
            g_ = got.reshape(-1)[e0:e1]
            if out_f32:
                close_f32(g_.cpu().numpy(), want[e0:e1], f"{nm} y {b0}:{b1}")
            else:
                eq(h16(g_), want[e0:e1], f"{nm} y {b0}:{b1}")
        for nm, got, want in (("guided", cg, wcg), ("rtn shared", cr, wcr), ("rtn own", co, wco)):
            eq(h8(got[e0 // 2:e1 // 2]), want[e0 // 2:e1 // 2], f"{nm} codes {b0}:{b1}")
        eq(h8(so[b0:b1]), wso[b0:b1], f"own scales {b0}:{b1}")


@pytest.mark.parametrize("wl,rows,ti", [(1, None, 0), (2, 2, 0), (3, 1024, 0), (4, 2048, 1), (5, 1, 0)])
def test_mx_workload_small_full_parity(tq, wl, rows, ti):
    name, shape = synth.tensor_specs(wl, rows)[ti]
    X, Y = synth.make_pair(wl, ti, shape, DEV)
    for k in (1, 2, 3, 4):
        check_all(tq, X, Y, k, out_f32=(k == 3))


@pytest.mark.parametrize("wl,ti", [(2, 0), (5, 0)])
def test_mx_full_size_sampled(tq, wl, ti):
    name, shape = synth.tensor_specs(wl)[ti]
    X, Y = synth.make_pair(wl, ti, shape, DEV)
    nb = X.numel() // 32
    rng = np.random.default_rng(wl + 50)
    wins = [(0, 300), (nb - 300, nb)] + [(int(s), int(s) + 150) for s in rng.integers(0, nb - 150, 6)]
    for k in (2, 4):
        check_all(tq, X, Y, k, out_f32=False, windows=wins)
    del X, Y
    torch.cuda.empty_cache()


def all_finite_bf16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return b[(b & 0x7F80) != 0x7F80]


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_mx_bruteforce_rollout_and_rtn(tq, k):
    """Every finite bf16 value, 31 per block after an anchor that sets the
    block scale, for anchors across the whole exponent range."""
    vals = all_finite_bf16()
    pad = (-vals.size) % 31
    vals = np.concatenate([vals, vals[:pad]]).reshape(-1, 31)
    blocks = []
    for a in (0.0, 1e-38, 1e-30, 1.0, 6.0, 7.99, 2688.0, 1e20, 3.0e38):
        ab = torch.tensor([a], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        blocks.append(np.concatenate([np.full((vals.shape[0], 1), ab[0], np.uint16), vals], 1))
    Y = to_dev(np.concatenate(blocks).reshape(-1))
    check_all(tq, Y, Y, k, out_f32=False)


@pytest.mark.parametrize("k", [1, 2, 3, 4])
@pytest.mark.parametrize("out_f32", [False, True])
def test_mx_bruteforce_guided_all_bf16(tq, k, out_f32):
    """Every finite bf16 training value under a set of E8M0 scale codes (both
    ends of the range included) and every guidance value."""
    vals = all_finite_bf16()
    pad = (-vals.size) % 32
    vals = np.concatenate([vals, vals[:pad]])
    per = vals.size // 32
    codes = [0, 1, 60, 125, 126, 127, 128, 131, 200, 252, 254]
    reps = 16 if k == 4 else (1 << k)
    Xh = np.tile(vals, len(codes) * reps)
    n = Xh.size
    nb = n // 32
    blk_code = np.array([codes[(b // per) // reps] for b in range(nb)], np.uint8)
    blk_rep = (np.arange(nb) // per) % reps
    gd = np.zeros(oracle.mx_guidance_bytes(n, k), np.uint8)
    gd[:nb] = blk_code
    off = oracle.mx_bitplane_offset(n)
    gbv = blk_rep[np.arange(n) // 32].astype(np.uint8)
    bits = ((gbv[:, None] >> np.arange(k)) & 1).astype(np.uint8).reshape(-1)
    gd[off:] = np.packbits(bits, bitorder="little")
    X = to_dev(Xh)
    od = tq.OUT_F32 if out_f32 else tq.OUT_BF16
    y, c = tq.mx_fakequant_guided(X, torch.from_numpy(gd).to(DEV), k, od, codes_out=True)
    oy, oc = oracle.mx_fakequant_guided(Xh, gd, k, out_f32)
    torch.cuda.synchronize()
    eq(h8(c), oc, f"chosen codes k={k}")
    if out_f32:
        close_f32(y.cpu().numpy(), oy, f"y k={k}")
    else:
        eq(h16(y), oy, f"y k={k}")


@pytest.mark.parametrize("case", ["zeros", "negzeros", "tiny", "huge", "ragged"])
def test_mx_degenerate_and_sizes(tq, case):
    rng = np.random.default_rng(3)
    n = 32 * (1 if case == "ragged" else 2048)
    x = {"zeros": np.zeros(n), "negzeros": -np.zeros(n), "tiny": rng.standard_normal(n) * 1e-39,
         "huge": rng.uniform(-2.5e38, 2.5e38, n), "ragged": rng.standard_normal(n)}[case]
    X = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(DEV)
    Yf = X.float() + 0.02 * X.float().abs() * torch.randn(n, device=DEV, generator=torch.Generator(DEV).manual_seed(5))
    Y = Yf.to(torch.bfloat16)
    for k in (1, 2, 3, 4):
        check_all(tq, X, Y, k, out_f32=(k % 2 == 0))
    for nb in (3, 2048 * 8 + 5):                          # odd block counts, several tiles and a ragged tail
        x2 = rng.standard_normal(32 * nb) * np.exp(rng.uniform(-4, 4, 32 * nb))
        X2 = torch.from_numpy(x2.astype(np.float32)).to(torch.bfloat16).to(DEV)
        check_all(tq, X2, X2, 2, out_f32=False)


def test_mx_guard_bytes(tq):
    n = 32 * (256 * 3 + 5)
    X, Y = synth.make_pair(1, 0, (n // 2048 + 1, 2048), DEV)
    X, Y = X.reshape(-1)[:n].contiguous(), Y.reshape(-1)[:n].contiguous()
    pad = 4096
    for k in (1, 2, 3, 4):
        gb = tq.mx_guidance_bytes(n, k)
        big_c = torch.full((n // 2 + 2 * pad,), 0xA5, dtype=torch.uint8, device=DEV)
        big_s = torch.full((n // 32 + 2 * pad,), 0xA5, dtype=torch.uint8, device=DEV)
        big_g = torch.full((gb + 2 * pad,), 0xA5, dtype=torch.uint8, device=DEV)
        big_y = torch.full((n + 2 * pad,), 1.5, dtype=torch.bfloat16, device=DEV)
        c, s, g = big_c[pad:pad + n // 2], big_s[pad:pad + n // 32], big_g[pad:pad + gb]
        tq.mx_quant_rollout(Y, k, guidance=g, codes=c, scales=s)
        tq.mx_fakequant_guided(X, g, k, out=big_y[pad:pad + n])
        torch.cuda.synchronize()
        for big, m in ((big_c, n // 2), (big_s, n // 32), (big_g, gb)):
            assert bool((big[:pad] == 0xA5).all()) and bool((big[pad + m:] == 0xA5).all())
        assert bool((big_y[:pad] == 1.5).all()) and bool((big_y[pad + n:] == 1.5).all())
