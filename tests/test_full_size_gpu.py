"""Whole-tensor parity at full size on every workload (GPU).

Each workload's tensors are run through the step exactly as bench.py times
it: the same tensors (a KV layer's K and V in one [2, T, H, D] buffer with
one global scale each), the same entry points and the same path choice (the
one-pass kernels when a global-scale group fits on chip, else amax and the
streaming kernel), for every guidance width the workload lists.  Every byte
of every output is then compared with the oracle over the whole tensor: the
global scales, codes, block scales, the guidance stream (pad included), the
full-code stream from trace_guidance_pack, and the bf16 outputs of the
guided, full-code and own-scale RTN fake-quant.  The oracle runs over block
ranges on the host threads of one GPU's share (ctypes releases the GIL;
each range writes only its own blocks' bytes)."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from precision_numerics_block_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
THREADS = min(16, os.cpu_count() or 1)


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


def bench_tensors(wl):
    """(name, X, Y, G) as bench.py builds them."""
    specs = synth.tensor_specs(wl)
    pairs = [synth.make_pair(wl, pos, shape, DEV) for pos, (_, shape) in enumerate(specs)]
    out = [(nm, X, Y, 1) for (nm, _), (X, Y) in zip(specs, pairs)]
    if [nm for nm, _ in specs][-2:] == ["k", "v"]:
        (_, K, Ky, _), (_, V, Vy, _) = out[-2:]
        out = out[:-2] + [("kv", torch.stack([K, V]), torch.stack([Ky, Vy]), 2)]
    return out


def fits_on_chip(tq, n, G):
    return -(-(n // G) // 8192) * 8192 <= tq.onepass_capacity()


def first_diff(got, want, what):
    if got.shape != want.shape:
        raise AssertionError(f"{what}: shape {got.shape} vs {want.shape}")
    if not np.array_equal(got, want):
        idx = np.flatnonzero(got != want)
        raise AssertionError(f"{what}: {idx.size} of {got.size} differ; first at {idx[0]}: "
                             f"got {got[idx[0]]} want {want[idx[0]]}")


def ranges(nblk, parts=64):
    cut = sorted({nblk * i // parts for i in range(parts + 1)})
    return list(zip(cut[:-1], cut[1:]))


def run_parallel(fn, nblk):
    with ThreadPoolExecutor(max_workers=THREADS) as ex:
        list(ex.map(lambda r: fn(*r), ranges(nblk)))


def gpu_step(tq, X, Y, G, ks, onepass):
    """The step on the GPU for each guidance width; host copies of every
    output.  Full code, pack and plain QAT do not depend on k: once."""
    n = X.numel()
    st = torch.zeros(4, dtype=torch.int32, device=DEV)
    r = {}
    for k in ks:
        if onepass:
            gY, codes, scales, gd = tq.quant_rollout_onepass(Y, k, G, status=st)
        else:
            gY = tq.amax(Y, G, status=st)
            codes, scales, gd = tq.quant_rollout(Y, gY, k, G)
        yg, _ = tq.fakequant_guided(X, gY, gd, k, G) if k < 4 else tq.fakequant_fullcode(X, gY, gd, G)
        r[k] = dict(gY=gY.cpu().numpy(), codes=h8(codes), scales=h8(scales), gd=h8(gd), yg=h16(yg))
        del yg, gd
    gd4 = tq.guidance_pack(codes, scales, n, 4)
    yf, _ = tq.fakequant_fullcode(X, gY, gd4, G)
    if onepass:
        gX, yr, _, _ = tq.fakequant_rtn_onepass(X, G, status=st)
    else:
        gX = tq.amax(X, G)
        yr, _, _ = tq.fakequant_rtn(X, gX, None, G)
    torch.cuda.synchronize()
    assert int(st[0].item()) == 0
    r["common"] = dict(gd4=h8(gd4), yf=h16(yf), gX=gX.cpu().numpy(), yr=h16(yr))
    return r


def oracle_check(Xh, Yh, G, ks, r, what):
    n = Xh.size
    nblk = n // 16
    gY, st = oracle.amax(Yh, G)
    assert st == 0
    gX, _ = oracle.amax(Xh, G)
    first_diff(r[ks[0]]["gY"].view(np.uint32), gY.view(np.uint32), f"{what}: rollout global scales")
    first_diff(r["common"]["gX"].view(np.uint32), gX.view(np.uint32), f"{what}: training global scales")
    codes = np.zeros(n // 2, np.uint8)
    scales = np.zeros(n // 16, np.uint8)
    y = np.zeros(n, np.uint16)
    for k in ks:
        gd = np.zeros(oracle.guidance_bytes(n, k), np.uint8)
        run_parallel(lambda b0, b1: oracle.quant_rollout(Yh, gY, k, G, b0, b1, out=(codes, scales, gd)), nblk)
        first_diff(r[k]["codes"], codes, f"{what} k={k}: codes")
        first_diff(r[k]["scales"], scales, f"{what} k={k}: scales")
        first_diff(r[k]["gd"], gd, f"{what} k={k}: guidance stream")
        if k < 4:
            run_parallel(lambda b0, b1: oracle.fakequant_guided(Xh, gY, gd, k, G, False, b0, b1, codes=False,
                                                                out=(y, None)), nblk)
        else:
            run_parallel(lambda b0, b1: oracle.fakequant_fullcode(Xh, gY, gd, G, False, b0, b1, codes=False,
                                                                  out=(y, None)), nblk)
        first_diff(r[k]["yg"], y, f"{what} k={k}: guided output")
        del gd
    gd4 = np.zeros(oracle.guidance_bytes(n, 4), np.uint8)
    run_parallel(lambda b0, b1: oracle.guidance_pack(codes, scales, n, 4, b0, b1, out=gd4), nblk)
    first_diff(r["common"]["gd4"], gd4, f"{what}: full-code stream (pack)")
    run_parallel(lambda b0, b1: oracle.fakequant_fullcode(Xh, gY, gd4, G, False, b0, b1, codes=False,
                                                          out=(y, None)), nblk)
    first_diff(r["common"]["yf"], y, f"{what}: full-code output")
    sc = np.zeros(n // 16, np.uint8)
    run_parallel(lambda b0, b1: oracle.fakequant_rtn(Xh, gX, None, G, False, b0, b1, codes=False,
                                                     out=(y, None, sc)), nblk)
    first_diff(r["common"]["yr"], y, f"{what}: own-scale RTN output")


@pytest.mark.parametrize("wl", [1, 2, 3, 4, 5])
def test_full_size_every_element(tq, wl):
    ks = tuple(synth.WORKLOADS[wl].ks)
    if 2 not in ks:
        ks = (2,) + ks
    for name, X, Y, G in bench_tensors(wl):
        onepass = fits_on_chip(tq, X.numel(), G)
        what = f"workload {wl} {name} {'x'.join(map(str, X.shape))} G={G} {'one-pass' if onepass else 'two-kernel'}"
        print(f"[full-size] {what} ks={ks}", flush=True)
        r = gpu_step(tq, X, Y, G, ks, onepass)
        Xh, Yh = h16(X), h16(Y)
        del X, Y
        torch.cuda.empty_cache()
        oracle_check(Xh, Yh, G, ks, r, what)
        del r, Xh, Yh


def test_full_size_per_expert_scales(tq):
    """The batched MoE step's activations with one global scale per expert
    (G = 128, the bench's per-expert line): the one-pass entry points in one
    launch by teams of workgroups (each team holds one expert's activations
    on chip at a time), every element against the oracle."""
    (name, shape), = synth.tensor_specs(5)[:1]
    X, Y = synth.make_pair(5, 0, shape, DEV)
    G = shape[0]
    assert fits_on_chip(tq, X.numel(), G) and X.numel() > tq.onepass_capacity()   # several launches
    r = gpu_step(tq, X, Y, G, (2,), True)
    Xh, Yh = h16(X), h16(Y)
    del X, Y
    torch.cuda.empty_cache()
    oracle_check(Xh, Yh, G, (2,), r, f"workload 5 {name} G={G} one-pass per block of experts")
