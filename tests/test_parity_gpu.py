"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: global scales, packed codes, block scales and guidance bytes bit-exact;
bf16 fake-quant outputs bit-exact (bf16 has no slack below one rounding);
fp32 fake-quant outputs within a relative 1e-6 (expected bit-exact, counted);
chosen-code nibbles bit-exact.  Inputs come from the seeded generators or are
constructed here; the oracle computes every expected value from those inputs
alone (its own global scales, its own guidance), never from a GPU output.
"""
import numpy as np
import pytest
import torch

import oracle
from precision_numerics_block_amd import synth

pytestmark = pytest.mark.gpu

REL_TOL = 1e-6


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


DEV = "cuda:0"


def h16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)


def h8(t):
    return t.contiguous().cpu().numpy().reshape(-1)


def to_dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def assert_f32_close(got, want, what):
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: finite positions differ"
    assert np.array_equal(got[~fin], want[~fin]), f"{what}: overflow values differ"
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    err[~fin] = 0.0
    lim = REL_TOL * np.abs(np.where(fin, want, 0).astype(np.float64))
    bad = err > lim
    assert not bad.any(), f"{what}: {bad.sum()} outside rel {REL_TOL}, first at {np.argmax(bad)}"
    assert np.array_equal(np.signbit(got), np.signbit(want)), f"{what}: sign bits differ"


def assert_eq(got, want, what):
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if not np.array_equal(got, want):
        idx = np.flatnonzero(got != want)
        raise AssertionError(f"{what}: {idx.size} of {got.size} differ; first at {idx[0]}: "
                             f"got {got[idx[0]]} want {want[idx[0]]}")


def blocks_of(n_blocks, windows):
    out = []
    for b0, b1 in windows:
        b0, b1 = max(0, b0), min(n_blocks, b1)
        if b0 < b1:
            out.append((b0, b1))
    return out


class Checker:
    """Runs every entry point on the GPU once and compares chosen windows of
    blocks (or everything) with the oracle."""

    def __init__(self, tq, X, Y, k, G=1, onepass=None):
        """onepass: None = trace_amax + trace_quant_rollout; an int = the
        one-pass rollout with that workgroup cap (0 = one per CU)."""
        self.tq, self.X, self.Y, self.k, self.G = tq, X, Y, k, G
        self.onepass = onepass
        self.n = X.numel()
        self.nblk = self.n // 16
        self.Xh, self.Yh = h16(X), h16(Y)

    def run_gpu(self, out_f32=False):
        tq, X, Y, k, G = self.tq, self.X, self.Y, self.k, self.G
        od = tq.OUT_F32 if out_f32 else tq.OUT_BF16
        r = {}
        st = torch.zeros(4, dtype=torch.int32, device=DEV)
        if self.onepass is None:
            r["gY"] = tq.amax(Y, G, status=st)
            r["codes"], r["scales"], r["gd"] = tq.quant_rollout(Y, r["gY"], k, G)
        else:
            r["gY"], r["codes"], r["scales"], r["gd"] = tq.quant_rollout_onepass(
                Y, k, G, max_workgroups=self.onepass, status=st)
        r["gX"] = tq.amax(X, G)
        r["pack"] = tq.guidance_pack(r["codes"], r["scales"], self.n, k)
        if k in (1, 2, 3):
            r["yg"], r["cg"] = tq.fakequant_guided(X, r["gY"], r["gd"], k, G, od, codes_out=True)
        else:
            r["yg"], r["cg"] = tq.fakequant_fullcode(X, r["gY"], r["gd"], G, od, codes_out=True)
        r["yr"], r["cr"], _ = tq.fakequant_rtn(X, r["gY"], r["scales"], G, od, codes_out=True)
        r["yo"], r["co"], r["so"] = tq.fakequant_rtn(X, r["gX"], None, G, od, codes_out=True, scales_out=True)
        torch.cuda.synchronize()
        r["status"] = int(st[0].item())
        self.r = r
        self.out_f32 = out_f32
        return r

    def check(self, windows=None):
        r, k, G, n = self.r, self.k, self.G, self.n
        assert r["status"] == 0
        gY, st = oracle.amax(self.Yh, G)
        gX, _ = oracle.amax(self.Xh, G)
        assert st == 0
        assert_eq(r["gY"].cpu().numpy().view(np.uint32), gY.view(np.uint32), "global scales (rollout)")
        assert_eq(r["gX"].cpu().numpy().view(np.uint32), gX.view(np.uint32), "global scales (training)")
        full = windows is None
        if full:
            windows = [(0, self.nblk)]
        codes = np.zeros(n // 2, np.uint8)
        scales = np.zeros(n // 16, np.uint8)
        gd = np.zeros(oracle.guidance_bytes(n, k), np.uint8)
        off = oracle.bitplane_offset(n)
        for b0, b1 in windows:
            oracle.quant_rollout(self.Yh, gY, k, G, b0, b1, out=(codes, scales, gd))
        for b0, b1 in windows:
            e0, e1 = 16 * b0, 16 * b1
            bk0, bk1 = off + b0 * 2 * k, off + b1 * 2 * k
            assert_eq(h8(r["codes"][e0 // 2:e1 // 2]), codes[e0 // 2:e1 // 2], f"codes {b0}:{b1}")
            assert_eq(h8(r["scales"][b0:b1]), scales[b0:b1], f"scales {b0}:{b1}")
            assert_eq(h8(r["gd"][b0:b1]), gd[b0:b1], f"guidance scale plane {b0}:{b1}")
            assert_eq(h8(r["gd"][bk0:bk1]), gd[bk0:bk1], f"guidance bits {b0}:{b1}")
            assert_eq(h8(r["pack"][b0:b1]), gd[b0:b1], f"packed scale plane {b0}:{b1}")
            assert_eq(h8(r["pack"][bk0:bk1]), gd[bk0:bk1], f"packed bits {b0}:{b1}")
        if full:
            assert_eq(h8(r["gd"]), gd, "whole guidance stream (with pad)")
            assert_eq(h8(r["pack"]), gd, "whole packed stream (with pad)")
        f32 = self.out_f32
        for b0, b1 in windows:
            e0, e1 = 16 * b0, 16 * b1
            if k in (1, 2, 3):
                yg, cg = oracle.fakequant_guided(self.Xh, gY, gd, k, G, f32, b0, b1)
            else:
                yg, cg = oracle.fakequant_fullcode(self.Xh, gY, gd, G, f32, b0, b1)
            yr, cr, _ = oracle.fakequant_rtn(self.Xh, gY, scales, G, f32, b0, b1)
            yo, co, so = oracle.fakequant_rtn(self.Xh, gX, None, G, f32, b0, b1)
            for name, got, want in (("guided", r["yg"], yg), ("rtn shared", r["yr"], yr),
                                    ("rtn own", r["yo"], yo)):
                g_ = got.reshape(-1)[e0:e1]
                if f32:
                    assert_f32_close(g_.cpu().numpy(), want[e0:e1], f"{name} y {b0}:{b1}")
                else:
                    assert_eq(h16(g_), want[e0:e1], f"{name} y {b0}:{b1}")
            for name, got, want in (("guided", r["cg"], cg), ("rtn shared", r["cr"], cr),
                                    ("rtn own", r["co"], co)):
                assert_eq(h8(got[e0 // 2:e1 // 2]), want[e0 // 2:e1 // 2], f"{name} codes {b0}:{b1}")
            assert_eq(h8(r["so"][b0:b1]), so[b0:b1], f"own scales {b0}:{b1}")


# ---------------------------------------------------------------------------
# Workloads at reduced row counts: the oracle checks every element
# ---------------------------------------------------------------------------
SMALL = [  # (workload, rows, tensor index)
    (1, None, 0), (2, 2, 0), (3, 1024, 0), (3, 1024, 1), (4, 2048, 0), (4, 2048, 1), (5, 1, 0), (5, 1024, 2),
]


@pytest.mark.parametrize("wl,rows,ti", SMALL)
def test_workload_small_full_parity(tq, wl, rows, ti):
    name, shape = synth.tensor_specs(wl, rows)[ti]
    X, Y = synth.make_pair(wl, ti, shape, DEV)
    for k in sorted(set(synth.WORKLOADS[wl].ks) | {3, 4}):
        for G in (1, 4):
            c = Checker(tq, X, Y, k, G)
            c.run_gpu(out_f32=(k == 2 and G == 1))
            c.check()


# ---------------------------------------------------------------------------
# Full sizes, in the launch configuration the benchmark times: windows of
# blocks (head, tail, the amax block, random) against the oracle
# ---------------------------------------------------------------------------
FULL = [(1, 0, 1), (2, 0, 1), (2, 0, 64), (3, 0, 1), (3, 1, 1), (4, 0, 1), (4, 1, 1), (5, 0, 1), (5, 1, 1),
        (5, 2, 1)]


@pytest.mark.parametrize("wl,ti,G", FULL)
def test_workload_full_size_sampled(tq, wl, ti, G):
    name, shape = synth.tensor_specs(wl)[ti]
    X, Y = synth.make_pair(wl, ti, shape, DEV)
    nblk = X.numel() // 16
    rng = np.random.default_rng(wl * 100 + ti)
    amax_blk = int(torch.argmax(Y.float().abs().reshape(-1)).item()) // 16
    wins = [(0, 600), (nblk - 600, nblk), (amax_blk - 40, amax_blk + 40)]
    for s in rng.integers(0, nblk - 300, 6):
        wins.append((int(s), int(s) + 300))
    wins = blocks_of(nblk, wins)
    for k in synth.WORKLOADS[wl].ks:
        c = Checker(tq, X, Y, k, G)
        c.run_gpu(out_f32=False)
        c.check(wins)
    del X, Y
    torch.cuda.empty_cache()


@pytest.mark.parametrize("k", [1, 3, 4])
def test_full_size_other_widths(tq, k):
    """The activations 64 x 512 x 2048 at the guidance widths the benchmark
    also times (k = 1, 3) and the full code, in its launch configuration:
    windows of blocks against the oracle."""
    name, shape = synth.tensor_specs(2)[0]
    X, Y = synth.make_pair(2, 0, shape, DEV)
    nblk = X.numel() // 16
    rng = np.random.default_rng(200 + k)
    wins = [(0, 600), (nblk - 600, nblk)] + [(int(s), int(s) + 300) for s in rng.integers(0, nblk - 300, 6)]
    c = Checker(tq, X, Y, k, 1)
    c.run_gpu(out_f32=False)
    c.check(blocks_of(nblk, wins))
    del c, X, Y
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# Brute force over every finite bf16 value
# ---------------------------------------------------------------------------
def all_finite_bf16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    fin = (b & 0x7F80) != 0x7F80
    return b[fin]                                                  # 65280 values


ANCHORS = [1e-38, 1.0, 6.0, 144.0, 2688.0, 3.0e37]


def anchored_blocks():
    """Every finite bf16 value, 15 per block after an anchor, for each anchor
    (the anchor sets the block scale of most blocks)."""
    vals = all_finite_bf16()
    pad = (-vals.size) % 15
    vals = np.concatenate([vals, vals[:pad]]).reshape(-1, 15)
    out = []
    for a in ANCHORS:
        ab = torch.tensor([a], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        out.append(np.concatenate([np.full((vals.shape[0], 1), ab[0], np.uint16), vals], 1))
    return np.concatenate(out).reshape(-1)


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_bruteforce_rollout_and_rtn(tq, k):
    Yh = anchored_blocks()
    nblk = Yh.size // 16
    Y = to_dev_bf16(Yh)
    # one global-scale group per block, so every anchor sets its own g
    for G in (nblk, nblk // 8 if nblk % 8 == 0 else 1):
        c = Checker(tq, Y, Y, k, G)
        c.run_gpu(out_f32=False)
        c.check()


def synthetic_guidance(n, k, scale_bytes, gb_fn):
    gd = np.zeros(oracle.guidance_bytes(n, k), np.uint8)
    gd[: n // 16] = scale_bytes
    off = oracle.bitplane_offset(n)
    vals = gb_fn(np.arange(n)).astype(np.uint8)
    bits = ((vals[:, None] >> np.arange(k)) & 1).astype(np.uint8).reshape(-1)
    gd[off:] = np.packbits(bits, bitorder="little")
    return gd


# (g, E4M3 scale byte) pairs: powers of two (exact normalisation, so every
# tie point is reached), an ordinary scale, subnormal scales, saturation.
COMBOS = [(1.0, 0x38), (2.0 ** -10, 0x28), (1.0 / 2688.0, 0x7E), (3.7e-3, 0x5C), (1e-30, 0x01),
          (1.0e20, 0x7E), (0.3, 0x00), (5.0e-3, 0x33)]


@pytest.mark.parametrize("k", [1, 2, 3, 4])
@pytest.mark.parametrize("out_f32", [False, True])
def test_bruteforce_guided_all_bf16(tq, k, out_f32):
    vals = all_finite_bf16()                                       # 4080 blocks
    reps = 16 if k == 4 else (1 << k)
    per = vals.size
    Xh = np.tile(vals, len(COMBOS) * reps)
    n = Xh.size
    nblk = n // 16
    blk_combo = (np.arange(nblk) // (per // 16)) // reps
    blk_rep = (np.arange(nblk) // (per // 16)) % reps
    g = np.array([COMBOS[c][0] for c in blk_combo], np.float32)
    sb = np.array([COMBOS[c][1] for c in blk_combo], np.uint8)
    gd = synthetic_guidance(n, k, sb, lambda i: blk_rep[i // 16])
    X = to_dev_bf16(Xh)
    gdev = torch.from_numpy(g).to(DEV)
    gddev = torch.from_numpy(gd).to(DEV)
    od = tq.OUT_F32 if out_f32 else tq.OUT_BF16
    if k == 4:
        y, c = tq.fakequant_fullcode(X, gdev, gddev, nblk, od, codes_out=True)
        oy, oc = oracle.fakequant_fullcode(Xh, g, gd, nblk, out_f32)
    else:
        y, c = tq.fakequant_guided(X, gdev, gddev, k, nblk, od, codes_out=True)
        oy, oc = oracle.fakequant_guided(Xh, g, gd, k, nblk, out_f32)
    torch.cuda.synchronize()
    assert_eq(h8(c), oc, f"chosen codes k={k}")
    if out_f32:
        assert_f32_close(y.cpu().numpy(), oy, f"y k={k}")
    else:
        assert_eq(h16(y), oy, f"y k={k}")


# ---------------------------------------------------------------------------
# Edge cases
# ---------------------------------------------------------------------------
def _pair_from_np(x, rel, seed):
    rng = np.random.default_rng(seed)
    X = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    xf = X.float().numpy()
    y = xf + rel * np.abs(xf) * rng.standard_normal(xf.shape).astype(np.float32)
    Y = torch.from_numpy(y).to(torch.bfloat16)
    return X.to(DEV), Y.to(DEV)


@pytest.mark.parametrize("nblk,G", [(1, 1), (2, 2), (37, 1), (512 + 37, 1), (3 * 512 + 6, 3),
                                    (2048 * 512 + 1234, 1), (2048 * 513, 513)])
def test_sizes_and_ragged_tails(tq, nblk, G):
    rng = np.random.default_rng(nblk)
    x = rng.standard_normal(16 * nblk) * np.exp(rng.uniform(-3, 3, 16 * nblk))
    X, Y = _pair_from_np(x, 0.01, nblk)
    for k in (1, 2, 3, 4):
        c = Checker(tq, X, Y, k, G)
        c.run_gpu(out_f32=(k == 1))
        if nblk > 100000:
            c.check(blocks_of(nblk, [(0, 700), (nblk - 700, nblk), (nblk // 2, nblk // 2 + 700)]))
        else:
            c.check()


@pytest.mark.parametrize("case", ["zeros", "negzeros", "tiny_amax", "huge", "mixed_tiny_blocks", "ties"])
def test_degenerate_inputs(tq, case):
    n = 16 * 1024
    rng = np.random.default_rng(7)
    if case == "zeros":
        x = np.zeros(n)
    elif case == "negzeros":
        x = -np.zeros(n)
    elif case == "tiny_amax":                        # g falls into fp32 subnormals
        x = rng.standard_normal(n) * 1e-39
    elif case == "huge":                             # near the bf16 maximum
        x = rng.uniform(-2.5e38, 2.5e38, n)
    elif case == "mixed_tiny_blocks":                # most block scales round to 0
        x = rng.standard_normal(n) * 1e-6
        x[::97] = 1e4
    else:                                            # exact E2M1 ties at g = 1, s = 1
        x = rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 2.25, 4.5, 3.75], n) * rng.choice([-1, 1], n)
        x[::16] = 6.0                                # block amax 6 -> t = 1 -> s = 1
        x[0] = 2688.0                                # tensor amax -> g = 1
    X, Y = _pair_from_np(x, 0.02, 11)
    for k in (1, 2, 3, 4):
        c = Checker(tq, X, Y, k, 1)
        c.run_gpu(out_f32=(k != 2))
        c.check()


def test_in_place_and_determinism(tq):
    X, Y = synth.make_pair(1, 0, (256, 2048), DEV)
    g = tq.amax(Y)
    codes, scales, gd = tq.quant_rollout(Y, g, 2)
    y1, c1 = tq.fakequant_guided(X, g, gd, 2, codes_out=True)
    y2, c2 = tq.fakequant_guided(X, g, gd, 2, codes_out=True)
    xin = X.clone()
    y3, c3 = tq.fakequant_guided(xin, g, gd, 2, out=xin, codes_out=True)
    codes2, scales2, gd2 = tq.quant_rollout(Y, g, 2)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(y1.view(torch.int16), xin.view(torch.int16))
    assert torch.equal(c1, c2) and torch.equal(c1, c3)
    assert torch.equal(codes, codes2) and torch.equal(gd, gd2) and torch.equal(scales, scales2)


def test_in_place_every_fakequant(tq):
    """Every fake-quant entry point with the output in the input's buffer
    (bf16) gives the out-of-place result, codes included; the one-pass RTN in
    one launch, with the excess read twice (one group larger than a capped
    chip) and with one launch per group."""
    X, Y = synth.make_pair(1, 0, (256, 2048), DEV)
    g = tq.amax(Y)
    codes, scales, gd2 = tq.quant_rollout(Y, g, 2)
    gd4 = tq.guidance_pack(codes, scales, X.numel(), 4)
    gx = tq.amax(X)
    _, mxs, mxgd = tq.mx_quant_rollout(Y, 2)
    cases = {
        "guided": lambda x, o: tq.fakequant_guided(x, g, gd2, 2, out=o, codes_out=True),
        "fullcode": lambda x, o: tq.fakequant_fullcode(x, g, gd4, out=o, codes_out=True),
        "rtn shared": lambda x, o: tq.fakequant_rtn(x, g, scales, out=o, codes_out=True)[:2],
        "rtn own": lambda x, o: tq.fakequant_rtn(x, gx, None, out=o, codes_out=True)[:2],
        "mx guided": lambda x, o: tq.mx_fakequant_guided(x, mxgd, 2, out=o, codes_out=True),
        "mx rtn own": lambda x, o: tq.mx_fakequant_rtn(x, None, out=o, codes_out=True)[:2],
    }
    for G, cap in ((1, 0), (1, 1), (4, 1)):            # one launch; excess read twice; one launch per 2 groups
        cases[f"rtn one-pass G={G} cap={cap}"] = (
            lambda x, o, G=G, cap=cap: tq.fakequant_rtn_onepass(x, G, out=o, codes_out=True, max_workgroups=cap)[1:3])
    for name, fn in cases.items():
        y_ref, c_ref = fn(X, None)
        xin = X.clone()
        y_in, c_in = fn(xin, xin)
        torch.cuda.synchronize()
        assert y_in.data_ptr() == xin.data_ptr(), name
        assert torch.equal(xin.view(torch.int16), y_ref.view(torch.int16)), name
        assert torch.equal(c_in, c_ref), name


def test_guard_bytes_untouched(tq):
    """Outputs carved out of larger buffers filled with a canary: nothing
    outside the documented extents is written."""
    n = 16 * (512 * 3 + 7)
    X, Y = synth.make_pair(1, 0, (n // 2048 + 1, 2048), DEV)
    X, Y = X.reshape(-1)[:n].contiguous(), Y.reshape(-1)[:n].contiguous()
    pad = 4096
    for k in (1, 2, 3, 4):
        gb = tq.guidance_bytes(n, k)
        big_codes = torch.full((n // 2 + 2 * pad,), 0xA5, dtype=torch.uint8, device=DEV)
        big_scales = torch.full((n // 16 + 2 * pad,), 0xA5, dtype=torch.uint8, device=DEV)
        big_gd = torch.full((gb + 2 * pad,), 0xA5, dtype=torch.uint8, device=DEV)
        big_y = torch.full((n + 2 * pad,), 1.5, dtype=torch.bfloat16, device=DEV)
        g = tq.amax(Y)
        codes, scales, gd = big_codes[pad:pad + n // 2], big_scales[pad:pad + n // 16], big_gd[pad:pad + gb]
        tq.quant_rollout(Y, g, k, 1, guidance=gd, codes=codes, scales=scales)
        y = big_y[pad:pad + n]
        if k == 4:
            tq.fakequant_fullcode(X, g, gd, out=y)
        else:
            tq.fakequant_guided(X, g, gd, k, out=y)
        torch.cuda.synchronize()
        for big, m, fill in ((big_codes, n // 2, 0xA5), (big_scales, n // 16, 0xA5), (big_gd, gb, 0xA5)):
            assert bool((big[:pad] == fill).all()) and bool((big[pad + m:] == fill).all())
        assert bool((big_y[:pad] == 1.5).all()) and bool((big_y[pad + n:] == 1.5).all())


def test_nonfinite_flag(tq):
    x = np.ones(16 * 64, np.float32)
    x[5] = np.inf
    x[700] = np.nan
    x[300] = 12.0
    X = torch.from_numpy(x).to(torch.bfloat16).to(DEV)
    st = torch.zeros(4, dtype=torch.int32, device=DEV)
    g = tq.amax(X, status=st)
    torch.cuda.synchronize()
    assert int(st[0]) == -7
    og, ost = oracle.amax(h16(X))
    assert ost == -7
    assert np.array_equal(g.cpu().numpy().view(np.uint32), og.view(np.uint32))


def test_graph_replay_matches_eager(tq):
    """The whole step captured into a HIP graph: every replay (with eager work
    and synchronisation between replays) reproduces the eager outputs."""
    X, Y = synth.make_pair(1, 0, (256, 2048), DEV)
    n = X.numel()
    g, gx = torch.empty(1, device=DEV), torch.empty(1, device=DEV)
    codes = torch.empty(n // 2, dtype=torch.uint8, device=DEV)
    scales = torch.empty(n // 16, dtype=torch.uint8, device=DEV)
    gd = torch.empty(tq.guidance_bytes(n, 2), dtype=torch.uint8, device=DEV)
    gd4 = torch.empty(tq.guidance_bytes(n, 4), dtype=torch.uint8, device=DEV)
    yg, yf, yr = (torch.empty_like(X) for _ in range(3))

    def step():
        tq.amax(Y, out=g)
        tq.quant_rollout(Y, g, 2, guidance=gd, codes=codes, scales=scales)
        tq.guidance_pack(codes, scales, n, 4, out=gd4)
        tq.fakequant_guided(X, g, gd, 2, out=yg)
        tq.fakequant_fullcode(X, g, gd4, out=yf)
        tq.amax(X, out=gx)
        tq.fakequant_rtn(X, gx, out=yr)

    outs = (g, gx, codes, scales, gd, gd4, yg, yf, yr)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        for t in outs:
            t.view(torch.uint8).fill_(0xA5 if rep % 2 else 0x00)   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, r in zip(outs, ref):
            assert torch.equal(t.view(torch.uint8), r.view(torch.uint8)), f"replay {rep} differs"


def _saturating_pair(n, seed):
    """A training tensor much wider than its rollout copy (relative noise 0.3),
    so that many training values leave the rollout's block range and the
    forward saturates there."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(n) * np.exp(rng.uniform(-2, 2, n))
    Y, X = _pair_from_np(x, 0.3, seed)          # X = the noisy copy: the wider one
    return X, Y


def _bf16_grad(n, seed):
    rng = np.random.default_rng(seed)
    return torch.from_numpy(rng.standard_normal(n).astype(np.float32)).to(torch.bfloat16).to(DEV)


@pytest.mark.parametrize("ste", ["clipped", "identity"])
def test_qat_autograd_wrappers(tq, ste):
    """Each autograd wrapper against the oracle: the forward equals the
    oracle's fake-quant bit for bit (guided, full code, shared-scale RTN,
    own-scale RTN with a given g, and plain QAT with its own scales on both
    kernel paths, G = 1 and 4); the backward equals the oracle's clipped
    straight-through gradient (gy where |v| <= 6, +0 where the forward
    saturated) or gy itself with ste="identity".  The wrappers get the
    oracle's global scales and guidance as inputs, so every expected value
    comes from the oracle alone."""
    from precision_numerics_block_amd import qat

    n = 16 * 8192
    X, Y = _saturating_pair(n, 77)
    Xh, Yh = h16(X), h16(Y)
    og, _ = oracle.amax(Yh)
    oc, os_, ogd2 = oracle.quant_rollout(Yh, og, 2)
    ogd4 = oracle.guidance_pack(oc, os_, n, 4)
    ogx, _ = oracle.amax(Xh)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    g, gd2, gd4, sc, gx = dev(og), dev(ogd2), dev(ogd4), dev(os_), dev(ogx)
    cases = [("guided k=2", lambda x: qat.guided_fake_quant(x, g, gd2, 2, ste=ste),
              oracle.fakequant_guided(Xh, og, ogd2, 2)[0], og, os_, 1),
             ("full code", lambda x: qat.fullcode_fake_quant(x, g, gd4, ste=ste),
              oracle.fakequant_fullcode(Xh, og, ogd4)[0], og, os_, 1),
             ("rtn shared scales", lambda x: qat.rtn_fake_quant(x, g, sc, ste=ste),
              oracle.fakequant_rtn(Xh, og, os_)[0], og, os_, 1)]
    oy, _, own = oracle.fakequant_rtn(Xh, ogx, None)
    cases.append(("rtn own scales", lambda x: qat.rtn_fake_quant(x, gx, ste=ste), oy, ogx, own, 1))
    for G in (1, 4):
        ogG, _ = oracle.amax(Xh, G)
        oyG, _, ownG = oracle.fakequant_rtn(Xh, ogG, None, G)
        for path in qat.PATHS:
            cases.append((f"own scales G={G} {path}",
                          lambda x, G=G, path=path: qat.own_scale_fake_quant(x, G, path=path, ste=ste),
                          oyG, ogG, ownG, G))
    saturated = 0
    for i, (what, fwd, want_y, og_, osc, G) in enumerate(cases):
        x = X.clone().requires_grad_(True)
        y = fwd(x)
        assert_eq(h16(y), want_y, f"{what}: forward")
        gy = _bf16_grad(n, 100 + i)
        y.backward(gy)
        want_g = h16(gy)
        if ste == "clipped":
            want_g = oracle.ste_grad(Xh, og_, osc, h16(gy), G)
            saturated += int((oracle.ste_mask(Xh, og_, osc, G) == 0).sum())
        assert_eq(h16(x.grad), want_g, f"{what}: gradient")
    if ste == "clipped":
        assert saturated > 100, "the case must exercise the clipped gradient"
    # a tiny training step through the guided fake-quant
    w = torch.randn(2048, 64, device=DEV, dtype=torch.float32, requires_grad=True)
    x = X.reshape(-1, 2048).clone().requires_grad_(True)
    loss = (qat.guided_fake_quant(x, g, gd2, 2, ste=ste).float() @ w).square().mean()
    loss.backward()
    assert torch.isfinite(w.grad).all() and x.grad is not None and torch.isfinite(x.grad.float()).all()


def test_qat_onepass_recovers_from_barrier_timeout(tq, monkeypatch):
    """Plain QAT on the one-pass path with the grid barrier forced to give
    up (a zero time limit set from the host): the wrapper reads the status
    word, warns, and recomputes through the two-kernel path; the result is
    the oracle's, and the work buffer is zeroed for the next call."""
    from precision_numerics_block_amd import qat

    X, _ = synth.make_pair(2, 0, (8, 512, 2048), DEV)
    work = torch.zeros(tq.onepass_work_bytes(1), dtype=torch.uint8, device=DEV)
    monkeypatch.setenv("TRACE_ONEPASS_WAIT_US", "0")
    with pytest.warns(RuntimeWarning, match="timed out"):
        y = qat.own_scale_fake_quant(X, 1, work=work, path="onepass")
    monkeypatch.delenv("TRACE_ONEPASS_WAIT_US")
    torch.cuda.synchronize()
    assert bool((work == 0).all())
    Xh = h16(X)
    og, _ = oracle.amax(Xh)
    assert_eq(h16(y), oracle.fakequant_rtn(Xh, og, None)[0], "recomputed forward")
    y2 = qat.own_scale_fake_quant(X, 1, work=work, path="onepass")
    assert_eq(h16(y2), h16(y), "the next one-pass call")


@pytest.mark.parametrize("f32", [False, True])
def test_ste_grad_bruteforce(tq, f32):
    """trace_fakequant_ste_grad over every finite bf16 value (anchored
    blocks) with block scales drawn over the whole E4M3 range and global
    scales over many binades (one group per block), against the oracle;
    bf16 and f32 gradients, and in place (gx = gy)."""
    Xh = anchored_blocks()
    n = Xh.size
    nblk = n // 16
    rng = np.random.default_rng(41 + f32)
    scales = rng.integers(0, 127, nblk).astype(np.uint8)
    g = (2.0 ** rng.uniform(-40, 20, nblk)).astype(np.float32)
    g[::97] = 0.0
    X = to_dev_bf16(Xh)
    gy = torch.from_numpy(rng.standard_normal(n).astype(np.float32)).to(DEV)
    if not f32:
        gy = gy.to(torch.bfloat16)
    gd, sd = torch.from_numpy(g).to(DEV), torch.from_numpy(scales).to(DEV)
    gx = tq.fakequant_ste_grad(X, gd, sd, gy, nblk)
    gy_np = gy.cpu().numpy() if f32 else h16(gy)
    want = oracle.ste_grad(Xh, g, scales, gy_np, nblk)
    got = gx.cpu().numpy() if f32 else h16(gx)
    assert_eq(got.view(np.uint32) if f32 else got, want.view(np.uint32) if f32 else want, "ste grad")
    m = oracle.ste_mask(Xh, g, scales, nblk)
    assert 0.05 < (m == 0).mean() < 0.95, "both sides of the edge must be covered"
    tq.fakequant_ste_grad(X, gd, sd, gy, nblk, out=gy)          # in place
    got = gy.cpu().numpy() if f32 else h16(gy)
    assert_eq(got.view(np.uint32) if f32 else got, want.view(np.uint32) if f32 else want, "in place")
    # one group, ragged sizes
    for nb in (1, 37, 513 * 4 + 3):
        Xs = Xh[: 16 * nb]
        gs = np.float32([2.0 ** -7])
        ss = scales[:nb]
        gy_s = torch.from_numpy(rng.standard_normal(16 * nb).astype(np.float32)).to(DEV)
        got = tq.fakequant_ste_grad(to_dev_bf16(Xs), torch.from_numpy(gs).to(DEV), torch.from_numpy(ss).to(DEV),
                                    gy_s).cpu().numpy()
        want = oracle.ste_grad(Xs, gs, ss, gy_s.cpu().numpy())
        assert_eq(got.view(np.uint32), want.view(np.uint32), f"one group, {nb} blocks")


@pytest.mark.parametrize("wl", [3, 4, 5])
def test_kv_one_buffer_two_groups(tq, wl):
    """K and V of a layer in one [2, T, H, D] buffer with one global scale per
    tensor (G = 2), as the benchmark runs the KV workloads, through both the
    two-kernel path and the one-pass path the benchmark picks (one launch for
    the 2 x 32768 x 8 x 128 layer; one per group for the larger ones, which
    exceed the on-chip capacity); windows straddle the K/V boundary."""
    specs = synth.tensor_specs(wl)
    pk, pv = (1, 2) if wl == 5 else (0, 1)
    shape = specs[pk][1]
    K, Ky = synth.make_pair(wl, pk, shape, DEV)
    V, Vy = synth.make_pair(wl, pv, shape, DEV)
    X, Y = torch.stack([K, V]), torch.stack([Ky, Vy])
    del K, Ky, V, Vy
    nblk = X.numel() // 16
    half = nblk // 2
    wins = blocks_of(nblk, [(0, 400), (half - 300, half + 300), (nblk - 400, nblk)])
    for onepass in (None, 0):
        for k in synth.WORKLOADS[wl].ks:
            c = Checker(tq, X, Y, k, 2, onepass=onepass)
            c.run_gpu(out_f32=False)
            c.check(wins)
            del c
    check_rtn_onepass(tq, X, 2, 0, False, wins)
    del X, Y
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# One-pass rollout (amax and quantisation from one read): the same oracle
# comparisons.  A small workgroup cap makes small tensors use every storage
# path of a workgroup (registers, LDS, read twice) and group changes inside
# a workgroup's run of tiles.
# ---------------------------------------------------------------------------
ONEPASS_SMALL = [  # (workload, rows, tensor index, workgroup caps)
    (1, None, 0, (0, 1, 2)), (2, 2, 0, (0, 3)), (3, 1024, 0, (0, 3)), (4, 2048, 1, (0, 5)), (5, 1024, 2, (0, 7)),
]


@pytest.mark.parametrize("wl,rows,ti,caps", ONEPASS_SMALL)
def test_onepass_small_full_parity(tq, wl, rows, ti, caps):
    name, shape = synth.tensor_specs(wl, rows)[ti]
    X, Y = synth.make_pair(wl, ti, shape, DEV)
    for cap in caps:
        for k in (1, 2, 3, 4):
            for G in (1, 4):
                c = Checker(tq, X, Y, k, G, onepass=cap)
                c.run_gpu(out_f32=False)
                c.check()


@pytest.mark.parametrize("G,cap", [(2, 0), (4, 1), (8, 1), (8, 2), (16, 3), (64, 0), (64, 5)])
def test_onepass_group_scale_tables(tq, G, cap):
    """Groups of whole tiles (256 x 2048, 64 tiles): with no workgroup run
    spanning more than four groups the rollout uses per-group scale tables,
    otherwise the per-block divisions; both against the oracle (G, cap pairs
    chosen to land on each side: 8 groups with one workgroup spans 8)."""
    X, Y = synth.make_pair(1, 0, (256, 2048), DEV)
    for k in (2, 3):
        c = Checker(tq, X, Y, k, G, onepass=cap)
        c.run_gpu(out_f32=False)
        c.check()


ONEPASS_FULL = [(2, 0, 1), (2, 0, 64), (3, 0, 1), (4, 0, 1), (5, 0, 1), (5, 1, 1)]


def test_onepass_capacity(tq):
    """The 64x512x2048 activation tensor (and a layer's K and V together)
    fits on chip on one MI355X; a workgroup cap shrinks the capacity."""
    cap = tq.onepass_capacity()
    assert cap >= 64 * 512 * 2048, cap
    assert 0 < tq.onepass_capacity(16) < cap


@pytest.mark.parametrize("wl,ti,G", ONEPASS_FULL)
def test_onepass_full_size_sampled(tq, wl, ti, G):
    name, shape = synth.tensor_specs(wl)[ti]
    X, Y = synth.make_pair(wl, ti, shape, DEV)
    nblk = X.numel() // 16
    rng = np.random.default_rng(wl * 100 + ti + 7)
    amax_blk = int(torch.argmax(Y.float().abs().reshape(-1)).item()) // 16
    wins = [(0, 600), (nblk - 600, nblk), (amax_blk - 40, amax_blk + 40)]
    for s in rng.integers(0, nblk - 300, 6):
        wins.append((int(s), int(s) + 300))
    wins = blocks_of(nblk, wins)
    for k in synth.WORKLOADS[wl].ks:
        c = Checker(tq, X, Y, k, G, onepass=0)
        c.run_gpu(out_f32=False)
        c.check(wins)
    del X, Y
    torch.cuda.empty_cache()


# Tensors beyond the on-chip capacity with several groups: when one group
# fits, the one-pass entry points run one launch per block of whole groups,
# writing into the whole tensor's planes; when a group is larger than the
# chip, one launch reads the excess twice.  Outputs start as a canary so that
# every byte must come from a launch.  (tensor, size, G, workgroup cap, ks):
# "act" = size x 512 x 2048 activations (128 tiles of 8192 per row); "ragged"
# = size blocks of random data, groups ending mid-tile.
GROUP_BLOCKS = [
    ("act", 2, 4, 1, (2,)),              # 64-tile groups, 33 tiles on chip: excess read twice
    ("act", 2, 2, 3, (2,)),              # 128-tile groups, 99 on chip: excess read twice
    ("act", 2, 4, 2, (1, 2, 3, 4)),      # 66 on chip: 4 launches of one group
    ("act", 2, 4, 5, (1, 2, 3, 4)),      # 165 on chip: 2 launches of two groups
    ("act", 2, 8, 3, (1, 2, 3, 4)),      # 32-tile groups, 99 on chip: launches of 3, 3 and 2 groups
    ("ragged", 3 * 7001, 3, 1, (1, 2, 3, 4)),   # 14-tile groups (last tile short): launches of 2 and 1
    # one launch by teams of workgroups (groups of whole tiles, a team holds a
    # group on chip, at least two teams under the cap; 32 tiles per workgroup
    # on MI355X, 31 with f32 output):
    ("act", 4, 8, 8, (1, 2, 3, 4)),      # 64-tile groups: 4 teams of 2, two groups each (f32: 2 teams of 3)
    ("act", 3, 4, 7, (2,)),              # 96-tile groups: 2 teams of 3, LDS tiles in use (f32: launches)
    ("ragged", 5 * 37 * 512, 5, 4, (1, 2, 3, 4)),   # random data, 37-tile groups: shares of 18 and 19 tiles,
                                                    # team 0 takes three groups, team 1 two
    ("ragged", 300 * 512, 300, 8, (2,)),            # one-tile groups: 8 teams of one, 38 rounds (the last short)
    ("ragged", 2400 * 512, 2400, 70, (1, 4)),       # 64 teams (every team line in use), 38 rounds
]


def _group_blocks_pair(kind, size):
    if kind == "act":
        return synth.make_pair(2, 0, (size, 512, 2048), DEV)
    rng = np.random.default_rng(size)
    x = rng.standard_normal(16 * size) * np.exp(rng.uniform(-3, 3, 16 * size))
    return _pair_from_np(x, 0.01, size)


def _canary(n, dtype=torch.uint8):
    return torch.full((n,), 0xA5, dtype=torch.uint8, device=DEV).view(dtype)


@pytest.mark.parametrize("kind,size,G,cap,ks", GROUP_BLOCKS)
def test_onepass_group_blocks(tq, kind, size, G, cap, ks):
    X, Y = _group_blocks_pair(kind, size)
    n = X.numel()
    group_tiles = -(-(n // G // 8) // 1024)
    cap_tiles = tq.onepass_capacity(cap) // 8192
    assert G * group_tiles > cap_tiles, "the case must exceed the on-chip capacity"
    Xh, Yh = h16(X), h16(Y)
    gY, _ = oracle.amax(Yh, G)
    gX, _ = oracle.amax(Xh, G)
    for k in ks:
        g = torch.full((G,), -1.0, device=DEV)
        codes, scales, gd = _canary(n // 2), _canary(n // 16), _canary(tq.guidance_bytes(n, k))
        st = torch.zeros(4, dtype=torch.int32, device=DEV)
        tq.quant_rollout_onepass(Y, k, G, g=g, guidance=gd, codes=codes, scales=scales, max_workgroups=cap,
                                 status=st)
        torch.cuda.synchronize()
        assert int(st[0]) == 0
        oc, os_, ogd = oracle.quant_rollout(Yh, gY, k, G)
        assert_eq(g.cpu().numpy().view(np.uint32), gY.view(np.uint32), f"k={k} global scales")
        assert_eq(h8(codes), oc, f"k={k} codes")
        assert_eq(h8(scales), os_, f"k={k} scales")
        assert_eq(h8(gd), ogd, f"k={k} guidance stream (with pad)")
    for out_f32 in (False, True):
        g = torch.full((G,), -1.0, device=DEV)
        y = _canary(n * (4 if out_f32 else 2), torch.float32 if out_f32 else torch.bfloat16)
        c, sc = _canary(n // 2), _canary(n // 16)
        st = torch.zeros(4, dtype=torch.int32, device=DEV)
        tq.fakequant_rtn_onepass(X, G, g=g, out_dtype=tq.OUT_F32 if out_f32 else tq.OUT_BF16, out=y.view(X.shape),
                                 codes_out=c, scales_out=sc, max_workgroups=cap, status=st)
        torch.cuda.synchronize()
        assert int(st[0]) == 0
        oy, oc, os_ = oracle.fakequant_rtn(Xh, gX, None, G, out_f32)
        assert_eq(g.cpu().numpy().view(np.uint32), gX.view(np.uint32), "rtn global scales")
        if out_f32:
            assert_f32_close(y.cpu().numpy(), oy, "rtn y f32")
        else:
            assert_eq(h16(y), oy, "rtn y bf16")
        assert_eq(h8(c), oc, "rtn codes")
        assert_eq(h8(sc), os_, "rtn scales")


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_onepass_bruteforce(tq, k):
    Yh = anchored_blocks()
    nblk = Yh.size // 16
    Y = to_dev_bf16(Yh)
    for G, cap in ((nblk, 0), (nblk // 8 if nblk % 8 == 0 else 1, 0), (1, 5)):
        c = Checker(tq, Y, Y, k, G, onepass=cap)
        c.run_gpu(out_f32=False)
        c.check()


@pytest.mark.parametrize("nblk,G,cap", [(1, 1, 0), (2, 2, 0), (37, 1, 0), (3 * 512 + 6, 3, 1),
                                        (2048 * 512 + 1234, 1, 0), (2048 * 513, 513, 0), (2048 * 513, 513, 9)])
def test_onepass_sizes_and_degenerate(tq, nblk, G, cap):
    rng = np.random.default_rng(nblk + cap)
    x = rng.standard_normal(16 * nblk) * np.exp(rng.uniform(-3, 3, 16 * nblk))
    X, Y = _pair_from_np(x, 0.01, nblk)
    for k in (1, 2, 3, 4):
        c = Checker(tq, X, Y, k, G, onepass=cap)
        c.run_gpu(out_f32=False)
        if nblk > 100000:
            c.check(blocks_of(nblk, [(0, 700), (nblk - 700, nblk), (nblk // 2, nblk // 2 + 700)]))
        else:
            c.check()
    for case in ("zeros", "negzeros", "tiny"):
        z = {"zeros": np.zeros(16 * 64), "negzeros": -np.zeros(16 * 64),
             "tiny": rng.standard_normal(16 * 64) * 1e-39}[case]
        X, Y = _pair_from_np(z, 0.02, 3)
        c = Checker(tq, X, Y, 2, 1, onepass=cap)
        c.run_gpu(out_f32=False)
        c.check()


def test_onepass_nonfinite_flag_and_repeat(tq):
    x = np.ones(16 * 4096, np.float32)
    x[5] = np.inf
    x[7000] = np.nan
    x[300] = 12.0
    X = torch.from_numpy(x).to(torch.bfloat16).to(DEV)
    st = torch.zeros(4, dtype=torch.int32, device=DEV)
    work = torch.zeros(tq.onepass_work_bytes(2), dtype=torch.uint8, device=DEV)
    g, codes, scales, gd = tq.quant_rollout_onepass(X, 2, status=st, work=work)
    torch.cuda.synchronize()
    assert int(st[0]) == -7
    assert bool((work == 0).all()), "the call leaves its work buffer zeroed"
    og, _ = oracle.amax(h16(X))
    assert np.array_equal(g.cpu().numpy().view(np.uint32), og.view(np.uint32))
    # the same work buffer again, several calls with other sizes, group
    # counts (up, down and up again) and workgroup caps: each call finds it
    # zeroed by the previous one
    X2, Y2 = synth.make_pair(1, 0, (256, 2048), DEV)
    for G, cap in ((1, 0), (2, 0), (1, 3), (2, 5), (1, 0), (8, 0), (1, 0), (8, 2), (4, 0), (8, 0)):
        st.zero_()
        g2, c2, s2, gd2 = tq.quant_rollout_onepass(Y2, 2, G, status=st, work=work, max_workgroups=cap)
        torch.cuda.synchronize()
        assert int(st[0]) == 0
        assert bool((work == 0).all())
        og2, _ = oracle.amax(h16(Y2), G)
        oc, os_, ogd = oracle.quant_rollout(h16(Y2), og2, 2, G)
        assert_eq(g2.cpu().numpy().view(np.uint32), og2.view(np.uint32), f"g G={G} cap={cap}")
        assert_eq(h8(c2), oc, f"codes G={G} cap={cap}")
        assert_eq(h8(s2), os_, f"scales G={G} cap={cap}")
        assert_eq(h8(gd2), ogd, f"guidance G={G} cap={cap}")


def test_onepass_teams_nonfinite_and_work_reuse(tq):
    """The launch by teams (8 groups of 64 tiles under a cap of 8 workgroups:
    4 teams of 2, two rounds each) on input with an inf and a NaN in two
    groups of different teams and rounds (one in an LDS tile, one in a
    register tile): the status word reports TRACE_E_NONFINITE and the global
    scales equal the oracle's (which skips non-finite values in the group
    maxima).  Non-finite inputs are outside the contract, so the outputs of
    the two blocks that hold them are left unchecked; every other byte must
    equal the oracle's.  The same work buffer then serves a one-launch call
    and the launch by teams again, each exact."""
    G, cap = 8, 8
    X, Y = synth.make_pair(2, 0, (4, 512, 2048), DEV)
    n = Y.numel()
    per = n // G
    bad_el = (1 * per + 123, 6 * per + 4567 + 16 * 512 * 30)   # LDS tile 0, register tile 30 (member 0)
    yb = Y.reshape(-1).clone()
    yb[bad_el[0]] = float("inf")
    yb[bad_el[1]] = float("nan")
    bad_blk = [e // 16 for e in bad_el]

    def keep(nbytes, per_block):
        m = np.ones(nbytes, bool)
        for b in bad_blk:
            m[b * per_block:(b + 1) * per_block] = False
        return m

    work = torch.zeros(tq.onepass_work_bytes(G), dtype=torch.uint8, device=DEV)
    st = torch.zeros(4, dtype=torch.int32, device=DEV)
    for Yc, Gc, capc, flag in ((yb.view_as(Y), G, cap, -7), (Y, 2, 0, 0), (Y, G, cap, 0)):
        st.zero_()
        g, codes, scales, gd = tq.quant_rollout_onepass(Yc, 2, Gc, status=st, work=work, max_workgroups=capc)
        torch.cuda.synchronize()
        assert int(st[0]) == flag
        assert bool((work == 0).all()), "the call leaves its work buffer zeroed"
        Yh = h16(Yc)
        og, _ = oracle.amax(Yh, Gc)
        oc, os_, ogd = oracle.quant_rollout(Yh, og, 2, Gc)
        what = f"G={Gc} cap={capc}"
        assert_eq(g.cpu().numpy().view(np.uint32), og.view(np.uint32), f"g {what}")
        mc, ms = keep(n // 2, 8), keep(n // 16, 1)
        bits0 = tq.guidance_bytes(n, 2) - n // 4
        mg = np.concatenate([ms, np.ones(bits0 - n // 16, bool), keep(n // 4, 4)])
        if flag == 0:
            mc[:], ms[:], mg[:] = True, True, True
        assert_eq(h8(codes)[mc], oc[mc], f"codes {what}")
        assert_eq(h8(scales)[ms], os_[ms], f"scales {what}")
        assert_eq(h8(gd)[mg], ogd[mg], f"guidance {what}")
    xb = X.reshape(-1).clone()
    xb[bad_el[0]] = float("-inf")
    st.zero_()
    gx, y, _, _ = tq.fakequant_rtn_onepass(xb.view_as(X), G, status=st, work=work, max_workgroups=cap)
    torch.cuda.synchronize()
    assert int(st[0]) == -7 and bool((work == 0).all())
    Xh = h16(xb)
    ogx, _ = oracle.amax(Xh, G)
    oy, _, _ = oracle.fakequant_rtn(Xh, ogx, None, G, False)
    assert_eq(gx.cpu().numpy().view(np.uint32), ogx.view(np.uint32), "rtn g")
    my = keep(n, 16)
    my[bad_blk[1] * 16:(bad_blk[1] + 1) * 16] = True       # only the first block holds a non-finite x here
    assert_eq(h16(y)[my], oy[my], "rtn y")


def test_onepass_graph_replay_matches_eager(tq):
    X, Y = synth.make_pair(2, 0, (4, 512, 2048), DEV)
    n = Y.numel()
    g = torch.empty(2, device=DEV)
    codes = torch.empty(n // 2, dtype=torch.uint8, device=DEV)
    scales = torch.empty(n // 16, dtype=torch.uint8, device=DEV)
    gd = torch.empty(tq.guidance_bytes(n, 2), dtype=torch.uint8, device=DEV)
    work = torch.zeros(tq.onepass_work_bytes(2), dtype=torch.uint8, device=DEV)

    def step():
        tq.quant_rollout_onepass(Y, 2, 2, g=g, guidance=gd, codes=codes, scales=scales, work=work)

    outs = (g, codes, scales, gd)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    og, _ = oracle.amax(h16(Y), 2)
    assert_eq(ref[0].cpu().numpy().view(np.uint32), og.view(np.uint32), "g")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        for t in outs:
            t.view(torch.uint8).fill_(0xA5 if rep % 2 else 0x00)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, r in zip(outs, ref):
            assert torch.equal(t.view(torch.uint8), r.view(torch.uint8)), f"replay {rep} differs"
        assert bool((work == 0).all()), f"replay {rep} left the work buffer dirty"


def test_onepass_barrier_timeout_reported(tq, monkeypatch):
    """The failure path of the bounded grid barrier, forced from the host with
    a zero time limit: the workgroups that wait give up, every kernel exits,
    and the status word reports TRACE_E_BARRIER.  Every workgroup still counts
    out, so the work buffer comes back zeroed, and the next calls on the same
    buffer (rollout, then own-scale RTN, with no fill in between) are exact."""
    X, Y = synth.make_pair(2, 0, (8, 512, 2048), DEV)
    work = torch.zeros(tq.onepass_work_bytes(1), dtype=torch.uint8, device=DEV)
    st = torch.zeros(4, dtype=torch.int32, device=DEV)
    monkeypatch.setenv("TRACE_ONEPASS_WAIT_US", "0")
    tq.quant_rollout_onepass(Y, 2, status=st, work=work)
    torch.cuda.synchronize()
    assert int(st[0]) == -10
    assert bool((work == 0).all()), "a timed-out call leaves the work buffer zeroed"
    st.zero_()
    tq.fakequant_rtn_onepass(X, status=st, work=work)
    torch.cuda.synchronize()
    assert int(st[0]) == -10
    assert bool((work == 0).all()), "a timed-out RTN call leaves the work buffer zeroed"
    monkeypatch.delenv("TRACE_ONEPASS_WAIT_US")
    st.zero_()
    g, codes, scales, gd = tq.quant_rollout_onepass(Y, 2, status=st, work=work)
    torch.cuda.synchronize()
    assert int(st[0]) == 0 and bool((work == 0).all())
    og, _ = oracle.amax(h16(Y))
    oc, os_, ogd = oracle.quant_rollout(h16(Y), og, 2)
    assert_eq(g.cpu().numpy().view(np.uint32), og.view(np.uint32), "g")
    assert_eq(h8(codes), oc, "codes")
    assert_eq(h8(gd), ogd, "guidance")
    gx, y, _, _ = tq.fakequant_rtn_onepass(X, status=st, work=work)
    torch.cuda.synchronize()
    assert int(st[0]) == 0 and bool((work == 0).all())
    ogx, _ = oracle.amax(h16(X))
    oy, _, _ = oracle.fakequant_rtn(h16(X), ogx, None, 1, False)
    assert_eq(gx.cpu().numpy().view(np.uint32), ogx.view(np.uint32), "rtn g")
    assert_eq(h16(y), oy, "rtn y")


def test_onepass_teams_barrier_timeout_reported(tq, monkeypatch):
    """The failure path of the per-team barriers of the launch by teams
    (8 groups of 64 tiles under a cap of 8 workgroups: 4 teams of 2, two
    rounds each), forced from the host with a zero time limit: the status
    word reports TRACE_E_BARRIER, every kernel exits, the work buffer comes
    back zeroed, and the next calls on it (rollout and own-scale RTN) are
    exact against the oracle."""
    X, Y = synth.make_pair(2, 0, (4, 512, 2048), DEV)
    G, cap = 8, 8
    work = torch.zeros(tq.onepass_work_bytes(G), dtype=torch.uint8, device=DEV)
    st = torch.zeros(4, dtype=torch.int32, device=DEV)
    monkeypatch.setenv("TRACE_ONEPASS_WAIT_US", "0")
    tq.quant_rollout_onepass(Y, 2, G, status=st, work=work, max_workgroups=cap)
    tq.fakequant_rtn_onepass(X, G, status=st, work=work, max_workgroups=cap)
    torch.cuda.synchronize()
    assert int(st[0]) == -10
    assert bool((work == 0).all()), "timed-out calls leave the work buffer zeroed"
    monkeypatch.delenv("TRACE_ONEPASS_WAIT_US")
    st.zero_()
    g, codes, scales, gd = tq.quant_rollout_onepass(Y, 2, G, status=st, work=work, max_workgroups=cap)
    gx, y, _, _ = tq.fakequant_rtn_onepass(X, G, status=st, work=work, max_workgroups=cap)
    torch.cuda.synchronize()
    assert int(st[0]) == 0 and bool((work == 0).all())
    Yh, Xh = h16(Y), h16(X)
    og, _ = oracle.amax(Yh, G)
    oc, os_, ogd = oracle.quant_rollout(Yh, og, 2, G)
    assert_eq(g.cpu().numpy().view(np.uint32), og.view(np.uint32), "g")
    assert_eq(h8(codes), oc, "codes")
    assert_eq(h8(scales), os_, "scales")
    assert_eq(h8(gd), ogd, "guidance")
    ogx, _ = oracle.amax(Xh, G)
    oy, _, _ = oracle.fakequant_rtn(Xh, ogx, None, G, False)
    assert_eq(gx.cpu().numpy().view(np.uint32), ogx.view(np.uint32), "rtn g")
    assert_eq(h16(y), oy, "rtn y")


@pytest.mark.parametrize("cap", [1, 2, 5])
def test_onepass_many_groups_per_workgroup(tq, cap):
    """More groups in one workgroup's run of items than its 128 LDS slots of
    global scales (3000 groups of one block, 1500 of two, 375 of eight, over
    1, 2 or 5 workgroups): groups past the slots take the per-item read of the
    group maxima, which every wave must finish before its workgroup counts
    out and the last one out clears them.  Rollout at every k and own-scale
    RTN in bf16 and f32, against the oracle."""
    rng = np.random.default_rng(300 + cap)
    nblk = 3000
    x = rng.standard_normal(16 * nblk) * np.exp(rng.uniform(-3, 3, 16 * nblk))
    X, Y = _pair_from_np(x, 0.01, nblk + cap)
    for G in (nblk, nblk // 2, nblk // 8):
        for k in (1, 2, 3, 4):
            c = Checker(tq, X, Y, k, G, onepass=cap)
            c.run_gpu(out_f32=False)
            c.check()
        for out_f32 in (False, True):
            check_rtn_onepass(tq, X, G, cap, out_f32)


# ---------------------------------------------------------------------------
# One-pass plain QAT (amax(x) + own-scale RTN from one read): against the
# oracle's amax and own-scale RTN
# ---------------------------------------------------------------------------
def check_rtn_onepass(tq, X, G, cap, out_f32, windows=None):
    od = tq.OUT_F32 if out_f32 else tq.OUT_BF16
    st = torch.zeros(4, dtype=torch.int32, device=DEV)
    g, y, c, s = tq.fakequant_rtn_onepass(X, G, out_dtype=od, codes_out=True, scales_out=True,
                                          max_workgroups=cap, status=st)
    torch.cuda.synchronize()
    assert int(st[0]) == 0
    Xh = h16(X)
    og, _ = oracle.amax(Xh, G)
    assert_eq(g.cpu().numpy().view(np.uint32), og.view(np.uint32), "g")
    nblk = X.numel() // 16
    for b0, b1 in (windows or [(0, nblk)]):
        e0, e1 = 16 * b0, 16 * b1
        oy, oc, os_ = oracle.fakequant_rtn(Xh, og, None, G, out_f32, b0, b1)
        yy = y.reshape(-1)[e0:e1]
        if out_f32:
            assert_f32_close(yy.cpu().numpy(), oy[e0:e1], f"y {b0}:{b1}")
        else:
            assert_eq(h16(yy), oy[e0:e1], f"y {b0}:{b1}")
        assert_eq(h8(c[e0 // 2:e1 // 2]), oc[e0 // 2:e1 // 2], f"codes {b0}:{b1}")
        assert_eq(h8(s[b0:b1]), os_[b0:b1], f"scales {b0}:{b1}")


@pytest.mark.parametrize("wl,rows,ti,caps", ONEPASS_SMALL)
def test_rtn_onepass_small_full_parity(tq, wl, rows, ti, caps):
    name, shape = synth.tensor_specs(wl, rows)[ti]
    X, _ = synth.make_pair(wl, ti, shape, DEV)
    for cap in caps:
        for G in (1, 4):
            for out_f32 in (False, True):
                check_rtn_onepass(tq, X, G, cap, out_f32)


@pytest.mark.parametrize("wl,ti,G", [(2, 0, 1), (2, 0, 64), (3, 0, 1), (5, 0, 1)])
def test_rtn_onepass_full_size_sampled(tq, wl, ti, G):
    name, shape = synth.tensor_specs(wl)[ti]
    X, _ = synth.make_pair(wl, ti, shape, DEV)
    nblk = X.numel() // 16
    rng = np.random.default_rng(wl * 10 + ti + 3)
    amax_blk = int(torch.argmax(X.float().abs().reshape(-1)).item()) // 16
    wins = [(0, 600), (nblk - 600, nblk), (amax_blk - 40, amax_blk + 40)]
    wins += [(int(s), int(s) + 300) for s in rng.integers(0, nblk - 300, 6)]
    check_rtn_onepass(tq, X, G, 0, False, blocks_of(nblk, wins))
    del X
    torch.cuda.empty_cache()


def test_rtn_onepass_bruteforce_and_sizes(tq):
    Yh = anchored_blocks()
    nblk = Yh.size // 16
    X = to_dev_bf16(Yh)
    for G, cap in ((nblk, 0), (1, 5)):
        check_rtn_onepass(tq, X, G, cap, G == 1)
    rng = np.random.default_rng(21)
    for nb, G, cap in ((1, 1, 0), (37, 1, 0), (3 * 512 + 6, 3, 1), (2048 * 513, 513, 0)):
        x = rng.standard_normal(16 * nb) * np.exp(rng.uniform(-3, 3, 16 * nb))
        X, _ = _pair_from_np(x, 0.01, nb)
        w = None if nb < 100000 else blocks_of(nb, [(0, 700), (nb - 700, nb), (nb // 2, nb // 2 + 700)])
        check_rtn_onepass(tq, X, G, cap, False, w)


def test_rtn_onepass_graph_replay_and_work_reuse(tq):
    X, _ = synth.make_pair(2, 0, (4, 512, 2048), DEV)
    g = torch.empty(1, device=DEV)
    y = torch.empty_like(X)
    work = torch.zeros(tq.onepass_work_bytes(1), dtype=torch.uint8, device=DEV)
    step = lambda: tq.fakequant_rtn_onepass(X, 1, g=g, out=y, work=work)  # noqa: E731
    step()
    torch.cuda.synchronize()
    ref_g, ref_y = g.clone(), y.clone()
    gx = tq.amax(X)
    yr, _, _ = tq.fakequant_rtn(X, gx)
    torch.cuda.synchronize()
    assert torch.equal(ref_g, gx) and torch.equal(ref_y.view(torch.int16), yr.view(torch.int16))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        y.view(torch.uint8).fill_(0xA5 if rep % 2 else 0)
        g.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref_y.view(torch.int16)) and torch.equal(g, ref_g), rep
        assert bool((work == 0).all())
    # the same buffer alternating with the one-pass rollout (same layout)
    _, Y = synth.make_pair(2, 0, (4, 512, 2048), DEV)
    gy = tq.amax(Y)
    cy, sy, dy = tq.quant_rollout(Y, gy, 2)
    for rep in range(3):
        g1, c1, s1, d1 = tq.quant_rollout_onepass(Y, 2, work=work)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(g1, gy) and torch.equal(c1, cy) and torch.equal(s1, sy) and torch.equal(d1, dy), rep
        assert torch.equal(y.view(torch.int16), ref_y.view(torch.int16)) and torch.equal(g, ref_g), rep
        assert bool((work == 0).all())

