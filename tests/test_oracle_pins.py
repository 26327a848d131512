"""Pins of the CPU oracle against facts fixed outside it.

Each test checks the oracle against something other than its own formulas:
the pages' worked example, a hand-derived decision table, a library routine
that covers a special case (torch's fp8/bf16 conversions, numpy's rint), closed
forms and invariants that follow from the rule.  Plausible slips (a dropped
factor in the global scale, a wrong tie rule, a flipped sign, a transposed
operand, a wrong bit order) each break at least one of them.
"""
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

GOLD = os.path.join(os.path.dirname(__file__), "golden")
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def read_kv(name):
    out = {}
    for line in open(os.path.join(GOLD, name)):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split()
            out[k] = float(v)
    return out


def read_table():
    tables, cur = {}, None
    for line in open(os.path.join(GOLD, "guided_table.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        if line.startswith("k="):
            cur = int(line[2:])
            tables[cur] = []
            continue
        parts = line.split()
        tables[cur].append((float(parts[0]), float(parts[1]), parts[2:]))
    return tables


def f32(x):
    return np.float32(x)


def bf16_bits(vals):
    return torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bits_to_f32(bits):
    return np.asarray(bits, np.uint32).view(np.float32)


def next_up(x):
    return np.nextafter(np.float32(x), np.float32(np.inf))


def next_down(x):
    return np.nextafter(np.float32(x), np.float32(-np.inf))


# --------------------------------------------------------------------------
# Worked example (Figure 1 of the article)
# --------------------------------------------------------------------------
def test_worked_example_scalar(orc):
    W = read_kv("worked_example.txt")
    c = W["combined_scale"]
    # the combined scale follows from the printed numbers
    assert round(W["training_value"] / c, 2) == W["training_normalised"]
    assert round(W["rollout_value"] / c, 2) == W["rollout_normalised"]
    assert abs(W["training_value"] - W["rollout_value"] - W["raw_difference"]) < 1e-9
    inv = f32(1.0) / f32(c)
    vt = f32(W["training_value"]) * inv
    vr = f32(W["rollout_value"]) * inv
    jt, jr = orc.rtn_index(vt), orc.rtn_index(vr)
    assert E2M1[jt] == W["training_rtn"] and E2M1[jr] == W["rollout_rtn"]
    assert (E2M1[jt] - E2M1[jr]) * c == W["amplified_diff"]
    for k in (1, 2, 3):
        nib = orc.guided_nibble(vt, k, jr & ((1 << k) - 1))
        assert E2M1[nib & 7] == W["guided_training"]
    assert E2M1[orc.fullcode_nibble(vt, jr) & 7] == W["guided_training"]


def test_worked_example_tensor(orc):
    """Tensor-level replay: a tensor amax of 2688 gives g = 1, a block amax of
    144 gives block scale 24 (exact in E4M3), so the example's two values sit
    at a combined scale of 24.  bf16 keeps them on their sides of the 2.5
    boundary (60.24 -> 60.25, 59.76 -> 59.75)."""
    W = read_kv("worked_example.txt")
    x = np.zeros(32, np.float32)
    y = np.zeros(32, np.float32)
    x[0] = y[0] = 2688.0
    x[16] = y[16] = 6.0 * W["combined_scale"]
    x[17], y[17] = W["training_value"], W["rollout_value"]
    rng = np.random.default_rng(0)
    x[18:] = y[18:] = rng.uniform(-20, 20, 14)
    X, Y = bf16_bits(x), bf16_bits(y)
    g, st_ = orc.amax(Y)
    assert st_ == 0 and g[0] == 1.0
    for k in (1, 2, 3):
        codes, scales, gd = orc.quant_rollout(Y, g, k)
        assert orc.e4m3_value(scales[1]) == W["combined_scale"]
        rn = orc.unpack_nibbles(codes)
        assert E2M1[rn[17] & 7] == W["rollout_rtn"]
        yr, cr, _ = orc.fakequant_rtn(X, g, scales_in=scales, out_f32=True)
        yg, cg = orc.fakequant_guided(X, g, gd, k, out_f32=True)
        assert yr[17] == W["training_rtn"] * W["combined_scale"]
        assert yr[17] - orc.dequant(rn[17], scales[1], g[0]) == W["amplified_diff"]
        assert yg[17] == W["guided_training"] * W["combined_scale"]
    gd4 = orc.guidance_pack(codes, scales, 32, 4)
    yf, _ = orc.fakequant_fullcode(X, g, gd4, out_f32=True)
    assert yf[17] == W["guided_training"] * W["combined_scale"]


@pytest.mark.parametrize("e", [-30, -7, 3, 40])
def test_worked_example_scaled(orc, e):
    """Scaling every input by 2^e scales g by 2^e and leaves block scales and
    codes alone, so every dequantised value (and the difference of 24) scales
    by exactly 2^e (all products stay exact in fp32)."""
    W = read_kv("worked_example.txt")
    f = 2.0 ** e
    x = np.zeros(32, np.float32)
    y = np.zeros(32, np.float32)
    x[0] = y[0] = 2688.0 * f
    x[16] = y[16] = 6.0 * W["combined_scale"] * f
    x[17], y[17] = np.float32(W["training_value"]) * f, np.float32(W["rollout_value"]) * f
    X, Y = bf16_bits(x), bf16_bits(y)
    g, _ = orc.amax(Y)
    assert g[0] == f
    codes, scales, gd = orc.quant_rollout(Y, g, 2)
    yr, _, _ = orc.fakequant_rtn(X, g, scales_in=scales, out_f32=True)
    yg, _ = orc.fakequant_guided(X, g, gd, 2, out_f32=True)
    rn = orc.unpack_nibbles(codes)
    assert yr[17] == W["training_rtn"] * W["combined_scale"] * f
    assert orc.dequant(rn[17], scales[1], g[0]) == W["rollout_rtn"] * W["combined_scale"] * f
    assert yg[17] == W["guided_training"] * W["combined_scale"] * f
    yb, _ = orc.fakequant_guided(X, g, gd, 2, out_f32=False)
    assert yb[17] == bf16_bits([W["guided_training"] * W["combined_scale"] * f])[0]


# --------------------------------------------------------------------------
# Number formats against library routines
# --------------------------------------------------------------------------
def test_e2m1_codebook(orc):
    # OCP MX v1.0 FP4 E2M1 value table; 16 codes (the Russian commentary page
    # counts 16 values in four bits)
    table = E2M1 + [-v for v in E2M1]
    got = [orc.e2m1_value(n) for n in range(16)]
    assert got == table
    assert np.signbit(got[8])


def test_e4m3_decode_matches_torch(orc):
    codes = torch.arange(127, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).float().numpy()
    got = np.array([orc.e4m3_value(c) for c in range(127)])
    np.testing.assert_array_equal(got, ref)
    assert got.max() == 448.0 and got[1] == 2.0 ** -9


def test_e4m3_encode_matches_torch(orc):
    vals = np.array([orc.e4m3_value(c) for c in range(127)], np.float64)
    pts = [0.0]
    for a, b in zip(vals[:-1], vals[1:]):
        m = np.float32((a + b) / 2)
        pts += [a, b, m, next_up(m), next_down(m), next_up(next_up(m)), next_down(next_down(m))]
    rng = np.random.default_rng(1)
    pts += list(np.exp2(rng.uniform(-14, np.log2(464), 20000)).astype(np.float32))
    pts += [448.0, 455.0, next_down(464.0), 464.0]
    pts = np.array(pts, np.float32)
    ref = torch.from_numpy(pts).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.e4m3_encode(t) for t in pts], np.uint8)
    np.testing.assert_array_equal(got, ref)
    # saturation (closed form: satfinite clamps to the largest finite value)
    for t in [next_up(464.0), 480.0, 1e6, 3.0e38]:
        assert orc.e4m3_encode(t) == 126


def rint_rtn_value(a):
    """RTN onto E2M1 via numpy rint (round half to even) on each binade's
    integer grid: step 0.5 on [0,2], 1 on [2,4], 2 on [4,6]; saturate at 6."""
    a = min(float(abs(a)), 6.0)
    if a <= 2.0:
        return float(np.rint(2.0 * a)) / 2.0
    if a <= 4.0:
        return float(np.rint(a))
    return 2.0 * float(np.rint(a / 2.0))


def test_rtn_matches_rint(orc):
    pts = [0.0, 1e-40, 6.0, 6.5, 7.0, 1e30, np.inf]
    for a, b in zip(E2M1[:-1], E2M1[1:]):
        m = np.float32((a + b) / 2)
        pts += [a, m, next_up(m), next_down(m), next_up(a), next_down(b)]
    rng = np.random.default_rng(2)
    pts += list(rng.uniform(0, 7, 20000).astype(np.float32))
    for p in pts:
        for s in (1.0, -1.0):
            v = np.float32(s * p)
            nib = orc.rtn_nibble(v)
            assert E2M1[nib & 7] == rint_rtn_value(v), v
            assert bool(nib & 8) == bool(np.signbit(v))


def test_bf16_rounding_matches_torch(orc):
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 0x7F7F0000, 20000, dtype=np.uint32)
    ties = (bits & 0xFFFF0000) | 0x8000          # exact halfway cases
    near = (bits & 0xFFFF0000) | 0x7FFF
    top = np.arange(0x7F7F0000, 0x7F800001, 97, dtype=np.uint32)       # the top binade, overflow to inf
    special = np.array([0x7F7F7FFF, 0x7F7F8000, 0x7F7F8001, 0x7F7FFFFF, 0x7F800000, 0x00000001, 0x00008000,
                        0x00018000], np.uint32)
    allb = np.concatenate([bits, ties, near, top, special, bits | 0x80000000, ties | 0x80000000,
                           top | 0x80000000, special | 0x80000000])
    f = bits_to_f32(allb)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.f32_to_bf16(v) for v in f], np.uint16)
    np.testing.assert_array_equal(got, ref)


# --------------------------------------------------------------------------
# Guided rounding against the hand-derived table
# --------------------------------------------------------------------------
def _probe_points(lo, hi, thr):
    pts = [next_up(lo), next_down(hi), np.float32(lo + 0.25 * (hi - lo)),
           np.float32(lo + 0.5 * (hi - lo)), np.float32(lo + 0.75 * (hi - lo))]
    if thr is not None:
        t = np.float32(thr)
        pts += [t, next_up(t), next_down(t)]
    return pts


@pytest.mark.parametrize("k", [1, 2, 3])
def test_guided_matches_hand_table(orc, k):
    table = read_table()[k]
    assert len(table) == 7
    for lo, hi, cols in table:
        assert len(cols) == 1 << k
        jl, jh = E2M1.index(lo), E2M1.index(hi)
        for gb, entry in enumerate(cols):
            thr, tie_side = None, None
            if entry.startswith("T="):
                t, tie_side = entry[2:].split("/")
                thr = float(t)
            for p in _probe_points(lo, hi, thr):
                if thr is None:
                    want = jl if entry == "lo" else jh
                elif p < thr:
                    want = jl
                elif p > thr:
                    want = jh
                else:
                    want = jl if tie_side == "lo" else jh
                for s in (1.0, -1.0):
                    v = np.float32(s * p)
                    nib = orc.guided_nibble(v, k, gb)
                    assert (nib & 7) == want, (k, lo, hi, gb, float(v))
                    assert bool(nib & 8) == (s < 0)


def test_guided_on_grid_and_saturation(orc):
    for k in (1, 2):
        for gb in range(1 << k):
            for j, val in enumerate(E2M1):
                assert orc.guided_nibble(np.float32(val), k, gb) == j
                assert orc.guided_nibble(np.float32(-val), k, gb) == 8 | j
            for big in (6.0, 6.3, 100.0, 3e38, np.inf):
                assert orc.guided_nibble(np.float32(big), k, gb) == 7
                assert orc.guided_nibble(np.float32(-big), k, gb) == 15


def test_fullcode_rule(orc):
    """Full code: chosen = lo when the rollout value is at or below lo,
    otherwise hi (signed values), which is 'the adjacent point nearer the
    rollout code' for adjacent lo < hi."""
    rng = np.random.default_rng(4)
    signed = sorted(set(E2M1 + [-v for v in E2M1]))
    for v in list(rng.uniform(-6.5, 6.5, 4000).astype(np.float32)):
        if abs(v) >= 6 or float(v) in signed:
            continue
        lo = max(s for s in signed if s <= v)
        hi = min(s for s in signed if s >= v)
        for r in range(16):
            rv = orc.e2m1_value(r)
            want = lo if rv <= lo else hi
            nib = orc.fullcode_nibble(v, r)
            assert orc.e2m1_value(nib) == want or (want == 0 and (nib & 7) == 0)


# --------------------------------------------------------------------------
# Invariants (hypothesis)
# --------------------------------------------------------------------------
finite_f32 = st.floats(min_value=-8.0, max_value=8.0, width=32, allow_nan=False)


@settings(max_examples=3000, deadline=None)
@given(v=finite_f32, k=st.sampled_from([1, 2, 3]), gb=st.integers(0, 7))
def test_invariants_scalar(orc, v, k, gb):
    gb &= (1 << k) - 1
    v = np.float32(v)
    rt = orc.rtn_nibble(v)
    gd = orc.guided_nibble(v, k, gb)
    # I1: one adjacent step at most, same sign bit
    assert abs((gd & 7) - (rt & 7)) <= 1 and (gd & 8) == (rt & 8)
    # I2: guidance bits equal to the training RTN code's bits -> RTN
    assert orc.guided_nibble(v, k, (rt & 7) & ((1 << k) - 1)) == rt
    assert orc.fullcode_nibble(v, rt) == rt
    # I4: odd symmetry
    assert orc.guided_nibble(-v, k, gb) == gd ^ 8
    # I3: a rollout code adjacent to v is reproduced (full code, k = 2; k = 1
    # except where the E2M1 step doubles: r = 3 with |v| in (2, 2.25] and
    # r = 6 with |v| in (4, 4.5])
    a = abs(float(v))
    if a < 6 and a not in E2M1:
        jl = max(j for j in range(8) if E2M1[j] <= a)
        for r in (jl, jl + 1):
            sign = 8 if np.signbit(v) else 0
            assert orc.fullcode_nibble(v, sign | r) & 7 == r
            assert orc.guided_nibble(v, 3, r) & 7 == r
            assert orc.guided_nibble(v, 2, r & 3) & 7 == r
            exc = (r == 5 and 2 < a <= 2.25) or (r == 7 and 4 < a <= 4.5)
            if not exc:
                assert orc.guided_nibble(v, 1, r & 1) & 7 == r


def _pair(seed, n, rel, scale=1.0):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(n) * scale).astype(np.float32)
    x[rng.random(n) < 0.01] *= 20
    X = bf16_bits(x)
    xf = bits_to_f32(X.astype(np.uint32) << 16)
    y = xf + rel * np.abs(xf) * rng.standard_normal(n).astype(np.float32)
    return X, bf16_bits(y)


@pytest.mark.parametrize("G", [1, 4])
def test_identical_inputs_never_mismatch(orc, G):
    """I5: Y == X bitwise -> every mode reproduces the rollout codes."""
    X, _ = _pair(5, 16 * 256, 0.0)
    g, _ = orc.amax(X, G)
    for k in (1, 2):
        codes, scales, gd = orc.quant_rollout(X, g, k, G=G)
        _, cg = orc.fakequant_guided(X, g, gd, k, G=G)
        _, cr, _ = orc.fakequant_rtn(X, g, scales_in=scales, G=G)
        _, co, so = orc.fakequant_rtn(X, g, G=G)
        np.testing.assert_array_equal(cg, codes)
        np.testing.assert_array_equal(cr, codes)
        np.testing.assert_array_equal(co, codes)
        np.testing.assert_array_equal(so, scales)
    gd4 = orc.guidance_pack(codes, scales, X.size, 4)
    _, cf = orc.fakequant_fullcode(X, g, gd4, G=G)
    np.testing.assert_array_equal(cf, codes)


def test_rollout_range_and_amax_block(orc):
    """Closed forms: the block holding a group's amax gets block scale 448 and
    its amax element index 7 (v = A / (448 * A / 2688) = 6); I6: every
    normalised rollout value with a normal E4M3 scale stays within
    6 / (1 - 2^-4) (E4M3 relative rounding error <= 2^-4)."""
    for seed in range(4):
        X, Y = _pair(10 + seed, 16 * 512, 0.01, scale=10.0 ** (seed - 2))
        G = 4
        g, _ = orc.amax(Y, G)
        codes, scales, _ = orc.quant_rollout(Y, g, 2, G=G, guidance=False)
        yf = bits_to_f32(Y.astype(np.uint32) << 16).reshape(G, -1)
        nib = orc.unpack_nibbles(codes).reshape(G, -1)
        for gi in range(G):
            i = int(np.argmax(np.abs(yf[gi])))
            b = (gi * yf.shape[1] + i) // 16
            assert scales[b] == 0x7E
            assert nib[gi, i] & 7 == 7
            assert np.float32(np.abs(yf[gi]).max()) / np.float32(2688.0) == g[gi]
        yb = bits_to_f32(Y.astype(np.uint32) << 16).reshape(-1, 16)
        for b in range(yb.shape[0]):
            s = orc.e4m3_value(scales[b])
            if s >= 2.0 ** -6:
                gg = g[b // (yb.shape[0] // G)]
                inv = np.float32(1.0) / (np.float32(s) * gg)
                assert np.abs(yb[b] * inv).max() <= 6.0 / (1 - 2.0 ** -4) * (1 + 2.0 ** -20)


def test_zero_and_tiny_blocks(orc):
    y = np.zeros(48, np.float32)
    y[0] = 1000.0                         # g = 1000 / 2688
    y[16:32] = -1e-6                      # t = 1e-6 / (6 g) -> E4M3 0
    y[33] = -0.0
    Y = bf16_bits(y)
    g, _ = orc.amax(Y)
    codes, scales, _ = orc.quant_rollout(Y, g, 2)
    assert scales[1] == 0 and scales[2] == 0
    nib = orc.unpack_nibbles(codes)
    assert all(nib[16:32] == 8)           # -tiny -> -0 code
    assert nib[33] == 8 and nib[34] == 0
    yr, _, _ = orc.fakequant_rtn(Y, g, scales_in=scales, out_f32=True)
    assert np.all(yr[16:32] == 0) and np.all(np.signbit(yr[16:32]))


def test_amax_nonfinite_and_groups(orc):
    x = np.ones(64, np.float32)
    x[40] = 2688.0
    X = bf16_bits(x)
    g, st_ = orc.amax(X, 2)
    assert st_ == 0 and g[0] == np.float32(1.0) / np.float32(2688.0) and g[1] == 1.0
    # the maximum at every position of a group, the group's first and last
    # included, and negative: g = |max| / 2688 for that group, the rest keep
    # g = 1 / 2688 (closed form: 2688 / 2688 = 1 exactly)
    for G in (1, 2, 4):
        per = 64 // G
        for grp in range(G):
            for pos in (0, 1, per // 2, per - 2, per - 1):
                for sign in (1.0, -1.0):
                    y = np.ones(64, np.float32)
                    y[grp * per + pos] = sign * 2688.0
                    g, st_ = orc.amax(bf16_bits(y), G)
                    want = np.full(G, np.float32(1.0) / np.float32(2688.0), np.float32)
                    want[grp] = 1.0
                    assert st_ == 0 and np.array_equal(g, want), (G, grp, pos, sign)
    Xb = X.copy()
    Xb[3] = 0x7F80                        # +inf
    assert orc.amax(Xb)[1] == -7
    Xb[3] = 0x7FC1                        # NaN
    assert orc.amax(Xb)[1] == -7


def test_layouts(orc):
    """Packed codes: element 2m in the low nibble.  Guidance: scale plane,
    zero pad to 256 bytes, then k bits per element, least significant first."""
    rng = np.random.default_rng(6)
    n = 16 * 40
    X, Y = _pair(7, n, 0.01)
    g, _ = orc.amax(Y)
    off = orc.bitplane_offset(n)
    assert off == 256 and orc.guidance_bytes(n, 2) == 256 + n // 4
    for k in (1, 2, 3, 4):
        codes, scales, gd = orc.quant_rollout(Y, g, k)
        nib = orc.unpack_nibbles(codes)
        np.testing.assert_array_equal(codes, (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8))
        np.testing.assert_array_equal(gd[: n // 16], scales)
        assert not gd[n // 16: off].any()
        plane = np.unpackbits(gd[off:], bitorder="little").reshape(-1, k)
        vals = (plane * (1 << np.arange(k))).sum(1)
        want = nib if k == 4 else (nib & 7) & ((1 << k) - 1)
        np.testing.assert_array_equal(vals, want)
        np.testing.assert_array_equal(orc.guidance_pack(codes, scales, n, k), gd)
    del rng


def test_k3_bitplane_literal(orc):
    """The 3-bit plane against bytes worked by hand (tests/golden/bitplane_k3.txt;
    fields straddle byte boundaries).  The values are E2M1 points times 448:
    the block maximum 6 * 448 = 2688 gives g = 1 and block scale 448, so every
    value normalises exactly onto its own point and RTN returns its index."""
    kv = {}
    for line in open(os.path.join(GOLD, "bitplane_k3.txt")):
        line = line.split("#")[0].split()
        if line:
            kv[line[0]] = line[1:]
    idx = [int(t) for t in kv["indices"]]
    want = bytes(int(t, 16) for t in kv["bytes"])
    block = idx + [7, 0, 0, 0, 0, 0, 0, 0]          # the second half carries the block maximum
    Y = bf16_bits(np.array([E2M1[j] for j in block], np.float32) * np.float32(448.0))
    g, _ = orc.amax(Y)
    assert g[0] == 1.0
    codes, scales, gd = orc.quant_rollout(Y, g, 3)
    assert orc.e4m3_value(scales[0]) == 448.0
    np.testing.assert_array_equal(orc.unpack_nibbles(codes) & 7, np.array(block))
    off = orc.bitplane_offset(16)
    assert bytes(gd[off:off + 3]) == want
    assert orc.guidance_bytes(16, 3) == off + 6


def test_k3_equals_fullcode_with_own_sign(orc):
    """k = 3 carries the whole magnitude index, so the reconstructed code is
    +-value(gb) with v's sign: the choice equals the full-code choice with the
    rollout sign replaced by v's."""
    rng = np.random.default_rng(9)
    vs = list(rng.uniform(-7, 7, 3000).astype(np.float32)) + [np.float32(x) for x in E2M1] + [np.float32(-0.0)]
    for v in vs:
        for gb in range(8):
            sign = 8 if np.signbit(v) else 0
            assert orc.guided_nibble(v, 3, gb) == orc.fullcode_nibble(v, sign | gb), (v, gb)


def test_one_step_mismatch_statistic(orc):
    """The pages report that over 99% of train/rollout mismatches are one
    adjacent codebook entry apart ("TRACE Core Concept"); on the single-tensor
    workload the RTN mismatches behave the same, and guidance removes most of
    them."""
    from precision_numerics_block_amd import synth

    X, Y = synth.make_pair(1, 0, (256, 2048), "cpu")
    Xb = X.view(torch.int16).numpy().view(np.uint16).reshape(-1)
    Yb = Y.view(torch.int16).numpy().view(np.uint16).reshape(-1)
    b1 = 4096                              # 65536 elements keep this quick
    n = Xb.size
    g, _ = orc.amax(Yb)
    codes, scales, gd = orc.quant_rollout(Yb, g, 2, b0=0, b1=b1)
    _, cr, _ = orc.fakequant_rtn(Xb, g, scales_in=scales, b0=0, b1=b1)
    _, cg = orc.fakequant_guided(Xb, g, gd, 2, b0=0, b1=b1)
    m = 16 * b1
    rn = orc.unpack_nibbles(codes)[:m].astype(int)
    tn = orc.unpack_nibbles(cr)[:m].astype(int)
    gn = orc.unpack_nibbles(cg)[:m].astype(int)
    sv = lambda c: np.where(c & 8, -1, 1) * (c & 7)  # noqa: E731
    mis = sv(rn) != sv(tn)
    mis &= ~(((rn & 7) == 0) & ((tn & 7) == 0))
    assert mis.sum() > 50
    steps = np.abs(sv(rn) - sv(tn))[mis]
    assert (steps == 1).mean() >= 0.99
    gmis = (sv(gn) != sv(rn)) & ~(((rn & 7) == 0) & ((gn & 7) == 0))
    assert gmis.sum() < 0.2 * mis.sum()
    assert n == 256 * 2048


# --------------------------------------------------------------------------
# MXFP4 variant (32-element blocks, E8M0 scales)
# --------------------------------------------------------------------------
def read_mx():
    scales, blocks = [], []
    for line in open(os.path.join(GOLD, "mx_examples.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        if line.startswith("scale"):
            _, a, c = line.split()
            scales.append((float(a), int(c)))
        elif line.startswith("block"):
            vals, codes = line[5:].split("->")
            blocks.append(([float(t) for t in vals.split()], [int(t) for t in codes.split()]))
    return scales, blocks


def test_mx_hand_examples(orc):
    scales, blocks = read_mx()
    assert len(scales) >= 8 and len(blocks) >= 2
    for amax, code in scales:
        assert orc.mx_scale(amax) == code, (amax, code)
    for vals, want in blocks:
        y = np.zeros(32, np.float32)
        y[: len(vals)] = vals
        Y = bf16_bits(y)
        assert np.array_equal(bits_to_f32(Y.astype(np.uint32) << 16)[: len(vals)], np.float32(vals))
        codes, sc, gd = orc.mx_quant_rollout(Y, 2)
        nib = orc.unpack_nibbles(codes)
        np.testing.assert_array_equal(nib[: len(want)], want)
        assert not nib[len(want):].any()
        assert gd[0] == sc[0]


def test_mx_range_and_exact_round_trip(orc):
    """A nonzero block with an unclamped code has max |V / X| in [4, 8); E2M1
    points times a power of two come back exactly, codes and values."""
    rng = np.random.default_rng(12)
    for e in (-120, -20, -3, 0, 5, 60, 120):
        j = rng.integers(0, 8, 32)
        j[0] = 7                                           # the block maximum is 6 * 2^e
        sgn = rng.choice([0, 8], 32)
        vals = np.array([E2M1[t] for t in j], np.float64) * np.where(sgn, -1.0, 1.0) * 2.0 ** e
        Y = bf16_bits(vals.astype(np.float32))
        codes, sc, gd = orc.mx_quant_rollout(Y, 4)
        assert orc.mx_scale_value(sc[0]) == 2.0 ** e
        nib = orc.unpack_nibbles(codes)
        np.testing.assert_array_equal(nib & 7, j)
        np.testing.assert_array_equal(((nib & 8) != 0) & (j != 0), (sgn == 8) & (j != 0))
        for t in range(32):
            assert orc.mx_dequant(nib[t], sc[0]) == np.float32(vals[t]) or (j[t] == 0)
        yr, _, _ = orc.mx_fakequant_rtn(Y, out_f32=True)
        np.testing.assert_array_equal(yr, vals.astype(np.float32))
    for _ in range(200):
        a = np.float32(np.exp(rng.uniform(-80, 80)))
        c = orc.mx_scale(a)
        if 0 < c < 254:
            r = float(a) / orc.mx_scale_value(c)
            assert 4.0 <= r < 8.0, (a, c, r)


def test_mx_worked_example_and_rules(orc):
    """The worked example in MX form: a block whose maximum is 6 has X = 1,
    so 2.51 / 2.49 normalise to themselves; RTN gives 3 / 2, guided gives 2."""
    x = np.zeros(32, np.float32)
    y = np.zeros(32, np.float32)
    x[0] = y[0] = 6.0
    x[1], y[1] = 2.51, 2.49
    X, Y = bf16_bits(x), bf16_bits(y)
    for k in (1, 2, 3, 4):
        codes, sc, gd = orc.mx_quant_rollout(Y, k)
        assert orc.mx_scale_value(sc[0]) == 1.0
        assert orc.unpack_nibbles(codes)[1] == 4                    # rollout: 2.49 -> 2
        yr, _, _ = orc.mx_fakequant_rtn(X, scales_in=sc, out_f32=True)
        assert yr[1] == 3.0                                         # training RTN: 2.51 -> 3
        yg, cg = orc.mx_fakequant_guided(X, gd, k, out_f32=True)
        assert yg[1] == 2.0                                         # guided: the rollout side's 2
    # own scales agree with the rollout scales for the same tensor
    _, _, so = orc.mx_fakequant_rtn(Y)
    _, sc, _ = orc.mx_quant_rollout(Y, 2)
    np.testing.assert_array_equal(so, sc)



# --------------------------------------------------------------------------
# Gradient of the fake-quant: clipped straight-through mask
# --------------------------------------------------------------------------
def read_pairs(name):
    xs, ms = [], []
    for line in open(os.path.join(GOLD, name)):
        line = line.split("#")[0].strip()
        if line:
            a, b = line.split()
            xs.append(float(a))
            ms.append(int(b))
    return xs, ms


def test_ste_mask_worked_scale(orc):
    """At the worked example's combined scale 24 the saturation edge lies at
    6 x 24 = 144 (tests/golden/ste_saturation.txt, worked by hand)."""
    xs, want = read_pairs("ste_saturation.txt")
    assert np.float32(144) * (np.float32(1) / np.float32(24)) == np.float32(6)
    n = 16 * (-(-len(xs) // 16))
    x = np.zeros(n, np.uint16)
    x[: len(xs)] = bf16_bits(xs)
    scales = np.full(n // 16, 0x5C, np.uint8)
    assert orc.e4m3_value(0x5C) == 24.0
    m = orc.ste_mask(x, np.float32([1.0]), scales)
    assert list(m[: len(xs)]) == want
    gy = np.arange(1, n + 1, dtype=np.float32)
    gx = orc.ste_grad(x, np.float32([1.0]), scales, gy)
    assert np.array_equal(gx[: len(xs)], np.where(np.array(want) == 1, gy[: len(xs)], 0))


@pytest.mark.parametrize("code,g", [(0x40, 0.5), (0x08, 2.0 ** -4), (0x48, 2.0 ** -40)])
def test_ste_mask_bruteforce_exact_scales(orc, code, g):
    """Combined scales that are powers of two (2 x 0.5 = 1, 2^-6 x 2^-4 =
    2^-10, 4 x 2^-40 = 2^-38) have exact reciprocals, so v = x * inv is exact
    and the mask must equal |x| <= 6 c over every finite bf16 value, compared
    in double: the closed form of the saturation edge."""
    vals = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    xf = bits_to_f32(vals.astype(np.uint32) << 16)
    vals = vals[np.isfinite(xf)]
    vals = np.concatenate([vals, vals[: (-vals.size) % 16]])
    c = orc.e4m3_value(code) * g
    assert c == 2.0 ** round(np.log2(c))
    m = orc.ste_mask(vals, np.float32([g]), np.full(vals.size // 16, code, np.uint8))
    want = np.abs(bits_to_f32(vals.astype(np.uint32) << 16).astype(np.float64)) <= 6.0 * c
    assert np.array_equal(m.astype(bool), want)


def test_ste_mask_zero_scale_and_groups(orc):
    """A zero combined scale (an all-zero group, g = 0) normalises every
    element to 0: the gradient passes everywhere.  With several groups each
    block takes its own group's g (the same block, scale code 0x40, passes
    under g = 0.5 and saturates under g = 2^-10 for x = 3)."""
    x = bf16_bits([3.0] * 32)
    m = orc.ste_mask(x, np.float32([0.0]), np.full(2, 0x40, np.uint8))
    assert m.all()
    m = orc.ste_mask(x, np.float32([0.5, 2.0 ** -10]), np.full(2, 0x40, np.uint8), G=2)
    assert m[:16].all() and not m[16:].any()


def test_ste_mask_marks_exactly_the_saturated_outputs(orc):
    """Training values spread wider than the rollout's (relative noise 0.3
    instead of 0.01) often leave the rollout's block range.  Where the mask is
    0, the guided forward saturates: its code has magnitude index 7, its
    output is 6 s g (rounded to bf16) and stays there when |x| grows by one
    bf16 step.  The mask reads the same scales from the guidance stream's
    scale plane as from the scale array."""
    rng = np.random.default_rng(5)
    n = 16 * 4096
    yf = (rng.standard_normal(n) * np.exp(rng.uniform(-2, 2, n))).astype(np.float32)
    y = bf16_bits(yf)
    xf = bits_to_f32(y.astype(np.uint32) << 16) * (1 + 0.3 * rng.standard_normal(n)).astype(np.float32)
    x = bf16_bits(xf)
    g, _ = orc.amax(y)
    codes, scales, gd = orc.quant_rollout(y, g, 2)
    m = orc.ste_mask(x, g, gd)                   # the guidance stream's scale plane
    assert np.array_equal(m, orc.ste_mask(x, g, scales))
    assert 0 < (m == 0).sum() < n // 10
    yg, cg = orc.fakequant_guided(x, g, gd, 2)
    nib = orc.unpack_nibbles(cg)
    sat = m == 0
    assert np.all((nib[sat] & 7) == 7)
    # one bf16 step away from zero keeps a saturated output where it is
    x_up = (x.astype(np.int32) + 1).astype(np.uint16)
    x_up[~sat] = x[~sat]
    yg_up, _ = orc.fakequant_guided(x_up, g, gd, 2)
    assert np.array_equal(yg_up[sat], yg[sat])
    # and that output is 6 s g, rounded to bf16 (fp32 product, then bf16)
    s_val = np.array([orc.e4m3_value(int(c)) for c in scales], np.float32)[np.arange(n) // 16]
    want = torch.from_numpy((np.float32(6.0) * s_val[sat]) * g[0]).to(torch.bfloat16).view(torch.int16)
    assert np.array_equal(yg[sat] & 0x7FFF, want.numpy().view(np.uint16))
