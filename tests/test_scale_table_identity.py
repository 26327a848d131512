"""The identity behind the one-pass rollout's table-driven block scale.

The one-pass kernel replaces the per-block division t = fl(ab / fl(6 g)) and
the E4M3 encode of t with a 256-entry table per group: a bf16 block amax ab
is V * 2^(e1 - 127) (V = 1 + j/128 for exponent field e >= 1, e1 = e; V =
j/128 for e = 0, e1 = 1), fl(6 g) = Dm * 2^Xd with Dm in [1, 2), and
fl(ab / d) = fl(V / Dm) * 2^(e1 - 127 - Xd) wherever that is normal, because
scaling by a power of two commutes with rounding to fp32 in the normal range.

This checks the identity in numpy float32 (IEEE division, RNE), not the
kernel: the table form against the direct formula for every finite
non-negative bf16 block amax not above the group amax A, over a spread of A
(zero, bf16 subnormals, the largest bf16, random bf16 values and random
fp32 values).  The E4M3 encode here is the round-to-nearest-even,
saturating encode of the block scale ([en] "Why Does FP4 Rollout 'Break' RL
Training?": the same global and block scale on both sides).  The GPU parity
tests check the kernel itself against the oracle.
"""
import numpy as np

f32 = np.float32


def _bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


def _from_bits(u):
    return np.asarray(u, np.uint32).view(np.float32)


def _e4m3(t):
    """RNE, saturating at 448, subnormal step 2^-9."""
    t = np.asarray(t, np.float32)
    sub = np.rint(t * f32(512)).astype(np.uint32)
    u = _bits(t)
    r = u + np.uint32(0x7FFFF) + ((u >> np.uint32(20)) & np.uint32(1))
    nrm = (r >> np.uint32(20)) - np.uint32(960)
    return np.where(t >= f32(448), np.uint32(0x7E), np.where(t < f32(2.0 ** -6), sub, nrm))


HAB = np.arange(0, 0x7F80, dtype=np.uint32)               # every finite bf16 magnitude
AB = _from_bits(HAB << np.uint32(16))
_IDX = np.arange(256, dtype=np.uint32)
_V = np.where(_IDX >= 128, f32(1) + (_IDX - 128).astype(np.float32) / f32(128),
              _IDX.astype(np.float32) / f32(128)).astype(np.float32)


def _split(d):
    """d = Dm * 2^Xd, Dm in [1, 2), for finite d > 0 (subnormals included)."""
    u = int(_bits(d))
    e = u >> 23
    if e == 0:
        s = (32 - u.bit_length()) - 8
        u <<= s
        return _from_bits((u & 0x7FFFFF) | 0x3F800000), -126 - s
    return _from_bits((u & 0x7FFFFF) | 0x3F800000), e - 127


def _table_codes(g):
    if not g > 0:
        q, p, k = np.zeros(256, np.float32), np.zeros(256, np.int64), 0
    else:
        dm, xd = _split(f32(f32(6) * g))
        q = (_V / dm).astype(np.float32)
        u = _bits(q).astype(np.int64)
        p = ((u + 0x7FFFF + ((u >> 20) & 1)) >> 20) - 960 - 8 * (127 + xd)
        k = -118 - xd
    idx = np.minimum(HAB, (HAB & 127) | 128)
    e1 = np.maximum(HAB >> 7, 1).astype(np.int64)
    tt = np.ldexp(q[idx], (e1 + k).astype(np.int32)).astype(np.float32)
    sub = np.rint(tt).astype(np.int64)
    nrm = np.minimum((p[idx] + 8 * e1) & 0xFFFFFFFF, 0x7E)
    return np.where(tt < f32(8), sub, nrm).astype(np.uint32)


def _direct_codes(g):
    if not g > 0:
        return np.zeros(HAB.shape, np.uint32)
    return _e4m3((AB / f32(f32(6) * g)).astype(np.float32))


def test_table_block_scale_equals_division_and_encode():
    rng = np.random.default_rng(7)
    amaxes = [f32(0)]
    amaxes += [_from_bits(h << 16) for h in (1, 2, 3, 0x7F, 0x80, 0x81, 0x3F80, 0x4328, 0x7F00, 0x7F7F)]
    amaxes += [_from_bits(int(h) << 16) for h in rng.integers(1, 0x7F80, 600)]
    amaxes += [f32(x) for x in rng.uniform(0, 100, 100)]
    with np.errstate(all="ignore"):
        for A in amaxes:
            g = f32(A / f32(2688))
            mine = AB <= A                                 # the blocks a group with amax A can hold
            want, got = _direct_codes(g), _table_codes(g)
            bad = np.nonzero((want != got) & mine)[0]
            assert bad.size == 0, (float(A), hex(int(HAB[bad[0]])), int(want[bad[0]]), int(got[bad[0]]))


def test_worked_example_scale():
    """A group amax of 2688 gives g = 1; a block amax of 144 then has t = 24,
    an exact E4M3 value (code 0x5C), and the table form agrees."""
    g = f32(1)
    with np.errstate(all="ignore"):
        codes, direct = _table_codes(g), _direct_codes(g)
    h = int(_bits(f32(144)) >> 16)
    assert codes[h] == 0x5C == direct[h]
