"""ctypes wrapper around ``liboracle.so`` (built from ``trace_oracle.c``).

Test infrastructure only: see the package docstring.  Arrays are numpy; bf16
tensors travel as ``uint16`` bit patterns.  Every function mirrors one C
function, whose comment cites the passage of the pages it follows.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "trace_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11", "-Wall"]


def build(force=True):
    """Compile the oracle with gcc (plain C, no vector intrinsics)."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    """Load the oracle library.  TRACE_ORACLE_LIB names another build of
    ``trace_oracle.c`` to load instead (the pins' mutation test uses it to run
    the pins against copies with planted mistakes)."""
    global _lib
    if _lib is None:
        path = os.environ.get("TRACE_ORACLE_LIB") or _LIB
        if path == _LIB and not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(path)
        i64, i32, f32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double
        vp, u8 = ctypes.c_void_p, ctypes.c_uint8
        sig = {
            "oracle_e2m1_value": (f64, [i32]),
            "oracle_e4m3_value": (f64, [i32]),
            "oracle_e4m3_encode": (u8, [f32]),
            "oracle_rtn_index": (i32, [f32]),
            "oracle_rtn_nibble": (i32, [f32]),
            "oracle_f32_to_bf16": (ctypes.c_uint16, [f32]),
            "oracle_bf16_to_f32": (f32, [ctypes.c_uint16]),
            "oracle_guided_nibble": (i32, [f32, i32, i32]),
            "oracle_fullcode_nibble": (i32, [f32, i32]),
            "oracle_dequant": (f32, [i32, u8, f32]),
            "oracle_bitplane_offset": (i64, [i64]),
            "oracle_guidance_bytes": (i64, [i64, i32]),
            "oracle_amax": (i32, [vp, i64, i32, vp]),
            "oracle_quant_rollout": (None, [vp, i64, i32, vp, i32, i64, i64, vp, vp, vp]),
            "oracle_guidance_pack": (None, [vp, vp, i64, i32, i64, i64, vp]),
            "oracle_fakequant_guided": (None, [vp, i64, i32, vp, vp, i32, i64, i64, vp, i32, vp]),
            "oracle_fakequant_fullcode": (None, [vp, i64, i32, vp, vp, i64, i64, vp, i32, vp]),
            "oracle_fakequant_rtn": (None, [vp, i64, i32, vp, vp, i64, i64, vp, i32, vp, vp]),
            "oracle_ste_mask": (None, [vp, i64, i32, vp, vp, i64, i64, vp]),
            "oracle_mx_scale": (u8, [f32]),
            "oracle_mx_scale_value": (f64, [u8]),
            "oracle_mx_bitplane_offset": (i64, [i64]),
            "oracle_mx_guidance_bytes": (i64, [i64, i32]),
            "oracle_mx_quant_rollout": (None, [vp, i64, i32, i64, i64, vp, vp, vp]),
            "oracle_mx_dequant": (f32, [i32, u8]),
            "oracle_mx_fakequant_guided": (None, [vp, i64, vp, i32, i64, i64, vp, i32, vp]),
            "oracle_mx_fakequant_rtn": (None, [vp, i64, vp, i64, i64, vp, i32, vp, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _u16(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


# ---- scalar helpers ------------------------------------------------------
def e2m1_value(nibble):
    return lib().oracle_e2m1_value(int(nibble))


def e4m3_value(code):
    return lib().oracle_e4m3_value(int(code))


def e4m3_encode(t):
    return int(lib().oracle_e4m3_encode(float(t)))


def rtn_index(v):
    return lib().oracle_rtn_index(float(v))


def rtn_nibble(v):
    return lib().oracle_rtn_nibble(float(v))


def f32_to_bf16(f):
    return int(lib().oracle_f32_to_bf16(float(f)))


def bf16_to_f32(h):
    return float(lib().oracle_bf16_to_f32(int(h)))


def guided_nibble(v, k, gb):
    return lib().oracle_guided_nibble(float(v), int(k), int(gb))


def fullcode_nibble(v, r):
    return lib().oracle_fullcode_nibble(float(v), int(r))


def dequant(nibble, s, g):
    return float(lib().oracle_dequant(int(nibble), int(s), float(g)))


# ---- sizes ---------------------------------------------------------------
def bitplane_offset(n):
    return int(lib().oracle_bitplane_offset(int(n)))


def guidance_bytes(n, k):
    return int(lib().oracle_guidance_bytes(int(n), int(k)))


# ---- tensor functions (full tensor in, blocks [b0, b1) processed) --------
def amax(x, G=1):
    """Global scale per group: returns (g float32[G], status)."""
    x = _u16(x).reshape(-1)
    g = np.zeros(G, np.float32)
    st = lib().oracle_amax(_p(x), x.size, G, _p(g))
    return g, st


def _range(n, b0, b1):
    return (0 if b0 is None else b0), (n // 16 if b1 is None else b1)


def quant_rollout(y, g, k, G=1, b0=None, b1=None, guidance=True, out=None):
    """RTN quantisation: returns (codes u8[n/2], scales u8[n/16], guidance u8 or None)."""
    y = _u16(y).reshape(-1)
    n = y.size
    g = np.ascontiguousarray(g, np.float32)
    b0, b1 = _range(n, b0, b1)
    if out is None:
        codes = np.zeros(n // 2, np.uint8)
        scales = np.zeros(n // 16, np.uint8)
        gd = np.zeros(guidance_bytes(n, k), np.uint8) if guidance else None
    else:
        codes, scales, gd = out
    lib().oracle_quant_rollout(_p(y), n, G, _p(g), k, b0, b1, _p(codes), _p(scales), _p(gd))
    return codes, scales, gd


def guidance_pack(codes, scales, n, k, b0=None, b1=None, out=None):
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    b0, b1 = _range(n, b0, b1)
    gd = np.zeros(guidance_bytes(n, k), np.uint8) if out is None else out
    lib().oracle_guidance_pack(_p(codes), _p(scales), n, k, b0, b1, _p(gd))
    return gd


def _outbufs(n, out_f32, want_codes):
    y = np.zeros(n, np.float32 if out_f32 else np.uint16)
    c = np.zeros(n // 2, np.uint8) if want_codes else None
    return y, c


def _checked_out(out, n, out_f32, codes):
    """Caller-given output arrays (filled only over the blocks processed)."""
    y, c = out[0], out[1]
    assert y.dtype == (np.float32 if out_f32 else np.uint16) and y.size == n and y.flags.c_contiguous
    assert (c is None) == (not codes) and (c is None or (c.dtype == np.uint8 and c.size == n // 2))
    return y, c


def fakequant_guided(x, g, guidance, k, G=1, out_f32=False, b0=None, b1=None, codes=True, out=None):
    """out: optional (y, codes) arrays to fill over blocks [b0, b1) only."""
    x = _u16(x).reshape(-1)
    n = x.size
    g = np.ascontiguousarray(g, np.float32)
    gd = np.ascontiguousarray(guidance, np.uint8)
    b0, b1 = _range(n, b0, b1)
    y, c = _outbufs(n, out_f32, codes) if out is None else _checked_out(out, n, out_f32, codes)
    lib().oracle_fakequant_guided(_p(x), n, G, _p(g), _p(gd), k, b0, b1, _p(y), int(out_f32), _p(c))
    return y, c


def fakequant_fullcode(x, g, guidance, G=1, out_f32=False, b0=None, b1=None, codes=True, out=None):
    x = _u16(x).reshape(-1)
    n = x.size
    g = np.ascontiguousarray(g, np.float32)
    gd = np.ascontiguousarray(guidance, np.uint8)
    b0, b1 = _range(n, b0, b1)
    y, c = _outbufs(n, out_f32, codes) if out is None else _checked_out(out, n, out_f32, codes)
    lib().oracle_fakequant_fullcode(_p(x), n, G, _p(g), _p(gd), b0, b1, _p(y), int(out_f32), _p(c))
    return y, c


def fakequant_rtn(x, g, scales_in=None, G=1, out_f32=False, b0=None, b1=None, codes=True, out=None):
    """Plain RTN fake-quant: returns (y, codes or None, scales used).  out:
    optional (y, codes, scales) arrays to fill over blocks [b0, b1) only."""
    x = _u16(x).reshape(-1)
    n = x.size
    g = np.ascontiguousarray(g, np.float32)
    sin = None if scales_in is None else np.ascontiguousarray(scales_in, np.uint8)
    b0, b1 = _range(n, b0, b1)
    if out is None:
        y, c = _outbufs(n, out_f32, codes)
        sout = np.zeros(n // 16, np.uint8)
    else:
        y, c = _checked_out(out, n, out_f32, codes)
        sout = out[2]
        assert sout.dtype == np.uint8 and sout.size == n // 16
    lib().oracle_fakequant_rtn(_p(x), n, G, _p(g), _p(sin), b0, b1, _p(y), int(out_f32), _p(c), _p(sout))
    return y, c, sout


def ste_mask(x, g, scales, G=1, b0=None, b1=None):
    """Clipped straight-through gradient mask u8[n]: 1 where |x * inv| <= 6
    with the forward's scales (g f32[G], scales u8[n/16] or a guidance
    stream, whose first n/16 bytes are the scale plane)."""
    x = _u16(x).reshape(-1)
    n = x.size
    g = np.ascontiguousarray(g, np.float32)
    sc = np.ascontiguousarray(np.asarray(scales, np.uint8).reshape(-1)[: n // 16])
    b0, b1 = _range(n, b0, b1)
    m = np.zeros(n, np.uint8)
    lib().oracle_ste_mask(_p(x), n, G, _p(g), _p(sc), b0, b1, _p(m))
    return m


def ste_grad(x, g, scales, gy, G=1, b0=None, b1=None):
    """The gradient itself: gy where the mask is 1, +0 elsewhere (gy as
    float32 values or as uint16 bf16 bit patterns; the result has gy's
    dtype)."""
    m = ste_mask(x, g, scales, G, b0, b1)
    gy = np.asarray(gy).reshape(-1)
    return np.where(m.astype(bool), gy, np.zeros(1, gy.dtype))


def unpack_nibbles(codes):
    """u8[n/2] -> u8[n] (element 2m in the low nibble)."""
    codes = np.asarray(codes, np.uint8)
    out = np.empty(codes.size * 2, np.uint8)
    out[0::2] = codes & 0xF
    out[1::2] = codes >> 4
    return out


# ---- MXFP4 variant (32-element blocks, E8M0 scales, no global scale) -----
def mx_scale(amax):
    return int(lib().oracle_mx_scale(float(amax)))


def mx_scale_value(code):
    return float(lib().oracle_mx_scale_value(int(code)))


def mx_bitplane_offset(n):
    return int(lib().oracle_mx_bitplane_offset(int(n)))


def mx_guidance_bytes(n, k):
    return int(lib().oracle_mx_guidance_bytes(int(n), int(k)))


def mx_dequant(nibble, code):
    return float(lib().oracle_mx_dequant(int(nibble), int(code)))


def _mx_range(n, b0, b1):
    return (0 if b0 is None else b0), (n // 32 if b1 is None else b1)


def mx_quant_rollout(y, k, b0=None, b1=None, guidance=True, out=None):
    """MX RTN quantisation: returns (codes u8[n/2], scales u8[n/32], guidance or None)."""
    y = _u16(y).reshape(-1)
    n = y.size
    b0, b1 = _mx_range(n, b0, b1)
    if out is None:
        codes = np.zeros(n // 2, np.uint8)
        scales = np.zeros(n // 32, np.uint8)
        gd = np.zeros(mx_guidance_bytes(n, k), np.uint8) if guidance else None
    else:
        codes, scales, gd = out
    lib().oracle_mx_quant_rollout(_p(y), n, k, b0, b1, _p(codes), _p(scales), _p(gd))
    return codes, scales, gd


def mx_fakequant_guided(x, guidance, k, out_f32=False, b0=None, b1=None, codes=True):
    """Guided (k = 1, 2, 3) or full-code (k = 4) fake-quant with MX scales."""
    x = _u16(x).reshape(-1)
    n = x.size
    gd = np.ascontiguousarray(guidance, np.uint8)
    b0, b1 = _mx_range(n, b0, b1)
    y, c = _outbufs(n, out_f32, codes)
    lib().oracle_mx_fakequant_guided(_p(x), n, _p(gd), k, b0, b1, _p(y), int(out_f32), _p(c))
    return y, c


def mx_fakequant_rtn(x, scales_in=None, out_f32=False, b0=None, b1=None, codes=True):
    """Plain RTN with MX scales: returns (y, codes or None, scales used)."""
    x = _u16(x).reshape(-1)
    n = x.size
    sin = None if scales_in is None else np.ascontiguousarray(scales_in, np.uint8)
    b0, b1 = _mx_range(n, b0, b1)
    y, c = _outbufs(n, out_f32, codes)
    so = np.zeros(n // 32, np.uint8)
    lib().oracle_mx_fakequant_rtn(_p(x), n, _p(sin), b0, b1, _p(y), int(out_f32), _p(c), _p(so))
    return y, c, (sin if sin is not None else so)

