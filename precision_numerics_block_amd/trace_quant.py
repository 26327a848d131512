"""Thin ctypes binding of ``libtrace_quant.so`` (C ABI: include/trace_quant.h).

Argument marshalling only: every function checks dtypes and devices, takes
raw device pointers from torch tensors (``data_ptr()``) and the current HIP
stream, and calls the C entry point of the same name.  torch supplies device
memory and streams; every step of the computation runs in the library's HIP
kernels.  Importing this module fails loudly when the library is missing.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtrace_quant.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc --offload-arch=gfx950)")

lib = ctypes.CDLL(LIB_PATH)

_i64, _int, _vp, _sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
_SIGS = {
    "trace_code_bytes": (_sz, [_i64]),
    "trace_scale_bytes": (_sz, [_i64]),
    "trace_guidance_bytes": (_sz, [_i64, _int]),
    "trace_amax": (_int, [_vp, _i64, _int, _vp, _vp, _vp]),
    "trace_quant_rollout": (_int, [_vp, _i64, _int, _vp, _int, _vp, _vp, _vp, _vp]),
    "trace_quant_weight": (_int, [_vp, _i64, _int, _vp, _vp, _vp, _vp, _vp]),
    "trace_guidance_pack": (_int, [_vp, _vp, _i64, _int, _vp, _vp]),
    "trace_onepass_work_bytes": (_sz, [_int]),
    "trace_onepass_capacity": (_i64, [_int]),
    "trace_quant_rollout_onepass": (_int, [_vp, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp, _int, _vp, _vp]),
    "trace_quant_rollout_onepass_noalloc": (_int, [_vp, _i64, _int, _int, _vp, _vp, _vp, _vp, _int, _vp, _vp]),
    "trace_fakequant_rtn_onepass": (_int, [_vp, _i64, _int, _vp, _vp, _int, _vp, _vp, _vp, _int, _vp, _vp]),
    "trace_fakequant_guided": (_int, [_vp, _i64, _int, _vp, _vp, _int, _vp, _int, _vp, _vp]),
    "trace_fakequant_fullcode": (_int, [_vp, _i64, _int, _vp, _vp, _vp, _int, _vp, _vp]),
    "trace_fakequant_rtn": (_int, [_vp, _i64, _int, _vp, _vp, _vp, _int, _vp, _vp, _vp]),
    "trace_fakequant_ste_grad": (_int, [_vp, _i64, _int, _vp, _vp, _vp, _vp, _int, _vp]),
    "trace_mx_scale_bytes": (_sz, [_i64]),
    "trace_mx_guidance_bytes": (_sz, [_i64, _int]),
    "trace_mx_quant_rollout": (_int, [_vp, _i64, _int, _vp, _vp, _vp, _vp]),
    "trace_mx_fakequant_guided": (_int, [_vp, _i64, _vp, _int, _vp, _int, _vp, _vp]),
    "trace_mx_fakequant_rtn": (_int, [_vp, _i64, _vp, _vp, _int, _vp, _vp, _vp]),
    "trace_record_bytes": (_sz, [_i64, _int, _int]),
    "trace_record_to_host": (_int, [_vp, _vp, _i64, _int, _int, _vp, _sz, _vp]),
    "trace_record_seal": (_int, [_vp, _sz]),
    "trace_record_check": (_int, [_vp, _sz, ctypes.POINTER(_i64), ctypes.POINTER(_int), ctypes.POINTER(_int)]),
    "trace_record_from_host": (_int, [_vp, _sz, _vp, _vp, _vp]),
    "trace_record_write": (_int, [ctypes.c_char_p, _vp, _sz]),
    "trace_record_read": (_int, [ctypes.c_char_p, _vp, _sz, ctypes.POINTER(_sz)]),
    "trace_xxh64": (ctypes.c_uint64, [_vp, _sz]),
    "trace_status_str": (ctypes.c_char_p, [_int]),
    "trace_version": (_int, []),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

OUT_BF16, OUT_F32 = 0, 1

__all__ = [
    "lib", "TraceError", "code_bytes", "scale_bytes", "guidance_bytes", "amax", "quant_rollout", "quant_weight",
    "onepass_work_bytes", "onepass_capacity", "quant_rollout_onepass", "quant_rollout_onepass_noalloc",
    "fakequant_rtn_onepass",
    "guidance_pack", "fakequant_guided", "fakequant_fullcode", "fakequant_rtn", "fakequant_ste_grad", "version",
    "mx_scale_bytes", "mx_guidance_bytes", "mx_quant_rollout", "mx_fakequant_guided", "mx_fakequant_rtn",
    "record_bytes", "record_to_host", "record_seal", "record_check", "record_from_host", "record_write",
    "record_read", "xxh64",
]


class TraceError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn}: {lib.trace_status_str(status).decode()} (status {status})")
        self.status = status


def _check(fn, status):
    if status != 0:
        raise TraceError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t, dtype, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _u8(n, dev):
    return torch.empty(int(n), dtype=torch.uint8, device=dev)


def code_bytes(n):
    return int(lib.trace_code_bytes(int(n)))


def scale_bytes(n):
    return int(lib.trace_scale_bytes(int(n)))


def guidance_bytes(n, k):
    return int(lib.trace_guidance_bytes(int(n), int(k)))


def version():
    return int(lib.trace_version())


def amax(x, G=1, out=None, status=None):
    """Global scales f32[G] = amax(|x| per group) / 2688.  ``status``: optional
    int32 GPU tensor of one element that receives TRACE_E_NONFINITE (-7)."""
    _need(x, torch.bfloat16, "x")
    g = torch.empty(G, dtype=torch.float32, device=x.device) if out is None else out
    _check("trace_amax", lib.trace_amax(_ptr(x), x.numel(), int(G), _ptr(g), _ptr(status), _stream(x.device)))
    return g


def quant_rollout(y, g, k, G=1, guidance=True, codes=None, scales=None):
    """RTN codes u8[n/2], E4M3 scales u8[n/16] and (if ``guidance``) the
    guidance stream of width k.  ``guidance`` may be a preallocated tensor."""
    _need(y, torch.bfloat16, "y")
    _need(g, torch.float32, "g")
    n, dev = y.numel(), y.device
    codes = _u8(n // 2, dev) if codes is None else codes
    scales = _u8(n // 16, dev) if scales is None else scales
    if guidance is True:
        guidance = _u8(guidance_bytes(n, k), dev)
    elif guidance is False:
        guidance = None
    _check("trace_quant_rollout", lib.trace_quant_rollout(
        _ptr(y), n, int(G), _ptr(g), int(k), _ptr(codes), _ptr(scales), _ptr(guidance), _stream(dev)))
    return codes, scales, guidance


def quant_weight(w, G=1, g=None, codes=None, scales=None, status=None):
    """FP4 weights: global scale per matrix (G matrices), RTN codes u8[n/2]
    and E4M3 block scales u8[n/16] along the contiguous dimension; no
    guidance.  Returns (g, codes, scales)."""
    _need(w, torch.bfloat16, "w")
    n, dev = w.numel(), w.device
    g = torch.empty(G, dtype=torch.float32, device=dev) if g is None else g
    codes = _u8(n // 2, dev) if codes is None else codes
    scales = _u8(n // 16, dev) if scales is None else scales
    _check("trace_quant_weight", lib.trace_quant_weight(
        _ptr(w), n, int(G), _ptr(g), _ptr(codes), _ptr(scales), _ptr(status), _stream(dev)))
    return g, codes, scales


def onepass_work_bytes(G=1):
    return int(lib.trace_onepass_work_bytes(int(G)))


def onepass_capacity(max_workgroups=0):
    """Elements the one-pass rollout keeps on chip on the current device."""
    return int(lib.trace_onepass_capacity(int(max_workgroups)))


def quant_rollout_onepass(y, k, G=1, g=None, guidance=True, codes=None, scales=None, work=None,
                          max_workgroups=0, status=None):
    """amax and quant_rollout from one read of y (where it fits on chip).
    Returns (g, codes, scales, guidance).  ``work``: a uint8 GPU tensor of
    onepass_work_bytes(G) bytes, zero-filled before its first use (every call
    leaves it zeroed); a fresh zeroed one is allocated when None."""
    _need(y, torch.bfloat16, "y")
    n, dev = y.numel(), y.device
    g = torch.empty(G, dtype=torch.float32, device=dev) if g is None else g
    codes = _u8(n // 2, dev) if codes is None else codes
    scales = _u8(n // 16, dev) if scales is None else scales
    if guidance is True:
        guidance = _u8(guidance_bytes(n, k), dev)
    elif guidance is False:
        guidance = None
    if work is None:
        work = torch.zeros(max(onepass_work_bytes(G), 256), dtype=torch.uint8, device=dev)
    _check("trace_quant_rollout_onepass", lib.trace_quant_rollout_onepass(
        _ptr(y), n, int(G), int(k), _ptr(g), _ptr(codes), _ptr(scales), _ptr(guidance), _ptr(work),
        int(max_workgroups), _ptr(status), _stream(dev)))
    return g, codes, scales, guidance


def quant_rollout_onepass_noalloc(y, k, G=1, g=None, guidance=True, codes=None, scales=None, max_workgroups=0,
                                  status=None):
    """quant_rollout_onepass with the library's static per-device work
    array instead of a work buffer (G <= 4096; calls on one device must be
    ordered on one stream).  Outputs left as None are allocated here, by
    torch; pass them all to allocate nothing."""
    _need(y, torch.bfloat16, "y")
    n, dev = y.numel(), y.device
    g = torch.empty(G, dtype=torch.float32, device=dev) if g is None else g
    codes = _u8(n // 2, dev) if codes is None else codes
    scales = _u8(n // 16, dev) if scales is None else scales
    if guidance is True:
        guidance = _u8(guidance_bytes(n, k), dev)
    elif guidance is False:
        guidance = None
    _check("trace_quant_rollout_onepass_noalloc", lib.trace_quant_rollout_onepass_noalloc(
        _ptr(y), n, int(G), int(k), _ptr(g), _ptr(codes), _ptr(scales), _ptr(guidance), int(max_workgroups),
        _ptr(status), _stream(dev)))
    return g, codes, scales, guidance


def fakequant_rtn_onepass(x, G=1, g=None, out_dtype=OUT_BF16, out=None, codes_out=None, scales_out=None,
                          work=None, max_workgroups=0, status=None):
    """amax(x) and own-scale fakequant_rtn from one read of x (where it fits
    on chip).  Returns (g, y, codes or None, scales or None); ``work`` as for
    quant_rollout_onepass."""
    _need(x, torch.bfloat16, "x")
    dev = x.device
    g = torch.empty(G, dtype=torch.float32, device=dev) if g is None else g
    out, codes_out = _outputs(x, out_dtype, out, codes_out)
    if scales_out is True:
        scales_out = _u8(x.numel() // 16, dev)
    elif scales_out is False:
        scales_out = None
    if work is None:
        work = torch.zeros(max(onepass_work_bytes(G), 256), dtype=torch.uint8, device=dev)
    _check("trace_fakequant_rtn_onepass", lib.trace_fakequant_rtn_onepass(
        _ptr(x), x.numel(), int(G), _ptr(g), _ptr(out), int(out_dtype), _ptr(codes_out), _ptr(scales_out),
        _ptr(work), int(max_workgroups), _ptr(status), _stream(dev)))
    return g, out, codes_out, scales_out


def guidance_pack(codes, scales, n, k, out=None):
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.uint8, "scales")
    dev = codes.device
    out = _u8(guidance_bytes(n, k), dev) if out is None else out
    _check("trace_guidance_pack", lib.trace_guidance_pack(
        _ptr(codes), _ptr(scales), int(n), int(k), _ptr(out), _stream(dev)))
    return out


def _outputs(x, out_dtype, out, codes_out):
    if out is None:
        out = torch.empty(x.shape, dtype=torch.float32 if out_dtype == OUT_F32 else torch.bfloat16,
                          device=x.device)
    if codes_out is True:
        codes_out = _u8(x.numel() // 2, x.device)
    elif codes_out is False:
        codes_out = None
    return out, codes_out


def fakequant_guided(x, g, guidance, k, G=1, out_dtype=OUT_BF16, out=None, codes_out=None):
    """Rollout-guided fake-quant; returns (y, codes_out or None)."""
    _need(x, torch.bfloat16, "x")
    _need(g, torch.float32, "g")
    _need(guidance, torch.uint8, "guidance")
    out, codes_out = _outputs(x, out_dtype, out, codes_out)
    _check("trace_fakequant_guided", lib.trace_fakequant_guided(
        _ptr(x), x.numel(), int(G), _ptr(g), _ptr(guidance), int(k), _ptr(out), int(out_dtype),
        _ptr(codes_out), _stream(x.device)))
    return out, codes_out


def fakequant_fullcode(x, g, guidance, G=1, out_dtype=OUT_BF16, out=None, codes_out=None):
    _need(x, torch.bfloat16, "x")
    _need(g, torch.float32, "g")
    _need(guidance, torch.uint8, "guidance")
    out, codes_out = _outputs(x, out_dtype, out, codes_out)
    _check("trace_fakequant_fullcode", lib.trace_fakequant_fullcode(
        _ptr(x), x.numel(), int(G), _ptr(g), _ptr(guidance), _ptr(out), int(out_dtype),
        _ptr(codes_out), _stream(x.device)))
    return out, codes_out


def fakequant_rtn(x, g, scales_in=None, G=1, out_dtype=OUT_BF16, out=None, codes_out=None, scales_out=None):
    """Plain RTN fake-quant; own block scales when ``scales_in`` is None."""
    _need(x, torch.bfloat16, "x")
    _need(g, torch.float32, "g")
    out, codes_out = _outputs(x, out_dtype, out, codes_out)
    if scales_out is True:
        scales_out = _u8(x.numel() // 16, x.device)
    elif scales_out is False:
        scales_out = None
    _check("trace_fakequant_rtn", lib.trace_fakequant_rtn(
        _ptr(x), x.numel(), int(G), _ptr(g), _ptr(scales_in), _ptr(out), int(out_dtype),
        _ptr(codes_out), _ptr(scales_out), _stream(x.device)))
    return out, codes_out, scales_out


def fakequant_ste_grad(x, g, scales, gy, G=1, out=None):
    """Clipped straight-through gradient: gy where |x * inv| <= 6, else 0,
    with the forward's scales (g f32[G], scales u8[n/16]; a guidance stream
    may be passed as ``scales``: its first n/16 bytes are the scale plane).
    gy is bf16 or f32 with x's shape; ``out`` may be gy (in place)."""
    _need(x, torch.bfloat16, "x")
    _need(g, torch.float32, "g")
    _need(scales, torch.uint8, "scales")
    if not isinstance(gy, torch.Tensor) or gy.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("gy must be a bf16 or f32 GPU tensor")
    _need(gy, gy.dtype, "gy")
    if gy.numel() != x.numel():
        raise ValueError("gy must have x's number of elements")
    if scales.numel() < x.numel() // 16:
        raise ValueError("scales must hold n / 16 bytes")
    out = torch.empty_like(gy) if out is None else _need(out, gy.dtype, "out")
    _check("trace_fakequant_ste_grad", lib.trace_fakequant_ste_grad(
        _ptr(x), x.numel(), int(G), _ptr(g), _ptr(scales), _ptr(gy), _ptr(out),
        OUT_F32 if gy.dtype == torch.float32 else OUT_BF16, _stream(x.device)))
    return out


# ---- MXFP4 variant (32-element blocks, E8M0 scales, no global scale) ------
def mx_scale_bytes(n):
    return int(lib.trace_mx_scale_bytes(int(n)))


def mx_guidance_bytes(n, k):
    return int(lib.trace_mx_guidance_bytes(int(n), int(k)))


def mx_quant_rollout(y, k, guidance=True, codes=None, scales=None):
    """MX RTN codes u8[n/2], E8M0 scales u8[n/32] and (if ``guidance``) the
    guidance stream of width k."""
    _need(y, torch.bfloat16, "y")
    n, dev = y.numel(), y.device
    codes = _u8(n // 2, dev) if codes is None else codes
    scales = _u8(n // 32, dev) if scales is None else scales
    if guidance is True:
        guidance = _u8(mx_guidance_bytes(n, k), dev)
    elif guidance is False:
        guidance = None
    _check("trace_mx_quant_rollout", lib.trace_mx_quant_rollout(
        _ptr(y), n, int(k), _ptr(codes), _ptr(scales), _ptr(guidance), _stream(dev)))
    return codes, scales, guidance


def mx_fakequant_guided(x, guidance, k, out_dtype=OUT_BF16, out=None, codes_out=None):
    """MX guided (k = 1, 2, 3) or full-code (k = 4) fake-quant; returns (y, codes or None)."""
    _need(x, torch.bfloat16, "x")
    _need(guidance, torch.uint8, "guidance")
    out, codes_out = _outputs(x, out_dtype, out, codes_out)
    _check("trace_mx_fakequant_guided", lib.trace_mx_fakequant_guided(
        _ptr(x), x.numel(), _ptr(guidance), int(k), _ptr(out), int(out_dtype), _ptr(codes_out), _stream(x.device)))
    return out, codes_out


def mx_fakequant_rtn(x, scales_in=None, out_dtype=OUT_BF16, out=None, codes_out=None, scales_out=None):
    """MX plain RTN fake-quant; own scales when ``scales_in`` is None."""
    _need(x, torch.bfloat16, "x")
    out, codes_out = _outputs(x, out_dtype, out, codes_out)
    if scales_out is True:
        scales_out = _u8(x.numel() // 32, x.device)
    elif scales_out is False:
        scales_out = None
    _check("trace_mx_fakequant_rtn", lib.trace_mx_fakequant_rtn(
        _ptr(x), x.numel(), _ptr(scales_in), _ptr(out), int(out_dtype), _ptr(codes_out), _ptr(scales_out),
        _stream(x.device)))
    return out, codes_out, scales_out


# ---- guidance records (transport and persistence) -------------------------
def record_bytes(n, k, G=1):
    return int(lib.trace_record_bytes(int(n), int(k), int(G)))


def _host_ptr(buf):
    if isinstance(buf, torch.Tensor):
        if buf.is_cuda or buf.dtype != torch.uint8 or not buf.is_contiguous():
            raise TypeError("record buffers are contiguous uint8 host tensors")
        return ctypes.c_void_p(buf.data_ptr()), buf.numel()
    raise TypeError("record buffers are uint8 host tensors")


def record_to_host(guidance, g, n, k, G=1, out=None):
    """Enqueue the device->host copy of a guidance stream and its global
    scales into a record (a pinned uint8 host tensor, allocated when `out` is
    None).  Synchronise the stream, then call record_seal."""
    _need(guidance, torch.uint8, "guidance")
    _need(g, torch.float32, "g")
    if out is None:
        out = torch.empty(record_bytes(n, k, G), dtype=torch.uint8, pin_memory=True)
    p, nb = _host_ptr(out)
    _check("trace_record_to_host", lib.trace_record_to_host(
        _ptr(guidance), _ptr(g), int(n), int(k), int(G), p, nb, _stream(guidance.device)))
    return out


def record_seal(record):
    p, nb = _host_ptr(record)
    _check("trace_record_seal", lib.trace_record_seal(p, nb))


def record_check(record):
    """(n, k, G) of a sealed, intact record; raises TraceError otherwise."""
    p, nb = _host_ptr(record)
    n, k, G = ctypes.c_int64(), ctypes.c_int(), ctypes.c_int()
    _check("trace_record_check", lib.trace_record_check(p, nb, ctypes.byref(n), ctypes.byref(k), ctypes.byref(G)))
    return n.value, k.value, G.value


def record_from_host(record, guidance, g, device=None):
    """Enqueue the host->device copy of a record into `guidance` and `g`."""
    _need(guidance, torch.uint8, "guidance")
    _need(g, torch.float32, "g")
    p, nb = _host_ptr(record)
    _check("trace_record_from_host", lib.trace_record_from_host(
        p, nb, _ptr(guidance), _ptr(g), _stream(guidance.device)))
    return guidance, g


def record_write(path, record):
    p, nb = _host_ptr(record)
    _check("trace_record_write", lib.trace_record_write(str(path).encode(), p, nb))


def record_read(path, capacity, out=None):
    """Read a record file into a pinned host tensor of `capacity` bytes;
    returns the tensor trimmed to the record's size."""
    if out is None:
        out = torch.empty(int(capacity), dtype=torch.uint8, pin_memory=True)
    p, nb = _host_ptr(out)
    got = ctypes.c_size_t()
    _check("trace_record_read", lib.trace_record_read(str(path).encode(), p, nb, ctypes.byref(got)))
    return out[: got.value]


def xxh64(buf):
    p, nb = _host_ptr(buf)
    return int(lib.trace_xxh64(p, nb))
