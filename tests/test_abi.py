"""C-ABI contract checks that need no GPU: the library loads, exports every
function include/trace_quant.h declares, computes sizes on the host, and
rejects bad arguments before it touches the HIP runtime."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "trace_quant.h")

OK, E_NULL, E_SIZE, E_ALIGN, E_K, E_DTYPE, E_SCRATCH = 0, -1, -2, -3, -4, -5, -11
A = 0x100000          # a fake, 16-byte aligned "device" address (never dereferenced)


@pytest.fixture(scope="module")
def tq():
    from precision_numerics_block_amd import trace_quant

    return trace_quant


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(trace_[a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_exports_every_declared_symbol(tq):
    names = declared_functions()
    assert len(names) >= 11, names
    for name in names:
        assert hasattr(tq.lib, name), name
    # and the binding wraps each of them
    for name in names:
        assert name in tq._SIGS


def test_sizes(tq):
    n = 16 * 40
    assert tq.code_bytes(n) == n // 2
    assert tq.scale_bytes(n) == n // 16
    assert tq.guidance_bytes(n, 1) == 256 + n // 8
    assert tq.guidance_bytes(n, 2) == 256 + n // 4
    assert tq.guidance_bytes(n, 4) == 256 + n // 2
    n = 16 * 256 * 3                         # scale plane exactly 768 bytes: no pad
    assert tq.guidance_bytes(n, 2) == 768 + n // 4
    assert tq.guidance_bytes(n, 3) == 768 + 3 * n // 8
    assert tq.guidance_bytes(n, 5) == 0 and tq.guidance_bytes(n, 0) == 0
    assert tq.code_bytes(17) == 0 and tq.code_bytes(0) == 0
    assert tq.version() >= 100
    assert tq.lib.trace_status_str(-7).decode().startswith("an input")
    assert tq.onepass_work_bytes(1) == 25344 and tq.onepass_work_bytes(64) == 25344
    assert tq.onepass_work_bytes(65) == 25600 and tq.onepass_work_bytes(0) == 0
    assert "barrier" in tq.lib.trace_status_str(-10).decode()
    assert "4096" in tq.lib.trace_status_str(-11).decode()
    assert "2^34" in tq.lib.trace_status_str(-2).decode()
    assert tq.mx_scale_bytes(32 * 10) == 10 and tq.mx_scale_bytes(16) == 0
    assert tq.mx_guidance_bytes(32 * 10, 2) == 256 + 80 and tq.mx_guidance_bytes(32 * 10, 5) == 0
    assert tq.onepass_capacity(-1) == 0                 # argument error, before any device query


def test_argument_errors_before_any_hip_call(tq):
    L = tq.lib
    n = 16 * 64
    # sizes
    assert L.trace_amax(A, 0, 1, A, None, None) == E_SIZE
    assert L.trace_amax(A, 24, 1, A, None, None) == E_SIZE
    assert L.trace_amax(A, n, 3, A, None, None) == E_SIZE
    assert L.trace_amax(A, n, 0, A, None, None) == E_SIZE
    assert L.trace_amax(A, 1 << 36, 1, A, None, None) == E_SIZE
    assert L.trace_amax(A, 1 << 35, 1, A, None, None) == E_SIZE
    assert L.trace_amax(A, 1 << 34, 1, A, None, None) == E_SIZE         # chunk counts stay below 2^31
    # null pointers
    assert L.trace_amax(None, n, 1, A, None, None) == E_NULL
    assert L.trace_quant_rollout(A, n, 1, None, 2, A, A, None, None) == E_NULL
    assert L.trace_quant_rollout(A, n, 1, A, 2, None, A, None, None) == E_NULL
    assert L.trace_guidance_pack(A, None, n, 2, A, None) == E_NULL
    assert L.trace_fakequant_guided(A, n, 1, A, None, 2, A, 0, None, None) == E_NULL
    assert L.trace_fakequant_fullcode(A, n, 1, A, None, A, 0, None, None) == E_NULL
    assert L.trace_fakequant_rtn(A, n, 1, None, None, A, 0, None, None, None) == E_NULL
    # alignment
    assert L.trace_amax(A + 2, n, 1, A, None, None) == E_ALIGN
    assert L.trace_quant_rollout(A, n, 1, A, 2, A + 8, A, None, None) == E_ALIGN
    assert L.trace_fakequant_guided(A, n, 1, A, A + 1, 2, A, 0, None, None) == E_ALIGN
    assert L.trace_fakequant_rtn(A, n, 1, A, A + 4, A, 0, None, None, None) == E_ALIGN
    # guidance width and output dtype
    assert L.trace_quant_rollout(A, n, 1, A, 5, A, A, A, None) == E_K
    assert L.trace_guidance_pack(A, A, n, 0, A, None) == E_K
    assert L.trace_fakequant_guided(A, n, 1, A, A, 4, A, 0, None, None) == E_K
    assert L.trace_fakequant_guided(A, n, 1, A, A, 2, A, 7, None, None) == E_DTYPE
    assert L.trace_fakequant_rtn(A, n, 1, A, None, A, 2, None, None, None) == E_DTYPE
    # weight quantisation: its own checks come before the amax it enqueues
    qw = L.trace_quant_weight
    assert qw(A, 24, 1, A, A, A, None, None) == E_SIZE
    assert qw(A, n, 3, A, A, A, None, None) == E_SIZE
    assert qw(None, n, 1, A, A, A, None, None) == E_NULL
    assert qw(A, n, 1, None, A, A, None, None) == E_NULL
    assert qw(A, n, 1, A, None, A, None, None) == E_NULL
    assert qw(A, n, 1, A, A, None, None, None) == E_NULL
    assert qw(A, n, 1, A, A + 8, A, None, None) == E_ALIGN
    assert qw(A, n, 1, A, A, A + 4, None, None) == E_ALIGN
    assert qw(A, n, 1, A, A, A, A + 4, None) == E_ALIGN
    # one-pass rollout: every argument error is found before the device query
    op = L.trace_quant_rollout_onepass
    assert op(A, 24, 1, 2, A, A, A, None, A, 0, None, None) == E_SIZE
    assert op(A, n, 3, 2, A, A, A, None, A, 0, None, None) == E_SIZE
    assert op(A, n, 1, 2, A, A, A, None, A, -1, None, None) == E_SIZE
    assert op(A, n, 1, 2, A, A, A, None, None, 0, None, None) == E_NULL
    assert op(A, n, 1, 2, None, A, A, None, A, 0, None, None) == E_NULL
    assert op(A, n, 1, 2, A, A, A, None, A + 4, 0, None, None) == E_ALIGN
    assert op(A, n, 1, 2, A, A, A, A + 8, A, 0, None, None) == E_ALIGN
    assert op(A, n, 1, 2, A, A, A, None, A, 0, A + 2, None) == E_ALIGN
    assert op(A, n, 1, 5, A, A, A, None, A, 0, None, None) == E_K
    rop = L.trace_fakequant_rtn_onepass
    assert rop(A, 24, 1, A, A, 0, None, None, A, 0, None, None) == E_SIZE
    assert rop(A, n, 1, A, A, 0, None, None, None, 0, None, None) == E_NULL
    assert rop(A, n, 1, None, A, 0, None, None, A, 0, None, None) == E_NULL
    assert rop(A, n, 1, A, A + 2, 0, None, None, A, 0, None, None) == E_ALIGN
    assert rop(A, n, 1, A, A, 0, A + 8, None, A, 0, None, None) == E_ALIGN
    assert rop(A, n, 1, A, A, 5, None, None, A, 0, None, None) == E_DTYPE
    assert rop(A, n, 1, A, A, 0, None, None, A, -2, None, None) == E_SIZE
    # a workgroup cap that would give one workgroup a run of 2^30 chunks or
    # more (32-bit output spans): rejected before the device query
    assert op(A, 1 << 33, 1, 4, A, A, A, A, A, 1, None, None) == E_SIZE        # codes: 2^30 chunks x 4 B
    assert rop(A, 1 << 30, 1, A, A, 1, None, None, A, 1, None, None) == E_SIZE  # f32 y: 2^27 chunks x 32 B
    # the allocation-free one-pass rollout: the same checks (no work buffer),
    # then its static scratch limit of 4096 groups, all before any HIP call
    na = L.trace_quant_rollout_onepass_noalloc
    assert na(A, 24, 1, 2, A, A, A, None, 0, None, None) == E_SIZE
    assert na(A, n, 3, 2, A, A, A, None, 0, None, None) == E_SIZE
    assert na(A, n, 1, 2, A, A, A, None, -1, None, None) == E_SIZE
    assert na(A, 1 << 33, 1, 2, A, A, A, None, 1, None, None) == E_SIZE
    assert na(None, n, 1, 2, A, A, A, None, 0, None, None) == E_NULL
    assert na(A, n, 1, 2, A, None, A, None, 0, None, None) == E_NULL
    assert na(A, n, 1, 2, A, A, A + 8, None, 0, None, None) == E_ALIGN
    assert na(A, n, 1, 2, A, A, A, A + 4, 0, None, None) == E_ALIGN
    assert na(A, n, 1, 0, A, A, A, None, 0, None, None) == E_K
    assert na(A, 16 * 4097, 4097, 2, A, A, A, None, 0, None, None) == E_SCRATCH
    assert na(A, 16 * 8192 * 3, 8192, 2, A, A, A, A, 0, None, None) == E_SCRATCH
    # MX variant
    assert L.trace_mx_quant_rollout(A, 48, 2, A, A, None, None) == E_SIZE
    assert L.trace_mx_quant_rollout(A, n, 2, None, A, None, None) == E_NULL
    assert L.trace_mx_quant_rollout(A, n, 2, A, A + 4, None, None) == E_ALIGN
    assert L.trace_mx_quant_rollout(A, n, 0, A, A, None, None) == E_K
    assert L.trace_mx_fakequant_guided(A, n, None, 2, A, 0, None, None) == E_NULL
    assert L.trace_mx_fakequant_guided(A, n, A, 5, A, 0, None, None) == E_K
    assert L.trace_mx_fakequant_guided(A, n, A, 2, A, 3, None, None) == E_DTYPE
    assert L.trace_mx_fakequant_rtn(A, 16, None, A, 0, None, None, None) == E_SIZE
    assert L.trace_mx_fakequant_rtn(A, n, A + 8, A, 0, None, None, None) == E_ALIGN


def test_binding_rejects_cpu_tensors(tq):
    import torch

    x = torch.zeros(64, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        tq.amax(x)
    assert ctypes.sizeof(ctypes.c_void_p) == 8
