"""Host logic of the QAT wrappers (CPU, no GPU): which kernel path plain QAT
takes, how the one-pass path's status word is handled, and the argument
checks.  The binding is replaced by a recorder that returns CPU tensors, so
only the wrappers' own control flow runs here."""
import types

import pytest
import torch

from precision_numerics_block_amd import qat

E_NONFINITE, E_BARRIER = -7, -10


class Recorder:
    """Stands in for the ctypes binding: records calls, returns tensors of
    the right shapes, and writes `onepass_status` into the status word."""

    TraceError = type("TraceError", (RuntimeError,), {})

    def __init__(self, onepass_status=0):
        self.calls = []
        self.onepass_status = onepass_status

    def amax(self, x, G=1, out=None, status=None):
        self.calls.append("amax")
        return torch.full((G,), 0.5)

    def fakequant_rtn(self, x, g, scales_in=None, G=1, out_dtype=0, out=None, codes_out=None, scales_out=None):
        self.calls.append("fakequant_rtn")
        return x.clone(), None, (torch.zeros(x.numel() // 16, dtype=torch.uint8) if scales_out else None)

    def fakequant_rtn_onepass(self, x, G=1, g=None, out_dtype=0, out=None, codes_out=None, scales_out=None,
                              work=None, max_workgroups=0, status=None):
        self.calls.append("fakequant_rtn_onepass")
        status[0] = self.onepass_status
        return torch.full((G,), 0.25), x.clone() + 1, None, torch.zeros(x.numel() // 16, dtype=torch.uint8)

    def fakequant_ste_grad(self, x, g, scales, gy, G=1, out=None):
        self.calls.append(("fakequant_ste_grad", float(g[0])))
        return gy * 0.5


@pytest.fixture
def rec(monkeypatch):
    def make(status=0):
        r = Recorder(status)
        fake = types.SimpleNamespace(**{nm: getattr(r, nm) for nm in (
            "amax", "fakequant_rtn", "fakequant_rtn_onepass", "fakequant_ste_grad")}, TraceError=r.TraceError)
        monkeypatch.setattr(qat, "tq", fake)
        return r
    return make


def test_default_path_is_two_kernel(rec):
    r = rec()
    x = torch.zeros(64, dtype=torch.bfloat16, requires_grad=True)
    y = qat.own_scale_fake_quant(x)
    assert r.calls == ["amax", "fakequant_rtn"]
    y.backward(torch.ones(64, dtype=torch.bfloat16))
    assert r.calls[-1] == ("fakequant_ste_grad", 0.5)          # the two-kernel path's g
    assert torch.equal(x.grad, torch.full((64,), 0.5, dtype=torch.bfloat16))


def test_onepass_path_reads_its_status(rec):
    r = rec(0)
    x = torch.zeros(64, dtype=torch.bfloat16, requires_grad=True)
    y = qat.own_scale_fake_quant(x, path="onepass")
    assert r.calls == ["fakequant_rtn_onepass"]
    assert torch.equal(y, torch.ones(64, dtype=torch.bfloat16))
    y.backward(torch.ones(64, dtype=torch.bfloat16))
    assert r.calls[-1] == ("fakequant_ste_grad", 0.25)         # the one-pass path's own g


def test_onepass_barrier_timeout_recomputes_with_two_kernels(rec):
    r = rec(E_BARRIER)
    x = torch.zeros(64, dtype=torch.bfloat16, requires_grad=True)
    with pytest.warns(RuntimeWarning, match="timed out"):
        y = qat.own_scale_fake_quant(x, path="onepass")
    assert r.calls == ["fakequant_rtn_onepass", "amax", "fakequant_rtn"]
    assert torch.equal(y, x.detach())                            # the two-kernel result
    y.backward(torch.ones(64, dtype=torch.bfloat16))
    assert r.calls[-1] == ("fakequant_ste_grad", 0.5)


def test_onepass_nonfinite_raises(rec):
    rec(E_NONFINITE)
    with pytest.raises(RuntimeError):
        qat.own_scale_fake_quant(torch.zeros(64, dtype=torch.bfloat16), path="onepass")


def test_identity_ste_skips_the_mask(rec):
    r = rec()
    x = torch.zeros(64, dtype=torch.bfloat16, requires_grad=True)
    qat.own_scale_fake_quant(x, ste="identity").backward(torch.full((64,), 3.0, dtype=torch.bfloat16))
    assert all(c in ("amax", "fakequant_rtn") for c in r.calls)
    assert torch.equal(x.grad, torch.full((64,), 3.0, dtype=torch.bfloat16))


def test_bad_arguments(rec):
    rec()
    x = torch.zeros(64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        qat.own_scale_fake_quant(x, path="one_pass")
    with pytest.raises(ValueError):
        qat.own_scale_fake_quant(x, ste="clip")
    with pytest.raises(ValueError):
        qat.guided_fake_quant(x, torch.ones(1), torch.zeros(4, dtype=torch.uint8), ste="none")
