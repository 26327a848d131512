"""Rollout-guided FP4 (E2M1) fake-quant for MI355X (gfx950).

The compute lives in ``libtrace_quant.so`` (hand-written HIP kernels behind a
C ABI, declared in ``include/trace_quant.h``).  ``trace_quant`` is the thin
ctypes binding; importing it loads the library and fails loudly when it has
not been built.  ``qat`` wraps the fake-quant kernels as autograd functions
(straight-through backward).  ``synth`` draws the seeded synthetic workloads.
"""

__all__ = ["trace_quant", "synth", "qat"]


def __getattr__(name):
    if name in ("trace_quant", "synth", "qat"):
        import importlib

        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
