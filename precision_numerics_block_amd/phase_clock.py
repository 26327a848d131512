"""Phase split of the one-pass kernels, from their own clocks.

The measurement build of the library (build.build_phase_clock: the same
sources with TRACE_OP_PHASE_CLOCK=1) makes thread 0 of every workgroup of
k_quant_onepass write the wall clock at four points: the kernel's start, the
end of phase 1 (the workgroup's share read once, its maxima folded and
published), the moment the grid barrier let it through, and the end of
phase 2 (its share converted and stored).  This script runs the one-pass
rollout (k = 2) and the one-pass own-scale RTN (bf16 out) on tensors that
fit one launch and prints, per case, over the workgroups of one launch
(median of several launches): when phase 1 ends (first, median, last
workgroup), the barrier wait, phase 2, and the launch's span; and the median
phase-1 end per XCD (workgroup w runs on XCD w mod 8).

    python -m precision_numerics_block_amd.phase_clock build   # here (hipcc)
    python -m precision_numerics_block_amd.phase_clock run     # on the GPU

It loads the measurement library with ctypes and nothing else of the
package's binding; inputs come from synth.  The product library is not
touched."""
import ctypes
import json
import statistics
import sys

from precision_numerics_block_amd import build as _build

CASES = [  # (label, workload, tensor spec index or "kv", G)
    ("activations 64x512x2048, G=1", 2, 0, 1),
    ("KV layer 2x32768x8x128, G=2", 3, "kv", 2),
]


def _lib():
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib = ctypes.CDLL(_build.OUT_PHASE_CLOCK)
    lib.trace_debug_phase_clock.restype, lib.trace_debug_phase_clock.argtypes = i32, [vp]
    lib.trace_quant_rollout_onepass.argtypes = [vp, i64, i32, i32, vp, vp, vp, vp, vp, i32, vp, vp]
    lib.trace_fakequant_rtn_onepass.argtypes = [vp, i64, i32, vp, vp, i32, vp, vp, vp, i32, vp, vp]
    lib.trace_onepass_work_bytes.restype, lib.trace_onepass_work_bytes.argtypes = ctypes.c_size_t, [i32]
    lib.trace_guidance_bytes.restype, lib.trace_guidance_bytes.argtypes = ctypes.c_size_t, [i64, i32]
    return lib


def _tensor(torch, synth, wl, which, dev):
    specs = synth.tensor_specs(wl)
    if which == "kv":
        (K, _), (V, _) = [synth.make_pair(wl, i, specs[i][1], dev) for i in (len(specs) - 2, len(specs) - 1)]
        return torch.stack([K, V])
    return synth.make_pair(wl, which, specs[which][1], dev)[0]


def _stats(c, tick_us):
    """Phase times (us) of one launch from its clocks c[w] = (start, end of
    phase 1, barrier passed, end of phase 2), relative to the first start."""
    t0 = c[:, 0].min()
    e1 = (c[:, 1] - t0) * tick_us
    return dict(
        workgroups=len(c),
        start_spread=(c[:, 0].max() - t0) * tick_us,
        phase1_end_first=e1.min(), phase1_end_median=float(statistics.median(e1)), phase1_end_last=e1.max(),
        barrier_wait_median=float(statistics.median((c[:, 2] - c[:, 1]) * tick_us)),
        phase2_median=float(statistics.median((c[:, 3] - c[:, 2]) * tick_us)),
        span=(c[:, 3].max() - t0) * tick_us,
        phase1_end_by_xcd=[float(statistics.median(e1[i::8])) for i in range(8)])


def run(reps=7):
    import torch

    from precision_numerics_block_amd import synth

    dev = "cuda:0"
    lib = _lib()
    P = lambda t: ctypes.c_void_p(t.data_ptr())                            # noqa: E731
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = {}
    for label, wl, which, G in CASES:
        x = _tensor(torch, synth, wl, which, dev)
        n = x.numel()
        work = torch.zeros(lib.trace_onepass_work_bytes(G), dtype=torch.uint8, device=dev)
        st = torch.zeros(4, dtype=torch.int32, device=dev)
        g = torch.empty(G, device=dev)
        codes = torch.empty(n // 2, dtype=torch.uint8, device=dev)
        scales = torch.empty(n // 16, dtype=torch.uint8, device=dev)
        gd = torch.empty(lib.trace_guidance_bytes(n, 2), dtype=torch.uint8, device=dev)
        y = torch.empty_like(x)
        clock = torch.zeros(4 * 4096, dtype=torch.int64, device=dev)
        khz = lib.trace_debug_phase_clock(P(clock))
        if khz <= 0:
            raise RuntimeError("no wall-clock rate for the current device")
        tick_us = 1e3 / khz
        calls = {
            "rollout k=2": lambda: lib.trace_quant_rollout_onepass(P(x), n, G, 2, P(g), P(codes), P(scales), P(gd),
                                                                   P(work), 0, P(st), s),
            "own-scale RTN, bf16 out": lambda: lib.trace_fakequant_rtn_onepass(P(x), n, G, P(g), P(y), 0, None, None,
                                                                               P(work), 0, P(st), s),
        }
        for name, call in calls.items():
            rows = []
            for r in range(reps + 2):
                clock.zero_()
                assert call() == 0
                torch.cuda.synchronize()
                assert int(st[0]) == 0
                c = clock.cpu().numpy().reshape(-1, 4)
                c = c[c[:, 0] != 0].astype("float64")
                if r >= 2:                                                   # two warm-up launches
                    rows.append(_stats(c, tick_us))
            med = {k: round(float(statistics.median([r[k] for r in rows])), 2) for k in rows[0]
                   if k != "phase1_end_by_xcd"}
            med["workgroups"] = int(med["workgroups"])
            med["phase1_end_by_xcd"] = [round(float(statistics.median([r["phase1_end_by_xcd"][i] for r in rows])), 2)
                                        for i in range(8)]
            out[f"{label}: {name}"] = med
            print(f"{label}: {name}: " + json.dumps(med), flush=True)
        lib.trace_debug_phase_clock(None)
    return out


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "build":
        print(_build.build_phase_clock(verbose=False))
    elif len(sys.argv) > 1 and sys.argv[1] == "run":
        run()
    else:
        sys.exit(__doc__)
