"""Host logic of the one-pass phase-clock measurement (CPU): the phase split
computed from fabricated clocks, and the measurement build's flag."""
import numpy as np

from precision_numerics_block_amd import build, phase_clock


def test_stats_from_clocks():
    # 16 workgroups, 10 ticks per us: start at 0..1.5 us, phase 1 ends at
    # 20 us + w * 0.5 us, the barrier passes for all at 29 us, phase 2 takes
    # 12 us for every workgroup
    w = np.arange(16, dtype=np.float64)
    c = np.stack([w, 200 + 5 * w, np.full(16, 290.0), np.full(16, 410.0)], axis=1) + 1000
    st = phase_clock._stats(c, 0.1)
    assert st["workgroups"] == 16
    assert abs(st["start_spread"] - 1.5) < 1e-9
    assert abs(st["phase1_end_first"] - 20.0) < 1e-9 and abs(st["phase1_end_last"] - 27.5) < 1e-9
    assert abs(st["phase1_end_median"] - 23.75) < 1e-9
    assert abs(st["barrier_wait_median"] - (29.0 - 23.75)) < 1e-9
    assert abs(st["phase2_median"] - 12.0) < 1e-9
    assert abs(st["span"] - 41.0) < 1e-9
    # workgroup w runs on XCD w mod 8: XCD 0 holds w = 0 and 8
    assert len(st["phase1_end_by_xcd"]) == 8
    assert abs(st["phase1_end_by_xcd"][0] - 22.0) < 1e-9


def test_measurement_build_is_not_the_product():
    assert build.OUT_PHASE_CLOCK != build.OUT
    assert build.OUT_PHASE_CLOCK.endswith("libtrace_quant_phaseclock.so")
