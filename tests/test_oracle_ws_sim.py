"""Pins of the warp-specialised GEMM event simulation (CPU only).

Each case has a schedule that follows from the kernel structure alone
(performance-model page for warp-specialised kernels: DMA loads A then B per
stage into a circular buffer, one MATH agent consumes stages in order), so
the expected start times are written in closed form:
- one slot: nothing overlaps, every stage costs T_A + T_B + T_MATH;
- loads slower than MATH: MATH starts each stage as soon as its B tile
  lands, at i (T_A + T_B);
- MATH slower than loads, with two or more slots: after the first load the
  MATH agent never waits, so stage i starts at T_A + T_B + i T_MATH;
- the wave and stage counts, and the two-point fit of a linear primitive.
Durations are dyadic so that every sum is exact.
"""
import math

import pytest

from oracle import ws_sim


def test_single_slot_is_fully_serial():
    ta, tb, tm, S = 1.5, 2.25, 4.0, 7
    st = ws_sim.simulate_wave(S, 1, ta, tb, tm)
    for i in range(S):
        assert st.load_a[i] == i * (ta + tb + tm)
        assert st.load_b[i] == i * (ta + tb + tm) + ta
        assert st.math[i] == i * (ta + tb + tm) + ta + tb
    assert st.math_end == S * (ta + tb + tm)
    assert st.math_wait == S * (ta + tb)


@pytest.mark.parametrize("ring", [2, 3, 8])
def test_load_bound_math_follows_each_load(ring):
    ta, tb, tm, S = 3.0, 2.5, 1.25, 9
    st = ws_sim.simulate_wave(S, ring, ta, tb, tm)
    for i in range(S):
        assert st.load_a[i] == i * (ta + tb)
        assert st.math[i] == (i + 1) * (ta + tb)
    assert st.math_end == S * (ta + tb) + tm
    assert st.math_wait == S * (ta + tb) - (S - 1) * tm


@pytest.mark.parametrize("ring", [2, 4, 16])
def test_math_bound_never_waits_after_the_first_load(ring):
    ta, tb, tm, S = 0.75, 0.5, 2.0, 12
    st = ws_sim.simulate_wave(S, ring, ta, tb, tm)
    for i in range(S):
        assert st.math[i] == ta + tb + i * tm
    assert st.math_end == ta + tb + S * tm
    assert st.math_wait == ta + tb
    # the DMA agent runs ahead by at most `ring` stages
    for i in range(ring, S):
        assert st.load_a[i] >= st.math[i - ring] + tm


def test_ring_bounds_how_far_dma_runs_ahead():
    """With two slots and loads much faster than MATH, stage i's A load
    starts exactly when MATH stage i - 2 ends."""
    ta, tb, tm, S = 0.25, 0.25, 4.0, 8
    st = ws_sim.simulate_wave(S, 2, ta, tb, tm)
    assert st.load_a[0] == 0 and st.load_a[1] == ta + tb
    for i in range(2, S):
        assert st.load_a[i] == st.math[i - 2] + tm


def test_empty_wave():
    st = ws_sim.simulate_wave(0, 2, 1.0, 1.0, 1.0)
    assert st.math_end == 0 and st.load_a == []


def test_wave_and_stage_counts():
    assert ws_sim.waves(1024, 1024, 128, 128, 84) == math.ceil(64 / 84)
    assert ws_sim.waves(8192, 8192, 256, 128, 256) == 8
    assert ws_sim.waves(8192, 8192, 256, 128, 248) == math.ceil(2048 / 248)
    assert ws_sim.waves(1000, 1000, 128, 64, 256) == 1
    assert ws_sim.stages(1024, 64) == 16 and ws_sim.stages(1000, 64) == 16
    assert ws_sim.stages(64, 128) == 1


def test_launch_time_composes_waves():
    """(end of the last MATH stage + T_EPILOGUE) W + T_INIT, math-bound."""
    ld_thr, ld_lat, c_thr, c_lat = 1024.0, 0.5, 32768.0, 0.25
    t = ws_sim.launch_time(512, 512, 1024, 128, 128, 64, 3, 4, ld_thr, ld_lat, c_thr, c_lat,
                           1.0, 2.0)
    ta = 128 * 64 / ld_thr + ld_lat
    tm = 128 * 128 * 64 / c_thr + c_lat
    assert tm > 2 * ta
    wave = ta + ta + 16 * tm
    assert t == (wave + 1.0) * 4 + 2.0


def test_two_point_recovers_linear_parameters():
    thr, lat = 640.0, 0.375
    s1, s2 = 8192, 16384
    got = ws_sim.two_point(s1, s1 / thr + lat, s2, s2 / thr + lat)
    assert got == pytest.approx((thr, lat), rel=1e-12)


# ---- planted slips ---------------------------------------------------------

SIM_MUTANTS = {
    "no ring limit": ("free_slots -= 1", "free_slots -= 0"),
    "B load takes no time": ('push(now + t_load_b, "b_done", stage)', 'push(now, "b_done", stage)'),
    "slot freed at MATH start": ("            free_slots += 1\n", "            pass\n"),
    "wave count floored": ("math.ceil(math.ceil(M / T_M) * math.ceil(N / T_N) / n_units)",
                           "math.ceil(M / T_M) * math.ceil(N / T_N) // n_units"),
    "epilogue once per launch": ("(st.math_end + t_epilogue) * waves(M, N, T_M, T_N, n_units)",
                                 "st.math_end * waves(M, N, T_M, T_N, n_units) + t_epilogue"),
}

SIM_PINS = [
    test_single_slot_is_fully_serial,
    lambda: test_load_bound_math_follows_each_load(2),
    lambda: test_math_bound_never_waits_after_the_first_load(2),
    test_ring_bounds_how_far_dma_runs_ahead,
    test_wave_and_stage_counts,
    test_launch_time_composes_waves,
]


@pytest.mark.parametrize("name", sorted(SIM_MUTANTS))
def test_pins_catch_planted_slip(name, monkeypatch):
    import types
    old, new = SIM_MUTANTS[name]
    src = open(ws_sim.__file__).read()
    assert src.count(old) == 1, "mutation site vanished: %s" % name
    if name == "slot freed at MATH start":
        new_src = src.replace(old, new).replace(
            "            math_busy = True\n", "            math_busy = True\n            free_slots += 1\n")
    else:
        new_src = src.replace(old, new)
    mod = types.ModuleType("ws_sim_mutant")
    mod.__dict__["__name__"] = "ws_sim_mutant"
    import sys
    sys.modules["ws_sim_mutant"] = mod
    exec(compile(new_src, "ws_sim_mutant", "exec"), mod.__dict__)
    monkeypatch.setattr(sys.modules[__name__], "ws_sim", mod)
    failed = 0
    for pin in SIM_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError, TypeError):
            failed += 1
    del sys.modules["ws_sim_mutant"]
    assert failed >= 1, "no pin caught: %s" % name
