"""Event simulation of a warp-specialised GEMM workgroup, as the oracle of
the analytic performance model.

TEST INFRASTRUCTURE ONLY. Only the tests may import this module. The HIP
library and its Python binding never import it, and it imports nothing
from them.

What it simulates (performance-model page for warp-specialised kernels,
sections "Warp specialization kernel structure" and "Algorithm 1"): one
output tile is computed in S = ceil(K / T_K) stages. A DMA agent loads the
stage's A tile, then its B tile, into a circular buffer of `ring` slots and
pushes the stage; a MATH agent pops stages in order, computes each one, and
releases its slot when done. At most one MATH agent is active. The DMA agent
waits while the buffer is full; the MATH agent waits while it is empty.

This module does not use the page's max-recurrences. It runs the two agents
as an event-driven simulation over a time-ordered queue, with the buffer as
a count of free slots and a queue of loaded stages, and records when each
action starts. The recurrences are the model's closed description of the
same schedule; the library's implementation of them is tested against this
simulation.

Durations follow the page's linear primitives (section "Core formulas"):
    T_MATH   = T_M T_N T_K / compute_throughput + compute_latency
    T_LOAD_A = T_M T_K / load_throughput + load_latency
    T_LOAD_B = T_K T_N / load_throughput + load_latency
and a whole launch takes W = ceil(ceil(M / T_M) ceil(N / T_N) / n_units)
waves of workgroups. The page writes the launch time as
(S_m(S) + T_EPILOGUE) W + T_INIT, with S_m the start of a MATH stage; the
reading taken here is that a wave ends when its last MATH stage ends, so a
wave lasts S_m(S) + T_MATH + T_EPILOGUE.
"""
from __future__ import annotations

import heapq
import math
from dataclasses import dataclass


@dataclass
class StageTimes:
    load_a: list   # start of stage i's A load, i = 0 .. S-1
    load_b: list   # start of stage i's B load
    math: list     # start of stage i's MATH
    math_end: float  # end of the last MATH stage
    math_wait: float  # total time the MATH agent spent waiting for data


def simulate_wave(S: int, ring: int, t_load_a: float, t_load_b: float, t_math: float) -> StageTimes:
    """One workgroup's S stages with a `ring`-slot circular buffer."""
    if S < 0 or ring < 1:
        raise ValueError("S >= 0 and ring >= 1")
    load_a = [None] * S
    load_b = [None] * S
    math_start = [None] * S
    free_slots = ring
    loaded = []          # stages pushed by DMA, in order, not yet popped
    dma_next = 0         # next stage the DMA agent will load
    dma_busy = False
    math_next = 0
    math_busy = False
    math_idle_since = 0.0
    math_wait = 0.0
    events = []          # (time, seq, kind, stage)
    seq = 0

    def push(t, kind, stage):
        nonlocal seq
        heapq.heappush(events, (t, seq, kind, stage))
        seq += 1

    now = 0.0
    last_end = 0.0

    def try_start(t):
        nonlocal free_slots, dma_next, dma_busy, math_next, math_busy, math_wait
        if not dma_busy and dma_next < S and free_slots > 0:
            free_slots -= 1
            load_a[dma_next] = t
            dma_busy = True
            push(t + t_load_a, "a_done", dma_next)
        if not math_busy and math_next < S and loaded and loaded[0] == math_next:
            loaded.pop(0)
            math_start[math_next] = t
            math_wait += t - math_idle_since
            math_busy = True
            push(t + t_math, "math_done", math_next)

    try_start(now)
    while events:
        now, _, kind, stage = heapq.heappop(events)
        if kind == "a_done":
            load_b[stage] = now
            push(now + t_load_b, "b_done", stage)
        elif kind == "b_done":
            loaded.append(stage)
            dma_busy = False
            dma_next += 1
        elif kind == "math_done":
            math_busy = False
            math_next += 1
            math_idle_since = now
            free_slots += 1
            last_end = now
        # start whatever became possible; equal-time events settle first
        if not events or events[0][0] > now:
            try_start(now)
    return StageTimes(load_a, load_b, math_start, last_end, math_wait)


def waves(M: int, N: int, T_M: int, T_N: int, n_units: int) -> int:
    """W = ceil(ceil(M / T_M) ceil(N / T_N) / n_units)."""
    return math.ceil(math.ceil(M / T_M) * math.ceil(N / T_N) / n_units)


def stages(K: int, T_K: int) -> int:
    """S = ceil(K / T_K)."""
    return math.ceil(K / T_K)


def primitives(T_M, T_N, T_K, load_throughput, load_latency, compute_throughput,
               compute_latency):
    """(T_LOAD_A, T_LOAD_B, T_MATH) from the linear primitives."""
    t_a = T_M * T_K / load_throughput + load_latency
    t_b = T_K * T_N / load_throughput + load_latency
    t_m = T_M * T_N * T_K / compute_throughput + compute_latency
    return t_a, t_b, t_m


def launch_time(M, N, K, T_M, T_N, T_K, ring, n_units, load_throughput, load_latency,
                compute_throughput, compute_latency, t_epilogue, t_init) -> float:
    """Predicted time of one launch: W waves of one simulated workgroup."""
    t_a, t_b, t_m = primitives(T_M, T_N, T_K, load_throughput, load_latency,
                               compute_throughput, compute_latency)
    st = simulate_wave(stages(K, T_K), ring, t_a, t_b, t_m)
    return (st.math_end + t_epilogue) * waves(M, N, T_M, T_N, n_units) + t_init


def two_point(size1, time1, size2, time2):
    """Throughput and start-up latency of a linear primitive time = size /
    throughput + latency, from two measurements (the page's two-point
    calibration)."""
    thr = (size1 - size2) / (time1 - time2)
    return thr, time1 - size1 / thr
