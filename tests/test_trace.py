"""The per-task trace analysis (persistent_megakernel_amd.trace.summarize) on synthetic traces.

A trace row holds six realtime-counter ticks per task (100 MHz): start, inputs observed, rows
done, end, first wave's rows done, outputs written. The analysis attributes each opcode's time
to waiting, computing and the epilogue, and finds the critical path of the launch: per phase
(opcode, layer) the moment its last task ended. The pages attribute the gap to their roofline to
a fixed cross-SM synchronisation cost per tile (AutoMegaKernel pages: page 2, "Performance
ceiling and gap"); this is the tool that measures that cost on this kernel. Here the timestamps
are built by hand, so every number the analysis reports is known exactly.
"""
from __future__ import annotations

import types

import numpy as np
import pytest

from persistent_megakernel_amd import _abi as A
from persistent_megakernel_amd.trace import TICK_US, summarize


def _sched(tasks, queues, waits=None, signals=None):
    """tasks: list of (opcode, layer); queues: list of lists of task ids; optional per-task waits
    [(counter, threshold)] and signalled counters."""
    n = len(tasks)
    waits = waits or [[] for _ in range(n)]
    signals = signals or [[] for _ in range(n)]
    ts = [types.SimpleNamespace(opcode=op, args=(layer, 0, 0, 0, 0), waits=waits[i], signals=signals[i])
          for i, (op, layer) in enumerate(tasks)]
    return types.SimpleNamespace(tasks=ts, queues=queues)


def _row(start, ready, done, end, w0=None, out=None):
    w0 = done if w0 is None else w0
    out = end if out is None else out
    return [start, ready, done, end, w0, out]


def test_two_cu_chain_attribution_and_critical_path():
    # CU 0: QKV (layer 0) then O (layer 0); CU 1: attention (layer 0)
    tasks = [(A.AMK_OP_QKV, 0), (A.AMK_OP_ATTN, 0), (A.AMK_OP_OPROJ, 0)]
    queues = [[0, 2], [1]]
    t0 = 1_000_000
    rows = {
        0: _row(t0, t0 + 100, t0 + 400, t0 + 500, w0=t0 + 350, out=t0 + 480),       # QKV: wait 1 us, compute 3 us
        1: _row(t0 + 50, t0 + 600, t0 + 900, t0 + 1000, out=t0 + 990),               # attention waits for QKV
        2: _row(t0 + 500, t0 + 1100, t0 + 1300, t0 + 1400, w0=t0 + 1290, out=t0 + 1380),
    }
    # trace rows are in queue order (CU 0's tasks, then CU 1's)
    order = [t for q in queues for t in q]
    tr = np.array([rows[t] for t in order], dtype=np.int64)
    res = summarize(_sched(tasks, queues), tr)
    assert res["n_cu"] == 2
    assert res["launch_us"] == pytest.approx(1400 * TICK_US)
    ops = res["ops_mean_us"]
    assert ops["qkv"]["wait"] == pytest.approx(100 * TICK_US)
    assert ops["qkv"]["compute"] == pytest.approx(300 * TICK_US)
    assert ops["qkv"]["epilogue"] == pytest.approx(100 * TICK_US)
    assert ops["qkv"]["wave_skew"] == pytest.approx(50 * TICK_US)
    assert ops["qkv"]["close"] == pytest.approx(20 * TICK_US)
    assert ops["attn"]["wait"] == pytest.approx(550 * TICK_US)
    assert ops["oproj"]["wait"] == pytest.approx(600 * TICK_US)
    # the critical path: phases by the time their last task ended, with the span from the previous
    phases = res["phases"]
    assert [p["op"] for p in phases] == ["qkv", "attn", "oproj"]
    assert [p["last_end_us"] for p in phases] == pytest.approx([500 * TICK_US, 1000 * TICK_US, 1400 * TICK_US])
    assert [p["span_us"] for p in phases] == pytest.approx([500 * TICK_US, 500 * TICK_US, 400 * TICK_US])
    assert phases[2]["last_inputs_us"] == pytest.approx(1100 * TICK_US)


def test_phase_end_is_the_last_task_of_the_phase():
    # one phase spread over three CUs: its end is the slowest CU's end, its inputs the latest
    tasks = [(A.AMK_OP_GATEUP, 3)] * 3
    queues = [[0], [1], [2]]
    tr = np.array([_row(10, 20, 30, 40), _row(10, 50, 70, 90), _row(10, 25, 35, 45)], dtype=np.int64)
    res = summarize(_sched(tasks, queues), tr)
    (p,) = res["phases"]
    assert p["op"] == "gateup" and p["layer"] == 3
    assert p["last_end_us"] == pytest.approx(80 * TICK_US)   # relative to the earliest start
    assert p["last_inputs_us"] == pytest.approx(40 * TICK_US)
    assert res["ops_mean_us"]["gateup"]["tasks"] == 3
    assert res["ops_mean_us"]["gateup"]["wait"] == pytest.approx(np.mean([10, 40, 15]) * TICK_US, abs=1e-3)   # rounded to ns


def test_merge_splits_at_its_chunk_weights_and_argmax_does_not_split():
    # merge: compute = inputs -> chunk weights, epilogue = the rest; argmax: all epilogue
    tasks = [(A.AMK_OP_MERGE, 0), (A.AMK_OP_ARGMAX, 1)]
    queues = [[0, 1]]
    tr = np.array([_row(0, 100, 120, 160, out=150), _row(160, 300, 0, 320, out=315)], dtype=np.int64)
    res = summarize(_sched(tasks, queues), tr)
    ops = res["ops_mean_us"]
    assert ops["merge"]["compute"] == pytest.approx(20 * TICK_US)
    assert ops["merge"]["epilogue"] == pytest.approx(40 * TICK_US)
    assert ops["argmax"]["compute"] == 0.0
    assert ops["argmax"]["epilogue"] == pytest.approx(20 * TICK_US)
    assert "wave_skew" not in ops["merge"]


def test_hops_from_the_last_producer_to_each_consumer():
    # two O tasks (CUs 0 and 1) signal counter 0; two gate/up tasks (CUs 1 and 2) wait on it
    tasks = [(A.AMK_OP_OPROJ, 4), (A.AMK_OP_OPROJ, 4), (A.AMK_OP_GATEUP, 4), (A.AMK_OP_GATEUP, 4)]
    queues = [[0], [1, 2], [3]]
    waits = [[], [], [(0, 2)], [(0, 2)]]
    signals = [[0], [0], [], []]
    rows = {
        0: _row(0, 10, 40, 60, out=50),
        1: _row(0, 10, 60, 80, out=70),          # the last producer publishes at 70 (CU 1)
        2: _row(80, 400, 500, 600),              # its own CU sees the inputs at 400: hop 330
        3: _row(20, 300, 450, 500),              # CU 2: hop 230
    }
    order = [t for q in queues for t in q]
    tr = np.array([rows[t] for t in order], dtype=np.int64)
    res = summarize(_sched(tasks, queues, waits, signals), tr)
    h = res["hops"]
    assert set(h) == {"gateup"}    # the O tasks wait on nothing here
    assert h["gateup"]["median_us"] == pytest.approx(280 * TICK_US)
    assert h["gateup"]["phase_max_median_us"] == pytest.approx(330 * TICK_US)
    assert h["gateup"]["slowest_on_last_producer_cu"] == 1.0
