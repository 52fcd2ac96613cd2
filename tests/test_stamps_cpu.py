"""The arithmetic of summarize_stamps (fc_stamped_call's per-block counter
readings into clock and cycle figures), pinned on hand-built readings."""
from __future__ import annotations

import numpy as np
import pytest

from sharded_fc_layer_amd import fcshard as F


def _block(t0, r0, clock_ghz, setup, prologue, per_stage, stages, epilogue, wall_mhz=100.0):
    t2 = t0 + setup
    t3 = t2 + prologue
    t4 = t3 + per_stage * stages
    t5 = t4 + epilogue
    r6 = r0 + (t5 - t0) * wall_mhz / (clock_ghz * 1e3)  # constant-rate ticks over the block's life
    return [t0, r0, t2, t3, t4, t5, r6, stages]


def test_one_block_figures():
    s = np.array([_block(10_000, 500, 2.0, 100, 2000, 2300, 128, 7000)], dtype=np.int64)
    r = F.summarize_stamps(s, 100.0)
    assert r["blocks"] == 1
    assert r["clock_GHz"] == pytest.approx(2.0, rel=1e-12)
    assert r["setup_cycles"] == 100 and r["prologue_cycles"] == 2000 and r["epilogue_cycles"] == 7000
    assert r["loop_cycles_per_stage"] == pytest.approx(2300)
    assert r["block_cycles"] == 100 + 2000 + 2300 * 128 + 7000
    assert r["stages"] == 128


def test_blocks_combine_by_elapsed_ticks():
    # two blocks of equal length at 2.0 and 1.0 GHz: the clock is total ticks
    # over total time (4/3 GHz), not the mean of the two clocks (1.5)
    a = _block(0, 0, 2.0, 0, 0, 1000, 10, 0)
    b = _block(0, 0, 1.0, 0, 0, 1000, 10, 0)
    r = F.summarize_stamps(np.array([a, b], dtype=np.float64), 100.0)
    assert r["clock_GHz"] == pytest.approx(4.0 / 3.0, rel=1e-12)
    # per-stage cycles average over blocks, each over its own stage count
    c = _block(0, 0, 2.0, 0, 0, 3000, 4, 0)
    r = F.summarize_stamps(np.array([a, c], dtype=np.float64), 100.0)
    assert r["loop_cycles_per_stage"] == pytest.approx(2000.0)
    assert r["stages"] == pytest.approx(7.0)


def test_wall_clock_rate_scales_the_clock():
    s = np.array([_block(0, 0, 2.4, 0, 0, 2000, 6, 0, wall_mhz=25.0)])
    assert F.summarize_stamps(s, 25.0)["clock_GHz"] == pytest.approx(2.4, rel=1e-12)


def test_malformed_readings_are_refused():
    with pytest.raises(ValueError):
        F.summarize_stamps(np.zeros((0, F.STAMP_SLOTS)), 100.0)
    with pytest.raises(ValueError):
        F.summarize_stamps(np.zeros((2, 7)), 100.0)
    blk = _block(0, 0, 2.0, 0, 0, 1000, 6, 0)
    frozen = list(blk)
    frozen[6] = frozen[1]  # no constant-rate ticks
    with pytest.raises(ValueError):
        F.summarize_stamps(np.array([frozen]), 100.0)
    no_stages = list(blk)
    no_stages[7] = 0
    with pytest.raises(ValueError):
        F.summarize_stamps(np.array([no_stages]), 100.0)


def test_launch_span_and_occupancy():
    # 4 CUs, 6 blocks: four start at 0 and run 1000 constant-rate ticks, two
    # start at 1000 and run 500 ticks: span 1500, lifetimes 5000 of 6000
    blocks = [[0, 0, 0, 0, 20_000, 20_000, 1000, 10]] * 4 + [[0, 1000, 0, 0, 10_000, 10_000, 1500, 10]] * 2
    r = F.summarize_stamps(np.array(blocks), 100.0, compute_units=4)
    assert r["launch_span_us"] == pytest.approx(15.0)
    assert r["cu_occupancy"] == pytest.approx(5000 / 6000)
    assert "cu_occupancy" not in F.summarize_stamps(np.array(blocks), 100.0)
