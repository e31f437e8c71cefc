"""Beacon coverage (Figure 6 (a)) on the CPU: the synthetic query stream has the intended
phases, and continual FPS over it (the oracle) keeps the plan clusters that late queries
revisit, which the recent window alone does not."""
import numpy as np

from oracle import bkv_oracle as O
from synth import WORKLOADS, bf16_bits
from synth.stream import query_stream


def _unit_max_cos(fut, sets):
    f = fut / np.linalg.norm(fut, axis=1, keepdims=True)
    s = sets / np.linalg.norm(sets, axis=1, keepdims=True)
    return (f @ s.T).max(axis=1)


def test_stream_phases_and_determinism():
    w = WORKLOADS["qwen14b_64k"]
    q1, c1 = query_stream(w, 0, 1, 2, 800, 200)
    q2, c2 = query_stream(w, 0, 1, 2, 800, 200)
    assert q1.shape == (w.group, 1000, w.head_dim)
    assert bf16_bits(q1).tobytes() == bf16_bits(q2).tobytes() and np.array_equal(c1, c2)
    early = int(0.05 * 800)
    assert np.all(c1[:, early:800] >= w.n_plan)                   # no plan cluster mid-stream
    assert (c1[:, :early] < w.n_plan).any()                        # the plan appears early
    assert abs((c1[:, 800:] < w.n_plan).mean() - w.recent_plan_p) < 0.08   # and is revisited


def test_continual_fps_keeps_the_plan_the_recent_window_lost():
    w = WORKLOADS["qwen14b_64k"]
    steps, future, chunk, nb, window = 640, 256, 128, w.nb_max, w.window
    q, cid = query_stream(w, 0, 0, 0, steps, future)
    bits = bf16_bits(q)                                            # [G, steps + future, D]
    beacons, n = np.zeros((nb, w.head_dim), np.uint16), 0
    for c0 in range(0, steps, chunk):
        rows, n, _ = O.update_beacons(beacons, n, bits[:, c0:c0 + chunk], nb)
        beacons = np.zeros((nb, w.head_dim), np.uint16)
        beacons[:n] = rows
    fut = O.bf16_to_f64(bits[:, steps:]).reshape(-1, w.head_dim)
    revisit = (cid[:, steps:] < w.n_plan).reshape(-1)
    cov_fps = _unit_max_cos(fut, O.bf16_to_f64(beacons[:n]))
    cov_recent = _unit_max_cos(fut, O.bf16_to_f64(bits[:, steps - window:steps]).reshape(-1, w.head_dim))
    assert cov_fps[revisit].mean() > 0.8            # a beacon sits in every plan cluster
    assert cov_recent[revisit].mean() < 0.3         # the window has moved on
    assert cov_fps[~revisit].mean() > 0.8 and cov_recent[~revisit].mean() > 0.8
