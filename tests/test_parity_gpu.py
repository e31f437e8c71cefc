"""GPU parity against the CPU oracle, every unit checked, on workloads small enough for
the oracle: the tiny workload at full size, the four model-shaped workloads with fewer
layers and shorter caches (still many tiles and ragged tails), and edge cases."""
import pytest
import torch

from synth import WORKLOADS
from parity import all_units, check_units, log, run_gpu

pytestmark = pytest.mark.gpu


def _run_all(w, aggregation="max", beacon_policy="fps"):
    log(f"[parity] {w.name}: layers {w.n_layers} batch {w.batch} cap {w.capacity} window {w.window} "
        f"nb {w.nb_init}/{w.nb_max} budget {w.budget} t_new {w.t_new} aggregation {aggregation} "
        f"beacons {beacon_policy}")
    ev, _ = run_gpu(w, aggregation=aggregation, beacon_policy=beacon_policy)
    worst = check_units(w, ev, all_units(w))
    log(f"[parity] {w.name}: worst {worst}")
    return worst


def test_tiny_full_size():
    _run_all(WORKLOADS["tiny"])


@pytest.mark.parametrize("name,kw", [
    ("qwen7b_16k", dict(n_layers=2, capacity=3000, seq_len=2989, budget=700)),
    ("llama8b_32k", dict(n_layers=1, batch=2, capacity=2304, seq_len=2304, budget=512)),
    ("qwen14b_64k", dict(n_layers=1, batch=1, capacity=4096, seq_len=4001, budget=1024)),
    ("qwen4b_serving", dict(n_layers=1, batch=3, capacity=2048, ragged=(700, 2048), budget=400)),
])
def test_model_shapes_reduced(name, kw):
    _run_all(WORKLOADS[name].replace(name=name + "_reduced", **kw))


EDGE = {
    # lengths around the budget, the window and tile edges; an empty sequence
    "lengths": WORKLOADS["tiny"].replace(batch=8, capacity=700,
                                         lengths=(0, 5, 127, 128, 129, 257, 511, 700), t_new=0),
    # head_dim 128, no beacons, no window: recent-only is empty, scores all zero
    "no_observers": WORKLOADS["tiny"].replace(head_dim=128, window=0, nb_init=0, nb_max=0, t_new=0,
                                              capacity=300, seq_len=300),
    # window only (recent-query scoring, n_beacon = 0)
    "recent_only": WORKLOADS["tiny"].replace(nb_init=0, nb_max=0, t_new=0, capacity=1000, seq_len=999),
    # beacons only, partial live count
    "beacons_only": WORKLOADS["tiny"].replace(window=0, nb_init=3, nb_max=8, t_new=0, capacity=600, seq_len=600,
                                              budget=64),
    # largest observation set: 4 * 120 + 32 = 512 rows
    "max_obs": WORKLOADS["qwen7b_16k"].replace(n_layers=1, n_q_heads=16, n_kv_heads=4, window=120, nb_init=32,
                                               nb_max=32, capacity=1500, seq_len=1500, budget=600),
    # head_dim 64 with 6 row blocks: two blocks on some waves of the register-resident stats pass
    "two_blocks_d64": WORKLOADS["tiny"].replace(n_q_heads=16, n_kv_heads=2, window=20, nb_init=16, nb_max=16,
                                                t_new=0, capacity=900, seq_len=877, budget=300),
    # exactly 256 observation rows (7 * 32 + 32), the most the 4-wave register-row stats pass takes
    "obs_256": WORKLOADS["qwen7b_16k"].replace(n_layers=1, capacity=1300, seq_len=1291, budget=400, nb_init=32,
                                               nb_max=32),
    # head_dim 64 with 11 row blocks (16 * 20 + 32 = 352 rows): three blocks on some waves
    "three_blocks_d64": WORKLOADS["tiny"].replace(n_q_heads=32, n_kv_heads=2, window=20, nb_init=32, nb_max=32,
                                                  t_new=0, capacity=1200, seq_len=1177, budget=300),
    # head_dim 128 with 9 row blocks (7 * 32 + 64 = 288 rows): the 8-wave register-row stats
    # pass with one wave holding two blocks and seven holding one
    "nine_blocks": WORKLOADS["qwen7b_16k"].replace(n_layers=2, capacity=1400, seq_len=1389, budget=500, nb_init=64,
                                                   nb_max=64),
    # head_dim 64 with 480 rows (8 * 56 + 32): above the register-row stats pass at head_dim 64,
    # so the LDS-staged stats pass
    "lds_stats_d64": WORKLOADS["tiny"].replace(n_q_heads=16, n_kv_heads=2, window=56, nb_init=32, nb_max=32,
                                               t_new=0, capacity=800, seq_len=777, budget=300),
    # window equals budget: nothing chosen by score
    "window_eq_budget": WORKLOADS["tiny"].replace(window=8, budget=8, t_new=0, capacity=400, seq_len=400),
    # more layers than one launch holds (48)
    "many_layers": WORKLOADS["tiny"].replace(n_layers=50, capacity=256, seq_len=250, budget=64, t_new=0),
    # FPS: pool smaller than capacity (copy path), then t_new < q_len
    "fps_small_pool": WORKLOADS["tiny"].replace(nb_init=2, nb_max=32, t_new=8),
    "fps_partial_new": WORKLOADS["qwen4b_serving"].replace(n_layers=1, batch=2, capacity=1024, ragged=(600, 1024),
                                                           t_new=48, window=16, budget=256, nb_init=5),
    "fps_empty_beacons": WORKLOADS["qwen4b_serving"].replace(n_layers=1, batch=2, capacity=512, ragged=(300, 512),
                                                             nb_init=0, budget=128),
}


@pytest.mark.parametrize("case", sorted(EDGE))
def test_edge_cases(case):
    _run_all(EDGE[case].replace(name=case))


def test_identical_keys_tie_to_lowest_positions():
    """All keys equal: every score is 1/L and the kept prefix is the lowest positions."""
    w = WORKLOADS["tiny"].replace(name="ties", t_new=0, capacity=512, seq_len=512)
    from parity import build_inputs, check_units
    inp = build_inputs(w)
    inp["k"][0][:] = inp["k"][0][0, 0, 0]
    ev, _ = run_gpu(w, inp)
    idx = ev.idx[0][0, 0].cpu().tolist()
    assert idx == list(range(w.budget - w.window)) + list(range(512 - w.window, 512))
    s = ev.scores[0][0, 0].cpu()
    assert torch.allclose(s, torch.full_like(s, 1 / 512), rtol=1e-5)


# Mean aggregation (Table 2's alternative to the max): same kernels up to the finish pass.
MEAN_CASES = {
    "tiny": WORKLOADS["tiny"],
    "qwen7b_reduced": WORKLOADS["qwen7b_16k"].replace(n_layers=2, capacity=3000, seq_len=2989, budget=700),
    "qwen4b_ragged_fps": WORKLOADS["qwen4b_serving"].replace(n_layers=1, batch=3, capacity=2048, ragged=(700, 2048),
                                                             budget=400),
    "qwen14b_352_rows": WORKLOADS["qwen14b_64k"].replace(n_layers=1, capacity=2048, seq_len=2001, budget=512),
    "lengths": EDGE["lengths"],
    "no_observers": EDGE["no_observers"],
}


@pytest.mark.parametrize("case", sorted(MEAN_CASES))
def test_mean_aggregation(case):
    _run_all(MEAN_CASES[case].replace(name="mean_" + case), aggregation="mean")


# Table 1's splits of the 32 observation slots per query step between recent queries and
# beacons (n_recent, n_beacon), on the serving shape with the continual-FPS update.
SPLITS = [(1, 31), (4, 28), (8, 24), (16, 16), (24, 8), (28, 4)]


@pytest.mark.parametrize("n_recent,n_beacon", SPLITS)
def test_recent_beacon_splits(n_recent, n_beacon):
    w = WORKLOADS["qwen4b_serving"].replace(name=f"split_{n_recent}_{n_beacon}", n_layers=1, batch=3, capacity=2048,
                                            ragged=(700, 2048), budget=512, window=n_recent, nb_init=n_beacon,
                                            nb_max=n_beacon)
    _run_all(w)


# Table 3's Initial+Recent: the beacon slots keep the earliest queries (filled in time
# order, frozen once full), scored with the recent window as usual.
INITIAL_CASES = {
    "tiny": WORKLOADS["tiny"],                                   # 4 live rows, slots full: frozen
    "empty_start": EDGE["fps_empty_beacons"],                    # no live rows: filled from new queries
    "partial_fill": EDGE["fps_small_pool"],                      # 2 live of 32 slots, pool smaller than slots
    "serving": WORKLOADS["qwen4b_serving"].replace(n_layers=1, batch=3, capacity=2048, ragged=(700, 2048),
                                                   budget=400, nb_init=5, t_new=3),
}


@pytest.mark.parametrize("case", sorted(INITIAL_CASES))
def test_initial_recent_beacons(case):
    _run_all(INITIAL_CASES[case].replace(name="initial_" + case), beacon_policy="initial")
