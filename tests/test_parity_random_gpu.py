"""GPU parity against the oracle on seeded random geometries, every unit checked: head_dim
64 and 128, GQA groups 1 to 8, windows and beacon counts from none to many, ragged and
empty sequences, budgets from one row to the whole cache, with and without the beacon
update, max and mean aggregation.  Complements the hand-picked edge cases with breadth;
all sizes stay small enough for the oracle."""
import random

import pytest

from synth import WORKLOADS
from parity import all_units, check_units, log, run_gpu

pytestmark = pytest.mark.gpu

N_CASES = 64


def _workload(seed: int):
    rng = random.Random(seed)
    d = rng.choice([64, 128])
    hkv = rng.choice([1, 2, 4])
    g = rng.choice([1, 2, 4, 7, 8])
    window = rng.choice([0, 1, 8, 17, 32, 40])
    nb_max = rng.choice([0, 4, 16, 32])
    while g * window + nb_max > 512:
        window //= 2
    t_new = rng.choice([0, 0, 8, 32]) if nb_max > 0 else 0
    if g * window + nb_max == 0 and rng.random() < 0.7:
        window = 4
    cap = rng.choice([64, 300, 777, 1024, 2049, 3000])
    batch = rng.choice([1, 2, 3])
    ragged = rng.random() < 0.5
    budget = rng.randint(max(window, 1), cap)
    w = WORKLOADS["tiny"].replace(
        name=f"random_{seed}", n_layers=rng.choice([1, 2]), n_q_heads=hkv * g, n_kv_heads=hkv, head_dim=d,
        batch=batch, capacity=cap, seq_len=None if ragged else rng.randint(0, cap),
        ragged=(0, cap) if ragged else None, window=window, nb_init=rng.randint(0, nb_max), nb_max=nb_max,
        budget=budget, t_new=t_new, kind=rng.choice(["gauss", "cluster"]), n_clusters=4, seed=0xBEA000 + seed)
    return w, rng.choice(["max", "max", "mean"])


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_geometry(seed):
    w, aggregation = _workload(seed)
    log(f"[random] {w.name}: d {w.head_dim} Hq/Hkv {w.n_q_heads}/{w.n_kv_heads} layers {w.n_layers} "
        f"batch {w.batch} cap {w.capacity} L {w.seq_len if w.ragged is None else 'ragged'} window {w.window} "
        f"nb {w.nb_init}/{w.nb_max} budget {w.budget} t_new {w.t_new} {w.kind} {aggregation}")
    ev, _ = run_gpu(w, aggregation=aggregation)
    worst = check_units(w, ev, all_units(w))
    log(f"[random] {w.name}: worst {worst}")
