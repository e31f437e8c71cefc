"""Parity where a logit lands far above its row's running max in the middle of a unit piece,
so the scorer's statistics passes take their exact branch (new max, earlier sum rescaled)
with a finite running max, and the finish pass merges partial statistics whose maxima
differ by hundreds (log2 units).  BeaconKV page, Figure 5 (b), (c): the scores are softmax
attention weights, so one key that dominates a row's softmax takes that row's whole mass.

Cases cover every statistics kernel class: observation rows in registers with one, two or
three 32-row blocks per wave (head_dim 128 and 64), the 8-wave register-row pass (nine
blocks), and the LDS-staged pass (480 rows at head_dim 64); units split over many
workgroups (one-tile pieces) and over pieces of several tiles; max and mean aggregation.
The CPU test checks the property of the inputs that makes the branch run; the GPU tests
compare every unit element by element with the oracle."""
import pytest

from synth import WORKLOADS
from parity import all_units, build_inputs, check_units, log, run_gpu
import planted

W = WORKLOADS
CASES = {
    # 240 rows (two blocks per wave, head_dim 128); 8 units of 12 one-tile pieces
    "qwen7b_split": W["qwen7b_16k"].replace(n_layers=2, capacity=3000, seq_len=2989, budget=700),
    # 240 rows; 768 tiles over the grid: pieces of one and two tiles
    "qwen7b_multitile": W["qwen7b_16k"].replace(n_layers=6, capacity=8192, seq_len=8000, budget=1500),
    # 20 rows at head_dim 64 (one block per wave)
    "tiny_d64": W["tiny"].replace(t_new=0, capacity=2000, seq_len=1999, budget=300),
    # 128 rows at head_dim 128 (one block per wave)
    "llama_one_block": W["llama8b_32k"].replace(n_layers=1, batch=2, window=28, capacity=2304, seq_len=2304,
                                                budget=512),
    # 288 rows at head_dim 128: the 8-wave register-row pass
    "nine_blocks": W["qwen7b_16k"].replace(n_layers=2, capacity=1400, seq_len=1389, budget=500, nb_init=64,
                                           nb_max=64),
    # 352 rows at head_dim 64: three blocks on some waves
    "three_blocks_d64": W["tiny"].replace(n_q_heads=32, n_kv_heads=2, window=20, nb_init=32, nb_max=32, t_new=0,
                                          capacity=1200, seq_len=1177, budget=300),
    # 480 rows at head_dim 64: the LDS-staged statistics pass
    "lds_stats_d64": W["tiny"].replace(n_q_heads=16, n_kv_heads=2, window=56, nb_init=32, nb_max=32, t_new=0,
                                       capacity=800, seq_len=777, budget=300),
}
MEAN = ["qwen7b_split", "nine_blocks", "lds_stats_d64"]


def _planted_inputs(w, device):
    inp = build_inputs(w, device)
    where = planted.plant(w, inp)
    return inp, where


@pytest.mark.parametrize("case", sorted(CASES))
def test_planted_keys_overflow_the_running_sum(case):
    """CPU: every planted key lies more than 64 (log2 units) above every earlier logit of
    its row, and in every unit at least two of them sit after the first 32-key fragment of
    their 64-key quarter, so any piece of the unit that reaches them has a finite running
    max below them by more than the cheap sum can hold.  (The spot at a tile start and the
    one in the last, partial fragment cover the first-fragment and masked-tail paths.)"""
    w = CASES[case]
    inp, where = _planted_inputs(w, "cpu")
    for (l, b, h), sp in where.items():
        mid = 0
        for (p, r), jump in zip(sp, planted.jumps(w, inp, l, b, h, sp)):
            assert jump > planted.OVERFLOW_LOG2, (l, b, h, p, r, jump)
            mid += p % 64 >= 32
        assert mid >= 2, f"unit {(l, b, h)}: spots {sp}"


def _run(case, aggregation):
    w = CASES[case].replace(name="rescale_" + case)
    inp, where = _planted_inputs(w, "cuda")
    log(f"[rescale] {case} ({aggregation}): layers {w.n_layers} batch {w.batch} cap {w.capacity} rows "
        f"{w.group * w.window + w.nb_init} d {w.head_dim}; spots of unit 0 {where[(0, 0, 0)]}")
    ev, _ = run_gpu(w, inp, aggregation=aggregation)
    worst = check_units(w, ev, all_units(w), inputs=inp)
    log(f"[rescale] {case} ({aggregation}): worst {worst}")


@pytest.mark.gpu
@pytest.mark.parametrize("case", sorted(CASES))
def test_rescale_parity_max(case):
    _run(case, "max")


@pytest.mark.gpu
@pytest.mark.parametrize("case", MEAN)
def test_rescale_parity_mean(case):
    _run(case, "mean")
