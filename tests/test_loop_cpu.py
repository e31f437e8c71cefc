"""Steady-state loop configuration checks that need no GPU."""
import pytest

from attention_guided_eviction_amd.loop import LoopConfig, SteadyStateLoop


def test_capacity_leaves_room_for_one_chunk():
    assert LoopConfig(1, 1, 4, 2, 64, budget=1024, window=32, nb_max=16, interval=128).capacity == 1152


@pytest.mark.parametrize("kw", [dict(window=200), dict(interval=0), dict(window=-1), dict(budget=16, window=32)])
def test_rejects_windows_that_do_not_fit(kw):
    base = dict(budget=1024, window=32, nb_max=16, interval=128)
    base.update(kw)
    with pytest.raises(ValueError):
        SteadyStateLoop(LoopConfig(1, 1, 4, 2, 64, **base), device="cpu")
