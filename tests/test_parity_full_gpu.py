"""GPU parity at the full sizes of the five workloads, in the same launch configuration
the benchmark times (one call covering every layer).  The oracle checks sampled units
one by one (it regenerates each unit's inputs on the CPU from the same seeds, so the
GPU-built caches are checked bit for bit through the compacted rows)."""
import gc

import pytest
import torch

from synth import WORKLOADS, WORKLOAD_ORDER, unit_inputs, bf16_bits
from parity import check_units, log, run_gpu, sample_units

pytestmark = pytest.mark.gpu

N_SAMPLE = {"tiny": 2, "qwen7b_16k": 6, "llama8b_32k": 5, "qwen14b_64k": 4, "qwen4b_serving": 6}


@pytest.mark.parametrize("name", WORKLOAD_ORDER)
def test_full_size(name):
    w = WORKLOADS[name]
    log(f"[full] {name}: building inputs on the GPU")
    ev, inputs = run_gpu(w)
    log(f"[full] {name}: event done; checking {N_SAMPLE[name]} sampled units")
    worst = check_units(w, ev, sample_units(w, N_SAMPLE[name], seed=len(name)))
    log(f"[full] {name}: worst {worst}")
    del ev, inputs
    gc.collect()
    torch.cuda.empty_cache()


def test_full_size_mean_aggregation():
    """Table 2's mean aggregation at the 7B shape's full size (sampled units)."""
    w = WORKLOADS["qwen7b_16k"]
    ev, inputs = run_gpu(w, aggregation="mean")
    worst = check_units(w, ev, sample_units(w, 4, seed=99))
    log(f"[full] qwen7b_16k mean: worst {worst}")
    del ev, inputs
    gc.collect()
    torch.cuda.empty_cache()


def test_device_generation_matches_host():
    w = WORKLOADS["qwen4b_serving"].replace(n_layers=1, batch=3)
    from synth import layer_tensors
    lt = layer_tensors(w, 0, "cuda")
    for b, h in [(0, 0), (2, 7)]:
        u = unit_inputs(w, 0, b, h, "cpu")
        L = u["L"]
        assert bf16_bits(lt["k"][0 if b == 0 else b, h, :L]).tobytes() == bf16_bits(u["k"]).tobytes()
        assert bf16_bits(lt["v"][b, h, :L]).tobytes() == bf16_bits(u["v"]).tobytes()
        assert bf16_bits(lt["q"][b, h * w.group:(h + 1) * w.group]).tobytes() == bf16_bits(u["q"]).tobytes()
