"""bench.py names the scorer's two kernels in its roofline object by mirroring the library's
dispatch rules.  The names are checked here against the kernels that rocprofv3 traced for
the same workloads (the kernel tables under profiles/), so the mirror cannot drift from
what actually runs."""
import re
from pathlib import Path

import pytest

import bench
from synth import WORKLOADS

ROOT = Path(__file__).resolve().parents[1]

# workload -> committed kernel-trace summary of one of its events
TRACES = {
    "qwen7b_16k": "score_qwen7b_16k_kernel_stats.md",
    "llama8b_32k": "kernels_llama8b_32k.md",
    "qwen14b_64k": "kernels_qwen14b_64k.md",
    "qwen4b_serving": "kernels_qwen4b_serving.md",
}


def _traced(name):
    text = (ROOT / "profiles" / TRACES[name]).read_text()
    return set(re.findall(r"^\| `([A-Za-z0-9_]+)<", text, flags=re.M))


def _base(label):
    return label.split("<", 1)[0]


@pytest.mark.parametrize("name", sorted(TRACES))
def test_score_kernel_names_match_the_traces(name):
    w = WORKLOADS[name]
    stats, finish = bench.score_kernel_names(w.head_dim, w.group * w.window + w.nb_max)
    traced = _traced(name)
    assert _base(stats) in traced, (stats, traced)
    assert _base(finish) in traced, (finish, traced)


def test_dispatch_classes():
    assert bench.score_kernel_names(128, 240) == ("qs_stats_kernel<D,BPW>", "score_kernel<D,true>")
    assert bench.score_kernel_names(128, 352) == ("qs_stats_kernel8<D>", "finish8_kernel<D>")
    assert bench.score_kernel_names(64, 300) == ("qs_stats_kernel_wide<D,3>", "score_kernel<D,true>")
    assert bench.score_kernel_names(128, 600)[0] == "score_kernel<D,false>"
