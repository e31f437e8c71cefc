"""bkv_compress_static (no workspace; statistics partials in the library's static device
scratch) against bkv_compress on the same inputs, through the C ABI, on two calls in a row
on one stream, the second smaller than the first:

* a call whose default launches' partials would not fit the scratch (16 layers, 6 ragged
  sequences, 512 observation rows), so the static call scores in smaller launch groups;
  its scores then come from another split of the keys over the workgroups and may differ
  in rounding: within 1e-3 relative, the selection exactly the top-K rule on its own
  scores and otherwise only near-tie swaps against bkv_compress's, compaction bit-exact
  for its own kept positions;
* then a smaller call that fits in the default grouping: every output bit-identical to
  bkv_compress's (same launches on the same inputs).

Every output tensor starts from the same sentinel fill for both entry points, so a write
outside the valid rows, or a missing one, shows up as a difference."""
import numpy as np
import pytest
import torch

import gc
from types import SimpleNamespace

from parity import build_inputs, check_selection, check_units, log, sample_units
from synth import WORKLOADS
from attention_guided_eviction_amd import bkv

pytestmark = pytest.mark.gpu

# 16 layers x 6 sequences x 8 KV heads x 12 slots x 512 rows x 8 bytes = 37.7 MB of
# partials by default, above the 32 MiB scratch
GROUPED = WORKLOADS["qwen4b_serving"].replace(name="static_grouped", n_layers=16, batch=6, n_q_heads=32,
                                              n_kv_heads=8, capacity=3072, ragged=(500, 3072), window=120,
                                              nb_init=32, nb_max=32, t_new=0, budget=600)
SMALL = WORKLOADS["qwen7b_16k"].replace(name="static_small", n_layers=2, capacity=3000, seq_len=2989, budget=700,
                                        t_new=0)


def _shape(w, inputs):
    return bkv.CacheShape(w.n_layers, w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.capacity,
                          inputs["seq_len"])


def _outputs(w):
    n, B, Hkv, D, cap, K = w.n_layers, w.batch, w.n_kv_heads, w.head_dim, w.capacity, w.budget
    dev = "cuda"
    return {
        "scores": [torch.full((B, Hkv, cap), float("nan"), device=dev) for _ in range(n)],
        "idx": [torch.full((B, Hkv, K), -7, dtype=torch.int32, device=dev) for _ in range(n)],
        "n_kept": [torch.full((B, Hkv), -9, dtype=torch.int32, device=dev) for _ in range(n)],
        "k_out": [torch.full((B, Hkv, K, D), -3.0, dtype=torch.bfloat16, device=dev) for _ in range(n)],
        "v_out": [torch.full((B, Hkv, K, D), -5.0, dtype=torch.bfloat16, device=dev) for _ in range(n)],
    }


def _prepare(w, inputs, out, static):
    s = _shape(w, inputs)
    args = (s, inputs["k"], inputs["v"], inputs["q"], w.q_len, w.window, inputs["beacons"], inputs["n_beacons"],
            w.nb_max, w.budget, out["scores"], out["idx"], out["n_kept"], out["k_out"], out["v_out"])
    if static:
        return bkv.prepare_compress_static(*args)
    ws = bkv.alloc_workspace(bkv.compress_workspace_bytes(s, w.window, w.nb_max, w.budget))
    return bkv.prepare_compress(*args, ws)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _assert_identical(w, ref, got):
    for key in ref:
        for l in range(w.n_layers):
            assert torch.equal(_bits(ref[key][l]), _bits(got[key][l])), f"{w.name}: {key} of layer {l} differs"


def _assert_equivalent(w, inputs, ref, got):
    worst_rel, swaps = 0.0, 0
    lens = inputs["seq_len"].cpu().numpy()
    for l in range(w.n_layers):
        sr, sg = ref["scores"][l].double(), got["scores"][l].double()
        written = ~torch.isnan(sr)
        assert torch.equal(written, ~torch.isnan(sg)), f"layer {l}: scores written at different keys"
        zero = sr == 0
        assert torch.equal(zero, sg == 0), f"layer {l}: zero scores differ"
        rel = ((sg - sr).abs() / torch.where(zero, torch.ones_like(sr), sr))[written]
        worst_rel = max(worst_rel, float(rel.max()) if rel.numel() else 0.0)
        assert torch.equal(ref["n_kept"][l], got["n_kept"][l]), f"layer {l}: kept counts differ"
        nk = got["n_kept"][l].cpu().numpy()
        idx = got["idx"][l].cpu().numpy()
        s_got, s_ref = sg.cpu().numpy(), sr.cpu().numpy()
        for b in range(w.batch):
            L = int(lens[b])
            for h in range(w.n_kv_heads):
                n = int(nk[b, h])
                st = check_selection(idx[b, h, :n].astype(np.int64), s_got[b, h, :L], s_ref[b, h, :L], L, w.budget,
                                     w.window)
                swaps += int(st["swaps"])
        # compaction: bit copies of the rows at the static call's own kept positions, and
        # the slots past each unit's count untouched (sentinel), as bkv_compress leaves them
        K, D = w.budget, w.head_dim
        gi = got["idx"][l].long()
        valid = torch.arange(K, device=gi.device)[None, None, :] < got["n_kept"][l][..., None]
        gidx = torch.where(valid, gi, torch.zeros_like(gi))[..., None].expand(-1, -1, -1, D)
        for src, key in ((inputs["k"][l], "k_out"), (inputs["v"][l], "v_out")):
            want = torch.gather(_bits(src), 2, gidx)
            have, base = _bits(got[key][l]), _bits(ref[key][l])
            assert torch.equal(have[valid], want[valid]), f"layer {l}: {key} not the kept rows"
            assert torch.equal(have[~valid], base[~valid]), f"layer {l}: {key} written past the kept count"
        assert torch.equal(got["idx"][l][~valid], ref["idx"][l][~valid]), f"layer {l}: idx written past the count"
    assert worst_rel <= 1e-3, worst_rel
    log(f"[static] {w.name}: scores within {worst_rel:.2e} of bkv_compress, {swaps} near-tie swaps")


def test_static_matches_compress_on_two_calls_in_a_row():
    big_in, small_in = build_inputs(GROUPED), build_inputs(SMALL)
    need = bkv.compress_workspace_bytes(_shape(GROUPED, big_in), GROUPED.window, GROUPED.nb_max, GROUPED.budget)
    assert need > bkv.STATIC_SCRATCH_BYTES, need
    ref_big, ref_small = _outputs(GROUPED), _outputs(SMALL)
    got_big, got_small = _outputs(GROUPED), _outputs(SMALL)
    calls = [_prepare(GROUPED, big_in, ref_big, False), _prepare(SMALL, small_in, ref_small, False),
             _prepare(GROUPED, big_in, got_big, True), _prepare(SMALL, small_in, got_small, True)]
    log(f"[static] {GROUPED.name} then {SMALL.name}: bkv_compress twice, then bkv_compress_static twice")
    for c in calls:
        c()
    torch.cuda.synchronize()
    _assert_equivalent(GROUPED, big_in, ref_big, got_big)
    _assert_identical(SMALL, ref_small, got_small)
    log(f"[static] {SMALL.name}: every output bit-identical to bkv_compress")


def test_static_repeats_bit_identically_after_a_larger_call():
    """The scratch keeps the last call's partials: a call after a larger one reads only
    what it wrote itself."""
    tiny = WORKLOADS["tiny"].replace(t_new=0)
    tin = build_inputs(tiny)
    first, again = _outputs(tiny), _outputs(tiny)
    _prepare(tiny, tin, first, True)()
    big_in = build_inputs(SMALL)
    _prepare(SMALL, big_in, _outputs(SMALL), True)()
    _prepare(tiny, tin, again, True)()
    torch.cuda.synchronize()
    _assert_identical(tiny, first, again)
    ref = _outputs(tiny)
    _prepare(tiny, tin, ref, False)()
    torch.cuda.synchronize()
    _assert_identical(tiny, ref, again)


def test_static_full_serving_shape_against_the_oracle():
    """The Qwen3-4B serving shape at full size (36 layers, batch 64 ragged 2048-8192, 135 MiB
    of partials by default): the static call scores it in launch groups that fit the
    scratch; sampled units checked against the oracle one by one."""
    w = WORKLOADS["qwen4b_serving"].replace(name="static_serving", t_new=0)
    inp = build_inputs(w)
    need = bkv.compress_workspace_bytes(_shape(w, inp), w.window, w.nb_max, w.budget)
    assert need > bkv.STATIC_SCRATCH_BYTES, need
    out = _outputs(w)
    log(f"[static] {w.name}: default partials {need / 2**20:.0f} MiB; one static call")
    _prepare(w, inp, out, True)()
    torch.cuda.synchronize()
    ev = SimpleNamespace(cfg=SimpleNamespace(aggregation="max"), **out)
    worst = check_units(w, ev, sample_units(w, 6, seed=5), inp)
    log(f"[static] {w.name}: worst {worst}")
    del inp, out, ev
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("seed", range(32))
def test_static_random_geometries_bit_identical(seed):
    """Random small geometries (those of the random parity cases, without the beacon
    update): the default grouping fits the scratch, so every output is bit-identical to
    bkv_compress's."""
    from test_parity_random_gpu import _workload
    w = _workload(seed)[0].replace(t_new=0)
    inp = build_inputs(w)
    ref, got = _outputs(w), _outputs(w)
    _prepare(w, inp, ref, False)()
    _prepare(w, inp, got, True)()
    torch.cuda.synchronize()
    _assert_identical(w, ref, got)


def test_static_grouped_with_an_empty_sequence_group_and_many_layers():
    """Edge cases of the launch grouping: the grouped shape with its first three sequences
    empty (the first sequence group has no keys at all), and a 50-layer model (a layer
    group of 48 and one of 2).  Compared with bkv_compress as in the grouped case."""
    w = GROUPED.replace(name="static_empty_group", ragged=None, seq_len=None, lengths=(0, 0, 0, 3072, 2000, 999))
    inp = build_inputs(w)
    assert bkv.compress_workspace_bytes(_shape(w, inp), w.window, w.nb_max, w.budget) > bkv.STATIC_SCRATCH_BYTES
    ref, got = _outputs(w), _outputs(w)
    _prepare(w, inp, ref, False)()
    _prepare(w, inp, got, True)()
    torch.cuda.synchronize()
    _assert_equivalent(w, inp, ref, got)
    many = WORKLOADS["tiny"].replace(name="static_many_layers", n_layers=50, capacity=256, seq_len=250, budget=64,
                                     t_new=0)
    inp = build_inputs(many)
    ref, got = _outputs(many), _outputs(many)
    _prepare(many, inp, ref, False)()
    _prepare(many, inp, got, True)()
    torch.cuda.synchronize()
    _assert_identical(many, ref, got)
