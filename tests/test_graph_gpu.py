"""The allocation-free event under HIP graph capture, its intended use: bkv_compress_static
captured once and replayed, against eager calls of the same entry point and of bkv_compress
on the same inputs.  Between replays the program does its own eager work (refilling the
outputs, rewriting part of the inputs, synchronising), and every replay is checked.  The
event records no memset, so the graph holds kernel nodes only."""
import pytest
import torch

from parity import build_inputs, log
from synth import WORKLOADS
from attention_guided_eviction_amd import bkv

pytestmark = pytest.mark.gpu

W = WORKLOADS["qwen7b_16k"].replace(name="graph_small", n_layers=2, capacity=3000, seq_len=2989, budget=700,
                                    t_new=0)


def _outputs(w):
    n, B, Hkv, D, cap, K = w.n_layers, w.batch, w.n_kv_heads, w.head_dim, w.capacity, w.budget
    return {
        "scores": [torch.full((B, Hkv, cap), float("nan"), device="cuda") for _ in range(n)],
        "idx": [torch.full((B, Hkv, K), -7, dtype=torch.int32, device="cuda") for _ in range(n)],
        "n_kept": [torch.full((B, Hkv), -9, dtype=torch.int32, device="cuda") for _ in range(n)],
        "k_out": [torch.full((B, Hkv, K, D), -3.0, dtype=torch.bfloat16, device="cuda") for _ in range(n)],
        "v_out": [torch.full((B, Hkv, K, D), -5.0, dtype=torch.bfloat16, device="cuda") for _ in range(n)],
    }


def _args(w, inp, out):
    s = bkv.CacheShape(w.n_layers, w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.capacity, inp["seq_len"])
    return (s, inp["k"], inp["v"], inp["q"], w.q_len, w.window, inp["beacons"], inp["n_beacons"], w.nb_max,
            w.budget, out["scores"], out["idx"], out["n_kept"], out["k_out"], out["v_out"])


def _refill(out):
    for t in out["scores"]:
        t.fill_(float("nan"))
    for key, val in (("idx", -7), ("n_kept", -9), ("k_out", -3.0), ("v_out", -5.0)):
        for t in out[key]:
            t.fill_(val)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _assert_same(ref, got, what):
    for key in ref:
        for l, (a, b) in enumerate(zip(ref[key], got[key])):
            assert torch.equal(_bits(a), _bits(b)), f"{what}: {key} of layer {l} differs"


def test_static_event_replays_in_a_graph():
    inp = build_inputs(W)
    out = _outputs(W)
    static = bkv.prepare_compress_static(*_args(W, inp, out))
    static()                       # first call on the device: the scratch address is taken here
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        static()                   # warm on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        static()
    torch.cuda.synchronize()

    ref = _outputs(W)
    ws = bkv.alloc_workspace(bkv.compress_workspace_bytes(_args(W, inp, ref)[0], W.window, W.nb_max, W.budget))
    eager = bkv.prepare_compress(*_args(W, inp, ref), ws)
    gen = torch.Generator(device="cuda").manual_seed(7)
    for replay in range(3):
        if replay > 0:             # the program's own eager work: new keys in part of layer 0
            rows = 64 * replay
            inp["k"][0][:, :, :rows].copy_(
                torch.randn(inp["k"][0][:, :, :rows].shape, device="cuda", generator=gen).to(torch.bfloat16))
        _refill(out)
        _refill(ref)
        torch.cuda.synchronize()
        eager()                    # bkv_compress on the same inputs
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _assert_same(ref, out, f"replay {replay} against bkv_compress")
        log(f"[graph] replay {replay}: every output bit-identical to bkv_compress")
