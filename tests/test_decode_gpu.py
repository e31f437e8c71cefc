"""Decode attention on the GPU against the oracle: every (sequence, query head) checked.
Tolerance: |out_gpu - out| <= 1e-4 + 1e-3 |out| per element (fp32 accumulation of at
most a few thousand weighted rows; outputs are convex combinations of the value rows)."""
import numpy as np
import pytest
import torch

from oracle import bkv_oracle as O
from synth import WORKLOADS, bf16_bits
from parity import log, run_gpu
from attention_guided_eviction_amd import bkv

pytestmark = pytest.mark.gpu


def _check(shape, q, k, v, out):
    G = shape.n_q_heads // shape.n_kv_heads
    lens = shape.seq_len.cpu().numpy()
    worst = 0.0
    for l in range(shape.n_layers):
        o_gpu = out[l].cpu().numpy().astype(np.float64)
        for b in range(shape.batch):
            L = int(min(max(lens[b], 0), shape.capacity))
            for h in range(shape.n_kv_heads):
                qg = O.bf16_to_f64(bf16_bits(q[l][b, h * G:(h + 1) * G].cpu()))
                kk = O.bf16_to_f64(bf16_bits(k[l][b, h, :L].cpu()))
                vv = O.bf16_to_f64(bf16_bits(v[l][b, h, :L].cpu()))
                want = O.decode_attention(qg, kk, vv)
                got = o_gpu[b, h * G:(h + 1) * G]
                err = np.abs(got - want) - (1e-4 + 1e-3 * np.abs(want))
                assert err.max() <= 0, f"layer {l} b {b} h {h}: worst excess {err.max():.2e}"
                worst = max(worst, float(np.abs(got - want).max()))
    return worst


def _random(shape, gen, scale=1.0):
    n, B, Hq, Hkv, D, cap = shape.n_layers, shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.capacity
    mk = lambda *s: (torch.randn(*s, generator=gen, device="cuda") * scale).to(torch.bfloat16)
    return ([mk(B, Hq, D) for _ in range(n)], [mk(B, Hkv, cap, D) for _ in range(n)],
            [mk(B, Hkv, cap, D) for _ in range(n)])


@pytest.mark.parametrize("B,Hq,Hkv,D,cap,lens,scale", [
    (3, 8, 2, 128, 2500, (2500, 1, 1025), 2.0),        # several 1024-key chunks, ragged
    (2, 4, 2, 64, 700, (0, 699), 1.0),                 # empty sequence, head_dim 64
    (1, 28, 4, 128, 4096, (4096,), 1.5),               # GQA 7
    (2, 8, 1, 128, 300, (300, 64), 3.0),               # GQA 8 (the limit), peaked weights
])
def test_decode_random(B, Hq, Hkv, D, cap, lens, scale):
    gen = torch.Generator(device="cuda").manual_seed(B * 1000 + cap)
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    shape = bkv.CacheShape(2, B, Hq, Hkv, D, cap, seq)
    q, k, v = _random(shape, gen, scale)
    out = [torch.empty((B, Hq, D), dtype=torch.float32, device="cuda") for _ in range(2)]
    ws = bkv.alloc_workspace(bkv.decode_workspace_bytes(shape))
    bkv.decode_attention(shape, q, k, v, out, ws)
    torch.cuda.synchronize()
    log(f"[decode] worst abs error {_check(shape, q, k, v, out):.2e}")


def test_decode_over_compacted_cache():
    """Decode over the compacted caches of an event: capacity = budget, lengths = kept counts."""
    w = WORKLOADS["qwen4b_serving"].replace(name="decode_compacted", n_layers=1, batch=3, capacity=2048,
                                            ragged=(700, 2048), budget=400)
    ev, inp = run_gpu(w)
    kept = torch.minimum(inp["seq_len"], torch.tensor(w.budget, dtype=torch.int32, device="cuda"))
    shape = bkv.CacheShape(1, w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.budget, kept)
    q = [inp["q"][0][:, :, -1].contiguous()]                 # the newest stored query of every head
    out = [torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")]
    ws = bkv.alloc_workspace(bkv.decode_workspace_bytes(shape))
    bkv.decode_attention(shape, q, ev.k_out, ev.v_out, out, ws)
    torch.cuda.synchronize()
    log(f"[decode] compacted: worst abs error {_check(shape, q, ev.k_out, ev.v_out, out):.2e}")


@pytest.mark.parametrize("G", range(1, 9))
@pytest.mark.parametrize("D", [64, 128])
def test_decode_every_group_size(G, D):
    """One partial kernel per (head_dim, group size): each is checked, with a ragged tail
    inside the second 1024-key chunk and a sequence shorter than one 64-key block."""
    gen = torch.Generator(device="cuda").manual_seed(100 * G + D)
    seq = torch.tensor((1100, 37), dtype=torch.int32, device="cuda")
    shape = bkv.CacheShape(1, 2, 2 * G, 2, D, 1100, seq)
    q, k, v = _random(shape, gen, 1.5)
    out = [torch.empty((2, 2 * G, D), dtype=torch.float32, device="cuda")]
    ws = bkv.alloc_workspace(bkv.decode_workspace_bytes(shape))
    bkv.decode_attention(shape, q, k, v, out, ws)
    torch.cuda.synchronize()
    log(f"[decode] G {G} D {D}: worst abs error {_check(shape, q, k, v, out):.2e}")


@pytest.mark.parametrize("n_layers,B,Hkv,cap,lens", [
    (4, 16, 8, 1100, (1100, 1025, 3, 0, 700, 1024, 1099, 64, 65, 512, 1100, 2, 1023, 300, 0, 1100)),
    # ^ 512 units, 1024 workgroups of 1024 keys
    (4, 10, 8, 2000, (2000, 1, 1025, 513, 257, 0, 1999, 64, 1024, 1536)),       # 320 units: 512-key chunks
])
def test_decode_chunk_sizes(n_layers, B, Hkv, cap, lens):
    """The chunk size follows the launch size (1024 keys per workgroup for large launches,
    512 or 256 for small ones); these shapes take the 1024- and 512-key kernels."""
    gen = torch.Generator(device="cuda").manual_seed(n_layers * 100 + B)
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    shape = bkv.CacheShape(n_layers, B, 2 * Hkv, Hkv, 64, cap, seq)
    q, k, v = _random(shape, gen, 1.5)
    out = [torch.empty((B, 2 * Hkv, 64), dtype=torch.float32, device="cuda") for _ in range(n_layers)]
    ws = bkv.alloc_workspace(bkv.decode_workspace_bytes(shape))
    bkv.decode_attention(shape, q, k, v, out, ws)
    torch.cuda.synchronize()
    log(f"[decode] chunks {n_layers}x{B}x{Hkv}: worst abs error {_check(shape, q, k, v, out):.2e}")


def _random_geometry(seed):
    """Seeded geometry: head_dim 64/128, groups 1-8, 1-4 KV heads, one to three sequences,
    capacities around the 1024-key chunk (and tiny), lengths 0, 1, full or random."""
    import random
    rng = random.Random(seed)
    D = rng.choice([64, 128])
    hkv = rng.choice([1, 2, 4])
    g = rng.randint(1, 8)
    B = rng.choice([1, 2, 3])
    cap = rng.choice([1, 31, 64, 300, 1023, 1024, 1025, 2049, 4100])
    lens = tuple(rng.choice([0, 1, cap, rng.randint(0, cap)]) for _ in range(B))
    return B, hkv * g, hkv, D, cap, lens, rng.choice([0.5, 1.0, 2.0, 3.0]), rng.choice([1, 2])


@pytest.mark.parametrize("seed", range(24))
def test_decode_random_geometries(seed):
    B, Hq, Hkv, D, cap, lens, scale, nl = _random_geometry(3000 + seed)
    gen = torch.Generator(device="cuda").manual_seed(seed)
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    shape = bkv.CacheShape(nl, B, Hq, Hkv, D, cap, seq)
    q, k, v = _random(shape, gen, scale)
    out = [torch.empty((B, Hq, D), dtype=torch.float32, device="cuda") for _ in range(nl)]
    ws = bkv.alloc_workspace(bkv.decode_workspace_bytes(shape))
    bkv.decode_attention(shape, q, k, v, out, ws)
    torch.cuda.synchronize()
    log(f"[decode] seed {seed}: B{B} Hq/Hkv {Hq}/{Hkv} D{D} cap {cap} lens {lens}: "
        f"worst abs error {_check(shape, q, k, v, out):.2e}")
