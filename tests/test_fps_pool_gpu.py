"""Beacon updates over pools larger than the register-resident kernel takes (over 768
rows, up to BKV_MAX_POOL): the streaming kernel, e.g. the Naive FPS of Figure 7 over a
whole query history; and seeded random geometries that take either kernel.  Every unit's
picks are replayed on the oracle (continual FPS on the same pool), with the near-tie
tolerance of the other beacon parity tests."""
import numpy as np
import pytest
import torch

from oracle import bkv_oracle as O
from synth import bf16_bits
from parity import check_fps_replay, log
from attention_guided_eviction_amd import bkv

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,Hq,Hkv,D,nb_max,q_len,t_new,n_in", [
    (2, 8, 2, 128, 32, 300, 300, (32, 0, 5, 32)),       # 1232-row pools; an empty and a partial set
    (1, 8, 2, 128, 1, 192, 192, (1, 0)),                # 769 rows (the first streamed size); one slot
    (1, 10, 2, 128, 48, 1600, 1500, (48, 17)),          # 7548 rows, G = 5, history longer than t_new
    (2, 4, 2, 64, 16, 2000, 2000, (16, 3, 0, 16)),      # head_dim 64, 4016 rows
    (1, 8, 2, 128, 16, 4092, 4092, (16, 16)),           # 16384 rows: the largest pool
])
def test_fps_pool(B, Hq, Hkv, D, nb_max, q_len, t_new, n_in):
    gen = torch.Generator(device="cuda").manual_seed(B * 7919 + q_len)
    G = Hq // Hkv
    assert nb_max + G * t_new > 768   # the launch takes the streaming kernel (every unit of it)
    bc_in = torch.randn(B, Hkv, nb_max, D, generator=gen, device="cuda").to(torch.bfloat16)
    q = torch.randn(B, Hq, q_len, D, generator=gen, device="cuda").to(torch.bfloat16)
    nb_in = torch.tensor(n_in, dtype=torch.int32, device="cuda").reshape(B, Hkv)
    bc_out = torch.zeros_like(bc_in)
    nb_out = torch.full((B, Hkv), -1, dtype=torch.int32, device="cuda")
    seq = torch.ones(B, dtype=torch.int32, device="cuda")
    shape = bkv.CacheShape(1, B, Hq, Hkv, D, 1, seq)
    bkv.update_beacons(shape, [bc_in], [nb_in], nb_max, [q], q_len, t_new, [bc_out], [nb_out])
    torch.cuda.synchronize()
    bin_bits = bf16_bits(bc_in.cpu())
    q_bits = bf16_bits(q.cpu())
    out_bits = bf16_bits(bc_out.cpu())
    for b in range(B):
        for h in range(Hkv):
            c = int(n_in[b * Hkv + h])
            pool = O.beacon_pool(bin_bits[b, h], c, q_bits[b, h * G:(h + 1) * G, q_len - t_new:])
            n_out = int(nb_out[b, h])
            assert n_out == min(nb_max, pool.shape[0])
            check_fps_replay(pool, out_bits[b, h, :n_out], nb_max)
    log(f"[fps pool] B {B} G {G} D {D} pool {pool.shape[0]} nb_max {nb_max} ok")


def _random_geometry(seed):
    """Seeded beacon-update geometry for either kernel: head_dim 64/128, groups 1-8, 1-4 KV
    heads, up to 64 beacon slots, live counts empty, full or partial, new queries from one
    to the pool limit (about a third of the cases past the register-resident 768 rows)."""
    import random
    rng = random.Random(seed)
    D = rng.choice([64, 128])
    hkv = rng.choice([1, 2, 4])
    g = rng.randint(1, 8)
    B = rng.choice([1, 2, 3])
    nb_max = rng.choice([1, 4, 16, 32, 64])
    big = rng.random() < 0.3
    t_new = rng.randint(1, (16384 - nb_max) // g if big else max(1, (768 - nb_max) // g))
    q_len = t_new + rng.choice([0, 0, 5, 100])
    n_in = tuple(rng.choice([0, nb_max, rng.randint(0, nb_max)]) for _ in range(B * hkv))
    return B, hkv * g, hkv, D, nb_max, q_len, t_new, n_in


@pytest.mark.parametrize("seed", range(24))
def test_beacon_update_random_geometries(seed):
    B, Hq, Hkv, D, nb_max, q_len, t_new, n_in = _random_geometry(4000 + seed)
    G = Hq // Hkv
    gen = torch.Generator(device="cuda").manual_seed(4000 + seed)
    bc_in = torch.randn(B, Hkv, nb_max, D, generator=gen, device="cuda").to(torch.bfloat16)
    q = torch.randn(B, Hq, q_len, D, generator=gen, device="cuda").to(torch.bfloat16)
    nb_in = torch.tensor(n_in, dtype=torch.int32, device="cuda").reshape(B, Hkv)
    bc_out = torch.zeros_like(bc_in)
    nb_out = torch.full((B, Hkv), -1, dtype=torch.int32, device="cuda")
    seq = torch.ones(B, dtype=torch.int32, device="cuda")
    shape = bkv.CacheShape(1, B, Hq, Hkv, D, 1, seq)
    bkv.update_beacons(shape, [bc_in], [nb_in], nb_max, [q], q_len, t_new, [bc_out], [nb_out])
    torch.cuda.synchronize()
    bin_bits, q_bits, out_bits = bf16_bits(bc_in.cpu()), bf16_bits(q.cpu()), bf16_bits(bc_out.cpu())
    for b in range(B):
        for h in range(Hkv):
            c = int(n_in[b * Hkv + h])
            pool = O.beacon_pool(bin_bits[b, h], c, q_bits[b, h * G:(h + 1) * G, q_len - t_new:])
            n_out = int(nb_out[b, h])
            assert n_out == min(nb_max, pool.shape[0])
            check_fps_replay(pool, out_bits[b, h, :n_out], nb_max)
    log(f"[fps random] seed {seed}: B {B} G {G} D {D} pool up to {nb_max + G * t_new} nb_max {nb_max} ok")
