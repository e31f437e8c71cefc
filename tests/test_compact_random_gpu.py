"""bkv_compact and bkv_compact_into alone on seeded random kept-position lists, against the
oracle's gather (bit copies of the kept rows in list order), with the rows past each
unit's kept count left untouched: head_dim 64 and 128, budgets from one row to the whole
cache, kept counts from zero to the budget (and one past it, which the kernel clamps),
output buffers with room to spare."""
import random

import numpy as np
import pytest
import torch

from oracle import bkv_oracle as O
from synth import bf16_bits
from parity import log
from attention_guided_eviction_amd import bkv

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed", range(24))
def test_compact_random(seed):
    rng = random.Random(6000 + seed)
    D = rng.choice([64, 128])
    B, Hkv, n_layers = rng.choice([1, 2, 3]), rng.choice([1, 2, 4]), rng.choice([1, 2])
    cap = rng.choice([1, 17, 256, 1000, 4096, rng.randint(1, 8192)])
    budget = rng.randint(1, cap)
    out_cap = budget + rng.choice([0, 0, 1, 128])
    gen = torch.Generator(device="cuda").manual_seed(6000 + seed)
    nrng = np.random.default_rng(6000 + seed)
    k = [torch.randn(B, Hkv, cap, D, generator=gen, device="cuda").to(torch.bfloat16) for _ in range(n_layers)]
    v = [torch.randn(B, Hkv, cap, D, generator=gen, device="cuda").to(torch.bfloat16) for _ in range(n_layers)]
    idx_np, n_np = [], []
    for _ in range(n_layers):
        idx_l = np.zeros((B, Hkv, budget), dtype=np.int32)
        n_l = np.zeros((B, Hkv), dtype=np.int32)
        for b in range(B):
            for h in range(Hkv):
                n = rng.choice([0, budget, budget + 1, rng.randint(0, budget)])
                take = min(n, budget)
                idx_l[b, h, :take] = np.sort(nrng.choice(cap, size=take, replace=False))
                n_l[b, h] = n
        idx_np.append(idx_l)
        n_np.append(n_l)
    idx = [torch.from_numpy(a).cuda() for a in idx_np]
    n_kept = [torch.from_numpy(a).cuda() for a in n_np]
    k_out = [torch.full((B, Hkv, out_cap, D), -3.0, dtype=torch.bfloat16, device="cuda") for _ in range(n_layers)]
    v_out = [torch.full((B, Hkv, out_cap, D), -5.0, dtype=torch.bfloat16, device="cuda") for _ in range(n_layers)]
    shape = bkv.CacheShape(n_layers, B, Hkv, Hkv, D, cap, torch.full((B,), cap, dtype=torch.int32, device="cuda"))
    bkv.compact(shape, k, v, idx, n_kept, budget, k_out, v_out, out_capacity=None if out_cap == budget else out_cap)
    torch.cuda.synchronize()
    fill_k, fill_v = bf16_bits(torch.tensor([-3.0], dtype=torch.bfloat16))[0], bf16_bits(torch.tensor([-5.0], dtype=torch.bfloat16))[0]
    for l in range(n_layers):
        kb, vb = bf16_bits(k[l].cpu()), bf16_bits(v[l].cpu())
        kob, vob = bf16_bits(k_out[l].cpu()), bf16_bits(v_out[l].cpu())
        for b in range(B):
            for h in range(Hkv):
                take = min(int(n_np[l][b, h]), budget)
                keep = idx_np[l][b, h, :take].astype(np.int64)
                assert np.array_equal(kob[b, h, :take], O.compact_rows(kb[b, h], keep)), f"layer {l} b {b} h {h}: K rows"
                assert np.array_equal(vob[b, h, :take], O.compact_rows(vb[b, h], keep)), f"layer {l} b {b} h {h}: V rows"
                assert (kob[b, h, take:] == fill_k).all() and (vob[b, h, take:] == fill_v).all(), \
                    f"layer {l} b {b} h {h}: rows past the kept count were written"
    log(f"[compact] seed {seed}: D {D} cap {cap} budget {budget} out {out_cap} layers {n_layers} ok")
