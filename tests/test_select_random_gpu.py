"""bkv_select_topk alone on seeded random score arrays, against the oracle's selection rule
on the same scores, exactly (positions ascending, equal scores to the lower position, the
window always kept): capacities from 1 to 65536 (every per-thread element count of the
kernel, registers and LDS), budgets and windows from one row to the whole cache, ragged
and empty sequences, and score patterns with many ties, few non-zeros, subnormals only
and all zeros."""
import random

import numpy as np
import pytest
import torch

from oracle import bkv_oracle as O
from parity import log
from attention_guided_eviction_amd import bkv

pytestmark = pytest.mark.gpu


def _geometry(seed):
    rng = random.Random(seed)
    cap = rng.choice([1, 2, 100, 1023, 1025, 4096, 16384, 32769, 65536, rng.randint(1, 65536)])
    B = rng.choice([1, 2, 3])
    Hkv = rng.choice([1, 2, 4])
    budget = rng.randint(1, cap)
    window = rng.randint(0, budget)
    lens = tuple(rng.choice([0, cap, budget, budget + 1, rng.randint(0, cap)]) for _ in range(B))
    kind = rng.choice(["uniform", "ties", "few", "tiny", "zeros"])
    return cap, B, Hkv, budget, window, lens, kind


def _scores(kind, shape, rng):
    if kind == "uniform":
        return rng.random(shape, dtype=np.float32)
    if kind == "ties":
        return (rng.integers(0, 50, shape) / 64.0).astype(np.float32)
    if kind == "few":
        return np.where(rng.random(shape) < 0.01, rng.random(shape), 0.0).astype(np.float32)
    if kind == "tiny":
        return (rng.random(shape) * 1e-38).astype(np.float32)
    return np.zeros(shape, dtype=np.float32)


@pytest.mark.parametrize("seed", range(32))
def test_select_random(seed):
    cap, B, Hkv, budget, window, lens, kind = _geometry(5000 + seed)
    sc = _scores(kind, (B, Hkv, cap), np.random.default_rng(5000 + seed))
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    shape = bkv.CacheShape(1, B, Hkv, Hkv, 128, cap, seq)
    idx = [torch.full((B, Hkv, budget), -7, dtype=torch.int32, device="cuda")]
    n_kept = [torch.full((B, Hkv), -9, dtype=torch.int32, device="cuda")]
    bkv.select_topk(shape, [torch.from_numpy(sc).cuda()], budget, window, idx, n_kept)
    torch.cuda.synchronize()
    got_idx, got_n = idx[0].cpu().numpy(), n_kept[0].cpu().numpy()
    for b in range(B):
        L = min(max(lens[b], 0), cap)
        for h in range(Hkv):
            want = O.select_keep(sc[b, h].astype(np.float64), L, budget, window)
            assert got_n[b, h] == len(want), f"b {b} h {h}: kept {got_n[b, h]}, want {len(want)}"
            assert np.array_equal(got_idx[b, h, :len(want)], want), f"b {b} h {h}: kept positions differ"
    log(f"[select] seed {seed}: cap {cap} B {B} Hkv {Hkv} budget {budget} window {window} {kind} ok")
