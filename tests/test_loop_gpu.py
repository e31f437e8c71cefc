"""The steady-state loop (append a chunk, refresh beacons, compress into the other buffer)
against the CPU oracle, cycle by cycle: each cycle's beacons, scores, selection and
compacted rows are checked from the GPU's own state before that cycle, so a near-tie
resolved differently in one cycle cannot hide a real error in a later one."""
import numpy as np
import pytest
import torch

from oracle import bkv_oracle as O
from synth import bf16_bits
from parity import SCORE_RTOL, check_fps_replay, check_selection, log
from attention_guided_eviction_amd.loop import LoopConfig, SteadyStateLoop

pytestmark = pytest.mark.gpu


def _chunk(cfg, gen, scale=1.0):
    B, Hkv, Hq, T, D = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.interval, cfg.head_dim
    mk = lambda *s: (torch.randn(*s, generator=gen, device="cuda") * scale).to(torch.bfloat16)
    return ([mk(B, Hkv, T, D) for _ in range(cfg.n_layers)], [mk(B, Hkv, T, D) for _ in range(cfg.n_layers)],
            [mk(B, Hq, T, D) for _ in range(cfg.n_layers)])


def _run(cfg, cycles=3, n_live=None):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234)
    B, Hkv, D, G = cfg.batch, cfg.n_kv_heads, cfg.head_dim, cfg.n_q_heads // cfg.n_kv_heads
    loop = SteadyStateLoop(cfg)
    k0 = [(torch.randn(B, Hkv, cfg.budget, D, generator=gen, device="cuda")).to(torch.bfloat16)
          for _ in range(cfg.n_layers)]
    v0 = [(torch.randn(B, Hkv, cfg.budget, D, generator=gen, device="cuda")).to(torch.bfloat16)
          for _ in range(cfg.n_layers)]
    nbm = max(cfg.nb_max, 1)
    bc0 = [(torch.randn(B, Hkv, nbm, D, generator=gen, device="cuda")).to(torch.bfloat16) for _ in range(cfg.n_layers)]
    live = cfg.nb_max if n_live is None else n_live
    nb0 = [torch.full((B, Hkv), live, dtype=torch.int32, device="cuda") for _ in range(cfg.n_layers)]
    loop.start(k0, v0, bc0, nb0)
    cap = cfg.capacity
    for cyc in range(cycles):
        loop.append(*_chunk(cfg, gen))
        pre = {name: [t.cpu() for t in getattr(loop, name)] for name in ("k", "v", "beacons", "n_beacons")}
        q = [t.cpu() for t in loop.q]
        loop.compress()
        torch.cuda.synchronize()
        for l in range(cfg.n_layers):
            for b in range(B):
                for h in range(Hkv):
                    kb, vb = bf16_bits(pre["k"][l][b, h]), bf16_bits(pre["v"][l][b, h])
                    qg = bf16_bits(q[l][b, h * G:(h + 1) * G])
                    if cfg.nb_max > 0:
                        n_out = int(loop.n_beacons[l][b, h].item())
                        rows = bf16_bits(loop.beacons[l][b, h, :n_out].cpu())
                        pool = O.beacon_pool(bf16_bits(pre["beacons"][l][b, h]), int(pre["n_beacons"][l][b, h]), qg)
                        assert n_out == min(cfg.nb_max, pool.shape[0])
                        check_fps_replay(pool, rows, cfg.nb_max)
                        obs = O.observation_queries(O.bf16_to_f64(qg), cfg.window, O.bf16_to_f64(rows), n_out)
                    else:
                        obs = O.observation_queries(O.bf16_to_f64(qg), cfg.window, np.zeros((0, D)), 0)
                    s_or = O.aggregated_scores(obs, O.bf16_to_f64(kb), cfg.aggregation)
                    s_gpu = loop.scores[l][b, h].cpu().numpy().astype(np.float64)
                    rel = np.abs(s_gpu - s_or) / s_or
                    assert rel.max() <= SCORE_RTOL, f"cycle {cyc} unit {(l, b, h)}: score rel {rel.max():.2e}"
                    n = int(loop.n_kept[l][b, h].item())
                    assert n == cfg.budget
                    keep = loop.idx[l][b, h, :n].cpu().numpy().astype(np.int64)
                    check_selection(keep, s_gpu, s_or, cap, cfg.budget, cfg.window)
                    assert bf16_bits(loop.k[l][b, h, :n].cpu()).tobytes() == kb[keep].tobytes()
                    assert bf16_bits(loop.v[l][b, h, :n].cpu()).tobytes() == vb[keep].tobytes()
        log(f"[loop] cycle {cyc} ok")
    return loop


def test_loop_three_cycles_with_continual_fps():
    _run(LoopConfig(n_layers=2, batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, budget=192, window=16, nb_max=8,
                    interval=64))


def test_loop_beacons_filling_up_and_head_dim_64():
    # 3 live beacons of 12 slots: the first update fills the set from the chunk's queries
    _run(LoopConfig(n_layers=1, batch=3, n_q_heads=4, n_kv_heads=2, head_dim=64, budget=100, window=8, nb_max=12,
                    interval=40), cycles=3, n_live=3)


def test_loop_recent_only_and_mean():
    _run(LoopConfig(n_layers=1, batch=2, n_q_heads=8, n_kv_heads=4, head_dim=128, budget=256, window=32, nb_max=0,
                    interval=128, aggregation="mean"), cycles=2)


def _random_config(seed):
    """Seeded loop configuration: head_dim 64/128, groups 1-8, 1-4 KV heads, budgets of 1
    to 400 rows, intervals of 1 to 200 tokens, windows up to 32 (within both), 0-16
    beacon slots with a random number live, max or mean aggregation."""
    import random
    rng = random.Random(seed)
    D = rng.choice([64, 128])
    hkv = rng.choice([1, 2, 4])
    g = rng.randint(1, 8)
    budget = rng.randint(1, 400)
    interval = rng.randint(1, 200)
    window = rng.randint(0, min(budget, interval, 32))
    nb_max = rng.choice([0, 1, 4, 8, 16])
    while g * window + nb_max > 512:
        window //= 2
    if g * window + nb_max == 0:
        window = 1
    n_live = rng.randint(0, nb_max)
    cfg = LoopConfig(n_layers=rng.choice([1, 2]), batch=rng.choice([1, 2, 3]), n_q_heads=hkv * g, n_kv_heads=hkv,
                     head_dim=D, budget=budget, window=window, nb_max=nb_max, interval=interval,
                     aggregation=rng.choice(["max", "max", "mean"]))
    return cfg, n_live


@pytest.mark.parametrize("seed", range(12))
def test_loop_random_configurations(seed):
    cfg, n_live = _random_config(7000 + seed)
    log(f"[loop] seed {seed}: {cfg} live beacons {n_live}")
    _run(cfg, cycles=2, n_live=n_live)
