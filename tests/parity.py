"""Helpers for GPU-vs-oracle parity: run a synthetic workload through the library on the
GPU, then check chosen units against the CPU oracle with the stated tolerances.

Tolerances:
* scores: |S_gpu - S_oracle| <= 1e-3 * S_oracle for every valid key;
* selection: (a) the GPU's kept set equals the oracle's selection rule applied to the
  GPU's own fp32 scores (exact); (b) against the oracle's own selection, the sets agree
  except for swaps whose oracle scores differ by less than 1e-5; (c) window kept, count
  min(budget, L), ascending;
* compaction: bit-exact rows given the GPU's kept positions;
* beacons: replay check -- at every step, given the GPU's earlier picks, the GPU's pick
  reaches the largest nearest-pick distance within 1e-5 (cosine-distance units) and is the
  oracle's pick whenever the oracle's best and second-best differ by at least 1e-5; rows are
  bit copies of the picked pool rows.
"""
from __future__ import annotations

import sys
import time
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

from oracle import bkv_oracle as O
from synth import layer_tensors, seq_lengths, unit_inputs, bf16_bits
from synth.gen import Workload
from attention_guided_eviction_amd import bkv
from attention_guided_eviction_amd.event import CompressionEvent, EventConfig

SCORE_RTOL = 1e-3
TIE_GAP = 1e-5
FPS_GAP = 1e-5


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def event_config(w: Workload, aggregation: str = "max", beacon_policy: str = "fps") -> EventConfig:
    return EventConfig(w.n_layers, w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.capacity, w.q_len, w.window,
                       w.nb_max, w.budget, w.t_new, aggregation, beacon_policy)


def build_inputs(w: Workload, device="cuda") -> Dict[str, List[torch.Tensor]]:
    layers = [layer_tensors(w, l, device) for l in range(w.n_layers)]
    out = {key: [lt[key] for lt in layers] for key in layers[0]}
    out["seq_len"] = torch.from_numpy(seq_lengths(w)).to(device)
    return out


def run_gpu(w: Workload, inputs=None, device="cuda", aggregation: str = "max",
            beacon_policy: str = "fps") -> Tuple[CompressionEvent, Dict]:
    if inputs is None:
        inputs = build_inputs(w, device)
    ev = CompressionEvent(event_config(w, aggregation, beacon_policy), inputs["seq_len"], device)
    ev.run(inputs["k"], inputs["v"], inputs["q"], inputs["beacons"], inputs["n_beacons"])
    torch.cuda.synchronize()
    return ev, inputs


# ------------------------------------------------------------------------------------------------

def check_fps_replay(pool_bits: np.ndarray, gpu_rows: np.ndarray, n_pick: int) -> np.ndarray:
    """Check GPU beacon rows against continual FPS by replay; returns the GPU's pool indices."""
    P = pool_bits.shape[0]
    n_exp = min(n_pick, P)
    assert gpu_rows.shape[0] == n_exp
    pool = O.bf16_to_f64(pool_bits)
    # map each GPU row to the first pool row with the same bits (duplicates are interchangeable)
    lookup = {}
    for p in range(P - 1, -1, -1):
        lookup[pool_bits[p].tobytes()] = p
    picks = []
    for r in range(n_exp):
        key = gpu_rows[r].tobytes()
        assert key in lookup, f"beacon row {r} is not a pool row"
        picks.append(lookup[key])
    if P <= n_pick:
        assert picks == list(range(P)) or all(pool_bits[a].tobytes() == pool_bits[b].tobytes()
                                              for a, b in zip(picks, range(P)))
        return np.array(picks)
    assert picks[0] == 0 or pool_bits[picks[0]].tobytes() == pool_bits[0].tobytes()
    picks[0] = 0
    nearest = O.cosine_distance_to(pool, 0)
    taken = np.zeros(P, bool)
    taken[0] = True
    for t in range(1, n_exp):
        cand = np.where(taken, -np.inf, nearest)
        best = cand.max()
        order = np.argsort(-cand, kind="stable")
        g = picks[t]
        # duplicates of a taken row have distance 0; choose any untaken row with the same bits
        if taken[g]:
            dups = [p for p in range(P) if not taken[p] and pool_bits[p].tobytes() == pool_bits[g].tobytes()]
            assert dups, f"step {t}: GPU repeated pool row {g}"
            g = dups[0]
        assert cand[g] >= best - FPS_GAP, f"step {t}: GPU pick {g} at {cand[g]:.8f}, best {best:.8f}"
        second = cand[order[1]] if P - t > 1 else -np.inf
        if best - second >= FPS_GAP:
            assert g == order[0], f"step {t}: GPU pick {g}, oracle {order[0]} (gap {best - second:.2e})"
        picks[t] = g
        taken[g] = True
        nearest = np.minimum(nearest, O.cosine_distance_to(pool, g))
    return np.array(picks)


def check_selection(keep_gpu: np.ndarray, s_gpu: np.ndarray, s_or: np.ndarray, L: int, budget: int,
                    window: int) -> Dict[str, float]:
    n = min(budget, L)
    assert keep_gpu.shape == (n,)
    assert np.all(np.diff(keep_gpu) > 0), "kept positions not strictly ascending"
    if L > budget:
        assert set(range(L - window, L)) <= set(keep_gpu.tolist()), "window not kept"
    # (a) exact: oracle rule on the GPU's fp32 scores
    want_self = O.select_keep(s_gpu.astype(np.float64), L, budget, window)
    np.testing.assert_array_equal(keep_gpu, want_self, err_msg="selection differs from rule on GPU scores")
    # (b) against the oracle's own selection: only near-tie swaps
    want = O.select_keep(s_or, L, budget, window)
    extra = np.setdiff1d(keep_gpu, want)
    missing = np.setdiff1d(want, keep_gpu)
    assert extra.size == missing.size
    gap = 0.0
    if extra.size:
        a = np.sort(s_or[extra])[::-1]
        b = np.sort(s_or[missing])[::-1]
        gaps = np.abs(a - b)
        gap = float(gaps.max())
        assert gap < TIE_GAP, f"{extra.size} swaps, largest oracle-score gap {gap:.3e}"
    return {"swaps": float(extra.size), "gap": gap}


def unit_from_inputs(w: Workload, inputs: Dict[str, List[torch.Tensor]], layer: int, b: int, h: int):
    """The unit's slices of explicit input tensors (e.g. generator output with planted
    rows), in the layout `unit_inputs` returns: the oracle then sees exactly the bits the
    GPU consumed."""
    G = w.group
    L = int(inputs["seq_len"][b].item())
    return {"k": inputs["k"][layer][b, h, :L].cpu(), "v": inputs["v"][layer][b, h, :L].cpu(),
            "q": inputs["q"][layer][b, h * G:(h + 1) * G].cpu(), "beacons": inputs["beacons"][layer][b, h].cpu(),
            "nb": int(inputs["n_beacons"][layer][b, h].item()), "L": L}


def check_unit(w: Workload, ev: CompressionEvent, layer: int, b: int, h: int,
               inputs: Optional[Dict[str, List[torch.Tensor]]] = None) -> Dict[str, float]:
    """One unit's beacons, scores (under the event's aggregation), selection and compaction.
    The unit's inputs are regenerated from the workload's seeds, or taken from `inputs`."""
    u = unit_inputs(w, layer, b, h, "cpu") if inputs is None else unit_from_inputs(w, inputs, layer, b, h)
    L = u["L"]
    kb, vb, qb, bcb = bf16_bits(u["k"]), bf16_bits(u["v"]), bf16_bits(u["q"]), bf16_bits(u["beacons"])
    stats: Dict[str, float] = {}
    # beacons
    if w.runs_fps:
        n_out = int(ev.n_beacons_out[layer][b, h].item())
        gpu_rows = bf16_bits(ev.beacons_out[layer][b, h, :n_out])
        q_new = qb[:, w.q_len - w.t_new:, :]
        if ev.cfg.beacon_policy == "initial":
            want, n_want = O.initial_beacons(bcb, u["nb"], q_new, w.nb_max)
            assert n_out == n_want and gpu_rows.tobytes() == want.tobytes(), "initial beacons differ"
        else:
            pool_bits = O.beacon_pool(bcb, u["nb"], q_new)
            assert n_out == min(w.nb_max, pool_bits.shape[0])
            check_fps_replay(pool_bits, gpu_rows, w.nb_max)
        beacons_used, nb_used = gpu_rows, n_out
    else:
        beacons_used, nb_used = bcb, u["nb"]
    # scores
    obs = O.observation_queries(O.bf16_to_f64(qb), w.window, O.bf16_to_f64(beacons_used), nb_used)
    s_or = O.aggregated_scores(obs, O.bf16_to_f64(kb), ev.cfg.aggregation)
    s_gpu = ev.scores[layer][b, h, :L].cpu().numpy()
    if L:
        zero = s_or == 0.0
        assert np.all(s_gpu[zero] == 0.0), "scores should be exactly 0 without observers"
        rel = np.abs(s_gpu.astype(np.float64) - s_or) / np.where(zero, 1.0, s_or)
        stats["score_rel_max"] = float(rel.max())
        bad = np.flatnonzero(~(rel <= SCORE_RTOL))
        assert bad.size == 0, (f"{bad.size} scores off (layer {layer} b {b} h {h}); first j={bad[0]}: "
                               f"gpu {s_gpu[bad[0]]!r} oracle {s_or[bad[0]]!r}")
    # selection
    n = int(ev.n_kept[layer][b, h].item())
    assert n == min(w.budget, L), f"n_kept {n}, expected {min(w.budget, L)}"
    keep_gpu = ev.idx[layer][b, h, :n].cpu().numpy().astype(np.int64)
    stats.update(check_selection(keep_gpu, s_gpu, s_or, L, w.budget, w.window))
    # compaction
    ko = bf16_bits(ev.k_out[layer][b, h, :n])
    vo = bf16_bits(ev.v_out[layer][b, h, :n])
    assert ko.tobytes() == kb[keep_gpu].tobytes(), "compacted K not bit-exact"
    assert vo.tobytes() == vb[keep_gpu].tobytes(), "compacted V not bit-exact"
    return stats


def check_units(w: Workload, ev: CompressionEvent, units: Sequence[Tuple[int, int, int]],
                inputs: Optional[Dict[str, List[torch.Tensor]]] = None) -> Dict[str, float]:
    worst = {"score_rel_max": 0.0, "swaps": 0.0, "gap": 0.0}
    for (l, b, h) in units:
        t0 = time.time()
        st = check_unit(w, ev, l, b, h, inputs)
        for k, v in st.items():
            worst[k] = max(worst.get(k, 0.0), v)
        log(f"  unit (layer {l}, b {b}, h {h}) ok in {time.time() - t0:.1f}s: {st}")
    return worst


def all_units(w: Workload):
    return [(l, b, h) for l in range(w.n_layers) for b in range(w.batch) for h in range(w.n_kv_heads)]


def sample_units(w: Workload, n: int, seed: int = 0):
    rng = np.random.default_rng(seed)
    units = {(0, 0, 0), (w.n_layers - 1, w.batch - 1, w.n_kv_heads - 1)}
    lens = seq_lengths(w)
    units.add((w.n_layers // 2, int(np.argmin(lens)), 0))
    units.add((w.n_layers // 3, int(np.argmax(lens)), w.n_kv_heads - 1))
    while len(units) < n:
        units.add((int(rng.integers(w.n_layers)), int(rng.integers(w.batch)), int(rng.integers(w.n_kv_heads))))
    return sorted(units)
