"""Inputs with planted dominant keys, for parity cases that drive the online softmax's
exact rescale (BeaconKV page, Figure 5 (b), (c): the scores are softmax attention weights).

A key k_p = bf16(alpha * q_i) gives observation row i a logit of about
alpha * |q_i|^2 / sqrt(d), far above every other logit of that row (the oracle reads the same
bf16 bits the GPU does, so the rounding of the product does not matter).  The scorer's statistics pass keeps a running max and adds exp2 terms against it; a
logit more than 64 above that max (log2 units) overflows the cheap running sum, so the pass
must take its exact branch (new max, old sum rescaled by exp2(m_old - m_new)).  Positions
are chosen after the first 32-key fragment of any piece of a unit a workgroup can start
(pieces start at 256-key tiles; the LDS-staged pass also splits tiles into 64-key quarters,
one per wave), so the running max of that piece is already finite when the key arrives.

This module only edits inputs; the expected values still come from the oracle.
"""
from __future__ import annotations

import math
from typing import Dict, List, Tuple

import numpy as np
import torch

from synth.gen import Workload

ALPHA = 8.0
GROWTH = 1.5
OVERFLOW_LOG2 = 64.0


def obs_row(w: Workload, inputs, layer: int, b: int, h: int, r: int) -> torch.Tensor:
    """Observation row r of unit (layer, b, h): recent queries head-major, then beacons."""
    gw = w.group * w.window
    if r < gw:
        hq = h * w.group + r // w.window
        return inputs["q"][layer][b, hq, w.q_len - w.window + r % w.window]
    return inputs["beacons"][layer][b, h, r - gw]


def _after_first_fragment(p: int) -> int:
    """The position at or below p whose offset within its 64-key quarter is 32..63."""
    return p - (p % 64) + 32 + (p % 32)


def spots(w: Workload, L: int, n_obs: int) -> List[Tuple[int, int]]:
    """(position, observation row) pairs for a unit of L keys and n_obs rows: one key early
    in the second tile, one mid-unit, one just before the window, one in the last (often
    partial) 32-key fragment, and one at a tile start (first fragment of a piece)."""
    if n_obs == 0 or L < 128:
        return []
    nt = (L + 255) // 256
    cand = [
        (_after_first_fragment(256 + 100), 0),
        (_after_first_fragment(256 * (nt // 2) + 232), w.group * w.window - 1 if w.window else n_obs - 1),
        (_after_first_fragment(max(L - w.window - 40, 40)), min(1, n_obs - 1)),
        (L - 5, n_obs - 1),
        (512, min(2, n_obs - 1)),
    ]
    out, used_p, used_r = [], set(), set()
    for p, r in cand:
        if 0 <= p < L and p not in used_p and r not in used_r:
            out.append((p, r))
            used_p.add(p)
            used_r.add(r)
    return out


def plant(w: Workload, inputs, alpha: float = ALPHA) -> Dict[Tuple[int, int, int], List[Tuple[int, int]]]:
    """Plant alpha * q_i keys in every unit (in place); returns the spots per unit.  The
    factor grows by GROWTH from one spot to the next in position order, so a planted key
    stays far above the earlier planted keys of other rows even when the two rows are alike,
    while the largest logit stays small enough (a few thousand) for fp32 accumulation."""
    lens = inputs["seq_len"].cpu().numpy()
    where = {}
    for layer in range(w.n_layers):
        for b in range(w.batch):
            L = int(lens[b])
            for h in range(w.n_kv_heads):
                nb = int(inputs["n_beacons"][layer][b, h].item())
                n_obs = w.group * w.window + nb
                sp = sorted(spots(w, L, n_obs))
                for i, (p, r) in enumerate(sp):
                    row = obs_row(w, inputs, layer, b, h, r).to(torch.float32)
                    inputs["k"][layer][b, h, p] = (row * (alpha * GROWTH ** i)).to(torch.bfloat16)
                where[(layer, b, h)] = sp
    return where


def jumps(w: Workload, inputs, layer: int, b: int, h: int, sp: List[Tuple[int, int]]) -> List[float]:
    """For each planted spot, how far (log2 units) its logit for its row lies above every
    earlier key's logit for that row.  Above OVERFLOW_LOG2 the cheap running sum of any
    piece of the unit that holds earlier keys overflows at that key."""
    L = int(inputs["seq_len"][b].item())
    k = inputs["k"][layer][b, h, :L].to(torch.float64).cpu().numpy()
    c = math.log2(math.e) / math.sqrt(w.head_dim)
    out = []
    for p, r in sp:
        q = obs_row(w, inputs, layer, b, h, r).to(torch.float64).cpu().numpy()
        t = (k @ q) * c
        out.append(float(t[p] - t[:p].max()) if p > 0 else float("inf"))
    return out
