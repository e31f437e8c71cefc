"""Steady-state compression loop on one GPU (BeaconKV page, Figure 7: beacons kept by
continual FPS as decoding proceeds; Table 4: the serving setting in which decoding goes on
after every compression).

Decoding appends `interval` tokens to every sequence; then the beacons are refreshed from
that chunk's queries, and the cache is compressed back to the budget.  With every
sequence at the budget after the first compression, each cycle sees the same lengths:
the cache holds budget + interval rows when it is compressed, the kept rows go to rows
0 .. budget-1 of the other of two cache buffers (bkv_compact_into), and the next chunk is
appended after them.

Everything the loop computes runs through the C ABI; torch only holds the buffers and
appends the new tokens the caller hands in (the part a decoding engine would do).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List

import torch

from . import bkv


@dataclass
class LoopConfig:
    n_layers: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    budget: int          # kept keys per KV head after each compression (window included)
    window: int          # recent queries scoring the keys; also always-kept keys
    nb_max: int          # beacon slots per KV head
    interval: int = 128  # decode steps (new tokens per sequence) between compressions
    aggregation: str = "max"
    beacon_policy: str = "fps"

    @property
    def capacity(self) -> int:
        return self.budget + self.interval


class SteadyStateLoop:
    """Double-buffered caches and beacon sets for the steady state of one model.

    `start(k, v, beacons, n_beacons)` installs caches of exactly `budget` rows per
    sequence (the state right after a compression); each `cycle(new_k, new_v, new_q)`
    appends one chunk and compresses.  `k`, `v` name the live buffers afterwards.
    """

    def __init__(self, cfg: LoopConfig, device="cuda"):
        c = self.cfg = cfg
        if c.interval < 1 or not 0 <= c.window <= min(c.budget, c.interval):
            raise ValueError("need interval >= 1 and 0 <= window <= min(budget, interval)")
        n, B, Hkv, Hq, D, cap = c.n_layers, c.batch, c.n_kv_heads, c.n_q_heads, c.head_dim, c.capacity
        bf = dict(dtype=torch.bfloat16, device=device)
        self._kv = [[[torch.zeros((B, Hkv, cap, D), **bf) for _ in range(n)] for _ in range(2)] for _ in range(2)]
        self._bc = [[torch.zeros((B, Hkv, max(c.nb_max, 1), D), **bf) for _ in range(n)] for _ in range(2)]
        self._nb = [[torch.zeros((B, Hkv), dtype=torch.int32, device=device) for _ in range(n)] for _ in range(2)]
        self._update = c.nb_max > 0
        if not self._update:   # nothing to refresh: both sides read one (empty) beacon set
            self._bc[1], self._nb[1] = self._bc[0], self._nb[0]
        self.q = [torch.zeros((B, Hq, c.interval, D), **bf) for _ in range(n)]
        self.seq_len = torch.full((B,), cap, dtype=torch.int32, device=device)
        self.shape = bkv.CacheShape(n, B, Hq, Hkv, D, cap, self.seq_len)
        self.scores = [torch.empty((B, Hkv, cap), dtype=torch.float32, device=device) for _ in range(n)]
        self.idx = [torch.empty((B, Hkv, c.budget), dtype=torch.int32, device=device) for _ in range(n)]
        self.n_kept = [torch.empty((B, Hkv), dtype=torch.int32, device=device) for _ in range(n)]
        self.workspace = bkv.alloc_workspace(bkv.score_workspace_bytes(self.shape, c.window, c.nb_max), device)
        self.cur = 0
        self.cycles = 0
        self._calls = [self._prepare(i) for i in range(2)]

    # buffers of side i: K/V caches and the beacon set read by a cycle that starts there
    def _k(self, i) -> List[torch.Tensor]:
        return self._kv[0][i]

    def _v(self, i) -> List[torch.Tensor]:
        return self._kv[1][i]

    @property
    def k(self) -> List[torch.Tensor]:
        return self._k(self.cur)

    @property
    def v(self) -> List[torch.Tensor]:
        return self._v(self.cur)

    @property
    def beacons(self) -> List[torch.Tensor]:
        return self._bc[self.cur]

    @property
    def n_beacons(self) -> List[torch.Tensor]:
        return self._nb[self.cur]

    def _prepare(self, i: int):
        """The library calls of a cycle that reads side i and writes side 1 - i."""
        c, sh, o = self.cfg, self.shape, 1 - i
        calls = []
        if self._update:
            calls.append(bkv.prepare_update_beacons(sh, self._bc[i], self._nb[i], c.nb_max, self.q, c.interval,
                                                    c.interval, self._bc[o], self._nb[o], c.beacon_policy))
        bc, nb = self._bc[o], self._nb[o]
        calls.append(bkv.prepare_score(sh, self._k(i), self.q, c.interval, c.window, bc, nb, c.nb_max,
                                       self.scores, self.workspace, c.aggregation))
        calls.append(bkv.prepare_select_topk(sh, self.scores, c.budget, c.window, self.idx, self.n_kept))
        calls.append(bkv.prepare_compact(sh, self._k(i), self._v(i), self.idx, self.n_kept, c.budget, self._k(o),
                                         self._v(o), out_capacity=c.capacity))
        return calls

    def start(self, k, v, beacons, n_beacons) -> None:
        """Install the post-compression state: per layer k, v [B][Hkv][budget][D] and the
        beacon sets [B][Hkv][nb_max][D] with their live counts [B][Hkv]."""
        c = self.cfg
        for l in range(c.n_layers):
            self.k[l][:, :, :c.budget].copy_(k[l])
            self.v[l][:, :, :c.budget].copy_(v[l])
            if c.nb_max > 0:
                self.beacons[l].copy_(beacons[l])
                self.n_beacons[l].copy_(n_beacons[l])

    def append(self, new_k, new_v, new_q) -> None:
        """Decoding's share of a cycle: the chunk's K/V rows after the kept ones, and its
        queries (per layer [B][Hkv][interval][D], [B][Hq][interval][D])."""
        c = self.cfg
        for l in range(c.n_layers):
            self.k[l][:, :, c.budget:].copy_(new_k[l])
            self.v[l][:, :, c.budget:].copy_(new_v[l])
            self.q[l].copy_(new_q[l])

    def compress(self, stream=None) -> None:
        """Beacon update (if any beacons), score, select and compact into the other side."""
        for call in self._calls[self.cur]:
            call(stream)
        self.cur = 1 - self.cur
        self.cycles += 1

    def cycle(self, new_k, new_v, new_q, stream=None) -> None:
        self.append(new_k, new_v, new_q)
        self.compress(stream)
