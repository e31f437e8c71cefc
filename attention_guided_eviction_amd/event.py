"""One compression event over all layers of a model, on one GPU.

A CompressionEvent owns the output buffers (scores, kept positions and counts,
compacted K/V, refreshed beacons) and the workspace for a fixed geometry, and runs the
path through the C ABI: optionally the continual-FPS beacon update (BeaconKV page,
Figure 7), then scoring, top-K selection and compaction (Figure 5 (b), (c); Abstract).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import torch

from . import bkv


@dataclass
class EventConfig:
    n_layers: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    capacity: int
    q_len: int          # stored queries per query head
    window: int         # recent queries per head scoring the keys; also always-kept keys
    nb_max: int         # beacon slots per KV head
    budget: int         # kept keys per KV head (window included)
    t_new: int = 0      # new queries per head fed to the beacon update (0: no update)
    aggregation: str = "max"   # "max" (the method) or "mean" (Table 2's alternative)
    beacon_policy: str = "fps"  # "fps" (continual FPS, the method) or "initial" (Table 3's Initial+Recent)


class CompressionEvent:
    def __init__(self, cfg: EventConfig, seq_len: torch.Tensor, device="cuda"):
        self.cfg = cfg
        c = cfg
        self.shape = bkv.CacheShape(c.n_layers, c.batch, c.n_q_heads, c.n_kv_heads, c.head_dim, c.capacity,
                                    seq_len)
        n = c.n_layers
        self.scores = [torch.empty((c.batch, c.n_kv_heads, c.capacity), dtype=torch.float32, device=device)
                       for _ in range(n)]
        self.idx = [torch.empty((c.batch, c.n_kv_heads, c.budget), dtype=torch.int32, device=device)
                    for _ in range(n)]
        self.n_kept = [torch.empty((c.batch, c.n_kv_heads), dtype=torch.int32, device=device) for _ in range(n)]
        self.k_out = [torch.empty((c.batch, c.n_kv_heads, c.budget, c.head_dim), dtype=torch.bfloat16,
                                  device=device) for _ in range(n)]
        self.v_out = [torch.empty_like(t) for t in self.k_out]
        if c.t_new > 0:
            self.beacons_out = [torch.empty((c.batch, c.n_kv_heads, c.nb_max, c.head_dim), dtype=torch.bfloat16,
                                            device=device) for _ in range(n)]
            self.n_beacons_out = [torch.empty((c.batch, c.n_kv_heads), dtype=torch.int32, device=device)
                                  for _ in range(n)]
        else:
            self.beacons_out = self.n_beacons_out = None
        need = bkv.compress_workspace_bytes(self.shape, c.window, c.nb_max, c.budget)
        self.workspace = bkv.alloc_workspace(need, device)

    def bind(self, k, v, q, beacons, n_beacons) -> "CompressionEvent":
        """Check the inputs once and prepare every library call of an event over them."""
        c = self.cfg
        sh = self.shape
        self.calls = {}
        if c.t_new > 0:
            self.calls["update_beacons"] = bkv.prepare_update_beacons(sh, beacons, n_beacons, c.nb_max, q, c.q_len,
                                                                      c.t_new, self.beacons_out, self.n_beacons_out,
                                                                      c.beacon_policy)
            beacons, n_beacons = self.beacons_out, self.n_beacons_out
        self.calls["compress"] = bkv.prepare_compress(sh, k, v, q, c.q_len, c.window, beacons, n_beacons, c.nb_max,
                                                      c.budget, self.scores, self.idx, self.n_kept, self.k_out,
                                                      self.v_out, self.workspace)
        # the three stages of compress, separately (for per-stage timing)
        self.calls["score"] = bkv.prepare_score(sh, k, q, c.q_len, c.window, beacons, n_beacons, c.nb_max,
                                                self.scores, self.workspace, c.aggregation)
        self.calls["select"] = bkv.prepare_select_topk(sh, self.scores, c.budget, c.window, self.idx, self.n_kept)
        self.calls["compact"] = bkv.prepare_compact(sh, k, v, self.idx, self.n_kept, c.budget, self.k_out,
                                                    self.v_out)
        return self

    def step(self, stream=None) -> None:
        """One event over the bound inputs: beacon update (if configured), then compress
        (max aggregation) or score, select and compact (any other aggregation)."""
        if "update_beacons" in self.calls:
            self.calls["update_beacons"](stream)
        if self.cfg.aggregation == "max":
            self.calls["compress"](stream)
        else:
            for name in ("score", "select", "compact"):
                self.calls[name](stream)

    def run(self, k, v, q, beacons, n_beacons, stream=None) -> None:
        """Bind the inputs and run one event."""
        self.bind(k, v, q, beacons, n_beacons).step(stream)
