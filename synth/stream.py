"""A decode-time query stream for the beacon-coverage experiment (inputs only).

For one (layer, sequence, KV head) of a clustered workload, the G query heads of the
group emit one query each per decode step.  Steps before plan_frac * steps may come from
any cluster (the "plan" the reasoning lays out early); later steps come only from the
other clusters; then `future` held-out steps revisit the plan clusters with probability
future_plan_p.  This mirrors the page's observation that queries form a few recurring
cosine clusters that late decoding returns to (Figure 4; Figure 6 (a) measures how well a
kept query set covers future queries).
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np
import torch

from .gen import Workload, _compose, _rng, _rows, centres

TAG_STREAM_C, TAG_STREAM_Z = 21, 22


def query_stream(w: Workload, layer: int, b: int, h: int, steps: int, future: int, plan_frac: float = 0.05,
                 future_plan_p: Optional[float] = None, device="cpu") -> Tuple[torch.Tensor, np.ndarray]:
    """(bf16 [G, steps + future, D] queries, int64 [G, steps + future] cluster ids)."""
    if w.kind != "cluster" or w.n_plan == 0:
        raise ValueError("the stream needs a clustered workload with plan clusters")
    G, total = w.group, steps + future
    p = w.recent_plan_p if future_plan_p is None else future_plan_p
    rng = _rng(w.seed, TAG_STREAM_C, layer, b, h)
    cid = np.empty((G, total), dtype=np.int64)
    early = int(plan_frac * steps)
    cid[:, :early] = rng.integers(0, w.n_clusters, size=(G, early))
    cid[:, early:steps] = rng.integers(w.n_plan, w.n_clusters, size=(G, steps - early))
    revisit = rng.random((G, future)) < p
    cid[:, steps:] = np.where(revisit, rng.integers(0, w.n_plan, size=(G, future)),
                              rng.integers(w.n_plan, w.n_clusters, size=(G, future)))
    z = _rows(w, TAG_STREAM_Z, [(layer, b, h * G + r) for r in range(G)], total, device)
    ctr = torch.from_numpy(np.stack([centres(w, layer, h)] * G)).to(device)
    return _compose(z, torch.from_numpy(cid).to(device), ctr, w.spread), cid
