"""Beacon coverage of future queries: how close the kept query set stays to the queries
decoding will issue later (BeaconKV page, Figure 6 (a): how similar later queries are to
the best match in each choice of kept past queries; Figure 7: continual versus naive FPS;
Table 3: Initial+Recent).

The beacon sets are built on the GPU by the library's beacon update, chunk after chunk of a
query stream; the similarity readout is a small evaluation, not part of the compression
path, and uses torch.

    python -m attention_guided_eviction_amd.coverage [--workload qwen14b_64k] [--units 8]
"""
from __future__ import annotations

import argparse
import json
from typing import Dict, List, Tuple

import torch

from . import bkv


def beacon_stream(q: torch.Tensor, nb_max: int, chunk: int, policy: str = "fps") -> Tuple[torch.Tensor, torch.Tensor]:
    """Beacon sets after feeding a query stream chunk by chunk.

    q: bf16 [U, G, steps, D] on the GPU, U independent groups of G query heads (one KV
    head each), steps a multiple of `chunk`.  Starts from empty sets.  Returns
    (beacons [U, nb_max, D], live counts [U]).
    """
    U, G, S, D = q.shape
    if S % chunk:
        raise ValueError("steps must be a multiple of chunk")
    dev = q.device
    shape = bkv.CacheShape(1, U, G, 1, D, 1, torch.ones(U, dtype=torch.int32, device=dev))
    bc = [torch.zeros((U, 1, nb_max, D), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    nb = [torch.zeros((U, 1), dtype=torch.int32, device=dev) for _ in range(2)]
    cur = 0
    for c0 in range(0, S, chunk):
        qn = q[:, :, c0:c0 + chunk].contiguous()
        o = 1 - cur
        bkv.update_beacons(shape, [bc[cur]], [nb[cur]], nb_max, [qn], chunk, chunk, [bc[o]], [nb[o]], policy=policy)
        cur = o
    return bc[cur][:, 0], nb[cur][:, 0]


def max_cosine(future: torch.Tensor, sets: torch.Tensor, counts: torch.Tensor) -> torch.Tensor:
    """[U, F] largest cosine similarity of each future query to the first counts[u] rows of
    sets[u] (-1 where a set is empty)."""
    f = torch.nn.functional.normalize(future.float(), dim=-1)
    s = torch.nn.functional.normalize(sets.float(), dim=-1)
    cos = torch.bmm(f, s.transpose(1, 2).contiguous())
    live = torch.arange(sets.shape[1], device=sets.device)[None, None, :] < counts[:, None, None]
    return torch.where(live, cos, torch.full_like(cos, -1.0)).amax(dim=-1)


def coverage(w, units: List[Tuple[int, int, int]], steps: int, future: int, chunk: int, window: int, nb_max: int,
             device="cuda") -> Dict[str, Dict[str, float]]:
    """Mean max-cosine coverage of the held-out queries by: the continual-FPS beacons, the
    initial-query beacons, naive FPS over the whole history in one pool (when the history
    fits the largest pool), and the recent window alone; split into plan revisits and the
    rest."""
    from synth.stream import query_stream
    qs, cids = [], []
    for (layer, b, h) in units:
        q, c = query_stream(w, layer, b, h, steps, future, device=device)
        qs.append(q)
        cids.append(torch.from_numpy(c))
    q = torch.stack(qs)                                   # [U, G, steps + future, D]
    cid = torch.stack(cids).to(device)
    U, G, _, D = q.shape
    past, fut = q[:, :, :steps], q[:, :, steps:].reshape(U, G * future, D)
    revisit = (cid[:, :, steps:] < w.n_plan).reshape(U, G * future)
    sets = {}
    for policy in ("fps", "initial"):
        sets[policy] = beacon_stream(past.contiguous(), nb_max, chunk, policy)
    if G * steps <= bkv.MAX_POOL:   # Figure 7's naive FPS: one pick over the whole history
        sets["naive_fps"] = beacon_stream(past.contiguous(), nb_max, steps, "fps")
    recent = past[:, :, steps - window:].reshape(U, G * window, D)
    sets["recent"] = (recent, torch.full((U,), G * window, dtype=torch.int32, device=device))
    for policy in [k for k in ("fps", "initial", "naive_fps") if k in sets]:
        b, n = sets[policy]
        sets[policy + "+recent"] = (torch.cat([recent, b], dim=1), n + G * window)
    out = {}
    for name, (s, n) in sets.items():
        m = max_cosine(fut, s, n)
        out[name] = {"plan_revisits": float(m[revisit].mean()), "other": float(m[~revisit].mean()),
                     "all": float(m.mean())}
    out["_counts"] = {"plan_revisits": int(revisit.sum()), "other": int((~revisit).sum())}
    return out


def main():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--workload", default="qwen14b_64k")
    p.add_argument("--units", type=int, default=8)
    p.add_argument("--steps", type=int, default=3200)
    p.add_argument("--future", type=int, default=512)
    p.add_argument("--chunk", type=int, default=128)
    args = p.parse_args()
    from synth import WORKLOADS
    w = WORKLOADS[args.workload]
    units = [(0, u % w.batch, (u // w.batch) % w.n_kv_heads) for u in range(args.units)]
    res = coverage(w, units, args.steps, args.future, args.chunk, w.window, w.nb_max)
    print(json.dumps({"workload": w.name, "steps": args.steps, "future": args.future, "chunk": args.chunk,
                      "window": w.window, "beacons": w.nb_max, "coverage": res}))


if __name__ == "__main__":
    main()
