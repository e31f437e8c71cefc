"""Seeded synthetic inputs for KV-cache compression workloads.

This module produces inputs only: KV caches, observation queries, beacon sets and
sequence lengths. It holds none of the compression arithmetic (no scoring, no
selection, no sampling of beacons), so both the CPU oracle and the GPU path can
consume what it makes without sharing any of the method.

The BeaconKV page (thelatestinai.com/papers/2609.04971) evaluates on real
reasoning traces of four models (Fig. 8 caption) with outputs of roughly 4k-15k
tokens (Table 6), and finds that the queries of thought-revisiting tokens
cluster in a few cosine-similarity groups (Abstract; Fig. 4).  None of that data
is available, so these workloads stand in for it:

* shapes follow the four models' attention geometry (layers, query / KV heads,
  head_dim 128) plus a tiny case;
* keys are contiguous "segments" (mean length 64, geometric) that either carry
  one cluster centre plus a small deviation or are plain noise tokens;
* queries are drawn near the same centres, so attention is peaked but not
  degenerate; the long-trace workload has four early "plan" clusters that only
  late queries and beacons revisit.

Determinism across devices
--------------------------
Every random element is a pure function of (seed, tensor tag, layer, sequence,
head, element index).  Uniform bits come from a counter-based integer hash
(Wellons' "lowbias32" 32-bit mixer, applied twice per 32-bit word), four
16-bit uniforms are summed (Irwin-Hall, n = 4, rescaled to unit variance) to
give an approximately standard normal deviate, and the only floating-point
steps are exact int->float conversion, correctly rounded fp32 multiply and add,
and round-to-nearest-even to bfloat16.  Hence the same code run with torch on
the CPU or on a GPU yields bit-identical tensors, so the oracle can regenerate
any single unit on the host while the GPU builds whole caches in HBM.

Host-side structure (segment layout, cluster choices, centres, lengths) is drawn
with NumPy's PCG64 from a SeedSequence keyed by the same fields.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

_M32 = 0xFFFFFFFF

# Tags that separate the random streams of different tensors.
TAG_K, TAG_V, TAG_QN, TAG_BC = 1, 2, 3, 4            # element noise streams
TAG_SEG, TAG_QC, TAG_BCC, TAG_CTR, TAG_LEN = 11, 12, 13, 14, 15  # host-side structure


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload.  All sizes are per GPU."""
    name: str
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    batch: int
    capacity: int                 # rows allocated per (sequence, KV head)
    seq_len: Optional[int]        # fixed length, or None for ragged
    ragged: Optional[tuple]       # (lo, hi) inclusive, uniform per sequence
    window: int                   # recent queries per query head and always-kept keys
    nb_init: int                  # beacons present before the call
    nb_max: int                   # beacon capacity per KV head
    budget: int                   # kept keys per KV head, window included
    t_new: int                    # new queries per query head fed to the beacon update (0: none)
    kind: str                     # "gauss" or "cluster"
    n_clusters: int = 0
    n_plan: int = 0               # clusters 0..n_plan-1 only appear early in the trace
    plan_frac: float = 0.05       # "early" = segment starts before plan_frac * L
    recent_plan_p: float = 0.0    # probability a recent query revisits a plan cluster
    beacon_plan_p: float = 0.0    # probability an initial beacon sits on a plan cluster
    noise_p: float = 0.25         # probability a key segment is pure noise
    seg_mean: float = 64.0        # mean key-segment length
    spread: float = 0.3           # RMS-per-coordinate deviation around a scaled centre
    seed: int = 0
    lengths: Optional[tuple] = None   # explicit per-sequence lengths (edge-case workloads)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def q_len(self) -> int:
        """Query rows stored per query head: the window is the last `window` of them."""
        return max(self.window, self.t_new)

    @property
    def runs_fps(self) -> bool:
        return self.t_new > 0

    @property
    def units(self) -> int:
        return self.n_layers * self.batch * self.n_kv_heads

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    # 1 layer, GQA 4/2, d 64, L 512, all N(0,1); beacons refreshed from the 8 recent queries.
    "tiny": Workload("tiny", 1, 4, 2, 64, 1, 512, 512, None, 8, 4, 4, 128, 8, "gauss",
                     seed=0xBEAC01),
    # R1-Distill-Qwen-7B attention geometry, one 16K trace.
    "qwen7b_16k": Workload("qwen7b_16k", 28, 28, 4, 128, 1, 16384, 16384, None, 32, 16, 16,
                           4096, 0, "cluster", n_clusters=8, seed=0xBEAC02),
    # R1-Distill-Llama-8B geometry, batch 8 x 32K.
    "llama8b_32k": Workload("llama8b_32k", 32, 32, 8, 128, 8, 32768, 32768, None, 32, 16, 16,
                            2048, 0, "cluster", n_clusters=16, seed=0xBEAC03),
    # Qwen3-14B geometry, batch 4 x 64K, four early plan clusters revisited late.
    "qwen14b_64k": Workload("qwen14b_64k", 40, 40, 8, 128, 4, 65536, 65536, None, 64, 32, 32,
                            8192, 0, "cluster", n_clusters=16, n_plan=4, recent_plan_p=0.25,
                            beacon_plan_p=0.5, seed=0xBEAC04),
    # Qwen3-4B geometry, 64 ragged sequences, beacon update over 128 new queries per head.
    "qwen4b_serving": Workload("qwen4b_serving", 36, 32, 8, 128, 64, 8192, None, (2048, 8192),
                               32, 16, 16, 1024, 128, "cluster", n_clusters=16, seed=0xBEAC05),
}
WORKLOAD_ORDER: List[str] = ["tiny", "qwen7b_16k", "llama8b_32k", "qwen14b_64k", "qwen4b_serving"]


# ----------------------------------------------------------------------------------------------
# counter-based hashing
# ----------------------------------------------------------------------------------------------

def _lowbias32_int(x: int) -> int:
    x &= _M32
    x ^= x >> 16
    x = (x * 0x7FEB352D) & _M32
    x ^= x >> 15
    x = (x * 0x846CA68B) & _M32
    x ^= x >> 16
    return x


def stream_key(*fields: int) -> tuple:
    """Two 32-bit keys for the stream named by `fields` (pure Python ints)."""
    h = 0x6A09E667
    for f in fields:
        h = _lowbias32_int(h ^ (int(f) & _M32))
        h = _lowbias32_int(h + ((int(f) >> 32) & _M32))
    return h, _lowbias32_int(h ^ 0x9E3779B9)


def _mul32(x: torch.Tensor, c: int) -> torch.Tensor:
    """(x * c) mod 2^32 for int64 x in [0, 2^32) without signed overflow."""
    lo = x & 0xFFFF
    hi = x >> 16
    return (lo * c + ((hi * (c & 0xFFFF)) << 16)) & _M32


def _lowbias32(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


_IH_MEAN = 2 * 65535            # mean of a sum of four uniforms on 0..65535, times 1
_IH_SCALE = float(np.float32(math.sqrt(3.0) / 65536.0))


def noise(keys: torch.Tensor, n: int, device) -> torch.Tensor:
    """Unit-variance, roughly Gaussian fp32 deviates.

    keys: int64 tensor [U, 2] (k1, k2 per stream).  Returns fp32 [U, n]; element e of
    stream u depends only on (k1_u, k2_u, e).
    """
    keys = keys.to(device)
    e = torch.arange(n, dtype=torch.int64, device=device).unsqueeze(0)
    k1 = keys[:, 0:1]
    k2 = keys[:, 1:2]
    a = _lowbias32(_lowbias32((2 * e) ^ k1) ^ k2)
    b = _lowbias32(_lowbias32((2 * e + 1) ^ k1) ^ k2)
    s = (a & 0xFFFF) + (a >> 16) + (b & 0xFFFF) + (b >> 16)
    del a, b
    scale = torch.full((1, 1), _IH_SCALE, dtype=torch.float32, device=device)
    return (s - _IH_MEAN).to(torch.float32) * scale


def _keys_tensor(pairs: Sequence[tuple]) -> torch.Tensor:
    return torch.tensor([[p[0], p[1]] for p in pairs], dtype=torch.int64)


def _rng(*fields: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(f) for f in fields])))


# ----------------------------------------------------------------------------------------------
# host-side structure
# ----------------------------------------------------------------------------------------------

def seq_lengths(w: Workload) -> np.ndarray:
    """Valid cached keys per sequence (int32 [batch])."""
    if w.lengths is not None:
        return np.asarray(w.lengths, dtype=np.int32)
    if w.ragged is None:
        return np.full(w.batch, w.seq_len, dtype=np.int32)
    lo, hi = w.ragged
    return _rng(w.seed, TAG_LEN).integers(lo, hi + 1, size=w.batch).astype(np.int32)


def centres(w: Workload, layer: int, h: int) -> np.ndarray:
    """fp32 [n_clusters, D]: sqrt(D) times a unit-norm direction, per (layer, KV head)."""
    if w.kind != "cluster":
        return np.zeros((0, w.head_dim), dtype=np.float32)
    u = _rng(w.seed, TAG_CTR, layer, h).standard_normal((w.n_clusters, w.head_dim))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    return (math.sqrt(w.head_dim) * u).astype(np.float32)


def key_clusters(w: Workload, layer: int, b: int, h: int, L: int) -> np.ndarray:
    """int64 [capacity]: cluster id of each cache row (-1 = noise token).

    Rows are cut into contiguous segments of geometric length; a segment is noise
    with probability noise_p, otherwise one cluster.  Plan clusters may only start
    segments that begin before plan_frac * L.
    """
    cap = w.capacity
    out = np.full(cap, -1, dtype=np.int64)
    if w.kind != "cluster":
        return out
    rng = _rng(w.seed, TAG_SEG, layer, b, h)
    n_seg = int(cap / w.seg_mean * 2) + 64
    lens = rng.geometric(1.0 / w.seg_mean, size=n_seg)
    while lens.sum() < cap:                       # practically never taken
        lens = np.concatenate([lens, rng.geometric(1.0 / w.seg_mean, size=n_seg)])
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    keep = starts < cap
    lens, starts = lens[keep], starts[keep]
    is_noise = rng.random(lens.size) < w.noise_p
    any_c = rng.integers(0, w.n_clusters, size=lens.size)
    late_c = rng.integers(w.n_plan, w.n_clusters, size=lens.size)
    early = starts < w.plan_frac * L
    cid = np.where(is_noise, -1, np.where(early, any_c, late_c))
    out[:] = np.repeat(cid, lens)[:cap]
    return out


def _query_clusters(w: Workload, rng: np.random.Generator, n: int, plan_p: float) -> np.ndarray:
    if w.kind != "cluster":
        return np.full(n, -1, dtype=np.int64)
    if w.n_plan == 0 or plan_p == 0.0:
        return rng.integers(0, w.n_clusters, size=n)
    plan = rng.random(n) < plan_p
    return np.where(plan, rng.integers(0, w.n_plan, size=n),
                    rng.integers(w.n_plan, w.n_clusters, size=n))


def query_clusters(w: Workload, layer: int, b: int, hq: int) -> np.ndarray:
    """int64 [q_len]: cluster of each stored query of one query head.

    For the beacon-update workloads the rows are the newest decode queries and the
    window is their tail; otherwise they are the recent window itself.
    """
    rng = _rng(w.seed, TAG_QC, layer, b, hq)
    return _query_clusters(w, rng, w.q_len, w.recent_plan_p)


def beacon_clusters(w: Workload, layer: int, b: int, h: int) -> np.ndarray:
    rng = _rng(w.seed, TAG_BCC, layer, b, h)
    return _query_clusters(w, rng, w.nb_max, w.beacon_plan_p)


# ----------------------------------------------------------------------------------------------
# element values
# ----------------------------------------------------------------------------------------------

def _compose(z: torch.Tensor, cid: torch.Tensor, ctr: torch.Tensor, spread: float) -> torch.Tensor:
    """z [U, R, D] fp32, cid [U, R] int64 (-1 noise), ctr [U, M, D] fp32 -> bf16 [U, R, D]."""
    if ctr.shape[1] == 0:
        return z.to(torch.bfloat16)
    idx = cid.clamp(min=0).unsqueeze(-1).expand(-1, -1, z.shape[-1])
    c = torch.gather(ctr, 1, idx)
    s = torch.full((1, 1, 1), spread, dtype=torch.float32, device=z.device)
    x = c + z * s
    x = torch.where(cid.unsqueeze(-1) >= 0, x, z)
    return x.to(torch.bfloat16)


def _rows(w: Workload, tag: int, unit_ids: Sequence[tuple], rows: int, device) -> torch.Tensor:
    keys = _keys_tensor([stream_key(w.seed, tag, *u) for u in unit_ids])
    return noise(keys, rows * w.head_dim, device).view(len(unit_ids), rows, w.head_dim)


def keys_for(w: Workload, layer: int, units: Sequence[tuple], rows: int, device) -> torch.Tensor:
    """bf16 [len(units), rows, D] key rows 0..rows-1 of the (b, h) units of one layer."""
    lens = seq_lengths(w)
    z = _rows(w, TAG_K, [(layer, b, h) for b, h in units], rows, device)
    cid = torch.from_numpy(np.stack([key_clusters(w, layer, b, h, int(lens[b]))[:rows]
                                     for b, h in units])).to(device)
    ctr = torch.from_numpy(np.stack([centres(w, layer, h) for _, h in units])).to(device)
    return _compose(z, cid, ctr, w.spread)


def values_for(w: Workload, layer: int, units: Sequence[tuple], rows: int, device) -> torch.Tensor:
    """bf16 [len(units), rows, D] value rows (plain noise)."""
    return _rows(w, TAG_V, [(layer, b, h) for b, h in units], rows, device).to(torch.bfloat16)


def queries_for(w: Workload, layer: int, heads: Sequence[tuple], device) -> torch.Tensor:
    """bf16 [len(heads), q_len, D] stored queries of (b, query head) pairs."""
    G = w.group
    z = _rows(w, TAG_QN, [(layer, b, hq) for b, hq in heads], w.q_len, device)
    cid = torch.from_numpy(np.stack([query_clusters(w, layer, b, hq) for b, hq in heads])).to(device)
    ctr = torch.from_numpy(np.stack([centres(w, layer, hq // G) for _, hq in heads])).to(device)
    return _compose(z, cid, ctr, w.spread)


def beacons_for(w: Workload, layer: int, units: Sequence[tuple], device) -> torch.Tensor:
    """bf16 [len(units), nb_max, D] beacon slots (the first nb_init are live)."""
    z = _rows(w, TAG_BC, [(layer, b, h) for b, h in units], w.nb_max, device)
    cid = torch.from_numpy(np.stack([beacon_clusters(w, layer, b, h) for b, h in units])).to(device)
    ctr = torch.from_numpy(np.stack([centres(w, layer, h) for _, h in units])).to(device)
    return _compose(z, cid, ctr, w.spread)


# ----------------------------------------------------------------------------------------------
# whole-layer tensors (device side) and single units (oracle side)
# ----------------------------------------------------------------------------------------------

def _chunks(items: list, per: int):
    for i in range(0, len(items), per):
        yield items[i:i + per]


def layer_tensors(w: Workload, layer: int, device, max_elems: int = 1 << 27) -> Dict[str, torch.Tensor]:
    """All inputs of one layer, laid out as the library expects.

    k, v:      bf16 [B, Hkv, capacity, D]
    q:         bf16 [B, Hq, q_len, D]
    beacons:   bf16 [B, Hkv, nb_max, D]
    n_beacons: int32 [B, Hkv]
    """
    B, Hq, Hkv, D, cap = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.capacity
    k = torch.empty((B, Hkv, cap, D), dtype=torch.bfloat16, device=device)
    v = torch.empty_like(k)
    units = [(b, h) for b in range(B) for h in range(Hkv)]
    per = max(1, max_elems // (cap * D))
    for part in _chunks(units, per):
        b0, h0 = part[0]
        kk = keys_for(w, layer, part, cap, device)
        vv = values_for(w, layer, part, cap, device)
        flat_k = k.view(B * Hkv, cap, D)
        flat_v = v.view(B * Hkv, cap, D)
        s = b0 * Hkv + h0
        flat_k[s:s + len(part)] = kk
        flat_v[s:s + len(part)] = vv
        del kk, vv
    heads = [(b, hq) for b in range(B) for hq in range(Hq)]
    q = queries_for(w, layer, heads, device).view(B, Hq, w.q_len, D)
    bc = beacons_for(w, layer, units, device).view(B, Hkv, w.nb_max, D)
    nb = torch.full((B, Hkv), w.nb_init, dtype=torch.int32, device=device)
    return {"k": k, "v": v, "q": q, "beacons": bc, "n_beacons": nb}


def unit_inputs(w: Workload, layer: int, b: int, h: int, device="cpu") -> Dict[str, object]:
    """Inputs of one unit (layer, sequence b, KV head h), bit-identical to the
    corresponding slices of `layer_tensors`.

    k, v:     bf16 [L, D]   (valid rows only)
    q:        bf16 [G, q_len, D]  (the group's query heads h*G .. h*G+G-1)
    beacons:  bf16 [nb_max, D]
    nb:       int (live beacons before the call)
    L:        int
    """
    G = w.group
    L = int(seq_lengths(w)[b])
    k = keys_for(w, layer, [(b, h)], L, device)[0]
    v = values_for(w, layer, [(b, h)], L, device)[0]
    q = queries_for(w, layer, [(b, h * G + r) for r in range(G)], device)
    bc = beacons_for(w, layer, [(b, h)], device)[0]
    return {"k": k, "v": v, "q": q, "beacons": bc, "nb": w.nb_init, "L": L}


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """uint16 NumPy view of a bf16 tensor's bit patterns (copied to host)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
