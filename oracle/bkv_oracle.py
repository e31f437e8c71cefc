"""Plain, slow CPU oracle for beacon-guided KV-cache compression (float64, NumPy).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call this
module: only the test suite, the graft smoke check and the CPU-baseline leg of the
benchmark use it.  It shares no code with the GPU library (no kernels, headers,
tables or helpers); the only thing both sides consume is the seeded input
generator in `synth/`, which holds none of this arithmetic.

Source: "BeaconKV: Key-Value Cache Compression Guided by Beacon Queries for
Efficient Large Reasoning Model Inference" (thelatestinai.com/papers/2609.04971).
What the page fixes, and where:

* Abstract - beacon queries are compact representatives of the global query
  clusters, kept without storing the whole query history; compression evicts KV
  pairs to bound the cache.
* Figure 5 (b) - eviction scores are attention-based scores computed from beacon
  queries together with the recent queries; (c) - the kept set is a top-K under
  max aggregation of those scores.
* Table 2 caption - the aggregation is applied consistently across heads and
  queries (max over both).
* Figure 7 caption - beacons are maintained by "Continual FPS" (farthest-point
  sampling that keeps running over new queries rather than the whole history).
* Figure 4 (a) / Figure 6 (a) - query similarity is cosine similarity.

The page prints no equations, listings or worked numbers.  Where it is silent the
oracle takes the plainest reading, each one named at the function that uses it:
softmax over the unit's valid keys with scale 1/sqrt(d) and no causal mask; the
window W both supplies each query head's last W queries and is always kept on the
key side; the budget counts the window; ties in the top-K go to the lower
position; FPS starts from pool index 0, breaks ties to the lower pool index and
uses cosine distance 1 - cos.

Every floating-point step runs in float64 on exact float64 copies of the bf16
inputs.  Row copies (beacons, compacted K/V) operate on the raw 16-bit patterns.
"""
from __future__ import annotations

import math
from typing import Dict, Tuple

import numpy as np

__all__ = [
    "bf16_to_f64", "observation_queries", "attention_probabilities", "max_aggregated_scores",
    "select_keep", "compact_rows", "cosine_distance_to", "farthest_point_picks",
    "beacon_pool", "update_beacons", "compress_unit",
]

NORM_FLOOR = 1e-30


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 values of bf16 bit patterns (uint16 array of any shape)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------------------------
# Observation set (Figure 5 (b))
# ---------------------------------------------------------------------------------------------

def observation_queries(q_group: np.ndarray, window: int, beacons: np.ndarray, n_beacons: int) -> np.ndarray:
    """Queries that score the keys of one KV head.

    q_group: [G, q_len, D] stored queries of the G query heads sharing the KV head
             (the newest query is the last row); beacons: [nb_max, D]; only the
             first n_beacons rows are live.
    Returns [G*window + n_beacons, D]: each head's last `window` queries (head-major,
    time order), then the live beacons in stored order.  Figure 5 (b) scores with
    beacon queries and recent queries; grouping the G heads that read the same KV
    head follows from one index set per KV head (the reading that K and V of a KV
    head are compacted identically).
    """
    G, q_len, D = q_group.shape
    if window > q_len:
        raise ValueError("window exceeds stored queries")
    recent = q_group[:, q_len - window:, :].reshape(G * window, D)
    return np.concatenate([recent, beacons[:n_beacons]], axis=0)


# ---------------------------------------------------------------------------------------------
# Scores (Figure 5 (b), (c); Table 2)
# ---------------------------------------------------------------------------------------------

def attention_probabilities(obs: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """Softmax attention weights [n_obs, L] of each observation query over the keys.

    Reading of "attention-based scores" (Figure 5): the standard scaled dot-product
    attention weight, exp(q.k / sqrt(d)) normalised over all L valid keys of the
    unit, with no causal mask (beacons have no position; window queries see every
    cached key).  The normaliser is a log-sum-exp with the row maximum removed.
    """
    d = keys.shape[1]
    logits = (obs @ keys.T) / math.sqrt(d)
    m = logits.max(axis=1, keepdims=True)
    lse = m + np.log(np.exp(logits - m).sum(axis=1, keepdims=True))
    return np.exp(logits - lse)


def max_aggregated_scores(obs: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """Per-key score [L]: the largest attention weight any observation query gives it.

    Figure 5 (c) selects with max aggregation; the Table 2 caption applies it over
    heads and queries alike, so the max runs over every query of the GQA group and
    every beacon of the KV head.
    """
    if keys.shape[0] == 0 or obs.shape[0] == 0:
        return np.zeros(keys.shape[0])     # no keys, or nobody observing: every score is 0
    return attention_probabilities(obs, keys).max(axis=0)


def mean_aggregated_scores(obs: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """Per-key score [L]: the mean attention weight over the observation queries.

    Table 2 compares max aggregation with mean aggregation, each applied the same way
    across heads and queries; the mean therefore runs over the same rows as the max
    (every query of the GQA group and every beacon of the KV head).  An empty
    observation set gives every key 0, as for the max.
    """
    if keys.shape[0] == 0 or obs.shape[0] == 0:
        return np.zeros(keys.shape[0])
    return attention_probabilities(obs, keys).mean(axis=0)


def aggregated_scores(obs: np.ndarray, keys: np.ndarray, aggregation: str = "max") -> np.ndarray:
    """Max (Figure 5 (c)) or mean (Table 2) aggregated scores."""
    if aggregation == "max":
        return max_aggregated_scores(obs, keys)
    if aggregation == "mean":
        return mean_aggregated_scores(obs, keys)
    raise ValueError(f"unknown aggregation {aggregation!r}")


# ---------------------------------------------------------------------------------------------
# Selection (Figure 5 (c)) and eviction (Abstract)
# ---------------------------------------------------------------------------------------------

def select_keep(scores: np.ndarray, L: int, budget: int, window: int) -> np.ndarray:
    """Ascending kept positions under the budget.

    If L <= budget nothing is evicted.  Otherwise the last `window` positions are
    always kept and the remaining budget - window slots go to the highest-scoring
    earlier positions; equal scores go to the lower position.  The kept count is
    min(budget, L).
    """
    if window < 0 or window > budget:
        raise ValueError("need 0 <= window <= budget")
    if L <= budget:
        return np.arange(L, dtype=np.int64)
    prefix = L - window
    s = np.asarray(scores[:prefix], dtype=np.float64)
    pos = np.arange(prefix)
    order = np.lexsort((pos, -s))          # primary: score descending; secondary: position
    top = order[: budget - window]
    kept = np.concatenate([top, np.arange(prefix, L)])
    return np.sort(kept).astype(np.int64)


def compact_rows(rows_bits: np.ndarray, keep: np.ndarray) -> np.ndarray:
    """Kept rows (bit copies) in ascending position order."""
    return rows_bits[keep]


# ---------------------------------------------------------------------------------------------
# Beacon maintenance: continual farthest-point sampling on cosine distance (Figure 7)
# ---------------------------------------------------------------------------------------------

def cosine_distance_to(pool: np.ndarray, j: int) -> np.ndarray:
    """1 - cos(x_p, x_j) for every pool row p, clamped to [0, 2] (Figure 4 (a) measures
    query similarity by cosine).  Norms below 1e-30 are floored."""
    norms = np.maximum(np.linalg.norm(pool, axis=1), NORM_FLOOR)
    unit = pool / norms[:, None]
    return np.clip(1.0 - unit @ unit[j], 0.0, 2.0)


def farthest_point_picks(pool: np.ndarray, n_pick: int) -> np.ndarray:
    """Greedy farthest-point sampling: pool indices in pick order.

    Start at pool index 0; each next pick is the not-yet-picked row whose distance
    to its nearest picked row is largest (ties to the lower index).  With no more
    rows than picks, every row is taken in pool order.
    """
    P = pool.shape[0]
    if P <= n_pick:
        return np.arange(P, dtype=np.int64)
    picks = [0]
    nearest = cosine_distance_to(pool, 0)
    taken = np.zeros(P, dtype=bool)
    taken[0] = True
    while len(picks) < n_pick:
        cand = np.where(taken, -np.inf, nearest)
        j = int(np.argmax(cand))            # first maximum = lowest index
        picks.append(j)
        taken[j] = True
        nearest = np.minimum(nearest, cosine_distance_to(pool, j))
    return np.asarray(picks, dtype=np.int64)


def beacon_pool(beacons_bits: np.ndarray, n_in: int, q_new_bits: np.ndarray) -> np.ndarray:
    """Candidate rows (bit patterns) for the continual update: the live beacons in stored
    order, then the new queries of the group's heads, head-major and in time order.
    Continuing from the previous beacons instead of the full history is what the
    Abstract and Figure 7 distinguish from naive FPS."""
    G, T, D = q_new_bits.shape
    return np.concatenate([beacons_bits[:n_in], q_new_bits.reshape(G * T, D)], axis=0)


def update_beacons(beacons_bits: np.ndarray, n_in: int, q_new_bits: np.ndarray,
                   nb_max: int) -> Tuple[np.ndarray, int, np.ndarray]:
    """Continual FPS step for one KV head.

    Returns (new beacon rows [n_out, D] as bit patterns in pick order, n_out, the pool
    indices picked).  n_out = min(nb_max, pool size).
    """
    n_in = max(0, min(int(n_in), nb_max))
    pool_bits = beacon_pool(beacons_bits, n_in, q_new_bits)
    picks = farthest_point_picks(bf16_to_f64(pool_bits), nb_max)
    return pool_bits[picks], int(picks.size), picks


def initial_beacons(beacons_bits: np.ndarray, n_in: int, q_new_bits: np.ndarray,
                    nb_max: int) -> Tuple[np.ndarray, int]:
    """Initial+Recent observation set (Table 3's baseline): the beacon slots hold the
    earliest queries seen and never change once full.

    Reading: "initial" queries are the first ones in time; the live rows stay in place
    and the new queries of the group take the free slots in time order, all heads of a
    step (head order) before the next step.  Returns (rows [n_out, D] as bit patterns,
    n_out) with n_out = min(nb_max, n_in + G * T).
    """
    n_in = max(0, min(int(n_in), nb_max))
    G, T, D = q_new_bits.shape
    rows = [beacons_bits[p] for p in range(n_in)]
    for t in range(T):
        for r in range(G):
            if len(rows) < nb_max:
                rows.append(q_new_bits[r, t])
    out = np.array(rows, dtype=beacons_bits.dtype).reshape(len(rows), beacons_bits.shape[1])
    return out, len(rows)


# ---------------------------------------------------------------------------------------------
# Decoding over the (compacted) cache (Abstract; Table 4)
# ---------------------------------------------------------------------------------------------

def decode_attention(q: np.ndarray, keys: np.ndarray, values: np.ndarray) -> np.ndarray:
    """One decoding step of attention for the query heads of one KV head: [n_q, D] outputs,
    each the softmax(q.k / sqrt(d))-weighted sum of the value rows.  With no rows the
    output is 0.  The compressed cache exists to be read this way: decoding attends over
    the kept KV pairs only."""
    if keys.shape[0] == 0:
        return np.zeros((q.shape[0], values.shape[1]))
    return attention_probabilities(q, keys) @ values


# ---------------------------------------------------------------------------------------------
# One unit end to end
# ---------------------------------------------------------------------------------------------

def compress_unit(k_bits: np.ndarray, v_bits: np.ndarray, q_bits: np.ndarray, beacons_bits: np.ndarray,
                  n_beacons: int, window: int, budget: int) -> Dict[str, np.ndarray]:
    """Scores, kept positions and compacted rows for one (layer, sequence, KV head).

    k_bits, v_bits: [L, D] uint16; q_bits: [G, q_len, D]; beacons_bits: [nb_max, D].
    """
    L = k_bits.shape[0]
    obs = observation_queries(bf16_to_f64(q_bits), window, bf16_to_f64(beacons_bits),
                              max(0, min(int(n_beacons), beacons_bits.shape[0])))
    scores = max_aggregated_scores(obs, bf16_to_f64(k_bits))
    keep = select_keep(scores, L, budget, window)
    return {"scores": scores, "keep": keep, "k_out": compact_rows(k_bits, keep),
            "v_out": compact_rows(v_bits, keep)}
