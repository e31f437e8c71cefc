"""Pins for the CPU oracle: each test ties it to something other than itself
(a library routine, a closed form, brute force on tiny inputs, an invariant or a
hand-worked fixture), chosen so that a dropped term, wrong sign, wrong index or
transposed operand fails at least one of them.  CPU only."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.spatial.distance import cdist

from oracle import bkv_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (via torch's RNE conversion) and return them as float64."""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def _bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------------------------------------
# input decoding
# ------------------------------------------------------------------------------------------------

def test_bf16_decoding_matches_torch_on_every_bit_pattern():
    """All 65,536 bf16 patterns decode to the value torch's own bf16 -> float64 conversion
    gives (signed zeros, subnormals, infinities and the sign of every value included; NaN
    patterns decode to NaN)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = O.bf16_to_f64(bits)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2 * (2 ** 7 - 1)                  # exponent all ones, mantissa non-zero
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))
    # shape is kept and a few patterns by hand: 1.0, -2.0, smallest subnormal, largest finite
    hand = O.bf16_to_f64(np.array([[0x3F80, 0xC000], [0x0001, 0x7F7F]], dtype=np.uint16))
    assert hand.shape == (2, 2)
    assert hand.tolist() == [[1.0, -2.0], [2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127]]


# ------------------------------------------------------------------------------------------------
# scores
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("n_obs,L,d", [(5, 37, 16), (12, 9, 64), (1, 200, 8)])
def test_probabilities_equal_torch_sdpa(n_obs, L, d):
    """torch's scaled_dot_product_attention with V = I returns the attention matrix itself;
    it applies its own default 1/sqrt(d) scale and softmax over keys."""
    rng = np.random.default_rng(n_obs * 1000 + L)
    q = rng.standard_normal((n_obs, d)) * 2.0
    k = rng.standard_normal((L, d)) * 2.0
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.eye(L, dtype=torch.float64)[None])[0]
    p = O.attention_probabilities(q, k)
    np.testing.assert_allclose(p, ref.numpy(), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(O.max_aggregated_scores(q, k), ref.numpy().max(axis=0), rtol=1e-12, atol=1e-15)


def test_scores_closed_form_fixture():
    g = _golden("scores_orthogonal.json")
    s = O.max_aggregated_scores(np.array(g["queries"], float), np.array(g["keys"], float))
    np.testing.assert_allclose(s, g["scores"], rtol=1e-14)


def test_identical_keys_give_uniform_scores():
    rng = np.random.default_rng(1)
    L = 33
    k = np.repeat(rng.standard_normal((1, 16)), L, axis=0)
    q = rng.standard_normal((7, 16)) * 3
    np.testing.assert_allclose(O.max_aggregated_scores(q, k), np.full(L, 1.0 / L), rtol=1e-13)


def test_one_key_dominates_when_aligned():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 32))
    k = rng.standard_normal((50, 32)) * 0.1
    k[17] = 40.0 * q[0]
    s = O.max_aggregated_scores(q, k)
    assert s[17] > 1 - 1e-12 and np.all(np.delete(s, 17) < 1e-12)


def test_probability_rows_sum_to_one_and_score_bounds():
    rng = np.random.default_rng(3)
    for _ in range(20):
        n, L, d = rng.integers(1, 30), rng.integers(1, 300), rng.choice([8, 64, 128])
        q = rng.standard_normal((n, d)) * rng.uniform(0.1, 4)
        k = rng.standard_normal((L, d)) * rng.uniform(0.1, 4)
        p = O.attention_probabilities(q, k)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)
        s = O.max_aggregated_scores(q, k)
        assert 1.0 - 1e-12 <= s.sum() <= n + 1e-12
        assert np.all(s[None, :] >= p - 1e-300)                      # max dominates every query
        assert np.all(np.isclose(p, s[None, :], rtol=0, atol=0).any(axis=0))  # and is attained


def test_scores_invariant_to_query_order_and_duplicates():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((9, 64))
    k = rng.standard_normal((120, 64)) * 2
    s = O.max_aggregated_scores(q, k)
    np.testing.assert_allclose(O.max_aggregated_scores(q[::-1], k), s, rtol=1e-14)
    np.testing.assert_allclose(O.max_aggregated_scores(np.concatenate([q, q[:3]]), k), s, rtol=1e-14)


def test_scores_follow_key_permutation():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((4, 16))
    k = rng.standard_normal((60, 16))
    perm = rng.permutation(60)
    np.testing.assert_allclose(O.max_aggregated_scores(q, k[perm]), O.max_aggregated_scores(q, k)[perm],
                               rtol=1e-13)


def test_brute_force_scores_pure_python():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((3, 5))
    k = rng.standard_normal((7, 5)) * 1.5
    want = []
    for j in range(7):
        best = 0.0
        for i in range(3):
            lg = [sum(q[i, t] * k[jj, t] for t in range(5)) / math.sqrt(5) for jj in range(7)]
            z = math.fsum(math.exp(x) for x in lg)
            best = max(best, math.exp(lg[j]) / z)
        want.append(best)
    np.testing.assert_allclose(O.max_aggregated_scores(q, k), want, rtol=1e-13)


def test_single_observer_selection_is_argsort_of_logits():
    """One observation query, no window: the kept set is the budget highest logits
    (softmax is monotone), i.e. a stable argsort of the negated logits."""
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 32))
    k = rng.standard_normal((300, 32))
    s = O.max_aggregated_scores(q, k)
    keep = O.select_keep(s, 300, 40, 0)
    logits = k @ q[0]
    np.testing.assert_array_equal(keep, np.sort(np.argsort(-logits, kind="stable")[:40]))


# ------------------------------------------------------------------------------------------------
# observation set
# ------------------------------------------------------------------------------------------------

def test_observation_set_uses_tail_window_then_live_beacons():
    rng = np.random.default_rng(8)
    G, q_len, W, D = 3, 10, 4, 8
    qg = rng.standard_normal((G, q_len, D))
    bc = rng.standard_normal((6, D))
    obs = O.observation_queries(qg, W, bc, 2)
    assert obs.shape == (G * W + 2, D)
    np.testing.assert_array_equal(obs[:W], qg[0, q_len - W:])
    np.testing.assert_array_equal(obs[W:2 * W], qg[1, q_len - W:])
    np.testing.assert_array_equal(obs[G * W:], bc[:2])


def test_old_queries_do_not_affect_scores_but_window_queries_do():
    rng = np.random.default_rng(9)
    G, q_len, W, D, L = 2, 12, 3, 16, 80
    qg = rng.standard_normal((G, q_len, D)) * 2
    bc = rng.standard_normal((4, D))
    k = rng.standard_normal((L, D)) * 2
    s0 = O.max_aggregated_scores(O.observation_queries(qg, W, bc, 4), k)
    q2 = qg.copy()
    q2[:, : q_len - W] = rng.standard_normal((G, q_len - W, D)) * 5
    np.testing.assert_array_equal(O.max_aggregated_scores(O.observation_queries(q2, W, bc, 4), k), s0)
    q3 = qg.copy()
    q3[1, q_len - 1] = rng.standard_normal(D) * 5
    assert not np.allclose(O.max_aggregated_scores(O.observation_queries(q3, W, bc, 4), k), s0)
    bc2 = bc.copy()
    bc2[3] = rng.standard_normal(D) * 5     # beacon beyond the live count: ignored
    np.testing.assert_array_equal(O.max_aggregated_scores(O.observation_queries(qg, W, bc2, 3), k),
                                  O.max_aggregated_scores(O.observation_queries(qg, W, bc, 3), k))


def test_splitting_queries_across_heads_is_metamorphic():
    rng = np.random.default_rng(10)
    D, L = 16, 50
    k = rng.standard_normal((L, D))
    flat = rng.standard_normal((6, D))
    one_head = O.observation_queries(flat[None], 6, np.zeros((0, D)), 0)
    three_heads = O.observation_queries(flat.reshape(3, 2, D), 2, np.zeros((0, D)), 0)
    np.testing.assert_array_equal(O.max_aggregated_scores(one_head, k), O.max_aggregated_scores(three_heads, k))


def test_recent_only_special_case():
    """G = 1 with no beacons is recent-query-only scoring (Figure 5 (a)): the scores are the
    max over that head's window rows alone."""
    rng = np.random.default_rng(11)
    qg = rng.standard_normal((1, 5, 8))
    k = rng.standard_normal((30, 8))
    got = O.max_aggregated_scores(O.observation_queries(qg, 5, np.zeros((2, 8)), 0), k)
    p = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(qg), torch.from_numpy(k)[None],
                                                         torch.eye(30, dtype=torch.float64)[None])[0]
    np.testing.assert_allclose(got, p.numpy().max(axis=0), rtol=1e-12)


# ------------------------------------------------------------------------------------------------
# selection
# ------------------------------------------------------------------------------------------------

def test_topk_fixture():
    g = _golden("topk_ties.json")
    s = np.array(g["scores"])
    for c in g["cases"]:
        np.testing.assert_array_equal(O.select_keep(s, len(s), c["budget"], c["window"]), c["keep"])


@pytest.mark.parametrize("seed", range(12))
def test_topk_equals_best_subset_by_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    L = int(rng.integers(1, 12))
    budget = int(rng.integers(1, 10))
    window = int(rng.integers(0, budget + 1))
    s = rng.random(L)                     # distinct with probability 1
    keep = O.select_keep(s, L, budget, window)
    if L <= budget:
        np.testing.assert_array_equal(keep, np.arange(L))
        return
    prefix = L - window
    best, best_set = -1.0, None
    for sub in itertools.combinations(range(prefix), budget - window):
        tot = sum(s[j] for j in sub)
        if tot > best:
            best, best_set = tot, sub
    np.testing.assert_array_equal(keep, sorted(list(best_set) + list(range(prefix, L))))


def test_topk_invariants_and_uniform_ties():
    rng = np.random.default_rng(12)
    for _ in range(50):
        L = int(rng.integers(0, 400))
        budget = int(rng.integers(1, 300))
        window = int(rng.integers(0, budget + 1))
        s = np.round(rng.random(L), 2)          # many exact ties
        keep = O.select_keep(s, L, budget, window)
        assert keep.size == min(budget, L)
        assert np.all(np.diff(keep) > 0)
        if L > budget:
            assert set(range(L - window, L)) <= set(keep.tolist())
            # every evicted prefix key scores no better than every kept prefix key
            kept_prefix = [j for j in keep if j < L - window]
            evicted = sorted(set(range(L - window)) - set(kept_prefix))
            if kept_prefix and evicted:
                assert s[kept_prefix].min() >= s[evicted].max()
                # among equal scores at the threshold, the lower positions are kept
                thr = s[kept_prefix].min()
                eq_kept = [j for j in kept_prefix if s[j] == thr]
                eq_evicted = [j for j in evicted if s[j] == thr]
                if eq_evicted:
                    assert max(eq_kept) < min(eq_evicted)
    flat = O.select_keep(np.full(100, 0.5), 100, 10, 3)
    np.testing.assert_array_equal(flat, list(range(7)) + [97, 98, 99])


def test_topk_permutation_metamorphic():
    rng = np.random.default_rng(13)
    L, budget, window = 200, 50, 8
    s = rng.random(L)
    perm = np.concatenate([rng.permutation(L - window), np.arange(L - window, L)])
    keep = O.select_keep(s, L, budget, window)
    keep_p = O.select_keep(s[perm], L, budget, window)
    np.testing.assert_array_equal(np.sort(perm[keep_p]), keep)


def test_compaction_identity_and_gather():
    rng = np.random.default_rng(14)
    bits = rng.integers(0, 1 << 16, size=(40, 8), dtype=np.uint16)
    np.testing.assert_array_equal(O.compact_rows(bits, np.arange(40)), bits)
    keep = np.array([0, 3, 39])
    out = O.compact_rows(bits, keep)
    for r, j in enumerate(keep):
        assert out[r].tobytes() == bits[j].tobytes()


# ------------------------------------------------------------------------------------------------
# farthest-point sampling
# ------------------------------------------------------------------------------------------------

def _plane_points(angles_deg, d):
    pts = np.zeros((len(angles_deg), d))
    for i, a in enumerate(angles_deg):
        pts[i, 0] = math.cos(math.radians(a))
        pts[i, 1] = math.sin(math.radians(a))
    return _bf16_round(pts)


@pytest.mark.parametrize("name", ["fps_circle.json", "fps_square_tie.json"])
def test_fps_fixtures(name):
    g = _golden(name)
    pts = _plane_points(g["angles_deg"], g["head_dim"])
    picks = O.farthest_point_picks(pts, g["n_pick"])
    np.testing.assert_array_equal(picks, g["picks"])
    if "covering_radii" in g:
        radii = [cdist(pts, pts[picks[:t]], "cosine").min(axis=1).max() for t in range(1, g["n_pick"])]
        np.testing.assert_allclose(radii, g["covering_radii"], atol=2e-3)


@pytest.mark.parametrize("seed", range(8))
def test_fps_each_pick_is_farthest_by_scipy_cosine(seed):
    """Definition check with scipy's cosine distance (1 - u.v/(|u||v|))."""
    rng = np.random.default_rng(200 + seed)
    P, d, n = int(rng.integers(5, 80)), int(rng.choice([4, 16, 64])), int(rng.integers(1, 12))
    pool = rng.standard_normal((P, d)) * rng.uniform(0.5, 3, size=(P, 1))
    picks = O.farthest_point_picks(pool, n)
    if P <= n:
        np.testing.assert_array_equal(picks, np.arange(P))
        return
    assert picks[0] == 0 and len(set(picks.tolist())) == n
    D = cdist(pool, pool, "cosine")
    radii = []
    for t in range(1, n):
        mind = D[:, picks[:t]].min(axis=1)
        mind[picks[:t]] = -np.inf
        best = mind.max()
        radii.append(best)
        assert mind[picks[t]] >= best - 1e-12
        assert picks[t] == np.flatnonzero(mind >= best - 1e-12)[0]
    assert all(a >= b - 1e-12 for a, b in zip(radii, radii[1:]))   # covering radius never grows


def test_fps_orthonormal_pool_takes_index_order():
    d = 16
    pool = np.eye(d)[:10] * np.arange(1, 11)[:, None]    # scaling must not matter
    np.testing.assert_array_equal(O.farthest_point_picks(pool, 6), np.arange(6))


def test_fps_antipode_is_second():
    rng = np.random.default_rng(15)
    x = rng.standard_normal(32)
    pool = np.stack([x, rng.standard_normal(32), -2.0 * x, rng.standard_normal(32)])
    assert O.farthest_point_picks(pool, 2).tolist() == [0, 2]


@pytest.mark.parametrize("seed", range(6))
def test_fps_gonzalez_two_approximation(seed):
    """Greedy FPS is a 2-approximation of the optimal k-center radius in a metric; on unit
    vectors the chord distance sqrt(2 (1 - cos)) is one, and FPS picks are unchanged by
    that monotone transform."""
    rng = np.random.default_rng(300 + seed)
    P, k = int(rng.integers(6, 12)), int(rng.integers(2, 5))
    pool = rng.standard_normal((P, 6))
    chord = np.sqrt(np.maximum(2.0 * cdist(pool, pool, "cosine"), 0.0))
    picks = O.farthest_point_picks(pool, k)
    greedy = chord[:, picks].min(axis=1).max()
    opt = min(chord[:, list(c)].min(axis=1).max() for c in itertools.combinations(range(P), k))
    assert greedy <= 2.0 * opt + 1e-12


def test_beacon_pool_order_and_update():
    D = 8
    bc = _bits(np.arange(5 * D).reshape(5, D) + 1.0)
    qn = _bits(-np.arange(2 * 3 * D).reshape(2, 3, D) - 1.0)
    pool = O.beacon_pool(bc, 2, qn)
    assert pool.shape == (2 + 6, D)
    np.testing.assert_array_equal(pool[:2], bc[:2])
    np.testing.assert_array_equal(pool[2:5], qn[0])
    np.testing.assert_array_equal(pool[5:], qn[1])
    out, n, picks = O.update_beacons(bc, 2, qn, 16)       # pool smaller than capacity: keep all
    assert n == 8 and picks.tolist() == list(range(8))
    np.testing.assert_array_equal(out, pool)
    out, n, picks = O.update_beacons(bc, 2, qn, 3)
    assert n == 3 and picks[0] == 0
    np.testing.assert_array_equal(out, pool[picks])


def test_compress_unit_window_and_count():
    rng = np.random.default_rng(16)
    L, D = 300, 16
    k = _bits(rng.standard_normal((L, D)))
    v = _bits(rng.standard_normal((L, D)))
    q = _bits(rng.standard_normal((2, 4, D)))
    bc = _bits(rng.standard_normal((3, D)))
    r = O.compress_unit(k, v, q, bc, 3, 4, 64)
    assert r["keep"].size == 64 and set(range(296, 300)) <= set(r["keep"].tolist())
    np.testing.assert_array_equal(r["k_out"], k[r["keep"]])
    np.testing.assert_array_equal(r["v_out"], v[r["keep"]])


# ------------------------------------------------------------------------------------------------
# mean aggregation (Table 2)
# ------------------------------------------------------------------------------------------------

def test_mean_scores_closed_form_fixture():
    g = _golden("scores_orthogonal_mean.json")
    s = O.mean_aggregated_scores(np.array(g["queries"], float), np.array(g["keys"], float))
    np.testing.assert_allclose(s, g["scores"], rtol=1e-14)


@pytest.mark.parametrize("n_obs,L,d", [(1, 7, 8), (5, 64, 32), (13, 200, 128)])
def test_mean_scores_equal_torch_sdpa_column_mean(n_obs, L, d):
    rng = np.random.default_rng(n_obs * 7 + L)
    q = rng.standard_normal((n_obs, d)) * 2.0
    k = rng.standard_normal((L, d)) * 2.0
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.eye(L, dtype=torch.float64)[None])[0]
    np.testing.assert_allclose(O.mean_aggregated_scores(q, k), ref.numpy().mean(axis=0), rtol=1e-12, atol=1e-15)


def test_mean_scores_sum_to_one_and_sit_between_max_over_n_and_max():
    rng = np.random.default_rng(31)
    for _ in range(20):
        n, L, d = rng.integers(1, 30), rng.integers(1, 300), rng.choice([8, 64, 128])
        q = rng.standard_normal((n, d)) * rng.uniform(0.1, 4)
        k = rng.standard_normal((L, d)) * rng.uniform(0.1, 4)
        m = O.mean_aggregated_scores(q, k)
        x = O.max_aggregated_scores(q, k)
        np.testing.assert_allclose(m.sum(), 1.0, atol=1e-12)
        assert np.all(m <= x * (1 + 1e-12)) and np.all(m >= x / n * (1 - 1e-12))


def test_mean_equals_max_for_one_observer_and_zero_for_none():
    rng = np.random.default_rng(32)
    q = rng.standard_normal((1, 16))
    k = rng.standard_normal((40, 16))
    np.testing.assert_allclose(O.mean_aggregated_scores(q, k), O.max_aggregated_scores(q, k), rtol=1e-14)
    np.testing.assert_array_equal(O.mean_aggregated_scores(q[:0], k), np.zeros(40))


def test_mean_brute_force_pure_python():
    rng = np.random.default_rng(33)
    q = rng.standard_normal((4, 6))
    k = rng.standard_normal((9, 6)) * 1.5
    want = []
    for j in range(9):
        tot = 0.0
        for i in range(4):
            lg = [sum(q[i, t] * k[jj, t] for t in range(6)) / math.sqrt(6) for jj in range(9)]
            tot += math.exp(lg[j]) / math.fsum(math.exp(x) for x in lg)
        want.append(tot / 4)
    np.testing.assert_allclose(O.mean_aggregated_scores(q, k), want, rtol=1e-13)
    np.testing.assert_allclose(O.aggregated_scores(q, k, "mean"), want, rtol=1e-13)
    with pytest.raises(ValueError):
        O.aggregated_scores(q, k, "median")


# ------------------------------------------------------------------------------------------------
# Initial+Recent beacon policy (Table 3's baseline)
# ------------------------------------------------------------------------------------------------

def _rand_bits(rng, shape):
    return rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)


def test_initial_beacons_take_earliest_queries_by_time_then_head():
    """The new rows are the queries with the smallest (step, head) in lexicographic order."""
    rng = np.random.default_rng(40)
    G, T, D, nb_max = 3, 5, 4, 9
    old = _rand_bits(rng, (nb_max, D))
    q = _rand_bits(rng, (G, T, D))
    for n_in in (0, 2, 9):
        rows, n = O.initial_beacons(old, n_in, q, nb_max)
        assert n == min(nb_max, n_in + G * T)
        assert rows[:n_in].tobytes() == old[:n_in].tobytes()
        heads, steps = np.meshgrid(np.arange(G), np.arange(T), indexing="ij")
        order = np.lexsort((heads.ravel(), steps.ravel()))[: n - n_in]   # by step, then head
        want = q.reshape(G * T, D)[order]
        assert rows[n_in:].tobytes() == want.tobytes()


def test_initial_beacons_frozen_once_full():
    rng = np.random.default_rng(41)
    G, T, D, nb_max = 4, 8, 6, 16
    old = _rand_bits(rng, (nb_max, D))
    rows, n = O.initial_beacons(old, 0, _rand_bits(rng, (G, T, D)), nb_max)
    assert n == nb_max
    again, n2 = O.initial_beacons(rows, n, _rand_bits(rng, (G, T, D)), nb_max)
    assert n2 == nb_max and again.tobytes() == rows.tobytes()


def test_initial_and_fps_keep_the_same_set_when_everything_fits():
    """With no more candidates than slots both policies keep every candidate (FPS in pool
    order, the initial policy in time order): the same set of rows."""
    rng = np.random.default_rng(42)
    G, T, D, nb_max = 2, 3, 8, 10
    old = _rand_bits(rng, (nb_max, D)) & 0x3FFF        # finite, non-zero bf16 patterns
    q = (_rand_bits(rng, (G, T, D)) & 0x3FFF) | 0x0080
    a, na = O.initial_beacons(old, 3, q, nb_max)
    b, nb, _ = O.update_beacons(old, 3, q, nb_max)
    assert na == nb == 3 + G * T
    assert sorted(r.tobytes() for r in a) == sorted(r.tobytes() for r in b)


# ------------------------------------------------------------------------------------------------
# decoding over the compacted cache
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("n_q,L,d", [(1, 5, 8), (4, 300, 64), (7, 1000, 128)])
def test_decode_attention_equals_torch_sdpa(n_q, L, d):
    rng = np.random.default_rng(n_q * 31 + L)
    q = rng.standard_normal((n_q, d)) * 1.5
    k = rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q)[None], torch.from_numpy(k)[None],
                                                           torch.from_numpy(v)[None])[0]
    np.testing.assert_allclose(O.decode_attention(q, k, v), ref.numpy(), rtol=1e-12, atol=1e-13)


def test_decode_attention_special_cases():
    rng = np.random.default_rng(50)
    d = 16
    v = rng.standard_normal((9, d))
    k_same = np.repeat(rng.standard_normal((1, d)), 9, axis=0)
    q = rng.standard_normal((3, d))
    np.testing.assert_allclose(O.decode_attention(q, k_same, v), np.repeat(v.mean(0, keepdims=True), 3, 0),
                               rtol=1e-13, atol=1e-14)          # equal keys: plain mean of the values
    k = rng.standard_normal((9, d)) * 0.01
    k[4] = 60.0 * q[0]
    np.testing.assert_allclose(O.decode_attention(q[:1], k, v)[0], v[4], atol=1e-9)   # one key dominates
    assert np.array_equal(O.decode_attention(q, k[:0], v[:0]), np.zeros((3, d)))


def test_decode_attention_brute_force():
    rng = np.random.default_rng(51)
    q = rng.standard_normal((2, 4))
    k = rng.standard_normal((5, 4))
    v = rng.standard_normal((5, 3))
    for i in range(2):
        lg = [sum(q[i, t] * k[j, t] for t in range(4)) / 2.0 for j in range(5)]
        z = math.fsum(math.exp(x) for x in lg)
        want = [math.fsum(math.exp(lg[j]) / z * v[j, c] for j in range(5)) for c in range(3)]
        np.testing.assert_allclose(O.decode_attention(q, k, v)[i], want, rtol=1e-13)
