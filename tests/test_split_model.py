"""Host-side model of the scorer's static work split (the arithmetic of the Split struct in
csrc/score_common.h and of the launcher in csrc/score.hip), checked on random shapes: every
share is non-empty and contiguous, the owner of a tile is the workgroup whose share holds
it, and no unit is met by more stats workgroups than the statistics slots the library
sizes its workspace for (read back through bkv_score_workspace_bytes).  A unit met by more
would lose a partial (the kernels then give it NaN scores; the library refuses any launch
whose closed-form bound, stats_span_bound in csrc/bkv_internal.h, exceeds the slots).  The
bound is checked here against the exact spans as well.  CPU only."""
import ctypes
import random

import pytest

from attention_guided_eviction_amd import bkv

TILE, MAX_GRID = 256, 1024
WEIGHTS = {"balanced": (3, 2), "default": (9, 7)}   # stats weights the launcher chooses from


class Split:
    """Shares of N tiles over G workgroups: the first H = G/2 weigh A, the rest B."""

    def __init__(self, N, G, A, B):
        self.N, self.G, self.H, self.A, self.B = N, G, G // 2, A, B

    def cum(self, w):
        return self.A * w if w <= self.H else self.A * self.H + self.B * (w - self.H)

    def begin(self, w):
        return self.cum(w) * self.N // self.cum(self.G)

    def owner(self, c):
        x = ((c + 1) * self.cum(self.G) + self.N - 1) // self.N - 1
        w = x // self.A if x < self.A * self.H else self.H + (x - self.A * self.H) // self.B
        return min(w, self.G - 1)


def stats_split(N, grid, paired, weights):
    G = min(grid, N)
    weighted = paired and G == grid and G % 2 == 0 and N >= 2 * G
    A, B = weights if weighted else (1, 1)
    return Split(N, G, A, B)


def span_bound(capacity, n_layers, n_kv_heads, grid, A, B):
    """Closed-form most workgroups meeting one unit (stats_span_bound in the library)."""
    u = n_layers * n_kv_heads
    c = A * (grid // 2) + B * (grid - grid // 2)
    return min(-(-c // (u * B)) + 1, -(-capacity // TILE), grid)


def library_slots(n_layers, batch, n_kv_heads, capacity, obs_pad):
    """Statistics slots per unit, read back from the workspace size (one launch)."""
    seq = (ctypes.c_int32 * 1)()
    s = bkv._Shape(n_layers, batch, 8 * n_kv_heads, n_kv_heads, 128, capacity, ctypes.addressof(seq))
    window = obs_pad // 8          # G = 8: 8 * window observation rows, no beacons
    nbytes = bkv.load().bkv_score_workspace_bytes(ctypes.byref(s), window, 0)
    per_slot = 2 * n_layers * batch * n_kv_heads * obs_pad * 4
    assert per_slot >= 512          # the 256-byte alignment adds less than one slot
    return nbytes // per_slot


def _check_random_shapes(seed):
    """Largest (span - slots) over 60 random shapes; asserts every split property."""
    rng = random.Random(seed)
    worst = -(1 << 30)
    for _ in range(60):
        n_layers = rng.choice([1, 2, 3, 7, 28, 36, 48])
        batch = rng.choice([1, 2, 3, 5, 8, 64])
        hkv = rng.choice([1, 2, 4, 8])
        cap = rng.choice([256, 257, 1000, 4096, 16384, 65536])
        if n_layers * batch * hkv * ((cap + TILE - 1) // TILE) > 2_000_000:
            continue
        lens = [rng.choice([0, 1, cap, rng.randint(0, cap), cap + 9, -3]) for _ in range(batch)]
        nt = [(min(max(l, 0), cap) + TILE - 1) // TILE for l in lens]
        N = n_layers * hkv * sum(nt)
        if N == 0:
            continue
        slots = library_slots(n_layers, batch, hkv, cap, 256)
        grid = rng.choice([256, 512, MAX_GRID, 250, 7])
        paired = rng.random() < 0.8
        sp = stats_split(N, grid, paired, rng.choice(list(WEIGHTS.values())))
        b = [sp.begin(w) for w in range(sp.G + 1)]
        assert b[0] == 0 and b[-1] == N and all(b[w + 1] > b[w] for w in range(sp.G))
        for c in rng.sample(range(N), min(N, 300)) + [0, N - 1]:
            w = sp.owner(c)
            assert b[w] <= c < b[w + 1]
        c = 0
        for _layer in range(n_layers):
            for bb in range(batch):
                for _h in range(hkv):
                    if nt[bb]:
                        span = sp.owner(c + nt[bb] - 1) - sp.owner(c) + 1
                        assert span <= slots, (span, slots, n_layers, batch, hkv, cap, lens, grid)
                        assert span <= span_bound(cap, n_layers, hkv, grid, sp.A, sp.B) <= slots
                        worst = max(worst, span - slots)
                        c += nt[bb]
        assert c == N
    return worst


def test_stats_split_fits_the_slots():
    worst = max(_check_random_shapes(seed) for seed in range(6))
    # some unit is met by exactly as many workgroups as there are slots: one slot fewer in
    # the library's sizing would lose partials on these shapes
    assert worst == 0


def _worst_span(n_layers, tiles_per_seq, hkv, grid, weights):
    N = n_layers * hkv * sum(tiles_per_seq)
    sp = stats_split(N, grid, True, weights)
    c, worst = 0, 0
    for _l in range(n_layers):
        for nt in tiles_per_seq:
            for _h in range(hkv):
                if nt:
                    worst = max(worst, sp.owner(c + nt - 1) - sp.owner(c) + 1)
                    c += nt
    return worst


@pytest.mark.parametrize("n_layers,hkv", [(1, 1), (1, 3), (1, 7), (3, 1), (1, 11), (2, 3)])
def test_few_units_with_long_caches(n_layers, hkv):
    """Few (layer, KV head) units and caches longer than the slot count (where the tile cap
    does not help): one short sequence ahead of a long one shifts the long units' start
    across the shares.  The bound holds, and the sweep comes within one workgroup of it."""
    u = n_layers * hkv
    gap = 1 << 30
    for weights in WEIGHTS.values():
        for tiles in range(1300, 1460, 7):
            cap = tiles * TILE
            slots = library_slots(n_layers, 1, hkv, cap, 256)
            for pre in (0, 1, 2, 3, 5, 8, 13, 21):
                lens = ([pre] if pre else []) + [tiles]
                worst = _worst_span(n_layers, lens, hkv, MAX_GRID, weights)
                bound = span_bound(cap, n_layers, hkv, MAX_GRID, *weights)
                assert worst <= bound <= slots, (worst, bound, slots, tiles, pre, weights)
                gap = min(gap, bound - worst)
    assert gap <= 1 or u == 1   # a single unit meets at most the grid, below the slots
