"""Beacon coverage on the GPU: the library's beacon stream matches continual FPS (replayed
on the oracle chunk by chunk from the GPU's own state), and the coverage readout agrees with
a float64 recomputation."""
import numpy as np
import pytest
import torch

from oracle import bkv_oracle as O
from synth import WORKLOADS, bf16_bits
from synth.stream import query_stream
from parity import check_fps_replay
from attention_guided_eviction_amd import bkv
from attention_guided_eviction_amd.coverage import beacon_stream, coverage, max_cosine

pytestmark = pytest.mark.gpu


def test_gpu_beacon_stream_replays_continual_fps():
    w = WORKLOADS["qwen14b_64k"]
    steps, chunk, nb = 512, 128, w.nb_max
    units = [(0, 0, 0), (0, 1, 3), (0, 3, 7)]
    q = torch.stack([query_stream(w, *u, steps, 0, device="cuda")[0] for u in units])   # [U, G, S, D]
    U, G, _, D = q.shape
    shape = bkv.CacheShape(1, U, G, 1, D, 1, torch.ones(U, dtype=torch.int32, device="cuda"))
    bc = [torch.zeros((U, 1, nb, D), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    n = [torch.zeros((U, 1), dtype=torch.int32, device="cuda") for _ in range(2)]
    cur = 0
    for c0 in range(0, steps, chunk):
        qn = q[:, :, c0:c0 + chunk].contiguous()
        bkv.update_beacons(shape, [bc[cur]], [n[cur]], nb, [qn], chunk, chunk, [bc[1 - cur]], [n[1 - cur]])
        torch.cuda.synchronize()
        for u in range(U):
            prev = bf16_bits(bc[cur][u, 0].cpu())
            pool = O.beacon_pool(prev, int(n[cur][u, 0]), bf16_bits(qn[u].cpu()))
            k = int(n[1 - cur][u, 0])
            assert k == min(nb, pool.shape[0])
            check_fps_replay(pool, bf16_bits(bc[1 - cur][u, 0, :k].cpu()), nb)
        cur = 1 - cur
    final, cnt = beacon_stream(q, nb, chunk)
    assert torch.equal(final, bc[cur][:, 0]) and torch.equal(cnt, n[cur][:, 0])


def test_coverage_readout_matches_float64():
    w = WORKLOADS["qwen14b_64k"]
    units = [(0, 0, 0), (0, 2, 5)]
    res = coverage(w, units, 512, 128, 128, w.window, w.nb_max)
    assert res["fps"]["plan_revisits"] > 0.8 and res["recent"]["plan_revisits"] < 0.3
    # max_cosine against a float64 recomputation on random data
    g = torch.Generator(device="cuda").manual_seed(3)
    fut = torch.randn(2, 50, 64, generator=g, device="cuda").to(torch.bfloat16)
    sets = torch.randn(2, 9, 64, generator=g, device="cuda").to(torch.bfloat16)
    cnt = torch.tensor([9, 4], dtype=torch.int32, device="cuda")
    got = max_cosine(fut, sets, cnt).cpu().numpy()
    for u in range(2):
        f = O.bf16_to_f64(bf16_bits(fut[u].cpu()))
        s = O.bf16_to_f64(bf16_bits(sets[u, :int(cnt[u])].cpu()))
        want = ((f / np.linalg.norm(f, axis=1, keepdims=True)) @ (s / np.linalg.norm(s, axis=1, keepdims=True)).T).max(1)
        np.testing.assert_allclose(got[u], want, atol=2e-6)
