"""The seeded input generator: deterministic, unit slices equal whole-layer tensors,
and the intended shape statistics.  CPU only."""
import numpy as np
import torch

from synth import WORKLOADS, WORKLOAD_ORDER, layer_tensors, seq_lengths, unit_inputs
from synth.gen import key_clusters, noise, stream_key


def _small(name, **kw):
    w = WORKLOADS[name]
    base = dict(n_layers=2, capacity=1024, batch=min(w.batch, 2))
    if w.ragged is None:
        base["seq_len"] = 1024
    else:
        base["ragged"] = (300, 1024)
    base.update(kw)
    return w.replace(**base)


def test_workloads_shapes():
    assert WORKLOAD_ORDER == list(WORKLOADS)
    for name in WORKLOAD_ORDER:
        w = WORKLOADS[name]
        assert w.n_q_heads % w.n_kv_heads == 0
        assert 0 <= w.window <= w.budget
        assert w.nb_init <= w.nb_max
        lens = seq_lengths(w)
        assert lens.shape == (w.batch,) and lens.max() <= w.capacity and lens.min() >= 1
    assert WORKLOADS["qwen7b_16k"].group * 32 + 16 == 240
    lens = seq_lengths(WORKLOADS["qwen4b_serving"])
    assert lens.min() >= 2048 and lens.max() <= 8192 and len(set(lens.tolist())) > 10


def test_noise_is_deterministic_and_standardised():
    keys = torch.tensor([list(stream_key(1, 2, 3)), list(stream_key(1, 2, 4))])
    a = noise(keys, 200000, "cpu")
    b = noise(keys, 200000, "cpu")
    assert torch.equal(a, b)
    assert abs(a.mean().item()) < 0.01 and abs(a.std().item() - 1) < 0.01
    assert not torch.equal(a[0], a[1])
    # prefix property: fewer elements give the same leading values
    assert torch.equal(noise(keys, 1000, "cpu"), a[:, :1000])


def test_unit_slices_match_layer_tensors():
    for name in WORKLOAD_ORDER:
        w = _small(name)
        lt = layer_tensors(w, 1, "cpu")
        lens = seq_lengths(w)
        G = w.group
        for b in range(w.batch):
            for h in range(w.n_kv_heads):
                u = unit_inputs(w, 1, b, h)
                L = int(lens[b])
                assert u["L"] == L
                assert torch.equal(u["k"], lt["k"][b, h, :L])
                assert torch.equal(u["v"], lt["v"][b, h, :L])
                assert torch.equal(u["q"], lt["q"][b, h * G:(h + 1) * G])
                assert torch.equal(u["beacons"], lt["beacons"][b, h])


def test_clustered_keys_have_segment_structure():
    w = WORKLOADS["qwen14b_64k"]
    cid = key_clusters(w, 0, 0, 0, w.seq_len)
    noise_frac = (cid < 0).mean()
    assert 0.15 < noise_frac < 0.35
    late = cid[int(0.2 * w.seq_len):]
    assert not np.isin(late, [0, 1, 2, 3]).any()       # plan clusters only early
    runs = np.count_nonzero(np.diff(cid)) + 1
    assert 400 < runs < 2000                             # mean segment ~64 rows


def test_queries_attend_their_cluster():
    w = _small("qwen7b_16k", n_layers=1)
    lt = layer_tensors(w, 0, "cpu")
    q = lt["q"][0, 0].float()
    k = lt["k"][0, 0].float()
    s = q @ k.T / np.sqrt(w.head_dim)
    # same-cluster logits ~ sqrt(d), others ~ N(0, 1)
    assert s.max().item() > 8 and s.median().item() < 2
