"""The C ABI: the library loads, exports every entry point include/bkv.h declares, and
rejects bad arguments on the host before touching the GPU.  CPU only: every call here
fails validation (fake device addresses are never dereferenced)."""
import ctypes
import os
import re
import subprocess

import pytest

from attention_guided_eviction_amd import bkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bkv.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bkv_[a-z_]+)\s*\(", text)))


def test_header_declares_binding_exports():
    assert _declared() == sorted(bkv.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = bkv.load()
    nm = subprocess.run(["nm", "-D", "--defined-only", bkv.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (bkv_\w+)", nm))
    for name in _declared():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_status_strings_and_version():
    for code in (0, -1, -2, -3, -4, -5):
        assert bkv.status_string(code).startswith("BKV_")
    assert "unknown" in bkv.status_string(7)
    assert re.match(r"\d+\.\d+\.\d+$", bkv.version())


def test_header_limits_match_binding():
    text = open(HEADER).read()
    assert int(re.search(r"#define BKV_MAX_OBS (\d+)", text).group(1)) == bkv.MAX_OBS
    assert int(re.search(r"#define BKV_MAX_POOL (\d+)", text).group(1)) == bkv.MAX_POOL
    mib = int(re.search(r"#define BKV_STATIC_SCRATCH_BYTES \(\(size_t\)(\d+) << 20\)", text).group(1))
    assert mib << 20 == bkv.STATIC_SCRATCH_BYTES


# ------------------------------------------------------------------------------------------------
# host-side validation with fake addresses
# ------------------------------------------------------------------------------------------------

FAKE = 0x7F0000000000


def shape(**kw):
    d = dict(n_layers=2, batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, capacity=1024, seq_len=FAKE)
    d.update(kw)
    return bkv._Shape(d["n_layers"], d["batch"], d["n_q_heads"], d["n_kv_heads"], d["head_dim"], d["capacity"],
                      d["seq_len"])


def arr(base, n=2, stride=1 << 32):
    return (ctypes.c_void_p * n)(*[base + i * stride for i in range(n)])


def nulls(n=2):
    return (ctypes.c_void_p * n)(*([None] * n))


def score_call(s=None, k=None, q=None, q_len=32, window=32, bc=None, nb=None, nb_max=16, sc=None, ws=FAKE + (1 << 40),
               ws_bytes=1 << 40):
    lib = bkv.load()
    s = s or shape()
    return lib.bkv_score(ctypes.byref(s), k or arr(FAKE + (1 << 36)), q or arr(FAKE + (2 << 36)), q_len, window,
                         bc or arr(FAKE + (3 << 36)), nb or arr(FAKE + (4 << 36)), nb_max, sc or arr(FAKE + (5 << 36)),
                         ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(s=shape(head_dim=96)), bkv.BKV_EUNSUPPORTED),
    (dict(s=shape(head_dim=0)), bkv.BKV_EINVAL),
    (dict(s=shape(n_q_heads=6, n_kv_heads=4)), bkv.BKV_EINVAL),
    (dict(s=shape(seq_len=0)), bkv.BKV_EINVAL),
    (dict(s=shape(n_layers=0)), bkv.BKV_EINVAL),
    (dict(s=shape(capacity=0)), bkv.BKV_EINVAL),
    (dict(window=33), bkv.BKV_EINVAL),
    (dict(window=-1), bkv.BKV_EINVAL),
    (dict(nb_max=-1), bkv.BKV_EINVAL),
    (dict(k=nulls()), bkv.BKV_EINVAL),
    (dict(sc=nulls()), bkv.BKV_EINVAL),
    (dict(bc=nulls()), bkv.BKV_EINVAL),
    (dict(window=32, q_len=200, nb_max=400), bkv.BKV_EUNSUPPORTED),   # 4*32 + 400 > 512 rows
    (dict(ws=None), bkv.BKV_EWORKSPACE),
    (dict(ws_bytes=16), bkv.BKV_EWORKSPACE),
    (dict(ws=FAKE + (1 << 40) + 8), bkv.BKV_EWORKSPACE),              # misaligned
    (dict(sc=arr(FAKE + (1 << 36) + 4096)), bkv.BKV_EALIAS),          # scores inside K
])
def test_score_rejects(kw, status):
    assert score_call(**kw) == status


def test_workspace_bytes_monotone():
    lib = bkv.load()
    a = lib.bkv_score_workspace_bytes(ctypes.byref(shape()), 32, 16)
    b = lib.bkv_score_workspace_bytes(ctypes.byref(shape(capacity=4096)), 32, 16)
    c = lib.bkv_score_workspace_bytes(ctypes.byref(shape(capacity=4096)), 64, 16)
    assert 0 < a < b < c
    assert lib.bkv_score_workspace_bytes(ctypes.byref(shape(head_dim=96)), 32, 16) == 0
    assert lib.bkv_compress_workspace_bytes(ctypes.byref(shape()), 32, 16, 256) >= a


def test_select_rejects():
    lib = bkv.load()
    s = shape()
    sc, idx, nk = arr(FAKE), arr(FAKE + (1 << 36)), arr(FAKE + (2 << 36))
    assert lib.bkv_select_topk(ctypes.byref(s), sc, 0, 0, idx, nk, None, 0, None) == bkv.BKV_EINVAL
    assert lib.bkv_select_topk(ctypes.byref(s), sc, 64, 65, idx, nk, None, 0, None) == bkv.BKV_EINVAL
    assert lib.bkv_select_topk(ctypes.byref(s), nulls(), 64, 8, idx, nk, None, 0, None) == bkv.BKV_EINVAL
    assert lib.bkv_select_topk(ctypes.byref(shape(capacity=70000)), sc, 64, 8, idx, nk, None, 0,
                               None) == bkv.BKV_EUNSUPPORTED
    assert lib.bkv_select_topk(ctypes.byref(s), sc, 64, 8, arr(FAKE + 64), nk, None, 0, None) == bkv.BKV_EALIAS


def test_compact_rejects_aliasing():
    lib = bkv.load()
    s = shape()
    k, v = arr(FAKE), arr(FAKE + (1 << 36))
    idx, nk = arr(FAKE + (2 << 36)), arr(FAKE + (3 << 36))
    ko, vo = arr(FAKE + (4 << 36)), arr(FAKE + (5 << 36))
    assert lib.bkv_compact(ctypes.byref(s), k, v, idx, nk, 0, ko, vo, None) == bkv.BKV_EINVAL
    assert lib.bkv_compact(ctypes.byref(s), k, v, idx, nk, 64, arr(FAKE + 256), vo, None) == bkv.BKV_EALIAS
    assert lib.bkv_compact(ctypes.byref(s), k, v, idx, nk, 64, ko, arr(FAKE + (1 << 36)), None) == bkv.BKV_EALIAS
    assert lib.bkv_compact(ctypes.byref(s), k, v, idx, nk, 64, ko, ko, None) == bkv.BKV_EALIAS
    assert lib.bkv_compact(ctypes.byref(s), k, nulls(), idx, nk, 64, ko, vo, None) == bkv.BKV_EINVAL
    # 2^27 kept rows of 16 pieces each: past what the kernel's 32-bit piece index covers
    assert lib.bkv_compact(ctypes.byref(s), k, v, idx, nk, 1 << 27, ko, vo, None) == bkv.BKV_EUNSUPPORTED


def test_update_beacons_rejects():
    lib = bkv.load()
    s = shape()
    bi, ni, qn = arr(FAKE), arr(FAKE + (1 << 36)), arr(FAKE + (2 << 36))
    bo, no = arr(FAKE + (3 << 36)), arr(FAKE + (4 << 36))
    f = lib.bkv_update_beacons
    assert f(ctypes.byref(s), bi, ni, 0, qn, 128, 128, bo, no, None) == bkv.BKV_EINVAL       # nb_max < 1
    assert f(ctypes.byref(s), bi, ni, 16, qn, 128, 129, bo, no, None) == bkv.BKV_EINVAL     # t_new > q_len
    assert f(ctypes.byref(s), bi, ni, 16, qn, 4093, 4093, bo, no, None) == bkv.BKV_EUNSUPPORTED  # pool 16+4*4093
    assert f(ctypes.byref(s), bi, ni, 16, qn, 128, 128, bi, no, None) == bkv.BKV_EALIAS
    assert f(ctypes.byref(s), bi, ni, 16, qn, 128, 128, bo, ni, None) == bkv.BKV_EALIAS
    assert f(ctypes.byref(s), bi, ni, 16, qn, 128, 128, qn, no, None) == bkv.BKV_EALIAS
    assert f(ctypes.byref(s), bi, ni, 16, nulls(), 128, 128, bo, no, None) == bkv.BKV_EINVAL
    assert f(ctypes.byref(shape(head_dim=32)), bi, ni, 16, qn, 128, 128, bo, no, None) == bkv.BKV_EUNSUPPORTED


def test_score_agg_rejects_unknown_aggregation_and_validates_like_score():
    lib = bkv.load()
    s = shape()

    def call(agg, **kw):
        a = dict(k=arr(FAKE + (1 << 36)), q=arr(FAKE + (2 << 36)), bc=arr(FAKE + (3 << 36)),
                 nb=arr(FAKE + (4 << 36)), sc=arr(FAKE + (5 << 36)), window=32)
        a.update(kw)
        return lib.bkv_score_agg(ctypes.byref(s), a["k"], a["q"], 32, a["window"], a["bc"], a["nb"], 16, agg,
                                 a["sc"], FAKE + (1 << 40), 1 << 40, None)

    assert call(2) == bkv.BKV_EINVAL
    assert call(-1) == bkv.BKV_EINVAL
    assert call(bkv.AGG_MEAN, window=33) == bkv.BKV_EINVAL
    assert call(bkv.AGG_MEAN, sc=arr(FAKE + (1 << 36) + 4096)) == bkv.BKV_EALIAS


def test_header_aggregation_values_match_binding():
    text = open(HEADER).read()
    assert int(re.search(r"BKV_AGG_MAX = (\d+)", text).group(1)) == bkv.AGG_MAX
    assert int(re.search(r"BKV_AGG_MEAN = (\d+)", text).group(1)) == bkv.AGG_MEAN


def test_update_beacons_policy_rejects_unknown_policy_and_keeps_fps_limits():
    lib = bkv.load()
    s = shape()

    def call(policy, t_new=8, nb_max=16, q_len=200):
        return lib.bkv_update_beacons_policy(ctypes.byref(s), arr(FAKE + (1 << 36)), arr(FAKE + (2 << 36)), nb_max,
                                             arr(FAKE + (3 << 36)), q_len, t_new, policy, arr(FAKE + (4 << 36)),
                                             arr(FAKE + (5 << 36)), None)

    assert call(2) == bkv.BKV_EINVAL
    # continual FPS is limited to BKV_MAX_POOL candidates; 16 + 4 * 4093 > 16384
    assert call(bkv.BEACON_FPS, t_new=4093, q_len=4093) == bkv.BKV_EUNSUPPORTED
    assert call(bkv.BEACON_INITIAL, t_new=201) == bkv.BKV_EINVAL                  # t_new > q_len


def test_header_beacon_policy_values_match_binding():
    text = open(HEADER).read()
    assert int(re.search(r"BKV_BEACON_FPS = (\d+)", text).group(1)) == bkv.BEACON_FPS
    assert int(re.search(r"BKV_BEACON_INITIAL = (\d+)", text).group(1)) == bkv.BEACON_INITIAL


def test_compact_into_validates_out_capacity():
    lib = bkv.load()
    s = shape()
    ks, vs = arr(FAKE + (1 << 36)), arr(FAKE + (2 << 36))

    def call(budget, out_cap, k_out=None):
        return lib.bkv_compact_into(ctypes.byref(s), ks, vs, arr(FAKE + (3 << 36)), arr(FAKE + (4 << 36)), budget,
                                    out_cap, k_out or arr(FAKE + (5 << 36)), arr(FAKE + (6 << 36)), None)

    assert call(64, 63) == bkv.BKV_EINVAL
    assert call(0, 64) == bkv.BKV_EINVAL
    # an output laid out with 2048 rows per (sequence, KV head) reaches into K here
    assert call(64, 2048, k_out=arr(FAKE + (1 << 36) - 2 * 2 * 2048 * 128 * 2 + 4096)) == bkv.BKV_EALIAS


def test_decode_attention_validation():
    lib = bkv.load()
    qs, ks, vs, os_ = arr(FAKE + (1 << 36)), arr(FAKE + (2 << 36)), arr(FAKE + (3 << 36)), arr(FAKE + (4 << 36))
    s = shape()
    need = lib.bkv_decode_workspace_bytes(ctypes.byref(s))
    assert need > 0
    ws = FAKE + (1 << 40)

    def call(s=s, q=qs, out=os_, ws=ws, nbytes=need):
        return lib.bkv_decode_attention(ctypes.byref(s), q, ks, vs, out, ws, nbytes, None)

    assert call(s=shape(n_q_heads=18, n_kv_heads=2)) == bkv.BKV_EUNSUPPORTED     # 9 query heads per KV head
    assert lib.bkv_decode_workspace_bytes(ctypes.byref(shape(n_q_heads=18, n_kv_heads=2))) == 0
    assert call(q=nulls()) == bkv.BKV_EINVAL
    assert call(nbytes=need - 1) == bkv.BKV_EWORKSPACE
    assert call(ws=ws + 8) == bkv.BKV_EWORKSPACE
    assert call(out=arr(FAKE + (2 << 36) + 512)) == bkv.BKV_EALIAS                # out inside K


def two(a, b):
    return (ctypes.c_void_p * 2)(a, b)


def test_outputs_may_not_overlap_anything_the_call_touches():
    """An output may overlap no input of any layer (nor the lengths), no workspace and no
    other output; every call below is refused before anything is enqueued."""
    lib = bkv.load()
    s = shape()
    # scoring
    assert score_call(sc=arr(FAKE + (1 << 40) + 4096)) == bkv.BKV_EALIAS                 # inside the workspace
    assert score_call(sc=two(FAKE + (2 << 36) + (1 << 32) + 64, FAKE + (5 << 36))) == bkv.BKV_EALIAS   # layer 1's q
    assert score_call(sc=arr(FAKE - 4)) == bkv.BKV_EALIAS                                # the lengths
    assert score_call(sc=arr(FAKE + (5 << 36), stride=4096)) == bkv.BKV_EALIAS           # the two layers' scores
    assert score_call(sc=arr(FAKE + (4 << 36) + 8)) == bkv.BKV_EALIAS                    # beacon counts
    assert score_call(ws=FAKE + (1 << 36)) == bkv.BKV_EALIAS                             # workspace over K
    # selection
    sc = arr(FAKE + (1 << 36))
    assert lib.bkv_select_topk(ctypes.byref(s), sc, 64, 8, arr(FAKE - 8), arr(FAKE + (3 << 36)), None, 0,
                               None) == bkv.BKV_EALIAS                                     # idx over the lengths
    assert lib.bkv_select_topk(ctypes.byref(s), sc, 64, 8, arr(FAKE + (2 << 36)),
                               two(FAKE + (2 << 36) + (1 << 32) + 4, FAKE + (3 << 36)), None, 0,
                               None) == bkv.BKV_EALIAS                                     # n_kept in idx of layer 1
    # one event: the stages' outputs must not meet either
    assert lib.bkv_compress(ctypes.byref(s), arr(FAKE + (1 << 36)), arr(FAKE + (6 << 36)), arr(FAKE + (2 << 36)), 32,
                            32, arr(FAKE + (3 << 36)), arr(FAKE + (4 << 36)), 16, 64, arr(FAKE + (5 << 36)),
                            arr(FAKE + (7 << 36)), arr(FAKE + (8 << 36)), arr(FAKE + (5 << 36) + 64),
                            arr(FAKE + (10 << 36)), FAKE + (1 << 40), 1 << 40, None) == bkv.BKV_EALIAS   # k_out in scores
    # beacon update
    assert lib.bkv_update_beacons(ctypes.byref(s), arr(FAKE), arr(FAKE + (1 << 36)), 16, arr(FAKE + (2 << 36)), 128,
                                  128, two(FAKE + (1 << 36) + (1 << 32), FAKE + (3 << 36)), arr(FAKE + (4 << 36)),
                                  None) == bkv.BKV_EALIAS                                  # beacons_out on n_in[1]
    # decode
    qs, ks, vs = arr(FAKE + (1 << 36)), arr(FAKE + (2 << 36)), arr(FAKE + (3 << 36))
    need = lib.bkv_decode_workspace_bytes(ctypes.byref(s))
    assert lib.bkv_decode_attention(ctypes.byref(s), qs, ks, vs, arr(FAKE - 4), FAKE + (1 << 40), need,
                                    None) == bkv.BKV_EALIAS                                # out over the lengths
    assert lib.bkv_decode_attention(ctypes.byref(s), qs, ks, vs, arr(FAKE + (4 << 36)), FAKE + (1 << 36), need,
                                    None) == bkv.BKV_EALIAS                                # workspace over q


def test_misaligned_pointers_are_rejected():
    """bf16 rows move in 16-byte pieces, fp32 / int32 arrays element by element: a layer
    pointer off those boundaries is BKV_EINVAL at every entry point, before any launch."""
    lib = bkv.load()
    s = shape()
    # score: K, queries, beacons on 16 bytes; scores and beacon counts on 4
    for kw in (dict(k=arr(FAKE + (1 << 36) + 8)), dict(q=arr(FAKE + (2 << 36) + 2)),
               dict(bc=arr(FAKE + (3 << 36) + 4)), dict(nb=arr(FAKE + (4 << 36) + 2)),
               dict(sc=arr(FAKE + (5 << 36) + 2)), dict(s=shape(seq_len=FAKE + 2))):
        assert score_call(**kw) == bkv.BKV_EINVAL, kw
    # select: scores, idx, n_kept on 4 bytes
    sc, idx, nk = arr(FAKE), arr(FAKE + (1 << 36)), arr(FAKE + (2 << 36))
    for a, b, c in ((arr(FAKE + 2), idx, nk), (sc, arr(FAKE + (1 << 36) + 1), nk), (sc, idx, arr(FAKE + (2 << 36) + 3))):
        assert lib.bkv_select_topk(ctypes.byref(s), a, 64, 8, b, c, None, 0, None) == bkv.BKV_EINVAL
    # compact: K, V, outputs on 16 bytes
    k, v = arr(FAKE), arr(FAKE + (1 << 36))
    idx, nk = arr(FAKE + (2 << 36)), arr(FAKE + (3 << 36))
    ko, vo = arr(FAKE + (4 << 36)), arr(FAKE + (5 << 36))
    assert lib.bkv_compact(ctypes.byref(s), arr(FAKE + 8), v, idx, nk, 64, ko, vo, None) == bkv.BKV_EINVAL
    assert lib.bkv_compact(ctypes.byref(s), k, v, idx, nk, 64, ko, arr(FAKE + (5 << 36) + 4), None) == bkv.BKV_EINVAL
    assert lib.bkv_compact(ctypes.byref(s), k, v, arr(FAKE + (2 << 36) + 2), nk, 64, ko, vo, None) == bkv.BKV_EINVAL
    # beacon update: beacon rows and new queries on 16 bytes, counts on 4
    bi, ni, qn = arr(FAKE), arr(FAKE + (1 << 36)), arr(FAKE + (2 << 36))
    bo, no = arr(FAKE + (3 << 36)), arr(FAKE + (4 << 36))
    f = lib.bkv_update_beacons
    assert f(ctypes.byref(s), arr(FAKE + 4), ni, 16, qn, 128, 128, bo, no, None) == bkv.BKV_EINVAL
    assert f(ctypes.byref(s), bi, ni, 16, arr(FAKE + (2 << 36) + 8), 128, 128, bo, no, None) == bkv.BKV_EINVAL
    assert f(ctypes.byref(s), bi, ni, 16, qn, 128, 128, arr(FAKE + (3 << 36) + 2), no, None) == bkv.BKV_EINVAL
    assert f(ctypes.byref(s), bi, ni, 16, qn, 128, 128, bo, arr(FAKE + (4 << 36) + 2), None) == bkv.BKV_EINVAL
    # decode: q, K, V on 16 bytes
    out, ws = arr(FAKE + (3 << 36)), FAKE + (1 << 40)
    d = lib.bkv_decode_attention
    assert d(ctypes.byref(s), arr(FAKE + (4 << 36) + 2), k, v, out, ws, 1 << 40, None) == bkv.BKV_EINVAL
    assert d(ctypes.byref(s), arr(FAKE + (4 << 36)), arr(FAKE + 8), v, out, ws, 1 << 40, None) == bkv.BKV_EINVAL


def compress_static_call(s=None, ko=None, k=None, window=32, nb_max=16, budget=64):
    lib = bkv.load()
    s = s or shape()
    return lib.bkv_compress_static(ctypes.byref(s), k or arr(FAKE + (1 << 36)), arr(FAKE + (6 << 36)),
                                   arr(FAKE + (2 << 36)), window, window, arr(FAKE + (3 << 36)),
                                   arr(FAKE + (4 << 36)), nb_max, budget, arr(FAKE + (5 << 36)),
                                   arr(FAKE + (7 << 36)), arr(FAKE + (8 << 36)), ko or arr(FAKE + (9 << 36)),
                                   arr(FAKE + (10 << 36)), None)


def test_compress_static_validates_like_compress():
    assert compress_static_call(ko=arr(FAKE + (5 << 36) + 64)) == bkv.BKV_EALIAS      # k_out inside scores
    assert compress_static_call(k=arr(FAKE + (1 << 36) + 8)) == bkv.BKV_EINVAL        # misaligned K
    assert compress_static_call(s=shape(head_dim=96)) == bkv.BKV_EUNSUPPORTED
    assert compress_static_call(budget=16) == bkv.BKV_EINVAL                          # window > budget


def test_compress_static_refuses_what_its_scratch_cannot_hold():
    """8192 KV heads x 2 slots x 512 observation rows x 8 bytes = 64 MiB of partials for a
    single layer of a single sequence: more than the static scratch, and no smaller launch
    group exists, so the call is refused before anything is enqueued, with the need named."""
    s = shape(n_layers=1, batch=1, n_q_heads=8192, n_kv_heads=8192, capacity=1024)
    assert compress_static_call(s=s, window=480, nb_max=32, budget=600) == bkv.BKV_EUNSUPPORTED
    msg = bkv.load().bkv_last_error().decode()
    assert "67108864" in msg and str(bkv.STATIC_SCRATCH_BYTES) in msg, msg
