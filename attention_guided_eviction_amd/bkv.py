"""Python binding of libbkv.so (include/bkv.h) -- argument marshalling only.

Each function takes per-layer lists of torch tensors that already live on the GPU,
checks that they have the dtype, device, contiguity and shape the C ABI expects (so a
wrong tensor cannot make a kernel read or write out of bounds), and passes their
device pointers and the current HIP stream to the library.  All computation happens
in the library's HIP kernels; there is no fallback: if libbkv.so is missing or was
built for another architecture the first call raises.

Operations (BeaconKV page, thelatestinai.com/papers/2609.04971):
  update_beacons  continual farthest-point sampling of beacon queries (Figure 7)
  score           max-aggregated attention scores from recent + beacon queries (Figure 5 (b), (c))
  select_topk     top-K under the budget, recent window always kept (Figure 5 (c))
  compact         gather of the kept K/V rows (Abstract)
  compress        score + select_topk + compact
  compress_static the same with no workspace (the library's static device scratch)
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# BKV_LIBRARY names another build of the same library (e.g. the host-only sanitized build
# that the ABI tests load); by default the in-tree libbkv.so.
LIB_PATH = os.environ.get("BKV_LIBRARY") or os.path.join(_HERE, "libbkv.so")

BKV_OK, BKV_EINVAL, BKV_EUNSUPPORTED, BKV_EALIAS, BKV_EWORKSPACE, BKV_EHIP = 0, -1, -2, -3, -4, -5
MAX_OBS = 512
AGG_MAX, AGG_MEAN = 0, 1
AGGREGATIONS = {"max": AGG_MAX, "mean": AGG_MEAN}
BEACON_FPS, BEACON_INITIAL = 0, 1
BEACON_POLICIES = {"fps": BEACON_FPS, "initial": BEACON_INITIAL}
MAX_POOL = 16384

EXPORTS = ["bkv_status_string", "bkv_version", "bkv_last_error", "bkv_update_beacons", "bkv_update_beacons_policy",
           "bkv_score_workspace_bytes",
           "bkv_score", "bkv_score_agg", "bkv_select_workspace_bytes", "bkv_select_topk", "bkv_compact",
           "bkv_compact_into", "bkv_decode_workspace_bytes", "bkv_decode_attention",
           "bkv_compress_workspace_bytes", "bkv_compress", "bkv_compress_static"]
# Bytes of bkv_compress_static's device scratch (BKV_STATIC_SCRATCH_BYTES).
STATIC_SCRATCH_BYTES = 32 << 20


class BkvError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = f"{what}: {status_string(status)} ({status})"
        if status == BKV_EHIP or (status == BKV_EUNSUPPORTED and what == "bkv_compress_static"):
            msg += " -- " + load().bkv_last_error().decode()
        super().__init__(msg)
        self.status = status


class _Shape(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("seq_len", ctypes.c_void_p)]


_lib = None


def load() -> ctypes.CDLL:
    """Load libbkv.so once and declare its prototypes.  Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m attention_guided_eviction_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    P = ctypes.POINTER
    arr = P(vp)
    lib.bkv_status_string.restype = ctypes.c_char_p
    lib.bkv_status_string.argtypes = [ctypes.c_int]
    lib.bkv_version.restype = ctypes.c_char_p
    lib.bkv_version.argtypes = []
    lib.bkv_last_error.restype = ctypes.c_char_p
    lib.bkv_last_error.argtypes = []
    lib.bkv_update_beacons.restype = ctypes.c_int
    lib.bkv_update_beacons.argtypes = [P(_Shape), arr, arr, i32, arr, i32, i32, arr, arr, vp]
    lib.bkv_update_beacons_policy.restype = ctypes.c_int
    lib.bkv_update_beacons_policy.argtypes = [P(_Shape), arr, arr, i32, arr, i32, i32, ctypes.c_int, arr, arr, vp]
    lib.bkv_score_workspace_bytes.restype = sz
    lib.bkv_score_workspace_bytes.argtypes = [P(_Shape), i32, i32]
    lib.bkv_score.restype = ctypes.c_int
    lib.bkv_score.argtypes = [P(_Shape), arr, arr, i32, i32, arr, arr, i32, arr, vp, sz, vp]
    lib.bkv_score_agg.restype = ctypes.c_int
    lib.bkv_score_agg.argtypes = [P(_Shape), arr, arr, i32, i32, arr, arr, i32, ctypes.c_int, arr, vp, sz, vp]
    lib.bkv_select_workspace_bytes.restype = sz
    lib.bkv_select_workspace_bytes.argtypes = [P(_Shape), i32]
    lib.bkv_select_topk.restype = ctypes.c_int
    lib.bkv_select_topk.argtypes = [P(_Shape), arr, i32, i32, arr, arr, vp, sz, vp]
    lib.bkv_compact.restype = ctypes.c_int
    lib.bkv_compact.argtypes = [P(_Shape), arr, arr, arr, arr, i32, arr, arr, vp]
    lib.bkv_decode_workspace_bytes.restype = sz
    lib.bkv_decode_workspace_bytes.argtypes = [P(_Shape)]
    lib.bkv_decode_attention.restype = ctypes.c_int
    lib.bkv_decode_attention.argtypes = [P(_Shape), arr, arr, arr, arr, vp, sz, vp]
    lib.bkv_compact_into.restype = ctypes.c_int
    lib.bkv_compact_into.argtypes = [P(_Shape), arr, arr, arr, arr, i32, i32, arr, arr, vp]
    lib.bkv_compress_workspace_bytes.restype = sz
    lib.bkv_compress_workspace_bytes.argtypes = [P(_Shape), i32, i32, i32]
    lib.bkv_compress.restype = ctypes.c_int
    lib.bkv_compress.argtypes = [P(_Shape), arr, arr, arr, i32, i32, arr, arr, i32, i32, arr, arr, arr,
                                 arr, arr, vp, sz, vp]
    lib.bkv_compress_static.restype = ctypes.c_int
    lib.bkv_compress_static.argtypes = [P(_Shape), arr, arr, arr, i32, i32, arr, arr, i32, i32, arr, arr, arr,
                                        arr, arr, vp]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().bkv_status_string(int(status)).decode()


def version() -> str:
    return load().bkv_version().decode()


@dataclass
class CacheShape:
    """Geometry shared by every layer of one call (mirrors bkv_shape)."""
    n_layers: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    capacity: int
    seq_len: torch.Tensor          # int32 [batch] on the GPU

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def c(self) -> _Shape:
        _check(self.seq_len, torch.int32, (self.batch,), "seq_len")
        return _Shape(self.n_layers, self.batch, self.n_q_heads, self.n_kv_heads, self.head_dim, self.capacity,
                      self.seq_len.data_ptr())


def _check(t: torch.Tensor, dtype, shape, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _layers(ts: Sequence[torch.Tensor], n: int, dtype, shape, name: str):
    if len(ts) != n:
        raise ValueError(f"{name}: {len(ts)} layers, expected {n}")
    for i, t in enumerate(ts):
        _check(t, dtype, shape, f"{name}[{i}]")
    return (ctypes.c_void_p * n)(*[t.data_ptr() for t in ts])


def _null_layers(n: int):
    return (ctypes.c_void_p * n)(*([None] * n))


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ok(status: int, what: str):
    if status != BKV_OK:
        raise BkvError(status, what)


def _workspace(ws: Optional[torch.Tensor], need: int):
    if need == 0:
        return None, 0
    if ws is None or not ws.is_cuda:
        raise ValueError(f"a GPU workspace of at least {need} bytes is required")
    return ws.data_ptr(), ws.numel() * ws.element_size()


# ------------------------------------------------------------------------------------------------
# Each operation is split into prepare_*() -- checks every tensor once and builds the ctypes
# argument list -- and a call of the returned object with an optional stream, so repeated
# events over the same buffers pay the Python checks once.

class Call:
    """A prepared library call: `call(stream=None)` enqueues it on `stream` (default: the
    current torch stream) and raises BkvError on a non-zero status."""

    def __init__(self, fn, args, what: str, keep):
        self._fn, self._args, self.what, self._keep = fn, args, what, keep

    def __call__(self, stream=None) -> None:
        _ok(self._fn(*self._args, _stream(stream)), self.what)


def prepare_update_beacons(s: CacheShape, beacons_in, n_in, nb_max: int, q_new, q_len: int, t_new: int,
                           beacons_out, n_out, policy: str = "fps") -> Call:
    """bkv_update_beacons for continual FPS, bkv_update_beacons_policy for any other policy."""
    lib = load()
    if policy not in BEACON_POLICIES:
        raise ValueError(f"policy must be one of {sorted(BEACON_POLICIES)}, got {policy!r}")
    B, Hq, Hkv, D, n = s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim, s.n_layers
    shape = s.c()
    bi = _layers(beacons_in, n, torch.bfloat16, (B, Hkv, nb_max, D), "beacons_in")
    ni = _layers(n_in, n, torch.int32, (B, Hkv), "n_in")
    qn = _layers(q_new, n, torch.bfloat16, (B, Hq, q_len, D), "q_new") if t_new > 0 else _null_layers(n)
    bo = _layers(beacons_out, n, torch.bfloat16, (B, Hkv, nb_max, D), "beacons_out")
    no = _layers(n_out, n, torch.int32, (B, Hkv), "n_out")
    keep = (shape, s.seq_len, beacons_in, n_in, q_new, beacons_out, n_out)
    if policy == "fps":
        args = (ctypes.byref(shape), bi, ni, nb_max, qn, q_len, t_new, bo, no)
        return Call(lib.bkv_update_beacons, args, "bkv_update_beacons", keep)
    args = (ctypes.byref(shape), bi, ni, nb_max, qn, q_len, t_new, BEACON_POLICIES[policy], bo, no)
    return Call(lib.bkv_update_beacons_policy, args, "bkv_update_beacons_policy", keep)


def update_beacons(s: CacheShape, beacons_in, n_in, nb_max: int, q_new, q_len: int, t_new: int,
                   beacons_out, n_out, stream=None, policy: str = "fps") -> None:
    """Beacon update of every layer: continual FPS (bkv_update_beacons) or the first
    queries kept (bkv_update_beacons_policy, policy "initial")."""
    prepare_update_beacons(s, beacons_in, n_in, nb_max, q_new, q_len, t_new, beacons_out, n_out, policy)(stream)


def score_workspace_bytes(s: CacheShape, window: int, nb_max: int) -> int:
    return int(load().bkv_score_workspace_bytes(ctypes.byref(s.c()), window, nb_max))


def alloc_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A byte tensor usable as workspace (torch allocations are 256-byte aligned)."""
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def _score_inputs(s: CacheShape, k, q, q_len, window, beacons, n_beacons, nb_max):
    B, Hq, Hkv, D, cap, n = s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim, s.capacity, s.n_layers
    kp = _layers(k, n, torch.bfloat16, (B, Hkv, cap, D), "k")
    qp = _layers(q, n, torch.bfloat16, (B, Hq, q_len, D), "q") if window > 0 else _null_layers(n)
    if nb_max > 0:
        bp = _layers(beacons, n, torch.bfloat16, (B, Hkv, nb_max, D), "beacons")
        nbp = _layers(n_beacons, n, torch.int32, (B, Hkv), "n_beacons")
    else:
        bp, nbp = _null_layers(n), _null_layers(n)
    return kp, qp, bp, nbp


def prepare_score(s: CacheShape, k, q, q_len: int, window: int, beacons, n_beacons, nb_max: int, scores,
                  workspace: Optional[torch.Tensor], aggregation: str = "max") -> Call:
    """bkv_score for max aggregation, bkv_score_agg for any other."""
    lib = load()
    if aggregation not in AGGREGATIONS:
        raise ValueError(f"aggregation must be one of {sorted(AGGREGATIONS)}, got {aggregation!r}")
    shape = s.c()
    kp, qp, bp, nbp = _score_inputs(s, k, q, q_len, window, beacons, n_beacons, nb_max)
    sp = _layers(scores, s.n_layers, torch.float32, (s.batch, s.n_kv_heads, s.capacity), "scores")
    wp, wn = _workspace(workspace, int(lib.bkv_score_workspace_bytes(ctypes.byref(shape), window, nb_max)))
    keep = (shape, s.seq_len, k, q, beacons, n_beacons, scores, workspace)
    if aggregation == "max":
        args = (ctypes.byref(shape), kp, qp, q_len, window, bp, nbp, nb_max, sp, wp, wn)
        return Call(lib.bkv_score, args, "bkv_score", keep)
    args = (ctypes.byref(shape), kp, qp, q_len, window, bp, nbp, nb_max, AGGREGATIONS[aggregation], sp, wp, wn)
    return Call(lib.bkv_score_agg, args, "bkv_score_agg", keep)


def score(s: CacheShape, k, q, q_len: int, window: int, beacons, n_beacons, nb_max: int, scores,
          workspace: Optional[torch.Tensor], stream=None, aggregation: str = "max") -> None:
    """Attention scores of every cached key, max- (bkv_score) or mean-aggregated (bkv_score_agg)."""
    prepare_score(s, k, q, q_len, window, beacons, n_beacons, nb_max, scores, workspace, aggregation)(stream)


def prepare_select_topk(s: CacheShape, scores, budget: int, window: int, idx, n_kept) -> Call:
    lib = load()
    B, Hkv, cap, n = s.batch, s.n_kv_heads, s.capacity, s.n_layers
    shape = s.c()
    sp = _layers(scores, n, torch.float32, (B, Hkv, cap), "scores")
    ip = _layers(idx, n, torch.int32, (B, Hkv, budget), "idx")
    np_ = _layers(n_kept, n, torch.int32, (B, Hkv), "n_kept")
    args = (ctypes.byref(shape), sp, budget, window, ip, np_, None, 0)
    return Call(lib.bkv_select_topk, args, "bkv_select_topk", (shape, s.seq_len, scores, idx, n_kept))


def select_topk(s: CacheShape, scores, budget: int, window: int, idx, n_kept, stream=None) -> None:
    """Top-K positions per KV head, window always kept, ascending (bkv_select_topk)."""
    prepare_select_topk(s, scores, budget, window, idx, n_kept)(stream)


def prepare_compact(s: CacheShape, k, v, idx, n_kept, budget: int, k_out, v_out,
                    out_capacity: Optional[int] = None) -> Call:
    """bkv_compact (outputs [B][Hkv][budget][D]) or, with out_capacity, bkv_compact_into
    (outputs [B][Hkv][out_capacity][D], kept rows first)."""
    lib = load()
    B, Hkv, D, cap, n = s.batch, s.n_kv_heads, s.head_dim, s.capacity, s.n_layers
    shape = s.c()
    rows = budget if out_capacity is None else out_capacity
    kp = _layers(k, n, torch.bfloat16, (B, Hkv, cap, D), "k")
    vp = _layers(v, n, torch.bfloat16, (B, Hkv, cap, D), "v")
    ip = _layers(idx, n, torch.int32, (B, Hkv, budget), "idx")
    np_ = _layers(n_kept, n, torch.int32, (B, Hkv), "n_kept")
    ko = _layers(k_out, n, torch.bfloat16, (B, Hkv, rows, D), "k_out")
    vo = _layers(v_out, n, torch.bfloat16, (B, Hkv, rows, D), "v_out")
    keep = (shape, s.seq_len, k, v, idx, n_kept, k_out, v_out)
    if out_capacity is None:
        return Call(lib.bkv_compact, (ctypes.byref(shape), kp, vp, ip, np_, budget, ko, vo), "bkv_compact", keep)
    args = (ctypes.byref(shape), kp, vp, ip, np_, budget, out_capacity, ko, vo)
    return Call(lib.bkv_compact_into, args, "bkv_compact_into", keep)


def compact(s: CacheShape, k, v, idx, n_kept, budget: int, k_out, v_out, stream=None,
            out_capacity: Optional[int] = None) -> None:
    """Gather the kept K/V rows into compacted caches (bkv_compact / bkv_compact_into)."""
    prepare_compact(s, k, v, idx, n_kept, budget, k_out, v_out, out_capacity)(stream)


def decode_workspace_bytes(s: CacheShape) -> int:
    return int(load().bkv_decode_workspace_bytes(ctypes.byref(s.c())))


def prepare_decode_attention(s: CacheShape, q, k, v, out, workspace: Optional[torch.Tensor]) -> Call:
    """One decoding step of attention over a cache (bkv_decode_attention): q per layer
    bf16 [B][Hq][D], k and v [B][Hkv][capacity][D], out fp32 [B][Hq][D]."""
    lib = load()
    B, Hq, Hkv, D, cap, n = s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim, s.capacity, s.n_layers
    shape = s.c()
    qp = _layers(q, n, torch.bfloat16, (B, Hq, D), "q")
    kp = _layers(k, n, torch.bfloat16, (B, Hkv, cap, D), "k")
    vp = _layers(v, n, torch.bfloat16, (B, Hkv, cap, D), "v")
    op = _layers(out, n, torch.float32, (B, Hq, D), "out")
    wp, wn = _workspace(workspace, int(lib.bkv_decode_workspace_bytes(ctypes.byref(shape))))
    args = (ctypes.byref(shape), qp, kp, vp, op, wp, wn)
    return Call(lib.bkv_decode_attention, args, "bkv_decode_attention", (shape, s.seq_len, q, k, v, out, workspace))


def decode_attention(s: CacheShape, q, k, v, out, workspace: Optional[torch.Tensor], stream=None) -> None:
    prepare_decode_attention(s, q, k, v, out, workspace)(stream)


def compress_workspace_bytes(s: CacheShape, window: int, nb_max: int, budget: int) -> int:
    return int(load().bkv_compress_workspace_bytes(ctypes.byref(s.c()), window, nb_max, budget))


def _compress_args(s: CacheShape, k, v, q, q_len, window, beacons, n_beacons, nb_max, budget, scores, idx, n_kept,
                   k_out, v_out):
    B, Hkv, D, cap, n = s.batch, s.n_kv_heads, s.head_dim, s.capacity, s.n_layers
    kp, qp, bp, nbp = _score_inputs(s, k, q, q_len, window, beacons, n_beacons, nb_max)
    vp = _layers(v, n, torch.bfloat16, (B, Hkv, cap, D), "v")
    sp = _layers(scores, n, torch.float32, (B, Hkv, cap), "scores")
    ip = _layers(idx, n, torch.int32, (B, Hkv, budget), "idx")
    np_ = _layers(n_kept, n, torch.int32, (B, Hkv), "n_kept")
    ko = _layers(k_out, n, torch.bfloat16, (B, Hkv, budget, D), "k_out")
    vo = _layers(v_out, n, torch.bfloat16, (B, Hkv, budget, D), "v_out")
    return (kp, vp, qp, q_len, window, bp, nbp, nb_max, budget, sp, ip, np_, ko, vo)


def prepare_compress(s: CacheShape, k, v, q, q_len: int, window: int, beacons, n_beacons, nb_max: int,
                     budget: int, scores, idx, n_kept, k_out, v_out, workspace: Optional[torch.Tensor]) -> Call:
    lib = load()
    shape = s.c()
    args = _compress_args(s, k, v, q, q_len, window, beacons, n_beacons, nb_max, budget, scores, idx, n_kept,
                          k_out, v_out)
    need = int(lib.bkv_compress_workspace_bytes(ctypes.byref(shape), window, nb_max, budget))
    wp, wn = _workspace(workspace, need)
    return Call(lib.bkv_compress, (ctypes.byref(shape),) + args + (wp, wn), "bkv_compress",
                (shape, s.seq_len, k, v, q, beacons, n_beacons, scores, idx, n_kept, k_out, v_out, workspace))


def prepare_compress_static(s: CacheShape, k, v, q, q_len: int, window: int, beacons, n_beacons, nb_max: int,
                            budget: int, scores, idx, n_kept, k_out, v_out) -> Call:
    """bkv_compress_static: bkv_compress without a workspace (nothing is allocated; calls on
    one device must not overlap in time)."""
    lib = load()
    shape = s.c()
    args = _compress_args(s, k, v, q, q_len, window, beacons, n_beacons, nb_max, budget, scores, idx, n_kept,
                          k_out, v_out)
    return Call(lib.bkv_compress_static, (ctypes.byref(shape),) + args, "bkv_compress_static",
                (shape, s.seq_len, k, v, q, beacons, n_beacons, scores, idx, n_kept, k_out, v_out))


def compress(s: CacheShape, k, v, q, q_len: int, window: int, beacons, n_beacons, nb_max: int, budget: int,
             scores, idx, n_kept, k_out, v_out, workspace: Optional[torch.Tensor], stream=None) -> None:
    """One compression event over every layer: score, select, compact (bkv_compress)."""
    prepare_compress(s, k, v, q, q_len, window, beacons, n_beacons, nb_max, budget, scores, idx, n_kept, k_out,
                     v_out, workspace)(stream)


def compress_static(s: CacheShape, k, v, q, q_len: int, window: int, beacons, n_beacons, nb_max: int,
                    budget: int, scores, idx, n_kept, k_out, v_out, stream=None) -> None:
    """One compression event with no workspace argument (bkv_compress_static)."""
    prepare_compress_static(s, k, v, q, q_len, window, beacons, n_beacons, nb_max, budget, scores, idx, n_kept,
                            k_out, v_out)(stream)
