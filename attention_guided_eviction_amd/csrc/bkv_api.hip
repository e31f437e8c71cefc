// Host side of the libbkv C ABI (include/bkv.h): argument checks, workspace sizing,
// splitting long models into launches of at most kMaxLayers layers, and launches.
// Nothing here allocates, frees or synchronises (the partials of bkv_compress_static sit
// in a static device array that the code object brings).
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "bkv_internal.h"

// Statistics partials of bkv_compress_static: one copy of this array per device,
// allocated when the code object is loaded on that device and held until the process
// ends.  In host code the name stands for a host-side shadow, never for device memory:
// the device address comes from hipGetSymbolAddress, taken once per device with that
// device current (static_scratch below).
constexpr size_t kStaticScratchBytes = BKV_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace bkv {
namespace {

constexpr size_t kAlign = 256;

static_assert(BKV_MAX_POOL == kFpsThreads * kFpsPoolRowsPerThread, "pool limit of the streaming beacon kernel");
static_assert(BKV_MAX_OBS <= 512, "observation rows the score kernels take");

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Multiply sizes, returning false on overflow.
bool mul_ok(size_t a, size_t b, size_t* out) {
  if (a != 0 && b > SIZE_MAX / a) return false;
  *out = a * b;
  return true;
}

// The kernels move bf16 rows (K, V, queries, beacons, compacted caches) in 16-byte pieces
// and fp32 / int32 arrays element by element: every layer pointer must be aligned to that.
constexpr uintptr_t kRowAlign = 16, kElemAlign = 4;

bkv_status check_shape(const bkv_shape* s) {
  if (s == nullptr || s->seq_len == nullptr) return BKV_EINVAL;
  if (s->n_layers < 1 || s->batch < 1 || s->n_q_heads < 1 || s->n_kv_heads < 1 || s->capacity < 1 ||
      s->head_dim < 1)
    return BKV_EINVAL;
  if (s->n_q_heads % s->n_kv_heads != 0) return BKV_EINVAL;
  if (reinterpret_cast<uintptr_t>(s->seq_len) % kElemAlign != 0) return BKV_EINVAL;
  if (s->head_dim != 64 && s->head_dim != 128) return BKV_EUNSUPPORTED;
  return BKV_OK;
}

template <typename T>
bool all_set(T const* arr, int n) {
  if (arr == nullptr) return false;
  for (int i = 0; i < n; ++i)
    if (arr[i] == nullptr) return false;
  return true;
}

template <typename T>
bool all_aligned(T const* arr, int n, uintptr_t align) {
  for (int i = 0; i < n; ++i)
    if (reinterpret_cast<uintptr_t>(arr[i]) % align != 0) return false;
  return true;
}

// The device memory one call reads and writes.  No output may overlap anything else the
// call touches: an input of any layer, the workspace or another output; inputs may share
// memory.  clash() sorts the regions by address and sweeps them once.
class Footprint {
 public:
  void in(const void* p, size_t n) { add(p, n, false); }
  void out(const void* p, size_t n) { add(p, n, true); }
  template <typename T>
  void in_layers(T const* arr, int n_layers, size_t bytes) {
    for (int l = 0; l < n_layers; ++l) in(arr[l], bytes);
  }
  template <typename T>
  void out_layers(T const* arr, int n_layers, size_t bytes) {
    for (int l = 0; l < n_layers; ++l) out(arr[l], bytes);
  }
  bool clash() {
    std::sort(r_.begin(), r_.end(), [](const R& x, const R& y) { return x.b < y.b; });
    uintptr_t end_any = 0, end_out = 0;   // furthest end of the regions before, of the outputs before
    for (const R& x : r_) {
      if (x.b < (x.out ? end_any : end_out)) return true;
      end_any = std::max(end_any, x.e);
      if (x.out) end_out = std::max(end_out, x.e);
    }
    return false;
  }

 private:
  struct R {
    uintptr_t b, e;
    bool out;
  };
  void add(const void* p, size_t n, bool is_out) {
    if (p == nullptr || n == 0) return;
    const uintptr_t b = reinterpret_cast<uintptr_t>(p);
    r_.push_back(R{b, n > UINTPTR_MAX - b ? UINTPTR_MAX : b + n, is_out});
  }
  std::vector<R> r_;
};

// Bytes of one layer of a [batch][heads][rows][cols] array of `elem`-byte items.
size_t layer_bytes(const bkv_shape* s, int heads, long long rows, long long cols, size_t elem) {
  size_t n = 1;
  if (!mul_ok(n, static_cast<size_t>(s->batch), &n) || !mul_ok(n, static_cast<size_t>(heads), &n) ||
      !mul_ok(n, static_cast<size_t>(rows), &n) || !mul_ok(n, static_cast<size_t>(cols), &n) ||
      !mul_ok(n, elem, &n))
    return SIZE_MAX;
  return n;
}

// Observation rows per unit rounded up to whole 32-row MFMA blocks (at least one block,
// so the workspace is never empty).
int obs_pad_of(const bkv_shape* s, int window, int nb_max) {
  const int g = s->n_q_heads / s->n_kv_heads;
  return std::max(32, round_up(g * window + nb_max, 32));
}

int layers_per_launch(const bkv_shape* s) { return std::min(s->n_layers, kMaxLayers); }

struct ScoreWs {
  size_t part_bytes, total;
};

// Statistics partials of the largest launch when the score call goes out in launches of
// at most `layers` layers and `seqs` sequences (the launches run one after another on
// the stream and reuse the workspace).  Slots per unit depend on the layers of a launch
// only, so the largest launch is one of `seqs` sequences and either `layers` layers or
// the remainder.
ScoreWs score_ws(const bkv_shape* s, int window, int nb_max, int layers, int seqs) {
  ScoreWs w{};
  const size_t obs = static_cast<size_t>(obs_pad_of(s, window, nb_max));
  size_t cells = 0;
  for (int nl : {layers, s->n_layers % layers}) {
    if (nl == 0) continue;
    const size_t units = static_cast<size_t>(nl) * seqs * s->n_kv_heads;
    cells = std::max(cells, units * static_cast<size_t>(score_slots(s->capacity, nl, s->n_kv_heads)));
  }
  w.part_bytes = align_up(cells * obs * sizeof(float));
  w.total = 2 * w.part_bytes;
  return w;
}

// The default grouping: kMaxLayers layers (or all of them) and the whole batch per launch.
ScoreWs score_ws(const bkv_shape* s, int window, int nb_max) {
  return score_ws(s, window, nb_max, layers_per_launch(s), s->batch);
}

bkv_status check_score_args(const bkv_shape* s, const void* const* k, const void* const* q, int32_t q_len,
                            int32_t window, const void* const* beacons, const int32_t* const* n_beacons,
                            int32_t nb_max, float* const* scores) {
  bkv_status st = check_shape(s);
  if (st != BKV_OK) return st;
  if (q_len < 0 || window < 0 || window > q_len || nb_max < 0) return BKV_EINVAL;
  if (!all_set(k, s->n_layers) || !all_set(scores, s->n_layers)) return BKV_EINVAL;
  if (window > 0 && !all_set(q, s->n_layers)) return BKV_EINVAL;
  if (nb_max > 0 && (!all_set(beacons, s->n_layers) || !all_set(n_beacons, s->n_layers))) return BKV_EINVAL;
  if (!all_aligned(k, s->n_layers, kRowAlign) || !all_aligned(scores, s->n_layers, kElemAlign) ||
      (window > 0 && !all_aligned(q, s->n_layers, kRowAlign)) ||
      (nb_max > 0 && (!all_aligned(beacons, s->n_layers, kRowAlign) || !all_aligned(n_beacons, s->n_layers, kElemAlign))))
    return BKV_EINVAL;
  const int g = s->n_q_heads / s->n_kv_heads;
  if (static_cast<long long>(g) * window + nb_max > BKV_MAX_OBS) return BKV_EUNSUPPORTED;
  const size_t kb = layer_bytes(s, s->n_kv_heads, s->capacity, s->head_dim, 2);
  const size_t sb = layer_bytes(s, s->n_kv_heads, s->capacity, 1, 4);
  const size_t qb = layer_bytes(s, s->n_q_heads, q_len, s->head_dim, 2);
  const size_t bb = layer_bytes(s, s->n_kv_heads, nb_max, s->head_dim, 2);
  if (kb == SIZE_MAX || sb == SIZE_MAX || qb == SIZE_MAX || bb == SIZE_MAX) return BKV_EINVAL;
  return BKV_OK;
}

size_t seq_len_bytes(const bkv_shape* s) { return static_cast<size_t>(s->batch) * sizeof(int32_t); }

// What scoring reads: K, the stored queries (window > 0), the beacons and their counts
// (nb_max > 0), the lengths.  Sizes were checked by check_score_args.
void score_inputs(Footprint& f, const bkv_shape* s, const void* const* k, const void* const* q, int32_t q_len,
                  int32_t window, const void* const* beacons, const int32_t* const* n_beacons, int32_t nb_max) {
  f.in_layers(k, s->n_layers, layer_bytes(s, s->n_kv_heads, s->capacity, s->head_dim, 2));
  if (window > 0) f.in_layers(q, s->n_layers, layer_bytes(s, s->n_q_heads, q_len, s->head_dim, 2));
  if (nb_max > 0) {
    f.in_layers(beacons, s->n_layers, layer_bytes(s, s->n_kv_heads, nb_max, s->head_dim, 2));
    f.in_layers(n_beacons, s->n_layers, layer_bytes(s, s->n_kv_heads, 1, 1, 4));
  }
  f.in(s->seq_len, seq_len_bytes(s));
}

bkv_status check_select_args(const bkv_shape* s, const float* const* scores, int32_t budget, int32_t window,
                             int32_t* const* idx, int32_t* const* n_kept) {
  bkv_status st = check_shape(s);
  if (st != BKV_OK) return st;
  if (budget < 1 || window < 0 || window > budget) return BKV_EINVAL;
  if (!all_set(scores, s->n_layers) || !all_set(idx, s->n_layers) || !all_set(n_kept, s->n_layers))
    return BKV_EINVAL;
  if (!all_aligned(scores, s->n_layers, kElemAlign) || !all_aligned(idx, s->n_layers, kElemAlign) ||
      !all_aligned(n_kept, s->n_layers, kElemAlign))
    return BKV_EINVAL;
  if (s->capacity > 64 * kSelectThreads) return BKV_EUNSUPPORTED;
  const size_t sb = layer_bytes(s, s->n_kv_heads, s->capacity, 1, 4);
  const size_t ib = layer_bytes(s, s->n_kv_heads, budget, 1, 4);
  const size_t nb = layer_bytes(s, s->n_kv_heads, 1, 1, 4);
  if (sb == SIZE_MAX || ib == SIZE_MAX) return BKV_EINVAL;
  Footprint f;
  f.in_layers(scores, s->n_layers, sb);
  f.in(s->seq_len, seq_len_bytes(s));
  f.out_layers(idx, s->n_layers, ib);
  f.out_layers(n_kept, s->n_layers, nb);
  return f.clash() ? BKV_EALIAS : BKV_OK;
}

bkv_status check_compact_args(const bkv_shape* s, const void* const* k, const void* const* v,
                              const int32_t* const* idx, const int32_t* const* n_kept, int32_t budget,
                              int32_t out_capacity, void* const* k_out, void* const* v_out) {
  bkv_status st = check_shape(s);
  if (st != BKV_OK) return st;
  if (budget < 1 || out_capacity < budget) return BKV_EINVAL;
  // the kernel numbers a unit's 16-byte row pieces (budget * head_dim / 8) with 32-bit ints
  if (static_cast<long long>(budget) * (s->head_dim / 8) >= (1LL << 30)) return BKV_EUNSUPPORTED;
  if (!all_set(k, s->n_layers) || !all_set(v, s->n_layers) || !all_set(idx, s->n_layers) ||
      !all_set(n_kept, s->n_layers) || !all_set(k_out, s->n_layers) || !all_set(v_out, s->n_layers))
    return BKV_EINVAL;
  if (!all_aligned(k, s->n_layers, kRowAlign) || !all_aligned(v, s->n_layers, kRowAlign) ||
      !all_aligned(k_out, s->n_layers, kRowAlign) || !all_aligned(v_out, s->n_layers, kRowAlign) ||
      !all_aligned(idx, s->n_layers, kElemAlign) || !all_aligned(n_kept, s->n_layers, kElemAlign))
    return BKV_EINVAL;
  const size_t kb = layer_bytes(s, s->n_kv_heads, s->capacity, s->head_dim, 2);
  const size_t ob = layer_bytes(s, s->n_kv_heads, out_capacity, s->head_dim, 2);
  const size_t ib = layer_bytes(s, s->n_kv_heads, budget, 1, 4);
  if (kb == SIZE_MAX || ob == SIZE_MAX || ib == SIZE_MAX) return BKV_EINVAL;
  Footprint f;
  f.in_layers(k, s->n_layers, kb);
  f.in_layers(v, s->n_layers, kb);
  f.in_layers(idx, s->n_layers, ib);
  f.in_layers(n_kept, s->n_layers, layer_bytes(s, s->n_kv_heads, 1, 1, 4));
  f.out_layers(k_out, s->n_layers, ob);
  f.out_layers(v_out, s->n_layers, ob);
  return f.clash() ? BKV_EALIAS : BKV_OK;
}

bkv_status hip_status(hipError_t e) { return e == hipSuccess ? BKV_OK : BKV_EHIP; }

// A launch of nl layers has score_slots() statistics slots per unit; every stats
// workgroup that meets a unit needs one.  Checked for the largest grid the launcher
// uses (the bound grows with the grid) under each share weighting it may choose.  (The
// arithmetic in stats_span_bound shows it always holds; the kernels also turn a unit
// whose partials did not fit into NaN scores rather than drop them silently.)
bool slots_cover(const bkv_shape* s, int nl) {
  const int slots = score_slots(s->capacity, nl, s->n_kv_heads);
  for (const SplitWeights& w : {kWeightsBalanced, kWeightsDefault, SplitWeights{1, 1, 1, 1}})
    if (stats_span_bound(s->capacity, nl, s->n_kv_heads, kScoreMaxGrid, w.stats_old, w.stats_new) > slots)
      return false;
  return true;
}

// The score call's launches: groups of at most `layers` layers and `seqs` sequences, in
// layer-major order, all sharing the partials at `ws_base` (laid out as `ws` says).  A
// group of sequences b0 .. b0+n-1 is the same call on the arrays' sub-blocks that start at
// sequence b0 (every array is sequence-major) and on seq_len + b0.  Arguments were
// checked by check_score_args.
bkv_status run_score(const bkv_shape* shape, const void* const* k, const void* const* q, int32_t q_len,
                     int32_t window, const void* const* beacons, const int32_t* const* n_beacons, int32_t nb_max,
                     int mean, float* const* scores, char* ws_base, const ScoreWs& ws, int layers, int seqs,
                     hipStream_t stream) {
  ScoreArgs a;
  memset(&a, 0, sizeof(a));
  a.part_m = reinterpret_cast<float*>(ws_base);
  a.part_z = reinterpret_cast<float*>(ws_base + ws.part_bytes);
  a.n_q_heads = shape->n_q_heads;
  a.n_kv_heads = shape->n_kv_heads;
  a.group = shape->n_q_heads / shape->n_kv_heads;
  a.capacity = shape->capacity;
  a.q_len = q_len;
  a.window = window;
  a.nb_max = nb_max;
  a.obs_pad = obs_pad_of(shape, window, nb_max);
  a.scale_log2 = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(shape->head_dim)));
  a.mean = mean;
  for (int nl : {layers, shape->n_layers % layers})
    if (nl > 0 && !slots_cover(shape, nl)) return BKV_EUNSUPPORTED;
  const size_t hkv = static_cast<size_t>(shape->n_kv_heads), hq = static_cast<size_t>(shape->n_q_heads);
  const size_t d = static_cast<size_t>(shape->head_dim);
  for (int l0 = 0; l0 < shape->n_layers; l0 += layers) {
    const int nl = std::min(layers, shape->n_layers - l0);
    for (int b0 = 0; b0 < shape->batch; b0 += seqs) {
      const size_t b = static_cast<size_t>(b0);
      a.batch = std::min(seqs, shape->batch - b0);
      a.seq_len = shape->seq_len + b0;
      for (int i = 0; i < nl; ++i) {
        const int l = l0 + i;
        a.k[i] = static_cast<const uint16_t*>(k[l]) + b * hkv * shape->capacity * d;
        a.q[i] = window > 0 ? static_cast<const uint16_t*>(q[l]) + b * hq * q_len * d : nullptr;
        a.beacons[i] = nb_max > 0 ? static_cast<const uint16_t*>(beacons[l]) + b * hkv * nb_max * d : nullptr;
        a.n_beacons[i] = nb_max > 0 ? n_beacons[l] + b * hkv : nullptr;
        a.scores[i] = scores[l] + b * hkv * shape->capacity;
      }
      const bkv_status st = hip_status(launch_score(a, nl, shape->head_dim, stream));
      if (st != BKV_OK) return st;
    }
  }
  return BKV_OK;
}

struct DecodeWs {
  size_t m_bytes, o_bytes, total;
  int chunk_keys, chunks;
};

// Partials of the largest launch (kMaxLayers layers or all of them).
DecodeWs decode_ws(const bkv_shape* s) {
  DecodeWs w{};
  const long long launch_units = static_cast<long long>(std::min(s->n_layers, kMaxLayers)) * s->batch * s->n_kv_heads;
  w.chunk_keys = decode_chunk_keys(launch_units, s->capacity);
  w.chunks = (s->capacity + w.chunk_keys - 1) / w.chunk_keys;
  const size_t cells = static_cast<size_t>(launch_units) * kDecodeMaxGroup * w.chunks;
  w.m_bytes = align_up(cells * sizeof(float));
  w.o_bytes = align_up(cells * static_cast<size_t>(s->head_dim) * sizeof(float));
  w.total = 2 * w.m_bytes + w.o_bytes;
  return w;
}

thread_local char g_last_error[256] = "no HIP error recorded";

// Arguments of one compression event: those of the three stages, and no output of any
// stage may overlap another stage's output, an input or the workspace (later stages read
// the earlier ones' outputs).  `workspace` may be null (the static variant has none).
bkv_status check_compress_args(const bkv_shape* shape, const void* const* k, const void* const* v,
                               const void* const* q, int32_t q_len, int32_t window, const void* const* beacons,
                               const int32_t* const* n_beacons, int32_t nb_max, int32_t budget,
                               float* const* scores, int32_t* const* idx, int32_t* const* n_kept,
                               void* const* k_out, void* const* v_out, const void* workspace,
                               size_t workspace_bytes) {
  bkv_status st = check_score_args(shape, k, q, q_len, window, beacons, n_beacons, nb_max, scores);
  if (st == BKV_OK) st = check_select_args(shape, scores, budget, window, idx, n_kept);
  if (st == BKV_OK) st = check_compact_args(shape, k, v, idx, n_kept, budget, budget, k_out, v_out);
  if (st != BKV_OK) return st;
  Footprint f;
  score_inputs(f, shape, k, q, q_len, window, beacons, n_beacons, nb_max);
  f.in_layers(v, shape->n_layers, layer_bytes(shape, shape->n_kv_heads, shape->capacity, shape->head_dim, 2));
  f.out_layers(scores, shape->n_layers, layer_bytes(shape, shape->n_kv_heads, shape->capacity, 1, 4));
  f.out_layers(idx, shape->n_layers, layer_bytes(shape, shape->n_kv_heads, budget, 1, 4));
  f.out_layers(n_kept, shape->n_layers, layer_bytes(shape, shape->n_kv_heads, 1, 1, 4));
  f.out_layers(k_out, shape->n_layers, layer_bytes(shape, shape->n_kv_heads, budget, shape->head_dim, 2));
  f.out_layers(v_out, shape->n_layers, layer_bytes(shape, shape->n_kv_heads, budget, shape->head_dim, 2));
  if (workspace != nullptr) f.out(workspace, std::min(workspace_bytes, score_ws(shape, window, nb_max).total));
  return f.clash() ? BKV_EALIAS : BKV_OK;
}

// ---- the allocation-free compression event ----------------------------------------------
// Its statistics partials live in the file-scope array `scratch` (top of this file).

PerDeviceOnce g_scratch_once;
char* g_scratch_addr[kMaxDevices];

hipError_t static_scratch(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return note_hip_error(e, "compress_static: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return note_hip_error(hipErrorInvalidDevice, "compress_static: device");
  e = once_per_device(g_scratch_once, [dev] {
    void* p = nullptr;
    const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (r == hipSuccess) g_scratch_addr[dev] = static_cast<char*>(p);
    return r;
  });
  if (e != hipSuccess) return note_hip_error(e, "compress_static: hipGetSymbolAddress");
  *out = g_scratch_addr[dev];
  return hipSuccess;
}

struct ScoreGroups {
  int layers, seqs;   // per launch; layers == 0: even one layer of one sequence does not fit
};

// The launch grouping of the static variant: the fewest launches whose partials fit the
// scratch (ties to more layers per launch); the whole call in the default grouping when
// that fits.  Sequence groups are evened out over the batch.
ScoreGroups static_groups(const bkv_shape* s, int window, int nb_max) {
  ScoreGroups best{0, 0};
  long long best_launches = 0;
  for (int nl = layers_per_launch(s); nl >= 1; --nl) {
    if (score_ws(s, window, nb_max, nl, 1).total > kStaticScratchBytes) continue;
    int lo = 1, hi = s->batch;   // the most sequences per launch that fit
    while (lo < hi) {
      const int mid = lo + (hi - lo + 1) / 2;
      if (score_ws(s, window, nb_max, nl, mid).total <= kStaticScratchBytes)
        lo = mid;
      else
        hi = mid - 1;
    }
    const int seq_groups = (s->batch + lo - 1) / lo;
    const int seqs = (s->batch + seq_groups - 1) / seq_groups;
    const long long launches = static_cast<long long>((s->n_layers + nl - 1) / nl) * seq_groups;
    if (best.layers == 0 || launches < best_launches) {
      best = ScoreGroups{nl, seqs};
      best_launches = launches;
    }
  }
  return best;
}


}  // namespace

hipError_t note_hip_error(hipError_t e, const char* where) {
  if (e != hipSuccess) snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%d)", where, hipGetErrorString(e), e);
  return e;
}

}  // namespace bkv

using namespace bkv;

extern "C" {

const char* bkv_status_string(int32_t status) {
  switch (status) {
    case BKV_OK: return "BKV_OK: success";
    case BKV_EINVAL: return "BKV_EINVAL: invalid argument";
    case BKV_EUNSUPPORTED: return "BKV_EUNSUPPORTED: valid but unsupported size or head_dim";
    case BKV_EALIAS: return "BKV_EALIAS: output overlaps an input";
    case BKV_EWORKSPACE: return "BKV_EWORKSPACE: workspace missing or too small";
    case BKV_EHIP: return "BKV_EHIP: HIP runtime or launch failure";
  }
  return "BKV_?: unknown status";
}

const char* bkv_version(void) { return "0.2.0"; }

const char* bkv_last_error(void) { return g_last_error; }

size_t bkv_score_workspace_bytes(const bkv_shape* shape, int32_t window, int32_t nb_max) {
  if (check_shape(shape) != BKV_OK || window < 0 || nb_max < 0) return 0;
  return score_ws(shape, window, nb_max).total;
}

bkv_status bkv_score(const bkv_shape* shape, const void* const* k, const void* const* q, int32_t q_len,
                     int32_t window, const void* const* beacons, const int32_t* const* n_beacons, int32_t nb_max,
                     float* const* scores, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return bkv_score_agg(shape, k, q, q_len, window, beacons, n_beacons, nb_max, BKV_AGG_MAX, scores, workspace,
                       workspace_bytes, stream);
}

bkv_status bkv_score_agg(const bkv_shape* shape, const void* const* k, const void* const* q, int32_t q_len,
                         int32_t window, const void* const* beacons, const int32_t* const* n_beacons, int32_t nb_max,
                         int32_t aggregation, float* const* scores, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  if (aggregation != BKV_AGG_MAX && aggregation != BKV_AGG_MEAN) return BKV_EINVAL;
  bkv_status st = check_score_args(shape, k, q, q_len, window, beacons, n_beacons, nb_max, scores);
  if (st != BKV_OK) return st;
  const ScoreWs ws = score_ws(shape, window, nb_max);
  if (workspace == nullptr || workspace_bytes < ws.total ||
      reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
    return BKV_EWORKSPACE;
  Footprint f;
  score_inputs(f, shape, k, q, q_len, window, beacons, n_beacons, nb_max);
  f.out_layers(scores, shape->n_layers, layer_bytes(shape, shape->n_kv_heads, shape->capacity, 1, 4));
  f.out(workspace, ws.total);
  if (f.clash()) return BKV_EALIAS;
  return run_score(shape, k, q, q_len, window, beacons, n_beacons, nb_max, aggregation == BKV_AGG_MEAN ? 1 : 0,
                   scores, static_cast<char*>(workspace), ws, layers_per_launch(shape), shape->batch, stream);
}

size_t bkv_select_workspace_bytes(const bkv_shape* shape, int32_t budget) {
  (void)shape;
  (void)budget;
  return 0;
}

bkv_status bkv_select_topk(const bkv_shape* shape, const float* const* scores, int32_t budget, int32_t window,
                           int32_t* const* idx, int32_t* const* n_kept, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  (void)workspace;
  (void)workspace_bytes;
  bkv_status st = check_select_args(shape, scores, budget, window, idx, n_kept);
  if (st != BKV_OK) return st;
  SelectArgs a;
  memset(&a, 0, sizeof(a));
  a.seq_len = shape->seq_len;
  a.batch = shape->batch;
  a.n_kv_heads = shape->n_kv_heads;
  a.capacity = shape->capacity;
  a.budget = budget;
  a.window = window;
  for (int l0 = 0; l0 < shape->n_layers; l0 += kMaxLayers) {
    const int nl = std::min(kMaxLayers, shape->n_layers - l0);
    for (int i = 0; i < nl; ++i) {
      a.scores[i] = scores[l0 + i];
      a.idx[i] = idx[l0 + i];
      a.n_kept[i] = n_kept[l0 + i];
    }
    st = hip_status(launch_select(a, nl, stream));
    if (st != BKV_OK) return st;
  }
  return BKV_OK;
}

bkv_status bkv_compact(const bkv_shape* shape, const void* const* k, const void* const* v,
                       const int32_t* const* idx, const int32_t* const* n_kept, int32_t budget, void* const* k_out,
                       void* const* v_out, hipStream_t stream) {
  return bkv_compact_into(shape, k, v, idx, n_kept, budget, budget, k_out, v_out, stream);
}

bkv_status bkv_compact_into(const bkv_shape* shape, const void* const* k, const void* const* v,
                            const int32_t* const* idx, const int32_t* const* n_kept, int32_t budget,
                            int32_t out_capacity, void* const* k_out, void* const* v_out, hipStream_t stream) {
  bkv_status st = check_compact_args(shape, k, v, idx, n_kept, budget, out_capacity, k_out, v_out);
  if (st != BKV_OK) return st;
  CompactArgs a;
  memset(&a, 0, sizeof(a));
  a.batch = shape->batch;
  a.n_kv_heads = shape->n_kv_heads;
  a.capacity = shape->capacity;
  a.budget = budget;
  a.out_capacity = out_capacity;
  for (int l0 = 0; l0 < shape->n_layers; l0 += kMaxLayers) {
    const int nl = std::min(kMaxLayers, shape->n_layers - l0);
    for (int i = 0; i < nl; ++i) {
      a.k[i] = static_cast<const uint16_t*>(k[l0 + i]);
      a.v[i] = static_cast<const uint16_t*>(v[l0 + i]);
      a.idx[i] = idx[l0 + i];
      a.n_kept[i] = n_kept[l0 + i];
      a.k_out[i] = static_cast<uint16_t*>(k_out[l0 + i]);
      a.v_out[i] = static_cast<uint16_t*>(v_out[l0 + i]);
    }
    st = hip_status(launch_compact(a, nl, shape->head_dim, stream));
    if (st != BKV_OK) return st;
  }
  return BKV_OK;
}

bkv_status bkv_update_beacons(const bkv_shape* shape, const void* const* beacons_in, const int32_t* const* n_in,
                              int32_t nb_max, const void* const* q_new, int32_t q_len, int32_t t_new,
                              void* const* beacons_out, int32_t* const* n_out, hipStream_t stream) {
  return bkv_update_beacons_policy(shape, beacons_in, n_in, nb_max, q_new, q_len, t_new, BKV_BEACON_FPS, beacons_out,
                                   n_out, stream);
}

bkv_status bkv_update_beacons_policy(const bkv_shape* shape, const void* const* beacons_in,
                                     const int32_t* const* n_in, int32_t nb_max, const void* const* q_new,
                                     int32_t q_len, int32_t t_new, int32_t policy,
                                     void* const* beacons_out, int32_t* const* n_out, hipStream_t stream) {
  if (policy != BKV_BEACON_FPS && policy != BKV_BEACON_INITIAL) return BKV_EINVAL;
  bkv_status st = check_shape(shape);
  if (st != BKV_OK) return st;
  if (nb_max < 1 || q_len < 0 || t_new < 0 || t_new > q_len) return BKV_EINVAL;
  if (!all_set(beacons_in, shape->n_layers) || !all_set(n_in, shape->n_layers) ||
      !all_set(beacons_out, shape->n_layers) || !all_set(n_out, shape->n_layers))
    return BKV_EINVAL;
  if (t_new > 0 && !all_set(q_new, shape->n_layers)) return BKV_EINVAL;
  if (!all_aligned(beacons_in, shape->n_layers, kRowAlign) || !all_aligned(beacons_out, shape->n_layers, kRowAlign) ||
      !all_aligned(n_in, shape->n_layers, kElemAlign) || !all_aligned(n_out, shape->n_layers, kElemAlign) ||
      (t_new > 0 && !all_aligned(q_new, shape->n_layers, kRowAlign)))
    return BKV_EINVAL;
  const int g = shape->n_q_heads / shape->n_kv_heads;
  const long long pool_max = nb_max + static_cast<long long>(g) * t_new;
  if (policy == BKV_BEACON_FPS && pool_max > BKV_MAX_POOL) return BKV_EUNSUPPORTED;
  const size_t bb = layer_bytes(shape, shape->n_kv_heads, nb_max, shape->head_dim, 2);
  const size_t qb = layer_bytes(shape, shape->n_q_heads, q_len, shape->head_dim, 2);
  const size_t cb = layer_bytes(shape, shape->n_kv_heads, 1, 1, 4);
  if (bb == SIZE_MAX || qb == SIZE_MAX) return BKV_EINVAL;
  Footprint f;
  f.in_layers(beacons_in, shape->n_layers, bb);
  f.in_layers(n_in, shape->n_layers, cb);
  if (t_new > 0) f.in_layers(q_new, shape->n_layers, qb);
  f.out_layers(beacons_out, shape->n_layers, bb);
  f.out_layers(n_out, shape->n_layers, cb);
  if (f.clash()) return BKV_EALIAS;
  FpsArgs a;
  memset(&a, 0, sizeof(a));
  a.batch = shape->batch;
  a.n_q_heads = shape->n_q_heads;
  a.n_kv_heads = shape->n_kv_heads;
  a.group = g;
  a.nb_max = nb_max;
  a.q_len = q_len;
  a.t_new = t_new;
  for (int l0 = 0; l0 < shape->n_layers; l0 += kMaxLayers) {
    const int nl = std::min(kMaxLayers, shape->n_layers - l0);
    for (int i = 0; i < nl; ++i) {
      a.beacons_in[i] = static_cast<const uint16_t*>(beacons_in[l0 + i]);
      a.n_in[i] = n_in[l0 + i];
      a.q_new[i] = t_new > 0 ? static_cast<const uint16_t*>(q_new[l0 + i]) : nullptr;
      a.beacons_out[i] = static_cast<uint16_t*>(beacons_out[l0 + i]);
      a.n_out[i] = n_out[l0 + i];
    }
    st = hip_status(policy == BKV_BEACON_FPS ? launch_fps(a, nl, shape->head_dim, static_cast<int>(pool_max), stream)
                                             : launch_initial(a, nl, shape->head_dim, stream));
    if (st != BKV_OK) return st;
  }
  return BKV_OK;
}

size_t bkv_compress_workspace_bytes(const bkv_shape* shape, int32_t window, int32_t nb_max, int32_t budget) {
  (void)budget;
  return bkv_score_workspace_bytes(shape, window, nb_max);
}

bkv_status bkv_compress(const bkv_shape* shape, const void* const* k, const void* const* v, const void* const* q,
                        int32_t q_len, int32_t window, const void* const* beacons, const int32_t* const* n_beacons,
                        int32_t nb_max, int32_t budget, float* const* scores, int32_t* const* idx,
                        int32_t* const* n_kept, void* const* k_out, void* const* v_out, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  bkv_status st = check_compress_args(shape, k, v, q, q_len, window, beacons, n_beacons, nb_max, budget, scores, idx,
                                      n_kept, k_out, v_out, workspace, workspace_bytes);
  if (st != BKV_OK) return st;
  st = bkv_score(shape, k, q, q_len, window, beacons, n_beacons, nb_max, scores, workspace, workspace_bytes, stream);
  if (st != BKV_OK) return st;
  st = bkv_select_topk(shape, scores, budget, window, idx, n_kept, nullptr, 0, stream);
  if (st != BKV_OK) return st;
  return bkv_compact(shape, k, v, idx, n_kept, budget, k_out, v_out, stream);
}

bkv_status bkv_compress_static(const bkv_shape* shape, const void* const* k, const void* const* v,
                               const void* const* q, int32_t q_len, int32_t window, const void* const* beacons,
                               const int32_t* const* n_beacons, int32_t nb_max, int32_t budget,
                               float* const* scores, int32_t* const* idx, int32_t* const* n_kept,
                               void* const* k_out, void* const* v_out, hipStream_t stream) {
  bkv_status st = check_compress_args(shape, k, v, q, q_len, window, beacons, n_beacons, nb_max, budget, scores, idx,
                                      n_kept, k_out, v_out, nullptr, 0);
  if (st != BKV_OK) return st;
  const ScoreGroups g = static_groups(shape, window, nb_max);
  if (g.layers == 0) {
    snprintf(g_last_error, sizeof(g_last_error),
             "compress_static: one layer of one sequence needs %zu bytes of statistics partials; the static "
             "scratch holds %zu",
             score_ws(shape, window, nb_max, 1, 1).total, kStaticScratchBytes);
    return BKV_EUNSUPPORTED;
  }
  char* base = nullptr;
  st = hip_status(static_scratch(&base));
  if (st != BKV_OK) return st;
  st = run_score(shape, k, q, q_len, window, beacons, n_beacons, nb_max, 0, scores, base,
                 score_ws(shape, window, nb_max, g.layers, g.seqs), g.layers, g.seqs, stream);
  if (st != BKV_OK) return st;
  st = bkv_select_topk(shape, scores, budget, window, idx, n_kept, nullptr, 0, stream);
  if (st != BKV_OK) return st;
  return bkv_compact(shape, k, v, idx, n_kept, budget, k_out, v_out, stream);
}

size_t bkv_decode_workspace_bytes(const bkv_shape* shape) {
  if (check_shape(shape) != BKV_OK || shape->n_q_heads / shape->n_kv_heads > kDecodeMaxGroup) return 0;
  return decode_ws(shape).total;
}

bkv_status bkv_decode_attention(const bkv_shape* shape, const void* const* q, const void* const* k,
                                const void* const* v, float* const* out, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  bkv_status st = check_shape(shape);
  if (st != BKV_OK) return st;
  const int g = shape->n_q_heads / shape->n_kv_heads;
  if (g > kDecodeMaxGroup) return BKV_EUNSUPPORTED;
  if (!all_set(q, shape->n_layers) || !all_set(k, shape->n_layers) || !all_set(v, shape->n_layers) ||
      !all_set(out, shape->n_layers))
    return BKV_EINVAL;
  if (!all_aligned(q, shape->n_layers, kRowAlign) || !all_aligned(k, shape->n_layers, kRowAlign) ||
      !all_aligned(v, shape->n_layers, kRowAlign) || !all_aligned(out, shape->n_layers, kElemAlign))
    return BKV_EINVAL;
  const DecodeWs ws = decode_ws(shape);
  if (workspace == nullptr || workspace_bytes < ws.total || reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
    return BKV_EWORKSPACE;
  const size_t qb = layer_bytes(shape, shape->n_q_heads, 1, shape->head_dim, 2);
  const size_t ob = layer_bytes(shape, shape->n_q_heads, 1, shape->head_dim, 4);
  const size_t kb = layer_bytes(shape, shape->n_kv_heads, shape->capacity, shape->head_dim, 2);
  if (qb == SIZE_MAX || ob == SIZE_MAX || kb == SIZE_MAX) return BKV_EINVAL;
  Footprint f;
  f.in_layers(q, shape->n_layers, qb);
  f.in_layers(k, shape->n_layers, kb);
  f.in_layers(v, shape->n_layers, kb);
  f.in(shape->seq_len, seq_len_bytes(shape));
  f.out_layers(out, shape->n_layers, ob);
  f.out(workspace, ws.total);
  if (f.clash()) return BKV_EALIAS;
  DecodeArgs a;
  memset(&a, 0, sizeof(a));
  char* wsp = static_cast<char*>(workspace);
  a.part_m = reinterpret_cast<float*>(wsp);
  a.part_z = reinterpret_cast<float*>(wsp + ws.m_bytes);
  a.part_o = reinterpret_cast<float*>(wsp + 2 * ws.m_bytes);
  a.seq_len = shape->seq_len;
  a.batch = shape->batch;
  a.n_q_heads = shape->n_q_heads;
  a.n_kv_heads = shape->n_kv_heads;
  a.group = g;
  a.capacity = shape->capacity;
  a.chunk_keys = ws.chunk_keys;
  a.chunks = ws.chunks;
  a.scale_log2 = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(shape->head_dim)));
  for (int l0 = 0; l0 < shape->n_layers; l0 += kMaxLayers) {
    const int nl = std::min(kMaxLayers, shape->n_layers - l0);
    for (int i = 0; i < nl; ++i) {
      a.q[i] = static_cast<const uint16_t*>(q[l0 + i]);
      a.k[i] = static_cast<const uint16_t*>(k[l0 + i]);
      a.v[i] = static_cast<const uint16_t*>(v[l0 + i]);
      a.out[i] = out[l0 + i];
    }
    st = hip_status(launch_decode(a, nl, shape->head_dim, stream));
    if (st != BKV_OK) return st;
  }
  return BKV_OK;
}

}  // extern "C"
