// Internal declarations shared by the gfx950 kernels and the host side of libbkv.
// Not installed; the public interface is include/bkv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "bkv.h"

namespace bkv {

// One launch covers up to this many layers; the host splits longer models.
constexpr int kMaxLayers = 48;

// Kernel attributes (the dynamic LDS limit) belong to a device: `set` runs once for each
// device it is called on (the current one) and its result is returned on every later call
// there.  Devices past kMaxDevices are refused.
constexpr int kMaxDevices = 64;
struct PerDeviceOnce {
  std::once_flag flag[kMaxDevices];
  hipError_t err[kMaxDevices] = {};
};

template <class F>
hipError_t once_per_device(PerDeviceOnce& o, F set) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(o.flag[dev], [&] { o.err[dev] = set(); });
  return o.err[dev];
}

// ---- score ----------------------------------------------------------------------------------
// Two persistent kernels (see score.hip).  A tile is kScoreTile keys of one unit; the grid is
// at most kScoreMaxGrid workgroups, each taking an equal contiguous share of the launch's
// tiles, so at most grid / (n_layers * n_kv_heads) + 2 workgroups share one unit.
constexpr int kScoreTile = 256;
constexpr int kScoreMaxGrid = 1024;

// Share weights of the older : newer workgroup of each CU when two run on it (workgroups w
// and w + grid/2): the wave arbiter favours the older one, so equal shares leave the newer
// one finishing last.  Chosen per launch by the launcher from per-workgroup timestamps and
// interleaved timings on MI355X: where every wave of the register-row stats pass owns the
// same number of 32-row blocks (a multiple of 4 blocks), 3 : 2 for the stats pass and 4 : 3
// for the finish pass; otherwise 9 : 7 and 15 : 13.  The stats weights also number the
// statistics partials, so both passes of a call use the same ones.
struct SplitWeights {
  int stats_old, stats_new, finish_old, finish_new;
};
constexpr SplitWeights kWeightsBalanced = {3, 2, 4, 3};
constexpr SplitWeights kWeightsDefault = {9, 7, 15, 13};
// The most skewed stats weights any launch uses (the slot bound below depends on them).
constexpr int kMaxSkewOld = 3, kMaxSkewNew = 2;
static_assert(kWeightsBalanced.stats_old * kMaxSkewNew <= kMaxSkewOld * kWeightsBalanced.stats_new &&
                  kWeightsDefault.stats_old * kMaxSkewNew <= kMaxSkewOld * kWeightsDefault.stats_new,
              "stats weights within the slot bound");

struct ScoreArgs {
  const uint16_t* k[kMaxLayers];
  const uint16_t* q[kMaxLayers];
  const uint16_t* beacons[kMaxLayers];
  const int32_t* n_beacons[kMaxLayers];
  float* scores[kMaxLayers];
  const int32_t* seq_len;
  float* part_m;        // [unit][slot][obs_pad] running max (log2 domain)
  float* part_z;        // [unit][slot][obs_pad] sum of exp2(t - m)
  int n_layers;         // layers in this launch (set by the launcher)
  int batch, n_q_heads, n_kv_heads, group, capacity;
  int q_len, window, nb_max;
  int obs_pad;          // observation rows per unit rounded up to 32 (launch-wide)
  int slots;            // statistics slots per unit (set by the launcher)
  int stats_grid;       // workgroups of the stats pass, whose split numbers the partials
  int paired;           // stats pass: two workgroups per CU, w and w + grid/2
  int finish_paired;    // finish pass: the same on its own grid
  SplitWeights weights; // older : newer share weights of a pair (all set by the launcher)
  int mean;             // 1: mean of the observation rows' attention weights, 0: max
  float scale_log2;     // log2(e) / sqrt(head_dim)
};

// Statistics slots per unit for a launch of n_layers layers (the workspace is sized from
// this): one per workgroup that can share a unit, never more than the unit's tiles.  The
// smallest stats share is at least 2 B / (A + B) of the mean (weights A : B up to the
// most skewed), so at most grid (A + B) / (2 B) / units + 2 workgroups meet one unit.
inline int score_slots(int capacity, int n_layers, int n_kv_heads) {
  const int tiles = (capacity + kScoreTile - 1) / kScoreTile;
  const int sharing = kScoreMaxGrid * (kMaxSkewOld + kMaxSkewNew) / (2 * kMaxSkewNew) /
                          (n_layers * n_kv_heads) + 2;
  return tiles < sharing ? tiles : sharing;
}

// Most stats workgroups that can meet one unit of a launch over n_layers layers, for any
// sequence lengths: `grid` workgroups, the first half weighing A and the rest B (A >= B;
// A = B = 1 for equal shares), C = A * (grid / 2) + B * (grid - grid / 2).  Of N tiles,
// the owner of tile c is the workgroup at cum value x(c) = ceil((c + 1) C / N) - 1, and the
// workgroup index grows by at most one per B cum values.  A unit's nt tiles come with
// every other (layer, KV head) of its sequence at the same length, so nt <= N / U
// (U = n_layers * n_kv_heads); its first and last tiles' cum values then differ by at most
// ceil((nt - 1) C / N) <= ceil(C / U), their workgroups by at most ceil(C / (U B)).  Never
// more than the unit's tiles or the grid either.  Since C / B <= kScoreMaxGrid (A + B) /
// (2 B) at the most skewed weights, this never exceeds score_slots().
inline int stats_span_bound(int capacity, int n_layers, int n_kv_heads, int grid, int A, int B) {
  const long long u = static_cast<long long>(n_layers) * n_kv_heads;
  const long long c = static_cast<long long>(A) * (grid / 2) + static_cast<long long>(B) * (grid - grid / 2);
  long long span = (c + u * B - 1) / (u * B) + 1;
  const long long tiles = (capacity + kScoreTile - 1) / kScoreTile;
  span = span < tiles ? span : tiles;
  span = span < grid ? span : grid;
  return static_cast<int>(span);
}

// ---- select ------------------------------------------------------------------------------
constexpr int kSelectThreads = 1024;

struct SelectArgs {
  const float* scores[kMaxLayers];
  int32_t* idx[kMaxLayers];
  int32_t* n_kept[kMaxLayers];
  const int32_t* seq_len;
  int batch, n_kv_heads, capacity, budget, window;
};

// ---- compact -----------------------------------------------------------------------------
struct CompactArgs {
  const uint16_t* k[kMaxLayers];
  const uint16_t* v[kMaxLayers];
  const int32_t* idx[kMaxLayers];
  const int32_t* n_kept[kMaxLayers];
  uint16_t* k_out[kMaxLayers];
  uint16_t* v_out[kMaxLayers];
  int batch, n_kv_heads, capacity, budget;
  int out_capacity;     // rows per (sequence, KV head) of k_out / v_out (>= budget)
};

// ---- beacons -----------------------------------------------------------------------------
constexpr int kFpsThreads = 1024;       // workgroup of both beacon kernels
constexpr int kFpsRegisterPool = 768;   // pools up to this many rows: one row per thread, in registers
constexpr int kFpsPoolRowsPerThread = 16;   // larger pools: up to 16 rows per thread, streamed

struct FpsArgs {
  const uint16_t* beacons_in[kMaxLayers];
  const int32_t* n_in[kMaxLayers];
  const uint16_t* q_new[kMaxLayers];
  uint16_t* beacons_out[kMaxLayers];
  int32_t* n_out[kMaxLayers];
  int batch, n_q_heads, n_kv_heads, group, nb_max, q_len, t_new;
};

// ---- decode attention ----------------------------------------------------------------------

constexpr int kDecodeMaxGroup = 8;     // query heads per KV head

// Keys per decode workgroup (4 waves, each a quarter in blocks of 64 keys): 1024, or 512 or
// 256 when larger chunks would leave fewer than kDecodeMinGrid workgroups per launch (four
// per CU of MI355X).  Measured: a 64-unit launch over 2048 keys took 34 us with 1024-key
// chunks and 25 us with 256; a 112-unit launch over 4096 keys (448 workgroups of 1024 keys)
// took 62.5 us with 1024-key chunks, 68 us with 512 and 59 us with 256.
constexpr int kDecodeMaxChunk = 1024;
constexpr int kDecodeMinChunk = 256;
constexpr int kDecodeMinGrid = 1024;
inline int decode_chunk_keys(long long launch_units, int capacity) {
  int c = kDecodeMaxChunk;
  while (c > kDecodeMinChunk && launch_units * ((capacity + c - 1) / c) < kDecodeMinGrid)
    c /= 2;
  return c;
}

struct DecodeArgs {
  const uint16_t* q[kMaxLayers];     // [batch][n_q_heads][head_dim]
  const uint16_t* k[kMaxLayers];     // [batch][n_kv_heads][capacity][head_dim]
  const uint16_t* v[kMaxLayers];
  float* out[kMaxLayers];            // [batch][n_q_heads][head_dim]
  const int32_t* seq_len;
  float* part_m;                     // [unit][kDecodeMaxGroup][chunks] running max (log2 domain)
  float* part_z;                     // same cells: sum of exp2(t - m)
  float* part_o;                     // [cell][head_dim] unnormalised output
  int batch, n_q_heads, n_kv_heads, group, capacity;
  int chunk_keys;                    // keys per workgroup (decode_chunk_keys)
  int chunks;                        // ceil(capacity / chunk_keys)
  float scale_log2;
};

// Launchers (return hipSuccess or the launch error).  n_layers <= kMaxLayers.
hipError_t launch_score(const ScoreArgs& a, int n_layers, int head_dim, hipStream_t s);
// Statistics pass with the observation rows in registers, for units of at most 512 padded
// rows at head_dim 128 and kQsMaxRows at 64 (qs_stats_covers): resident workgroups per CU,
// and one launch on `grid` workgroups (a.n_layers, a.slots, a.stats_grid and a.paired set
// by the caller).
constexpr int kQsMaxRows = 384;
bool qs_stats_covers(int head_dim, int obs_pad);
hipError_t qs_stats_occupancy(int head_dim, int obs_pad, int* per_cu);
hipError_t launch_qs_stats(const ScoreArgs& a, int head_dim, int grid, hipStream_t s);
hipError_t launch_select(const SelectArgs& a, int n_layers, hipStream_t s);
hipError_t launch_compact(const CompactArgs& a, int n_layers, int head_dim, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int n_layers, int head_dim, hipStream_t s);
hipError_t launch_fps(const FpsArgs& a, int n_layers, int head_dim, int pool_max, hipStream_t s);
hipError_t launch_initial(const FpsArgs& a, int n_layers, int head_dim, hipStream_t s);

inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

// Remember the HIP error behind a BKV_EHIP (per calling thread) together with the name of
// the call that returned it; returns `e` unchanged.
hipError_t note_hip_error(hipError_t e, const char* where);

}  // namespace bkv
