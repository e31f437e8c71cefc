// Internal declarations shared by the gfx950 kernels and the host side of libbkv.
// Not installed; the public interface is include/bkv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "bkv.h"

namespace bkv {

// One launch covers up to this many layers; the host splits longer models.
constexpr int kMaxLayers = 48;

// ---- score ----------------------------------------------------------------------------------
// Two grid-stride kernels per chunk of units (see score.hip).  Key tiles are WAVES*64 keys;
// an item is kScoreTilesPerItem consecutive tiles of one unit.
constexpr int kScoreTilesPerItem = 4;

struct ScoreArgs {
  const uint16_t* k[kMaxLayers];
  const uint16_t* q[kMaxLayers];
  const uint16_t* beacons[kMaxLayers];
  const int32_t* n_beacons[kMaxLayers];
  float* scores[kMaxLayers];
  const int32_t* seq_len;
  float* part_m;        // [unit][split][obs_pad] running max (log2 domain)
  float* part_z;        // [unit][split][obs_pad] sum of exp2(t - m)
  int batch, n_q_heads, n_kv_heads, group, capacity;
  int q_len, window, nb_max;
  int obs_pad;          // observation rows per unit rounded up to 32 (launch-wide)
  int unit0;            // first unit of the current chunk (set by the launcher)
  int units;            // units in the chunk (the whole call on entry to the launcher)
  int tps;              // tiles per item
  int splits;           // items per unit (set by the launcher)
  float scale_log2;     // log2(e) / sqrt(head_dim)
};

// Waves per score workgroup for a given padded observation count, and the split count the
// launcher will use (the workspace is sized from these).
int score_waves(int obs_pad);
inline int score_splits(int capacity, int obs_pad) {
  const int tile = score_waves(obs_pad) * 64;
  const int ntiles = (capacity + tile - 1) / tile;
  return (ntiles + kScoreTilesPerItem - 1) / kScoreTilesPerItem;
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
};

// ---- beacons -----------------------------------------------------------------------------
constexpr int kFpsThreads = 512;

struct FpsArgs {
  const uint16_t* beacons_in[kMaxLayers];
  const int32_t* n_in[kMaxLayers];
  const uint16_t* q_new[kMaxLayers];
  uint16_t* beacons_out[kMaxLayers];
  int32_t* n_out[kMaxLayers];
  int batch, n_q_heads, n_kv_heads, group, nb_max, q_len, t_new;
};

// Launchers (return hipSuccess or the launch error).  n_layers <= kMaxLayers.
hipError_t launch_score(const ScoreArgs& a, int n_layers, int head_dim, hipStream_t s);
hipError_t launch_select(const SelectArgs& a, int n_layers, hipStream_t s);
hipError_t launch_compact(const CompactArgs& a, int n_layers, int head_dim, hipStream_t s);
hipError_t launch_fps(const FpsArgs& a, int n_layers, int head_dim, int pool_max, hipStream_t s);

inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

// Remember the HIP error behind a BKV_EHIP (per calling thread) together with the name of
// the call that returned it; returns `e` unchanged.
hipError_t note_hip_error(hipError_t e, const char* where);

}  // namespace bkv
