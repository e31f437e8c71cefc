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

// ---- score -------------------------------------------------------------------------------
// Keys per workgroup tile: 4 waves x 64 keys (two 32-key MFMA fragments per wave).
constexpr int kScoreWaves = 4;
constexpr int kKeysPerWave = 64;
constexpr int kScoreTile = kScoreWaves * kKeysPerWave;

struct ScoreArgs {
  const uint16_t* k[kMaxLayers];
  const uint16_t* q[kMaxLayers];
  const uint16_t* beacons[kMaxLayers];
  const int32_t* n_beacons[kMaxLayers];
  float* scores[kMaxLayers];
  const int32_t* seq_len;
  float* part_m;        // [unit][tile][obs_pad] running max (log2 domain)
  float* part_z;        // [unit][tile][obs_pad] sum of exp2(t - m)
  float* lse;           // [unit][obs_pad] log2-sum-exp2 per observation row
  int batch, n_q_heads, n_kv_heads, group, capacity;
  int q_len, window, nb_max;
  int obs_pad;          // observation rows per unit rounded up to 32 (launch-wide)
  int tiles;            // ceil(capacity / kScoreTile)
  int units;            // units in this launch (layers * batch * n_kv_heads)
  float scale_log2;     // log2(e) / sqrt(head_dim)
};

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

}  // namespace bkv
