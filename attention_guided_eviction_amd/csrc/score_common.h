// Work split and per-unit bookkeeping shared by the two scorer implementations
// (observation rows staged in LDS, or held in registers with keys streamed through LDS).
// Both cut a launch's 256-key tiles into one contiguous share per workgroup and number a
// unit's statistics partials by workgroup, so either finish pass finds the partials of
// its unit arithmetically.
#pragma once

#include "bkv_internal.h"

namespace bkv {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
static_assert(kScoreTile == kWaves * 64, "a tile is 64 keys per wave");

constexpr float kNegInf = -__builtin_inff();

// ---- work split -----------------------------------------------------------------------

__device__ inline int seq_tiles(const ScoreArgs& a, int b) {
  int L = a.seq_len[b];
  L = L < 0 ? 0 : (L > a.capacity ? a.capacity : L);
  return (L + kScoreTile - 1) / kScoreTile;
}

__device__ inline int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Tiles of one layer, all sequences and KV heads (computed by every wave).
__device__ inline int layer_tiles(const ScoreArgs& a) {
  const int lane = threadIdx.x & 63;
  int s = 0;
  for (int b0 = 0; b0 < a.batch; b0 += 64) {
    int x = b0 + lane < a.batch ? seq_tiles(a, b0 + lane) : 0;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    s += x;
  }
  return uniform(s * a.n_kv_heads);
}

struct Cursor {
  int u;      // unit (layer, sequence, KV head) of the launch
  int tile;   // tile within the unit
  int nt;     // tiles of the unit
};

// Unit and tile of global tile c (0 <= c < n_layers * T, T tiles per layer).
__device__ inline Cursor locate(const ScoreArgs& a, long long c, int T) {
  const int lane = threadIdx.x & 63;
  const int layer = static_cast<int>(c / T);
  const int r = static_cast<int>(c - static_cast<long long>(layer) * T);
  // the sequence b with H * S_b <= r < H * S_{b+1}, S_b = tiles of sequences before b
  int base = 0, b = 0, nt = 1, sb = 0;
  for (int b0 = 0; b0 < a.batch; b0 += 64) {
    const int x = b0 + lane < a.batch ? seq_tiles(a, b0 + lane) : 0;
    int incl = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    const unsigned long long hit = __ballot((base + incl) * a.n_kv_heads > r);
    if (hit) {
      const int j = __ffsll(static_cast<long long>(hit)) - 1;
      nt = __shfl(x, j);
      sb = base + __shfl(incl, j) - nt;
      b = b0 + j;
      break;
    }
    base += __shfl(incl, 63);
  }
  const int rr = r - sb * a.n_kv_heads;
  Cursor cur;
  cur.nt = uniform(nt);
  const int h = rr / cur.nt;
  cur.tile = uniform(rr - h * cur.nt);
  cur.u = uniform((layer * a.batch + b) * a.n_kv_heads + h);
  return cur;
}

// Move to the first tile of the next unit that has keys; false past the launch's units
// (never reached while the share has tiles left).
__device__ inline bool next_unit(const ScoreArgs& a, Cursor& cur) {
  const int units = a.n_layers * a.batch * a.n_kv_heads;
  int u = cur.u + 1;
  while (u < units) {
    const int b = (u / a.n_kv_heads) % a.batch;
    const int nt = seq_tiles(a, b);
    if (nt > 0) {
      cur.u = u;
      cur.nt = nt;
      cur.tile = 0;
      return true;
    }
    u = (u / a.n_kv_heads + 1) * a.n_kv_heads;   // the whole sequence is empty
  }
  return false;
}

// The launch's split of N tiles over G workgroups.  Workgroups w and w + G/2 share a CU
// (two per CU, dispatched in index order), and the SIMDs' arbiters favour the older waves,
// so the first half runs faster while both are resident: shares are weighted A : B
// between the halves so that both finish together.  cum(w) is the weight of
// workgroups 0 .. w-1; workgroup w owns tiles [cum(w) N / cum(G), cum(w+1) N / cum(G)).
struct Split {
  long long N;
  int G, H, A, B;
  __device__ long long cum(int w) const {
    return w <= H ? static_cast<long long>(A) * w : static_cast<long long>(A) * H + static_cast<long long>(B) * (w - H);
  }
  __device__ long long begin(int w) const { return cum(w) * N / cum(G); }
  // Workgroup whose share holds global tile c: the last w with begin(w) <= c.
  __device__ int owner(long long c) const {
    const long long x = ((c + 1) * cum(G) + N - 1) / N - 1;   // largest cum(w) allowed
    const long long w = x < static_cast<long long>(A) * H ? x / A : H + (x - static_cast<long long>(A) * H) / B;
    return static_cast<int>(w < G - 1 ? w : G - 1);
  }
};



// ---- per-unit data ------------------------------------------------------------------------

struct UnitInfo {
  int layer, b, h, L, n_obs, nqb;
};

__device__ inline UnitInfo unit_info(const ScoreArgs& a, int u) {
  UnitInfo ui;
  const int per_layer = a.batch * a.n_kv_heads;
  ui.layer = u / per_layer;
  const int rem = u - ui.layer * per_layer;
  ui.b = rem / a.n_kv_heads;
  ui.h = rem - ui.b * a.n_kv_heads;
  int L = a.seq_len[ui.b];
  ui.L = L < 0 ? 0 : (L > a.capacity ? a.capacity : L);
  int nb = 0;
  if (a.nb_max > 0) {
    nb = a.n_beacons[ui.layer][ui.b * a.n_kv_heads + ui.h];
    nb = nb < 0 ? 0 : (nb > a.nb_max ? a.nb_max : nb);
  }
  ui.n_obs = uniform(a.group * a.window + nb);
  ui.nqb = (ui.n_obs + 31) >> 5;
  return ui;
}

// Merge two (max, sum) pairs of exp2 statistics.
__device__ inline void merge_stats(float& m, float& z, float m2, float z2) {
  const float M = fmaxf(m, m2);
  if (M == kNegInf) return;
  z = z * __builtin_amdgcn_exp2f(m - M) + z2 * __builtin_amdgcn_exp2f(m2 - M);
  m = M;
}

}  // namespace
}  // namespace bkv
