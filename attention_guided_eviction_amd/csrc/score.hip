// Max-aggregated attention scores of cached keys (BeaconKV page, Figure 5 (b), (c);
// Table 2 caption: max over heads and queries).
//
// Per unit (layer, sequence, KV head) the observation rows are the last `window`
// queries of every query head of the group followed by the live beacons.  For key j
//     score_j = max_i exp(s_ij - lse_i),   s_ij = q_i . k_j / sqrt(d),
// where lse_i normalises row i over all valid keys.  Everything runs in the log2
// domain: t_ij = s_ij * log2(e) and score_j = exp2(max_i(t_ij - lse2_i)).
//
// Two passes over K, each one MFMA contraction of a 256-key tile with all observation
// rows (bf16 inputs, fp32 accumulation):
//   pass 1  per (unit, tile): row max and sum of exp2 over the tile's keys;
//   merge   per (unit, row):  lse2 = M + log2(sum_t z_t * exp2(m_t - M));
//   pass 2  per (unit, tile): recompute the logits, take max_i(t_ij - lse2_i), exp2.
//
// MFMA mapping (v_mfma_f32_32x32x16_bf16): the A operand is 32 keys x 16 dims, the B
// operand 16 dims x 32 observation rows, so one lane's 16 accumulators are 16 keys of
// one observation row.  Row statistics (pass 1) therefore reduce inside a lane, and the
// per-key max (pass 2) is one cross-lane reduction at the end of the tile.
#include <mutex>

#include "bkv_internal.h"

namespace bkv {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr float kNegInf = -__builtin_inff();

struct UnitInfo {
  int layer, b, h, L, n_obs;
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
  ui.n_obs = a.group * a.window + nb;
  return ui;
}

// Stage the unit's observation rows in LDS (row stride D*2+16 bytes keeps the 16-byte
// fragment reads of 8 consecutive rows on distinct banks); rows n_obs..nqb*32-1 are zero.
template <int D>
__device__ inline void stage_queries(const ScoreArgs& a, const UnitInfo& ui, int nqb, uint8_t* qs) {
  constexpr int kRowBytes = D * 2 + 16;
  constexpr int kChunks = D / 8;
  const int gw = a.group * a.window;
  const uint16_t* q = a.q[ui.layer];
  const uint16_t* bc = a.nb_max > 0 ? a.beacons[ui.layer] : nullptr;
  for (int c = threadIdx.x; c < nqb * 32 * kChunks; c += blockDim.x) {
    const int r = c / kChunks;
    const int cc = c - r * kChunks;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < gw) {
      const int hq = ui.h * a.group + r / a.window;
      const int t = a.q_len - a.window + r % a.window;
      v = *reinterpret_cast<const uint4*>(
          q + ((static_cast<size_t>(ui.b) * a.n_q_heads + hq) * a.q_len + t) * D + cc * 8);
    } else if (r < ui.n_obs) {
      v = *reinterpret_cast<const uint4*>(
          bc + ((static_cast<size_t>(ui.b) * a.n_kv_heads + ui.h) * a.nb_max + (r - gw)) * D + cc * 8);
    }
    *reinterpret_cast<uint4*>(qs + r * kRowBytes + cc * 16) = v;
  }
}

// Load two 32-key A fragments.  Lane l holds key (l & 31) of each fragment and, for
// k-step s, dims 16*s + 8*(l >> 5) .. +7.  Keys past the valid length read row L-1
// (always in bounds) and are masked by the caller.
template <int D>
__device__ inline void load_key_fragments(const uint16_t* kp, int kbase, int L, bf16x8 (&kf)[2][D / 16]) {
  const int lane = threadIdx.x & 63;
  const int row = lane & 31;
  const int half = lane >> 5;
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    int key = kbase + f * 32 + row;
    key = key < L ? key : L - 1;
    const uint16_t* src = kp + static_cast<size_t>(key) * D + half * 8;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) kf[f][s] = *reinterpret_cast<const bf16x8*>(src + s * 16);
  }
}

template <int D>
__device__ inline void mfma_block(const bf16x8 (&kf)[2][D / 16], const uint8_t* qs, int qb, f32x16 (&acc)[2]) {
  constexpr int kRowBytes = D * 2 + 16;
  const int lane = threadIdx.x & 63;
  const uint8_t* qrow = qs + (qb * 32 + (lane & 31)) * kRowBytes + (lane >> 5) * 16;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qrow + s * 32);
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    f32x16 c = {};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[f][s], qf[s], c, 0, 0, 0);
    acc[f] = c;
  }
}

// Key offset (within the wave's 64 keys) of accumulator r of fragment f in lane l.
__device__ inline int acc_key(int f, int r, int lane) {
  return f * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// Merge two (max, sum) pairs of exp2 statistics.
__device__ inline void merge_stats(float& m, float& z, float m2, float z2) {
  const float M = fmaxf(m, m2);
  if (M == kNegInf) return;
  z = z * __builtin_amdgcn_exp2f(m - M) + z2 * __builtin_amdgcn_exp2f(m2 - M);
  m = M;
}

template <int D>
__global__ __launch_bounds__(kScoreWaves * 64) void score_pass1(const ScoreArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int u = blockIdx.x / a.tiles;
  const int tile = blockIdx.x - u * a.tiles;
  const UnitInfo ui = unit_info(a, u);
  const int tile0 = tile * kScoreTile;
  if (tile0 >= ui.L) return;
  const int nqb = (ui.n_obs + 31) >> 5;
  uint8_t* qs = smem;
  float* st_m = reinterpret_cast<float*>(smem + a.obs_pad * (D * 2 + 16));
  float* st_z = st_m + kScoreWaves * a.obs_pad;
  stage_queries<D>(a, ui, nqb, qs);

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int kbase = tile0 + wave * kKeysPerWave;
  const uint16_t* kp = a.k[ui.layer] + (static_cast<size_t>(ui.b) * a.n_kv_heads + ui.h) * a.capacity * D;
  bf16x8 kf[2][D / 16];
  load_key_fragments<D>(kp, kbase, ui.L, kf);
  __syncthreads();

  for (int qb = 0; qb < nqb; ++qb) {
    f32x16 acc[2];
    mfma_block<D>(kf, qs, qb, acc);
    float m = kNegInf;
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float t = kbase + acc_key(f, r, lane) < ui.L ? acc[f][r] * a.scale_log2 : kNegInf;
        acc[f][r] = t;
        m = fmaxf(m, t);
      }
    float z = 0.f;
    if (m != kNegInf) {
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int r = 0; r < 16; ++r) z += __builtin_amdgcn_exp2f(acc[f][r] - m);
    }
    merge_stats(m, z, __shfl_xor(m, 32), __shfl_xor(z, 32));
    if (lane < 32) {
      st_m[wave * a.obs_pad + qb * 32 + lane] = m;
      st_z[wave * a.obs_pad + qb * 32 + lane] = z;
    }
  }
  __syncthreads();
  const size_t base = (static_cast<size_t>(u) * a.tiles + tile) * a.obs_pad;
  for (int i = threadIdx.x; i < nqb * 32; i += blockDim.x) {
    float m = st_m[i], z = st_z[i];
#pragma unroll
    for (int w = 1; w < kScoreWaves; ++w) merge_stats(m, z, st_m[w * a.obs_pad + i], st_z[w * a.obs_pad + i]);
    a.part_m[base + i] = m;
    a.part_z[base + i] = z;
  }
}

__global__ __launch_bounds__(256) void score_merge(const ScoreArgs a) {
  const int u = blockIdx.x;
  const UnitInfo ui = unit_info(a, u);
  const int ntiles = (ui.L + kScoreTile - 1) / kScoreTile;
  for (int i = threadIdx.x; i < a.obs_pad; i += blockDim.x) {
    float M = kNegInf;
    const size_t base = static_cast<size_t>(u) * a.tiles * a.obs_pad + i;
    for (int t = 0; t < ntiles; ++t) M = fmaxf(M, a.part_m[base + static_cast<size_t>(t) * a.obs_pad]);
    float Z = 0.f;
    if (M != kNegInf)
      for (int t = 0; t < ntiles; ++t) {
        const size_t o = base + static_cast<size_t>(t) * a.obs_pad;
        Z += a.part_z[o] * __builtin_amdgcn_exp2f(a.part_m[o] - M);
      }
    // Rows past n_obs (padding) and units without keys get +inf: they never win a max.
    a.lse[static_cast<size_t>(u) * a.obs_pad + i] =
        (i < ui.n_obs && Z > 0.f) ? M + log2f(Z) : __builtin_inff();
  }
}

template <int D>
__global__ __launch_bounds__(kScoreWaves * 64) void score_pass2(const ScoreArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int u = blockIdx.x / a.tiles;
  const int tile = blockIdx.x - u * a.tiles;
  const UnitInfo ui = unit_info(a, u);
  const int tile0 = tile * kScoreTile;
  if (tile0 >= ui.L) return;
  const int nqb = (ui.n_obs + 31) >> 5;
  uint8_t* qs = smem;
  float* lse_s = reinterpret_cast<float*>(smem + a.obs_pad * (D * 2 + 16));
  stage_queries<D>(a, ui, nqb, qs);
  for (int i = threadIdx.x; i < nqb * 32; i += blockDim.x) lse_s[i] = a.lse[static_cast<size_t>(u) * a.obs_pad + i];

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int kbase = tile0 + wave * kKeysPerWave;
  const uint16_t* kp = a.k[ui.layer] + (static_cast<size_t>(ui.b) * a.n_kv_heads + ui.h) * a.capacity * D;
  bf16x8 kf[2][D / 16];
  load_key_fragments<D>(kp, kbase, ui.L, kf);
  __syncthreads();

  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = kNegInf;
  for (int qb = 0; qb < nqb; ++qb) {
    f32x16 acc[2];
    mfma_block<D>(kf, qs, qb, acc);
    const float neg_lse = -lse_s[qb * 32 + (lane & 31)];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) v[f * 16 + r] = fmaxf(v[f * 16 + r], fmaf(acc[f][r], a.scale_log2, neg_lse));
  }
  // Max over the 32 observation rows held by lanes l ^ {1,2,4,8,16}: each exchange step
  // halves the values a lane keeps, so lane l ends with value index (l & 31).
#pragma unroll
  for (int step = 16, n = 16; step >= 1; step >>= 1, n >>= 1) {
    const bool upper = (lane & step) != 0;
#pragma unroll
    for (int i = 0; i < n; ++i) {
      const float send = upper ? v[i] : v[i + n];
      const float keep = upper ? v[i + n] : v[i];
      v[i] = fmaxf(keep, __shfl_xor(send, step));
    }
  }
  const int vi = lane & 31;
  const int key = kbase + acc_key(vi >> 4, vi & 15, lane);
  if (key < ui.L) {
    float* sp = a.scores[ui.layer] + (static_cast<size_t>(ui.b) * a.n_kv_heads + ui.h) * a.capacity;
    sp[key] = ui.n_obs > 0 ? exp2f(v[0]) : 0.f;
  }
}

template <int D>
size_t score_lds_bytes(int obs_pad) {
  return static_cast<size_t>(obs_pad) * (D * 2 + 16) + 2 * kScoreWaves * obs_pad * sizeof(float);
}

template <int D>
hipError_t launch_score_d(const ScoreArgs& a, hipStream_t s) {
  const size_t lds = score_lds_bytes<D>(a.obs_pad);
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [] {
    attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(&score_pass1<D>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (attr_err == hipSuccess)
      attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(&score_pass2<D>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  });
  if (attr_err != hipSuccess) return attr_err;
  const unsigned grid = static_cast<unsigned>(a.units) * a.tiles;
  hipLaunchKernelGGL(score_pass1<D>, dim3(grid), dim3(kScoreWaves * 64), lds, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(score_merge, dim3(a.units), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(score_pass2<D>, dim3(grid), dim3(kScoreWaves * 64), lds, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score(const ScoreArgs& a, int /*n_layers*/, int head_dim, hipStream_t s) {
  return head_dim == 128 ? launch_score_d<128>(a, s) : launch_score_d<64>(a, s);
}

}  // namespace bkv
