// Max-aggregated attention scores of cached keys (BeaconKV page, Figure 5 (b), (c);
// Table 2 caption: max over heads and queries).
//
// Per unit (layer, sequence, KV head) the observation rows are the last `window`
// queries of every query head of the group followed by the live beacons.  For key j
//     score_j = max_i exp(s_ij - lse_i),   s_ij = q_i . k_j / sqrt(d),
// where lse_i normalises row i over all valid keys.  Everything runs in the log2
// domain: t_ij = s_ij * log2(e) and score_j = exp2(max_i(t_ij - lse2_i)).
//
// Two kernels, each one launch over every unit and a grid-stride loop over items
// (unit, split); an item is a run of key tiles of one unit.  No workgroup ever waits for
// another:
//   score_stats   logits of the item's tiles against every observation row, per-row
//                 running max and sum of exp2 -> partial (m, z) per (unit, split, row);
//   score_finish  merges the unit's partials into lse2 per row (in LDS), recomputes
//                 the logits and writes exp2(max_i(t_ij - lse2_i)) for its keys.
// Both passes are bound by the matrix and vector units rather than by HBM, so the keys
// are simply read twice.
//
// MFMA mapping (v_mfma_f32_32x32x16_bf16): the A operand is 32 keys x 16 dims, the B
// operand 16 dims x 32 observation rows, so one lane's 16 accumulators are 16 keys of
// one observation row.  Row statistics reduce inside a lane; the per-key max is one
// cross-lane reduction per key tile.  Four waves per workgroup, each owning 64 keys of
// a 256-key tile; the exp2 work of one observation block is interleaved with the MFMAs
// of the next.
#include <algorithm>
#include <mutex>

#include "bkv_internal.h"

namespace bkv {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr float kNegInf = -__builtin_inff();
constexpr float kPosInf = __builtin_inff();

struct UnitInfo {
  int layer, b, h, L, n_obs, nqb, ntiles, nsplits;
};

template <int WAVES>
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
  ui.nqb = (ui.n_obs + 31) >> 5;
  ui.ntiles = (ui.L + WAVES * 64 - 1) / (WAVES * 64);
  ui.nsplits = (ui.ntiles + a.tps - 1) / a.tps;
  return ui;
}

// Stage the unit's observation rows in LDS, rows n_obs..nqb*32-1 zero.  Row r occupies
// D*2 bytes with its 16-byte chunk c stored at chunk slot c ^ (r mod D/8): the fragment
// reads of 16 consecutive rows at one chunk then touch 16 different slots, i.e. all 64
// banks once, with no padding.  Each thread issues its loads in batches of 8 before
// waiting, so staging costs about one memory latency per batch.
template <int D>
__device__ inline void stage_queries(const ScoreArgs& a, const UnitInfo& ui, uint8_t* qs) {
  constexpr int kChunks = D / 8;
  constexpr int kBatch = 8;
  const int gw = a.group * a.window;
  const uint16_t* q = a.q[ui.layer];
  const uint16_t* bc = a.nb_max > 0 ? a.beacons[ui.layer] : nullptr;
  const int total = ui.nqb * 32 * kChunks;
  for (int c0 = threadIdx.x; c0 < total; c0 += kBatch * blockDim.x) {
    uint4 v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int c = c0 + j * blockDim.x;
      const int r = c / kChunks;
      const int cc = c - r * kChunks;
      v[j] = make_uint4(0, 0, 0, 0);
      if (c < total) {
        if (r < gw) {
          const int hq = ui.h * a.group + r / a.window;
          const int t = a.q_len - a.window + r % a.window;
          v[j] = *reinterpret_cast<const uint4*>(
              q + ((static_cast<size_t>(ui.b) * a.n_q_heads + hq) * a.q_len + t) * D + cc * 8);
        } else if (r < ui.n_obs) {
          v[j] = *reinterpret_cast<const uint4*>(
              bc + ((static_cast<size_t>(ui.b) * a.n_kv_heads + ui.h) * a.nb_max + (r - gw)) * D + cc * 8);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int c = c0 + j * blockDim.x;
      const int r = c / kChunks;
      const int cc = c - r * kChunks;
      if (c < total) *reinterpret_cast<uint4*>(qs + r * (D * 2) + ((cc ^ (r & (kChunks - 1))) * 16)) = v[j];
    }
  }
}

// Two 32-key A fragments.  Lane l holds key (l & 31) of each fragment and, for k-step
// s, dims 16*s + 8*(l >> 5) .. +7.  Keys past the valid length read row L-1 (always in
// bounds) and are masked by the caller.
template <int D>
struct KeyFrag {
  bf16x8 v[2][D / 16];
};

template <int D>
__device__ inline void load_keys(const uint16_t* kp, int kbase, int L, KeyFrag<D>& kf) {
  const int lane = threadIdx.x & 63;
  const int row = lane & 31;
  const int half = lane >> 5;
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    int key = kbase + f * 32 + row;
    key = key < L ? key : L - 1;
    const uint16_t* src = kp + static_cast<size_t>(key) * D + half * 8;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) kf.v[f][s] = *reinterpret_cast<const bf16x8*>(src + s * 16);
  }
}

template <int D>
__device__ inline void load_qfrag(const uint8_t* qs, int qb, bf16x8 (&qf)[D / 16]) {
  constexpr int kChunks = D / 8;
  const int lane = threadIdx.x & 63;
  const int row = qb * 32 + (lane & 31);
  const uint8_t* base = qs + row * (D * 2);
  const int sw = row & (kChunks - 1);
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    qf[s] = *reinterpret_cast<const bf16x8*>(base + (((2 * s + (lane >> 5)) ^ sw) * 16));
}

template <int D>
__device__ inline void mfma_frags(const KeyFrag<D>& kf, const bf16x8 (&qf)[D / 16], f32x16 (&acc)[2]) {
  f32x16 c0 = {}, c1 = {};
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf.v[0][s], qf[s], c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf.v[1][s], qf[s], c1, 0, 0, 0);
  }
  acc[0] = c0;
  acc[1] = c1;
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

template <int D, int WAVES>
struct Smem {
  static constexpr int kRowBytes = D * 2;
  uint8_t* qs;
  float* st_m;   // [WAVES][2][obs_pad] (pass 1): per wave and lane half
  float* st_z;   // [WAVES][2][obs_pad] (pass 1)
  float* lse_s;  // [obs_pad]        (pass 2; aliases st_m)
  __device__ Smem(uint8_t* base, int obs_pad) {
    qs = base;
    st_m = reinterpret_cast<float*>(base + obs_pad * kRowBytes);
    st_z = st_m + 2 * WAVES * obs_pad;
    lse_s = st_m;
  }
};

// Keys at or past L (only in a unit's last tile) get -inf logits.
__device__ inline void mask_tail(f32x16 (&acc)[2], int kbase, int L, int lane) {
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (kbase + acc_key(f, r, lane) >= L) acc[f][r] = kNegInf;
}

// Exact (max, sum) update of one lane's 32 logits of one row: the block max is taken and
// the running sum rescaled.  Used for a row's first block and when the cheap update below
// reports a possible overflow.
__device__ inline void row_update_exact(const f32x16 (&acc)[2], float c, float& m, float& z) {
  float mx = kNegInf;
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[f][r]);
  if (mx == kNegInf) return;   // every key of this lane masked
  const float mt = fmaxf(mx * c, m);
  float zt = 0.f;
  const float neg = -mt;
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int r = 0; r < 16; ++r) zt += __builtin_amdgcn_exp2f(fmaf(acc[f][r], c, neg));
  z = (m == kNegInf ? 0.f : z * __builtin_amdgcn_exp2f(m - mt)) + zt;
  m = mt;
}

template <int D, int WAVES>
__device__ void pass1_item(const ScoreArgs& a, int u, int split, const UnitInfo& ui, uint8_t* smem) {
  Smem<D, WAVES> sm(smem, a.obs_pad);
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  stage_queries<D>(a, ui, sm.qs);
  for (int i = threadIdx.x; i < 2 * WAVES * a.obs_pad; i += blockDim.x) {
    sm.st_m[i] = kNegInf;
    sm.st_z[i] = 0.f;
  }
  const int t0 = split * a.tps;
  const int t1 = min(t0 + a.tps, ui.ntiles);
  const uint16_t* kp = a.k[ui.layer] + (static_cast<size_t>(ui.b) * a.n_kv_heads + ui.h) * a.capacity * D;
  const float c = a.scale_log2;
  // lane (l & 31, l >> 5) keeps the statistics of row qb*32 + (l & 31) over its key half
  float* my_m = sm.st_m + (wave * 2 + (lane >> 5)) * a.obs_pad + (lane & 31);
  float* my_z = sm.st_z + (wave * 2 + (lane >> 5)) * a.obs_pad + (lane & 31);
  KeyFrag<D> kf, kn;
  load_keys<D>(kp, t0 * WAVES * 64 + wave * 64, ui.L, kf);
  __syncthreads();
  for (int t = t0; t < t1; ++t) {
    const int kbase = t * WAVES * 64 + wave * 64;
    if (t + 1 < t1) load_keys<D>(kp, kbase + WAVES * 64, ui.L, kn);
    if (kbase < ui.L) {
      const bool full = kbase + 64 <= ui.L;
      bf16x8 qf[D / 16];
      f32x16 acc[2];
      load_qfrag<D>(sm.qs, 0, qf);
      mfma_frags<D>(kf, qf, acc);
      load_qfrag<D>(sm.qs, ui.nqb > 1 ? 1 : 0, qf);
      if (!full) mask_tail(acc, kbase, ui.L, lane);
      for (int qb = 0; qb < ui.nqb; ++qb) {
        // The next block's products (qf already holds its rows) are issued step by step
        // among this block's exponentials.  With the stale running max m the sum stays
        // finite unless a logit exceeds m by ~64 (it is +inf/NaN while m is still -inf);
        // then the exact update redoes the block.
        float m = my_m[qb * 32], z = my_z[qb * 32];
        const float neg = -m;
        f32x16 n0 = {}, n1 = {};
        float zs[4] = {0.f, 0.f, 0.f, 0.f};
        constexpr int kPer = 32 / (D / 16);   // logits handled per MFMA step
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
          n0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf.v[0][st], qf[st], n0, 0, 0, 0);
          n1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf.v[1][st], qf[st], n1, 0, 0, 0);
#pragma unroll
          for (int j = 0; j < kPer; ++j) {
            const int idx = st * kPer + j;
            zs[j & 3] += __builtin_amdgcn_exp2f(fmaf(acc[idx >> 4][idx & 15], c, neg));
          }
        }
        // keep the two MFMAs of each step among this block's exp work
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);           // MFMA
          __builtin_amdgcn_sched_group_barrier(0x402, 3 * kPer, 0);    // VALU / transcendental
        }
        load_qfrag<D>(sm.qs, qb + 2 < ui.nqb ? qb + 2 : qb, qf);   // unconditional: one scheduling region
        const float zt = (zs[0] + zs[1]) + (zs[2] + zs[3]);
        if (zt <= 1.8e19f)   // 2^64: no term overflowed (false for NaN and +inf)
          z += zt;
        else
          row_update_exact(acc, c, m, z);
        my_m[qb * 32] = m;
        my_z[qb * 32] = z;
        acc[0] = n0;
        acc[1] = n1;
        if (!full) mask_tail(acc, kbase, ui.L, lane);
      }
    }
    if (t + 1 < t1) kf = kn;
  }
  __syncthreads();
  const size_t base = (static_cast<size_t>(u) * a.splits + split) * a.obs_pad;
  for (int i = threadIdx.x; i < ui.nqb * 32; i += blockDim.x) {
    float m = kNegInf, z = 0.f;
#pragma unroll
    for (int w = 0; w < 2 * WAVES; ++w) merge_stats(m, z, sm.st_m[w * a.obs_pad + i], sm.st_z[w * a.obs_pad + i]);
    a.part_m[base + i] = m;
    a.part_z[base + i] = z;
  }
  __syncthreads();   // LDS is restaged by the next item
}

template <int D, int WAVES>
__device__ void pass2_item(const ScoreArgs& a, int u, int split, const UnitInfo& ui, uint8_t* smem) {
  Smem<D, WAVES> sm(smem, a.obs_pad);
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int t0 = split * a.tps;
  const int t1 = min(t0 + a.tps, ui.ntiles);
  const uint16_t* kp = a.k[ui.layer] + (static_cast<size_t>(ui.b) * a.n_kv_heads + ui.h) * a.capacity * D;
  float* sp = a.scores[ui.layer] + (static_cast<size_t>(ui.b) * a.n_kv_heads + ui.h) * a.capacity;
  KeyFrag<D> kf;   // no prefetch buffer: these keys were just read by the stats kernel
  load_keys<D>(kp, t0 * WAVES * 64 + wave * 64, ui.L, kf);
  stage_queries<D>(a, ui, sm.qs);
  // log2-sum-exp2 of every observation row from the unit's stats partials (the loads of
  // up to 8 splits are issued before any is used).
  for (int i = threadIdx.x; i < ui.nqb * 32; i += blockDim.x) {
    float M = kNegInf, Z = 0.f;
    for (int s0 = 0; s0 < ui.nsplits; s0 += 8) {
      float pm[8], pz[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const size_t o = (static_cast<size_t>(u) * a.splits + (s0 + j)) * a.obs_pad + i;
        pm[j] = s0 + j < ui.nsplits ? a.part_m[o] : kNegInf;
        pz[j] = s0 + j < ui.nsplits ? a.part_z[o] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) merge_stats(M, Z, pm[j], pz[j]);
    }
    // Padding rows get +inf: they never win the max.
    sm.lse_s[i] = (i < ui.n_obs && Z > 0.f) ? M + log2f(Z) : kPosInf;
  }
  __syncthreads();
  for (int t = t0; t < t1; ++t) {
    const int kbase = t * WAVES * 64 + wave * 64;
    if (t > t0) load_keys<D>(kp, kbase, ui.L, kf);
    if (kbase < ui.L) {
      float v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = kNegInf;
      bf16x8 qf[D / 16];
      f32x16 acc[2];
      load_qfrag<D>(sm.qs, 0, qf);
      mfma_frags<D>(kf, qf, acc);
      load_qfrag<D>(sm.qs, ui.nqb > 1 ? 1 : 0, qf);
      for (int qb = 0; qb < ui.nqb; ++qb) {
        const float neg_lse = -sm.lse_s[qb * 32 + (lane & 31)];
        f32x16 n0 = {}, n1 = {};
        constexpr int kPer = 32 / (D / 16);
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
          n0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf.v[0][st], qf[st], n0, 0, 0, 0);
          n1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf.v[1][st], qf[st], n1, 0, 0, 0);
#pragma unroll
          for (int j = 0; j < kPer; ++j) {
            const int idx = st * kPer + j;
            v[idx] = fmaxf(v[idx], fmaf(acc[idx >> 4][idx & 15], a.scale_log2, neg_lse));
          }
        }
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);           // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 2 * kPer, 0);    // VALU
        }
        load_qfrag<D>(sm.qs, qb + 2 < ui.nqb ? qb + 2 : qb, qf);   // unconditional: one scheduling region
        acc[0] = n0;
        acc[1] = n1;
      }
      // Max over the 32 observation rows held by lanes l ^ {16,8,4,2,1}: each exchange
      // halves the values a lane keeps, so lane l ends with value index (l & 31).
#pragma unroll
      for (int step = 16; step >= 1; step >>= 1) {
        const bool upper = (lane & step) != 0;
#pragma unroll
        for (int i = 0; i < step; ++i) {
          const float send = upper ? v[i] : v[i + step];
          const float keep = upper ? v[i + step] : v[i];
          v[i] = fmaxf(keep, __shfl_xor(send, step));
        }
      }
      const int vi = lane & 31;
      const int key = kbase + acc_key(vi >> 4, vi & 15, lane);
      if (key < ui.L) sp[key] = ui.n_obs > 0 ? exp2f(v[0]) : 0.f;
    }
  }
  __syncthreads();   // LDS is restaged by the next item
}

template <int D, int WAVES, bool FINISH>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 8))) void score_kernel(const ScoreArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int n_items = a.units * a.splits;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int u = a.unit0 + item / a.splits;
    const int split = item - (item / a.splits) * a.splits;
    const UnitInfo ui = unit_info<WAVES>(a, u);
    if (split >= ui.nsplits) continue;   // no keys in this split (uniform across the block)
    if (FINISH)
      pass2_item<D, WAVES>(a, u, split, ui, smem);
    else
      pass1_item<D, WAVES>(a, u, split, ui, smem);
  }
}

template <int D, int WAVES>
size_t lds_bytes(int obs_pad) {
  return static_cast<size_t>(obs_pad) * (D * 2) + 4 * WAVES * obs_pad * sizeof(float);
}

template <int D, int WAVES>
hipError_t launch_d(ScoreArgs a, hipStream_t s) {
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [] {
    attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(&score_kernel<D, WAVES, false>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (attr_err == hipSuccess)
      attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(&score_kernel<D, WAVES, true>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  });
  if (attr_err != hipSuccess) return note_hip_error(attr_err, "score: hipFuncSetAttribute");
  const size_t lds = lds_bytes<D, WAVES>(a.obs_pad);
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return note_hip_error(e, "score: hipGetDevice");
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return note_hip_error(e, "score: hipDeviceGetAttribute");
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, score_kernel<D, WAVES, true>, WAVES * 64, lds);
  if (e != hipSuccess) return note_hip_error(e, "score: hipOccupancyMaxActiveBlocksPerMultiprocessor");
  const int resident = std::max(1, per_cu) * cus;
  a.tps = kScoreTilesPerItem;
  a.splits = score_splits(a.capacity, a.obs_pad);
  // One stats launch and one finish launch over every unit: the passes are bound by the
  // matrix and vector units, not by memory (the finish pass re-reads the keys at a few
  // TB/s), and every extra launch costs its ramp-up and tail.
  const int total_units = a.units;
  const int per_chunk = total_units;
  for (int u0 = 0; u0 < total_units; u0 += per_chunk) {
    a.unit0 = u0;
    a.units = std::min(per_chunk, total_units - u0);
    const int grid = std::min(resident, a.units * a.splits);
    hipLaunchKernelGGL((score_kernel<D, WAVES, false>), dim3(grid), dim3(WAVES * 64), lds, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return note_hip_error(e, "score: launch score_stats");
    hipLaunchKernelGGL((score_kernel<D, WAVES, true>), dim3(grid), dim3(WAVES * 64), lds, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return note_hip_error(e, "score: launch score_finish");
  }
  return hipSuccess;
}

}  // namespace

// Four waves per workgroup: the LDS (observation rows + per-wave statistics) is
// obs_pad * (2D + 32) bytes, at most 160 KB, and up to 256 rows two workgroups share a CU.
int score_waves(int /*obs_pad*/) { return 4; }

hipError_t launch_score(const ScoreArgs& a, int /*n_layers*/, int head_dim, hipStream_t s) {
  const int w = score_waves(a.obs_pad);
  (void)w;
  return head_dim == 128 ? launch_d<128, 4>(a, s) : launch_d<64, 4>(a, s);
}

}  // namespace bkv
