// Max-aggregated attention scores of cached keys (BeaconKV page, Figure 5 (b), (c);
// Table 2 caption: max over heads and queries).
//
// Per unit (layer, sequence, KV head) the observation rows are the last `window`
// queries of every query head of the group followed by the live beacons.  For key j
//     score_j = max_i exp(s_ij - lse_i),   s_ij = q_i . k_j / sqrt(d),
// where lse_i normalises row i over all valid keys.  Everything runs in the log2
// domain: t_ij = s_ij * log2(e) and score_j = exp2(max_i(t_ij - lse2_i)).
//
// Two persistent kernels, each on its own grid.  The launch's key tiles (256 keys each, unit
// after unit) are cut into one contiguous share per workgroup (weighted where two
// workgroups share a CU); a share covers the end of one unit, whole units and the start
// of another.  Per unit piece ("segment") a workgroup stages the unit's observation rows
// in LDS once and then walks its tiles.  No workgroup ever waits for another:
//   score_stats   per-row running max and sum of exp2 over the segment's keys ->
//                 one partial (m, z) per (unit, segment) and row;
//   score_finish  merges the unit's partials into lse2 per row (in LDS), recomputes
//                 the logits and writes exp2(max_i(t_ij - lse2_i)) for its keys.
// Both passes are bound by the matrix and vector units rather than by HBM, so the keys
// are simply read twice.  The segments of a unit are numbered by stats workgroup (the
// workgroup holding a tile follows arithmetically from the split, see score_common.h), so
// the finish pass finds every partial of a unit without any table.  Where the rows fit in
// registers (up to 512 padded rows at head_dim 128, 384 at 64) the stats pass is the
// register-row one of score_qs.hip, which writes the same partials; the LDS-staged stats
// pass here takes the rest.  Where the staged rows leave room for only one 4-wave finish
// workgroup per CU, the 8-wave finish (finish8_kernel) runs instead.
//
// MFMA mapping (v_mfma_f32_32x32x16_bf16, four waves, each owning 64 keys of a tile).
// Stats pass: A = 32 keys x 16 dims, B = 16 dims x 32 observation rows, so a lane's 16
// accumulators are 16 keys of one row and the row sums reduce inside the lane.  Finish
// pass: A = rows, B = keys, so a lane's accumulators are 16 rows of one key and the max
// over rows reduces inside the lane.  Blocks of 32 rows run two at a time in ping-pong
// accumulators: the products of one block are issued among the vector work of the other.
#include <algorithm>

#include "score_common.h"

namespace bkv {
namespace {

// Stage the unit's observation rows in LDS, rows n_obs..nqb*32-1 zero.  Row r occupies
// D*2 bytes with its 16-byte chunk c stored at chunk slot c ^ (r mod D/8): the fragment
// reads of 16 consecutive rows at one chunk then touch 16 different slots, i.e. all 64
// banks once, with no padding.  Each thread issues its loads in batches of 8 before
// waiting, so staging costs about one memory latency per batch.
template <int D, int NT = kThreads>
__device__ inline void stage_queries(const ScoreArgs& a, const UnitInfo& ui, uint8_t* qs) {
  constexpr int kChunks = D / 8;
  constexpr int kBatch = 8;
  const int gw = a.group * a.window;
  // the unit's first recent-query row and first beacon row
  const uint16_t* q0 = a.window > 0 ? a.q[ui.layer] + ((static_cast<size_t>(ui.b) * a.n_q_heads + ui.h * a.group) *
                                                       a.q_len + (a.q_len - a.window)) * D : nullptr;
  const uint16_t* b0 = a.nb_max > 0 ? a.beacons[ui.layer] + (static_cast<size_t>(ui.b) * a.n_kv_heads + ui.h) *
                                                                a.nb_max * D : nullptr;
  const int total = ui.nqb * 32 * kChunks;
  for (int c0 = threadIdx.x; c0 < total; c0 += kBatch * NT) {
    uint4 v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int c = c0 + j * NT;
      const int r = c / kChunks;
      const int cc = c - r * kChunks;
      v[j] = make_uint4(0, 0, 0, 0);
      if (c < total) {
        if (r < gw)   // query head h * G + r / window, its row q_len - window + r % window
          v[j] = *reinterpret_cast<const uint4*>(
              q0 + (static_cast<size_t>(r / a.window) * a.q_len + r % a.window) * D + cc * 8);
        else if (r < ui.n_obs)
          v[j] = *reinterpret_cast<const uint4*>(b0 + static_cast<size_t>(r - gw) * D + cc * 8);
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int c = c0 + j * NT;
      const int r = c / kChunks;
      const int cc = c - r * kChunks;
      if (c < total) *reinterpret_cast<uint4*>(qs + r * (D * 2) + ((cc ^ (r & (kChunks - 1))) * 16)) = v[j];
    }
  }
}

// ---- fragments --------------------------------------------------------------------------

// Fragment s of observation rows blk*32 .. +31 from LDS: lane l holds row (l & 31), dims
// 16*s + 8*(l >> 5) .. +7.  With the chunk swizzle the byte offset inside the row is
// 16 * ((2s + half) ^ (row mod D/8)) = (32 s) ^ (16 * (half ^ (row mod D/8))), so each
// fragment's address is one XOR away from a per-lane base.
template <int D>
__device__ inline bf16x8 q_frag(const uint8_t* qs, int blk, int s) {
  const int lane = threadIdx.x & 63;
  const int row = blk * 32 + (lane & 31);
  const unsigned base = static_cast<unsigned>(row * (D * 2) + 16 * ((row & (D / 8 - 1)) ^ (lane >> 5)));
  return *reinterpret_cast<const bf16x8*>(qs + (base ^ (32u * s)));
}

template <int D>
struct Smem {
  uint8_t* qs;   // [obs_pad][D] bf16, swizzled
  float* st_m;   // [kWaves][2][obs_pad] (stats pass): per wave and lane half
  float* st_z;   // [kWaves][2][obs_pad] (stats pass)
  float* nlse;   // [obs_pad]            (finish pass; aliases st_m): -lse2_i / c
  __device__ Smem(uint8_t* base, int obs_pad) {
    qs = base;
    st_m = reinterpret_cast<float*>(base + obs_pad * (D * 2));
    st_z = st_m + 2 * kWaves * obs_pad;
    nlse = st_m;
  }
};

// Two 32-key fragments.  Lane l holds key (l & 31) of each fragment and, for k-step s,
// dims 16*s + 8*(l >> 5) .. +7 (the A layout of keys in the stats pass and the B layout
// in the finish pass are the same registers).  Keys past the valid length read row L-1
// (always in bounds) and are masked or dropped by the caller.
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

// Observation rows qb*32 .. +31 from LDS: lane l holds row (l & 31), dims of k-step s at
// 16*s + 8*(l >> 5).
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

// ---- key fragments ----------------------------------------------------------------------
//
// A wave takes the 64 keys it owns in a tile as two 32-key fragments, one after the other;
// each fragment's registers are refilled with the next tile's fragment as soon as it has
// been multiplied against every row block, a whole fragment pass before its use.

// One 32-key fragment: lane l holds key (l & 31) and, for k-step s, dims 16*s + 8*(l >> 5)
// .. +7 (the A layout of keys in the stats pass and the B layout in the finish pass are
// the same registers).  Keys past the valid length read row L-1 (in bounds) and are
// masked or dropped by the caller.
template <int D>
struct Frag {
  bf16x8 v[D / 16];
};

template <int D>
__device__ inline void load_frag(const uint16_t* kp, int key0, int L, Frag<D>& f) {
  const int lane = threadIdx.x & 63;
  int key = key0 + (lane & 31);
  key = key < L ? key : L - 1;
  const uint16_t* src = kp + static_cast<size_t>(key) * D + (lane >> 5) * 8;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) f.v[s] = *reinterpret_cast<const bf16x8*>(src + s * 16);
}

// ---- stats pass -------------------------------------------------------------------------

// Keys at or past L get -inf logits; accumulator r of lane l holds key
// key0 + 8 (r >> 2) + 4 (l >> 5) + (r & 3) in the stats layout.
__device__ inline void mask_frag(f32x16& acc, int key0, int L) {
  const int half = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (key0 + 8 * (r >> 2) + 4 * half + (r & 3) >= L) acc[r] = kNegInf;
}

// Exact (max, sum) update of one lane's 16 logits of one row: the block max is taken and
// the running sum rescaled.  Used for a row's first block and when the cheap update
// reports a possible overflow.
__device__ inline void row_update_exact(const f32x16& acc, float c, float& m, float& z) {
  float mx = kNegInf;
#pragma unroll
  for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[r]);
  if (mx == kNegInf) return;   // every key of this lane masked
  const float mt = fmaxf(mx * c, m);
  float zt = 0.f;
  const float neg = -mt;
#pragma unroll
  for (int r = 0; r < 16; ++r) zt += __builtin_amdgcn_exp2f(fmaf(acc[r], c, neg));
  z = (m == kNegInf ? 0.f : z * __builtin_amdgcn_exp2f(m - mt)) + zt;
  m = mt;
}

// With the running max m of earlier blocks the sum stays finite unless a logit exceeds
// m by ~64 (it is +inf/NaN while m is still -inf); then the exact update redoes the block.
__device__ inline void stats_commit(const f32x16& cur, float zt, float c, float m, float z, float* pm, float* pz) {
  if (zt <= 1.8e19f)   // 2^64: no term overflowed (false for NaN and +inf)
    z += zt;
  else
    row_update_exact(cur, c, m, z);
  *pm = m;
  *pz = z;
}

// The block in `cur` (its rows' running statistics in m, z; their LDS copies at pm, pz)
// is reduced to sums of exp2(c x - m) while the products of rows blk*32.. go into `nxt`.
// qpre holds fragments 0 and 1 of block blk on entry and of block blk_next on exit (the
// other fragments are read two MFMA steps ahead of their use); m, z hold the statistics
// of the next block on exit.
template <int D, bool MASK>
__device__ inline void stats_step(const Frag<D>& kf, bf16x8 (&qpre)[2], f32x16& cur, f32x16& nxt, const uint8_t* qs,
                                  int blk, int blk_next, float c, float* pm, float* pz, float& m, float& z, int key0,
                                  int L) {
  constexpr int S = D / 16;
  constexpr int kPer = 16 / S;   // logits handled per MFMA step
  if (MASK) mask_frag(cur, key0, L);
  const float m_next = pm[32], z_next = pz[32];
  const float neg = -m;
  f32x16 n = {};
  float zs[4] = {0.f, 0.f, 0.f, 0.f};
  bf16x8 qf[S + 2];
  qf[0] = qpre[0];
  qf[1] = qpre[1];
#pragma unroll
  for (int st = 0; st < S; ++st) {
    qf[st + 2] = q_frag<D>(qs, st + 2 < S ? blk : blk_next, (st + 2) % S);
    n = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf.v[st], qf[st], n, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int idx = st * kPer + j;
      zs[idx & 3] += __builtin_amdgcn_exp2f(fmaf(cur[idx], c, neg));
    }
  }
#pragma unroll
  for (int st = 0; st < S; ++st) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);           // LDS read
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);           // MFMA
    __builtin_amdgcn_sched_group_barrier(0x402, 3 * kPer, 0);    // VALU / transcendental
  }
  qpre[0] = qf[S];
  qpre[1] = qf[S + 1];
  stats_commit(cur, (zs[0] + zs[1]) + (zs[2] + zs[3]), c, m, z, pm, pz);
  m = m_next;
  z = z_next;
  nxt = n;
}

// The last block of a pass: no products left to overlap.
template <bool MASK>
__device__ inline void stats_last(f32x16& cur, float c, float* pm, float* pz, float m, float z, int key0, int L) {
  if (MASK) mask_frag(cur, key0, L);
  const float neg = -m;
  float zs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < 16; ++r) zs[r & 3] += __builtin_amdgcn_exp2f(fmaf(cur[r], c, neg));
  stats_commit(cur, (zs[0] + zs[1]) + (zs[2] + zs[3]), c, m, z, pm, pz);
}

// One 32-key fragment (keys key0..) against all nqb >= 1 row blocks.  pm/pz address the
// lane's statistics of row block 0; block qb is at +qb*32.
template <int D, bool MASK>
__device__ inline void stats_pass(const Frag<D>& kf, const uint8_t* qs, int nqb, float c, float* pm, float* pz,
                                  int key0, int L) {
  constexpr int S = D / 16;
  f32x16 A, B;
  {
    bf16x8 q[S];
#pragma unroll
    for (int s = 0; s < S; ++s) q[s] = q_frag<D>(qs, 0, s);
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < S; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf.v[s], q[s], acc, 0, 0, 0);
    A = acc;
  }
  const int b1 = nqb > 1 ? 1 : 0;
  bf16x8 qpre[2] = {q_frag<D>(qs, b1, 0), q_frag<D>(qs, b1, 1)};
  float m = pm[0], z = pz[0];
  int qb = 0;
  for (; qb + 2 < nqb; qb += 2) {
    stats_step<D, MASK>(kf, qpre, A, B, qs, qb + 1, qb + 2, c, pm + qb * 32, pz + qb * 32, m, z, key0, L);
    stats_step<D, MASK>(kf, qpre, B, A, qs, qb + 2, qb + 3 < nqb ? qb + 3 : nqb - 1, c, pm + (qb + 1) * 32,
                        pz + (qb + 1) * 32, m, z, key0, L);
  }
  if (qb + 1 < nqb) {
    stats_step<D, MASK>(kf, qpre, A, B, qs, qb + 1, qb + 1, c, pm + qb * 32, pz + qb * 32, m, z, key0, L);
    stats_last<MASK>(B, c, pm + (qb + 1) * 32, pz + (qb + 1) * 32, m, z, key0, L);
  } else {
    stats_last<MASK>(A, c, pm + qb * 32, pz + qb * 32, m, z, key0, L);
  }
}

template <int D>
__device__ inline void stats_fragment(const Frag<D>& kf, const uint8_t* qs, int nqb, float c, float* pm, float* pz,
                                      int key0, int L) {
  if (key0 >= L || nqb == 0) return;
  if (key0 + 32 <= L)
    stats_pass<D, false>(kf, qs, nqb, c, pm, pz, key0, L);
  else
    stats_pass<D, true>(kf, qs, nqb, c, pm, pz, key0, L);
}

// Tiles tile0 .. tile0+ntile-1 of one unit -> partial statistics out_m/out_z [nqb*32].
template <int D>
__device__ void stats_segment(const ScoreArgs& a, const UnitInfo& ui, int tile0, int ntile, float* out_m,
                              float* out_z, uint8_t* smem) {
  Smem<D> sm(smem, a.obs_pad);
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const uint16_t* kp = a.k[ui.layer] + (static_cast<size_t>(ui.b) * a.n_kv_heads + ui.h) * a.capacity * D;
  Frag<D> fa, fb;
  load_frag<D>(kp, tile0 * kScoreTile + (threadIdx.x >> 6) * 64, ui.L, fa);
  load_frag<D>(kp, tile0 * kScoreTile + (threadIdx.x >> 6) * 64 + 32, ui.L, fb);
  stage_queries<D>(a, ui, sm.qs);
  for (int i = threadIdx.x; i < 2 * kWaves * a.obs_pad; i += kThreads) {
    sm.st_m[i] = kNegInf;
    sm.st_z[i] = 0.f;
  }
  const float c = a.scale_log2;
  float* my_m = sm.st_m + (wave * 2 + (lane >> 5)) * a.obs_pad + (lane & 31);
  float* my_z = sm.st_z + (wave * 2 + (lane >> 5)) * a.obs_pad + (lane & 31);
  __syncthreads();
  const int t1 = tile0 + ntile;
  for (int t = tile0; t < t1; ++t) {
    const int kbase = t * kScoreTile + wave * 64;
    const int knext = t + 1 < t1 ? kbase + kScoreTile : kbase;
    stats_fragment<D>(fa, sm.qs, ui.nqb, c, my_m, my_z, kbase, ui.L);
    load_frag<D>(kp, knext, ui.L, fa);
    stats_fragment<D>(fb, sm.qs, ui.nqb, c, my_m, my_z, kbase + 32, ui.L);
    load_frag<D>(kp, knext + 32, ui.L, fb);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < ui.nqb * 32; i += kThreads) {
    float m = kNegInf, z = 0.f;
#pragma unroll
    for (int w = 0; w < 2 * kWaves; ++w) merge_stats(m, z, sm.st_m[w * a.obs_pad + i], sm.st_z[w * a.obs_pad + i]);
    out_m[i] = m;
    out_z[i] = z;
  }
  __syncthreads();   // LDS is restaged by the next segment
}

// ---- finish pass ------------------------------------------------------------------------

// The accumulators of a block start at -lse2_i / c instead of zero (c = log2(e) / sqrt(d)
// > 0), so they end at x_ij - lse2_i / c and the vector work per logit is a running max;
// score_j = exp2(c * max) once per key.  Register r = 4g + j of lane l is row
// 8g + 4(l >> 5) + j of the block.
__device__ inline f32x16 load_seed(const float* nlse, int qb) {
  const int lane = threadIdx.x & 63;
  const float* p = nlse + qb * 32 + 4 * (lane >> 5);
  f32x16 o;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const float4 v = *reinterpret_cast<const float4*>(p + 8 * g);
    o[4 * g] = v.x;
    o[4 * g + 1] = v.y;
    o[4 * g + 2] = v.z;
    o[4 * g + 3] = v.w;
  }
  return o;
}

// Products of block k (rows in qk, accumulators X already seeded with -lse2 / c) while the
// accumulators P of the previous block are folded into vm (FOLD); the rows of block kn go
// to qn at the start of the step and, once P is folded, the seed of block kn to P, so both
// loads are in flight behind this step's products.  MEAN: vm sums the attention weights
// exp2(c * acc); otherwise vm is the running max of acc.
//
// The max is IEEE-2019 maximum (v_maximum3_f32, NaN-propagating), not fmaxf: the operands
// come straight from the matrix unit, and fmaxf's number-preferring semantics make the
// compiler quiet each of them with an extra v_max_f32 first (3.5 vector instructions per
// two logits instead of one).  Logits of finite inputs are never NaN.
template <bool MEAN>
__device__ inline void fold2(float& vm, float x0, float x1, float c) {
  if (MEAN)
    vm += __builtin_amdgcn_exp2f(c * x0) + __builtin_amdgcn_exp2f(c * x1);
  else
    vm = __builtin_elementwise_maximum(__builtin_elementwise_maximum(vm, x0), x1);
}

template <int D, bool MEAN, bool FOLD>
__device__ inline void finish_step(const KeyFrag<D>& kf, const bf16x8 (&qk)[D / 16], bf16x8 (&qn)[D / 16],
                                   f32x16 (&X)[2], f32x16 (&P)[2], const uint8_t* qs, const float* nlse, int kn,
                                   float c, float (&vm)[2]) {
  constexpr int S = D / 16;
  constexpr int kHalf = S / 2;
  constexpr int kPer = 32 / kHalf;   // (row, key) pairs of each fragment folded per early k-step
  load_qfrag<D>(qs, kn, qn);
  f32x16 n0 = X[0], n1 = X[1];
#pragma unroll
  for (int st = 0; st < S; ++st) {
    n0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qk[st], kf.v[0][st], n0, 0, 0, 0);
    n1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qk[st], kf.v[1][st], n1, 0, 0, 0);
    if (FOLD && st < kHalf) {
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int j = 0; j < kPer / 2; j += 2) fold2<MEAN>(vm[f], P[f][st * kPer / 2 + j], P[f][st * kPer / 2 + j + 1], c);
    }
  }
  const f32x16 sd = load_seed(nlse, kn);
  P[0] = sd;
  P[1] = sd;
  __builtin_amdgcn_sched_group_barrier(0x100, S, 0);                           // DS read: rows
#pragma unroll
  for (int st = 0; st < kHalf; ++st) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                          // MFMA
    if (FOLD) __builtin_amdgcn_sched_group_barrier(MEAN ? 0x402 : 0x002, MEAN ? 3 * kPer / 2 : kPer / 2, 0);   // fold
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);                           // DS read: seed
  __builtin_amdgcn_sched_group_barrier(0x008, 2 * (S - kHalf), 0);             // MFMA
  X[0] = n0;
  X[1] = n1;
}

template <bool MEAN>
__device__ inline void finish_last(const f32x16 (&cur)[2], float c, float (&vm)[2]) {
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int r = 0; r < 16; r += 2) fold2<MEAN>(vm[f], cur[f][r], cur[f][r + 1], c);
}

// One wave's 64 keys: returns, in lane l, for key l of the wave (fragment l >> 5, key
// l & 31) the max over all rows of x - lse2 / c, or with MEAN the sum over all rows of the
// attention weights.  Blocks alternate between two row and two accumulator register sets.
template <int D, bool MEAN>
__device__ inline float finish_tile(const KeyFrag<D>& kf, const uint8_t* qs, const float* nlse, int nqb, float c) {
  const int lane = threadIdx.x & 63;
  float vm[2] = {MEAN ? 0.f : kNegInf, MEAN ? 0.f : kNegInf};
  bf16x8 q0[D / 16], q1[D / 16];
  f32x16 A[2], B[2];
  load_qfrag<D>(qs, 0, q0);
  A[0] = load_seed(nlse, 0);
  A[1] = A[0];
  const int last = nqb - 1;
  auto nxt = [&](int k) { return k < last ? k : last; };
  finish_step<D, MEAN, false>(kf, q0, q1, A, B, qs, nlse, nxt(1), c, vm);
  int k = 1;
  for (; k + 1 < nqb; k += 2) {
    finish_step<D, MEAN, true>(kf, q1, q0, B, A, qs, nlse, nxt(k + 1), c, vm);
    finish_step<D, MEAN, true>(kf, q0, q1, A, B, qs, nlse, nxt(k + 2), c, vm);
  }
  if (k < nqb) {
    finish_step<D, MEAN, true>(kf, q1, q0, B, A, qs, nlse, nxt(k + 1), c, vm);
    finish_last<MEAN>(B, c, vm);
  } else {
    finish_last<MEAN>(A, c, vm);
  }
  // lanes l and l ^ 32 hold the two row halves of the same keys
  const bool lo = lane < 32;
  const float keep = lo ? vm[0] : vm[1];
  const float other = __shfl_xor(lo ? vm[1] : vm[0], 32);
  return MEAN ? keep + other : fmaxf(keep, other);
}

// Scores of tiles tile0 .. tile0+ntile-1 of one unit.  Its statistics partials are the
// n_part slots at pm0/pz0 (stride obs_pad), slot s written by workgroup w0 + s.  A unit met
// by more stats workgroups than it has slots (n_part > a.slots; the host sizes the slots so
// that no launch gets there) lost the partials past the last slot: its scores are then NaN
// rather than a softmax over part of the keys.
template <int D, bool MEAN>
__device__ void finish_segment(const ScoreArgs& a, const UnitInfo& ui, int tile0, int ntile, const float* pm0,
                               const float* pz0, int n_part, uint8_t* smem) {
  Smem<D> sm(smem, a.obs_pad);
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const uint16_t* kp = a.k[ui.layer] + (static_cast<size_t>(ui.b) * a.n_kv_heads + ui.h) * a.capacity * D;
  float* sp = a.scores[ui.layer] + (static_cast<size_t>(ui.b) * a.n_kv_heads + ui.h) * a.capacity;
  KeyFrag<D> kf;
  load_keys<D>(kp, tile0 * kScoreTile + wave * 64, ui.L, kf);
  stage_queries<D>(a, ui, sm.qs);
  const bool lost = n_part > a.slots;
  const int n_kept = lost ? a.slots : n_part;
  // log2-sum-exp2 of every observation row from the unit's partials (the loads of up to
  // 8 slots are issued before any is used; slots of workgroups with no tiles are skipped).
  for (int i = threadIdx.x; i < ui.nqb * 32; i += kThreads) {
    float M = kNegInf, Z = 0.f;
    for (int s0 = 0; s0 < n_kept; s0 += 8) {
      float pm[8], pz[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool use = s0 + j < n_kept;
        const size_t o = static_cast<size_t>(s0 + j) * a.obs_pad + i;
        pm[j] = use ? pm0[o] : kNegInf;
        pz[j] = use ? pz0[o] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) merge_stats(M, Z, pm[j], pz[j]);
    }
    // -lse2_i / c; padding rows -inf: they never win the max.
    sm.nlse[i] = lost ? __builtin_nanf("") : (i < ui.n_obs && Z > 0.f) ? -(M + log2f(Z)) / a.scale_log2 : kNegInf;
  }
  __syncthreads();
  const int t1 = tile0 + ntile;
  for (int t = tile0; t < t1; ++t) {
    const int kbase = t * kScoreTile + wave * 64;
    if (t > tile0) load_keys<D>(kp, kbase, ui.L, kf);
    if (kbase < ui.L) {
      float v = kNegInf;
      if (ui.nqb > 0) v = finish_tile<D, MEAN>(kf, sm.qs, sm.nlse, ui.nqb, a.scale_log2);
      const int key = kbase + lane;
      if (key < ui.L) sp[key] = ui.n_obs > 0 ? (MEAN ? v / static_cast<float>(ui.n_obs) : exp2f(a.scale_log2 * v)) : 0.f;
    }
  }
  __syncthreads();   // LDS is restaged by the next segment
}

// Finish pass for observation sets whose staged rows leave room for one workgroup per CU
// (over 256 rows): one workgroup of 8 waves per CU, so every SIMD still runs two waves on
// one LDS copy of the rows.  The waves take the segment's 64-key items from an LDS counter
// as they free up, so no wave waits on a slower partner at the end of the share.
constexpr int kThreads8 = 512;

template <int D, bool MEAN>
__device__ void finish_segment8(const ScoreArgs& a, const UnitInfo& ui, int tile0, int ntile, const float* pm0,
                                const float* pz0, int n_part, uint8_t* smem) {
  Smem<D> sm(smem, a.obs_pad);
  int* next_item = reinterpret_cast<int*>(sm.nlse + a.obs_pad);
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const uint16_t* kp = a.k[ui.layer] + (static_cast<size_t>(ui.b) * a.n_kv_heads + ui.h) * a.capacity * D;
  float* sp = a.scores[ui.layer] + (static_cast<size_t>(ui.b) * a.n_kv_heads + ui.h) * a.capacity;
  const int n_items = ntile * (kScoreTile / 64);
  const int key0 = tile0 * kScoreTile;
  int item = wave;   // the first item of each wave is fixed, so its keys load before staging
  KeyFrag<D> kf;
  if (item < n_items) load_keys<D>(kp, key0 + item * 64, ui.L, kf);
  stage_queries<D, kThreads8>(a, ui, sm.qs);
  const bool lost = n_part > a.slots;
  const int n_kept = lost ? a.slots : n_part;
  for (int i = threadIdx.x; i < ui.nqb * 32; i += kThreads8) {
    float M = kNegInf, Z = 0.f;
    for (int s0 = 0; s0 < n_kept; s0 += 8) {
      float pm[8], pz[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool use = s0 + j < n_kept;
        const size_t o = static_cast<size_t>(s0 + j) * a.obs_pad + i;
        pm[j] = use ? pm0[o] : kNegInf;
        pz[j] = use ? pz0[o] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) merge_stats(M, Z, pm[j], pz[j]);
    }
    sm.nlse[i] = lost ? __builtin_nanf("") : (i < ui.n_obs && Z > 0.f) ? -(M + log2f(Z)) / a.scale_log2 : kNegInf;
  }
  if (threadIdx.x == 0) *next_item = kThreads8 / 64;
  __syncthreads();
  while (item < n_items) {
    const int kbase = key0 + item * 64;
    if (kbase < ui.L) {
      float v = kNegInf;
      if (ui.nqb > 0) v = finish_tile<D, MEAN>(kf, sm.qs, sm.nlse, ui.nqb, a.scale_log2);
      const int key = kbase + lane;
      if (key < ui.L) sp[key] = ui.n_obs > 0 ? (MEAN ? v / static_cast<float>(ui.n_obs) : exp2f(a.scale_log2 * v)) : 0.f;
    }
    int nx = 0;
    if (lane == 0) nx = atomicAdd(next_item, 1);
    item = __builtin_amdgcn_readfirstlane(nx);
    if (item < n_items) load_keys<D>(kp, key0 + item * 64, ui.L, kf);
  }
  __syncthreads();   // LDS is restaged by the next segment
}

template <int D, bool MEAN>
__global__ __launch_bounds__(kThreads8) __attribute__((amdgpu_waves_per_eu(2, 2))) void finish8_kernel(const ScoreArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int w = static_cast<int>(blockIdx.x);
  const int T = layer_tiles(a);
  const long long N = static_cast<long long>(T) * a.n_layers;
  // the partials are numbered by the stats pass's split
  Split ss;
  ss.N = N;
  ss.G = static_cast<int>(N < a.stats_grid ? N : a.stats_grid);
  ss.H = ss.G / 2;
  const bool weighted = a.paired && ss.G == a.stats_grid && (ss.G & 1) == 0 && N >= 2LL * ss.G;
  ss.A = weighted ? a.weights.stats_old : 1;
  ss.B = weighted ? a.weights.stats_new : 1;
  Split sp;
  sp.N = N;
  sp.G = static_cast<int>(N < gridDim.x ? N : gridDim.x);
  sp.H = sp.G / 2;
  sp.A = sp.B = 1;
  if (w >= sp.G) return;
  const long long c0 = sp.begin(w);
  const long long c1 = sp.begin(w + 1);
  Cursor cur = locate(a, c0, T);
  long long c = c0;
  for (;;) {
    const long long left = c1 - c;
    const int n = static_cast<int>(left < cur.nt - cur.tile ? left : cur.nt - cur.tile);
    const long long first = c - cur.tile;
    const int w0 = ss.owner(first);
    const UnitInfo ui = unit_info(a, cur.u);
    const size_t unit_part = static_cast<size_t>(cur.u) * a.slots * a.obs_pad;
    const int n_part = ss.owner(first + cur.nt - 1) - w0 + 1;
    finish_segment8<D, MEAN>(a, ui, cur.tile, n, a.part_m + unit_part, a.part_z + unit_part, n_part, smem);
    c += n;
    if (c >= c1 || !next_unit(a, cur)) break;
  }
}

// ---- kernels ----------------------------------------------------------------------------


template <int D, bool FINISH, bool MEAN = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 8))) void score_kernel(const ScoreArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int w = static_cast<int>(blockIdx.x);
  const int T = layer_tiles(a);
  const long long N = static_cast<long long>(T) * a.n_layers;
  // Partial slots are numbered by the stats pass's split (on its own grid) in both passes.
  // With fewer tiles than workgroups only the first N take part, so every share holds at
  // least one tile and a unit's shares are consecutive workgroups.  Weighted shares only
  // where the pairs are real and every share keeps two tiles or more.
  Split ss;
  ss.N = N;
  ss.G = static_cast<int>(N < a.stats_grid ? N : a.stats_grid);
  ss.H = ss.G / 2;
  const bool s_weighted = a.paired && ss.G == a.stats_grid && (ss.G & 1) == 0 && N >= 2LL * ss.G;
  ss.A = s_weighted ? a.weights.stats_old : 1;
  ss.B = s_weighted ? a.weights.stats_new : 1;
  Split sp = ss;
  if (FINISH) {
    sp.G = static_cast<int>(N < gridDim.x ? N : gridDim.x);
    sp.H = sp.G / 2;
    const bool f_weighted =
        a.finish_paired && sp.G == static_cast<int>(gridDim.x) && (sp.G & 1) == 0 && N >= 2LL * sp.G;
    sp.A = f_weighted ? a.weights.finish_old : 1;
    sp.B = f_weighted ? a.weights.finish_new : 1;
  }
  if (w >= sp.G) return;
  const long long c0 = sp.begin(w);
  const long long c1 = sp.begin(w + 1);
  Cursor cur = locate(a, c0, T);
  long long c = c0;
  for (;;) {
    const long long left = c1 - c;
    const int n = static_cast<int>(left < cur.nt - cur.tile ? left : cur.nt - cur.tile);
    const long long first = c - cur.tile;   // global index of the unit's first tile
    const int w0 = ss.owner(first);   // slot 0 of the unit's partials
    const UnitInfo ui = unit_info(a, cur.u);
    const size_t unit_part = static_cast<size_t>(cur.u) * a.slots * a.obs_pad;
    if (FINISH) {
      const int n_part = ss.owner(first + cur.nt - 1) - w0 + 1;
      finish_segment<D, MEAN>(a, ui, cur.tile, n, a.part_m + unit_part, a.part_z + unit_part, n_part, smem);
    } else if (w - w0 < a.slots) {   // past the slots: no partial (the finish pass gives NaN)
      const size_t o = unit_part + static_cast<size_t>(w - w0) * a.obs_pad;
      stats_segment<D>(a, ui, cur.tile, n, a.part_m + o, a.part_z + o, smem);
    }
    c += n;
    if (c >= c1 || !next_unit(a, cur)) break;
  }
}

size_t lds_bytes(int head_dim, int obs_pad) {
  return static_cast<size_t>(obs_pad) * (head_dim * 2) + 4 * kWaves * obs_pad * sizeof(float);
}

template <int D>
hipError_t launch_d(ScoreArgs a, int n_layers, hipStream_t s) {
  static PerDeviceOnce once;
  const hipError_t attr_err = once_per_device(once, [] {
    const void* kernels[] = {reinterpret_cast<const void*>(&score_kernel<D, false>),
                             reinterpret_cast<const void*>(&score_kernel<D, true>),
                             reinterpret_cast<const void*>(&score_kernel<D, true, true>),
                             reinterpret_cast<const void*>(&finish8_kernel<D, true>),
                             reinterpret_cast<const void*>(&finish8_kernel<D, false>)};
    for (const void* k : kernels) {
      const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  });
  if (attr_err != hipSuccess) return note_hip_error(attr_err, "score: hipFuncSetAttribute");
  const size_t lds = lds_bytes(D, a.obs_pad);
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return note_hip_error(e, "score: hipGetDevice");
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return note_hip_error(e, "score: hipDeviceGetAttribute");
  int per_cu_stats = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, score_kernel<D, true>, kThreads, lds);
  if (e != hipSuccess) return note_hip_error(e, "score: hipOccupancyMaxActiveBlocksPerMultiprocessor");
  // The stats pass keeps the observation rows in registers where they fit.
  const bool qs_stats = qs_stats_covers(D, a.obs_pad);
  if (qs_stats)
    e = qs_stats_occupancy(D, a.obs_pad, &per_cu_stats);
  else
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_stats, score_kernel<D, false>, kThreads, lds);
  if (e != hipSuccess) return note_hip_error(e, "score: hipOccupancyMaxActiveBlocksPerMultiprocessor");
  // Every workgroup resident at once (at most two per CU): the shares are static, so none
  // waits for a slot.  Each pass runs on its own grid; the stats grid numbers the partials.
  per_cu = std::max(1, std::min(2, per_cu));
  per_cu_stats = std::max(1, std::min(2, per_cu_stats));
  const int grid = std::min(kScoreMaxGrid, per_cu_stats * cus);
  const int grid_finish = std::min(kScoreMaxGrid, per_cu * cus);
  a.n_layers = n_layers;
  a.slots = score_slots(a.capacity, n_layers, a.n_kv_heads);
  a.stats_grid = grid;
  a.paired = per_cu_stats == 2 ? 1 : 0;
  a.finish_paired = per_cu == 2 ? 1 : 0;
  a.weights = qs_stats && (a.obs_pad / 32) % kWaves == 0 ? kWeightsBalanced : kWeightsDefault;
  if (qs_stats) {
    e = launch_qs_stats(a, D, grid, s);
    if (e != hipSuccess) return e;
  } else {
    hipLaunchKernelGGL((score_kernel<D, false>), dim3(grid), dim3(kThreads), lds, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return note_hip_error(e, "score: launch score_stats");
  }
  if (per_cu == 1) {   // one workgroup of 4 waves per CU: take the 8-wave finish instead
    const size_t lds8 = static_cast<size_t>(a.obs_pad) * (D * 2 + sizeof(float)) + 16;
    if (a.mean)
      hipLaunchKernelGGL((finish8_kernel<D, true>), dim3(cus), dim3(kThreads8), lds8, s, a);
    else
      hipLaunchKernelGGL((finish8_kernel<D, false>), dim3(cus), dim3(kThreads8), lds8, s, a);
  } else if (a.mean) {
    hipLaunchKernelGGL((score_kernel<D, true, true>), dim3(grid_finish), dim3(kThreads), lds, s, a);
  } else {
    hipLaunchKernelGGL((score_kernel<D, true>), dim3(grid_finish), dim3(kThreads), lds, s, a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return note_hip_error(e, "score: launch score_finish");
  return hipSuccess;
}

}  // namespace

hipError_t launch_score(const ScoreArgs& a, int n_layers, int head_dim, hipStream_t s) {
  if (head_dim == 128) return launch_d<128>(a, n_layers, s);
  return launch_d<64>(a, n_layers, s);
}

}  // namespace bkv
