// Statistics pass of the max-aggregated attention scores (per observation row the max
// and the sum of exp2 of its logits over a unit piece; BeaconKV page, Figure 5 (b), (c))
// with the observation rows held in registers and the keys streamed through LDS.  Same
// work split and statistics partials as the LDS-staged stats pass of score.hip, whose
// finish pass consumes them; used for up to 16 blocks of 32 observation rows at head_dim
// 128 and up to 12 at 64.
//
// Per workgroup (NW = 4 or 8 waves) the observation row blocks are dealt round-robin to the
// waves: wave w keeps blocks w, w + NW (and w + 2 NW) in registers for the whole unit
// piece.  Every wave works on every 32-key fragment, so a fragment is fetched from HBM once
// per workgroup, by all waves together, straight into LDS (`global_load_lds_dwordx4`, no
// registers), into a ring of kSlots slots that keeps kSlots - 1 fragments in flight.  Each
// 16-byte key chunk read from LDS into the MFMA layout serves one product per owned row
// block.
//
// Ring protocol, per fragment f: every wave waits for its own loads of f (in-order
// vmcnt), the workgroup meets at a barrier (now all of f is in LDS and every wave is done
// with f - 1), and the loads of f + kSlots - 1 go into the slot f - 1 used.
#include <algorithm>
#include <type_traits>

#include "score_common.h"

namespace bkv {
namespace {

constexpr int kSlots = 4;
constexpr int kAhead = kSlots - 1;

template <int D, int NW>
struct Qs {
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kChunks = D / 8;                    // 16-byte chunks per key row
  static constexpr int kFragBytes = 32 * kRowBytes;        // one 32-key fragment
  static constexpr int kInstr = kFragBytes / 1024;         // 64-lane 16-byte loads per fragment
  static constexpr int kPerWave = kInstr / NW;
  static constexpr int kRowsPerInstr = 1024 / kRowBytes;
  static constexpr int kS = D / 16;                        // MFMA k-steps per row
  static_assert(kPerWave >= 1 && kInstr % NW == 0, "fragment loads split evenly over the waves");
};

// s_waitcnt immediate: vector memory count <= vm and LDS count <= lgkm (export count
// unconstrained).
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8); }

// The wave's share of the loads of one fragment (keys key0 .. key0+31, rows past L read
// row L-1) into `slot`.  Lane i of load j lands at slot + 1024 j + 16 i, i.e. key row r
// = j * kRowsPerInstr + i / kChunks at chunk position p = i % kChunks; the lane fetches
// chunk p ^ (r mod kChunks) of that row, so LDS holds row r's chunk c at position
// c ^ (r mod kChunks) (the swizzle that makes the MFMA-layout reads conflict-free) while
// every load still covers whole key rows.
template <int D, int NW>
__device__ inline void issue_fragment(const uint16_t* kp, int key0, int L, uint8_t* slot) {
  using C = Qs<D, NW>;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < C::kPerWave; ++j) {
    const int ins = wave * C::kPerWave + j;
    const int r = ins * C::kRowsPerInstr + lane / C::kChunks;
    const int c = (lane % C::kChunks) ^ (r & (C::kChunks - 1));
    int key = key0 + r;
    key = key < L ? key : L - 1;
    __builtin_amdgcn_global_load_lds((const void*)(kp + static_cast<size_t>(key) * D + c * 8),
                                     (__attribute__((address_space(3))) void*)(slot + ins * 1024), 16, 0, 0);
  }
}

// k-step s of the fragment in `slot`: lane l gets key (l & 31), dims 16 s + 8 (l >> 5) .. +7.
template <int D>
__device__ inline bf16x8 key_chunk(const uint8_t* slot, int s) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 31;
  const unsigned base = static_cast<unsigned>(r * (2 * D) + 16 * ((r & (D / 8 - 1)) ^ (lane >> 5)));
  return *reinterpret_cast<const bf16x8*>(slot + (base ^ (32u * s)));
}

template <int D>
struct KeyRegs {
  bf16x8 v[D / 16];
};

template <int D>
__device__ inline void read_keys(const uint8_t* slot, KeyRegs<D>& k) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s) k.v[s] = key_chunk<D>(slot, s);
}

// Fragment f has landed in LDS for the whole workgroup, and no wave still reads the slot
// of f - 1.  kImm: vector memory count <= the operations this wave issued after its loads
// of f, LDS count 0.
template <int kImm>
__device__ inline void ring_wait() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kImm);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Observation row blocks of this wave: blk = wave + 4 b for b < BPW.  Lane l holds row
// blk*32 + (l & 31), dims 16 s + 8 (l >> 5) .. +7 of k-step s (the same registers serve
// as the B operand of the stats pass and the A operand of the finish pass); rows at or
// past n_obs are zero.
template <int D, int BPW>
struct RowRegs {
  bf16x8 v[BPW][D / 16];
};

template <int D, int BPW, int NW>
__device__ inline void load_rows(const ScoreArgs& a, const UnitInfo& ui, RowRegs<D, BPW>& q) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int gw = a.group * a.window;
  // the unit's first recent-query row and first beacon row (uniform across the wave)
  const uint16_t* q0 = a.window > 0 ? a.q[ui.layer] + ((static_cast<size_t>(ui.b) * a.n_q_heads + ui.h * a.group) *
                                                       a.q_len + (a.q_len - a.window)) * D : nullptr;
  const uint16_t* b0 = a.nb_max > 0 ? a.beacons[ui.layer] + (static_cast<size_t>(ui.b) * a.n_kv_heads + ui.h) *
                                                                a.nb_max * D : nullptr;
#pragma unroll
  for (int b = 0; b < BPW; ++b) {
    const int r = (wave + NW * b) * 32 + (lane & 31);
    const uint16_t* p = nullptr;
    if (r < gw)   // query head h * G + r / window, its row q_len - window + r % window
      p = q0 + (static_cast<size_t>(r / a.window) * a.q_len + r % a.window) * D;
    else if (r < ui.n_obs)
      p = b0 + static_cast<size_t>(r - gw) * D;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      bf16x8 v = {};
      if (p != nullptr) v = *reinterpret_cast<const bf16x8*>(p + 16 * s + 8 * (lane >> 5));
      q.v[b][s] = v;
    }
  }
}

// Row blocks this wave owns in a unit with nqb blocks (NW waves per workgroup).
template <int NW>
__device__ inline int owned_blocks(int nqb) {
  const int wave = threadIdx.x >> 6;
  return nqb > wave ? (nqb - wave + NW - 1) / NW : 0;
}

// ---- stats pass -------------------------------------------------------------------------
//
// A = 32 keys x 16 dims (from LDS), B = 16 dims x 32 rows (registers): register r of
// lane l holds key key0 + 8 (r >> 2) + 4 (l >> 5) + (r & 3) of row (l & 31), so each lane
// keeps a running (max, sum of exp2) for its row and half of the keys.  The products of
// fragment f (both owned blocks, two independent accumulator chains) are issued among the
// exp2 work of fragment f - 1.

struct RowStat {
  float m, z;
};

__device__ inline void mask_keys(f32x16& acc, int key0, int L) {
  const int half = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (key0 + 8 * (r >> 2) + 4 * half + (r & 3) >= L) acc[r] = kNegInf;
}

// Exact update: block max first, running sum rescaled.
__device__ inline void stat_exact(const f32x16& acc, float c, RowStat& st) {
  float mx = kNegInf;
#pragma unroll
  for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[r]);
  if (mx == kNegInf) return;
  const float mt = fmaxf(mx * c, st.m);
  float zt = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) zt += __builtin_amdgcn_exp2f(fmaf(acc[r], c, -mt));
  st.z = (st.m == kNegInf ? 0.f : st.z * __builtin_amdgcn_exp2f(st.m - mt)) + zt;
  st.m = mt;
}

// Cheap update against the running max of earlier fragments; falls back to the exact
// update when a term may have overflowed (a logit ~64 above the running max, or the
// row's first fragment while the max is still -inf).
constexpr float kFastSumLimit = 1.8e19f;

__device__ inline void stat_commit(const f32x16& acc, float zt, float c, RowStat& st) {
  if (zt <= kFastSumLimit)
    st.z += zt;
  else
    stat_exact(acc, c, st);
}

// Products of fragment k for NB blocks into `nxt` while the exp2 sums of `cur` (the
// previous fragment, when `has_cur`) are taken; per k-step the vector work comes first, so
// it covers the LDS reads of the keys.
template <int D, int BPW, int NB, bool MASK>
__device__ inline void stats_step(const KeyRegs<D>& k, const RowRegs<D, BPW>& q, f32x16 (&cur)[BPW],
                                  f32x16 (&nxt)[BPW], RowStat (&st)[BPW], int pkey0, int L, float c) {
  constexpr int S = D / 16;
  constexpr int kPer = 16 / S;   // exp2 items per block per k-step
  f32x16 x[NB];
  float neg[NB];
  float zs[NB][2];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    x[b] = cur[b];
    if (MASK) mask_keys(x[b], pkey0, L);
    neg[b] = -st[b].m;
    zs[b][0] = 0.f;
    zs[b][1] = 0.f;
  }
  f32x16 n[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) n[b] = f32x16{};
#pragma unroll
  for (int s = 0; s < S; ++s) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        zs[b][j & 1] += __builtin_amdgcn_exp2f(fmaf(x[b][s * kPer + j], c, neg[b]));
#pragma unroll
    for (int b = 0; b < NB; ++b) n[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k.v[s], q.v[b][s], n[b], 0, 0, 0);
  }
#pragma unroll
  for (int s = 0; s < S; ++s) {
    __builtin_amdgcn_sched_group_barrier(0x402, 3 * kPer * NB, 0);   // VALU / transcendental
    __builtin_amdgcn_sched_group_barrier(0x008, NB, 0);              // MFMA
  }
  // One branch for all blocks: every block's sum feeds its condition, so the exp2 work of
  // every block stays in the basic block of the products instead of sinking past an
  // earlier block's overflow branch.
  float zt[NB];
  bool fast = true;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    zt[b] = zs[b][0] + zs[b][1];
    fast = fast && zt[b] <= kFastSumLimit;
  }
  if (fast) {
#pragma unroll
    for (int b = 0; b < NB; ++b) st[b].z += zt[b];
  } else {
#pragma unroll
    for (int b = 0; b < NB; ++b) stat_commit(x[b], zt[b], c, st[b]);
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) nxt[b] = n[b];
}

template <int D, int BPW, int NB>
__device__ inline void stats_first(const KeyRegs<D>& k, const RowRegs<D, BPW>& q, f32x16 (&nxt)[BPW]) {
  f32x16 n[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) n[b] = f32x16{};
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
#pragma unroll
    for (int b = 0; b < NB; ++b) n[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k.v[s], q.v[b][s], n[b], 0, 0, 0);
#pragma unroll
  for (int b = 0; b < NB; ++b) nxt[b] = n[b];
}

template <int NB, int BPW, bool MASK>
__device__ inline void stats_drain(f32x16 (&cur)[BPW], RowStat (&st)[BPW], int pkey0, int L, float c) {
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    f32x16 x = cur[b];
    if (MASK) mask_keys(x, pkey0, L);
    const float neg = -st[b].m;
    float zs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 16; ++r) zs[r & 3] += __builtin_amdgcn_exp2f(fmaf(x[r], c, neg));
    stat_commit(x, (zs[0] + zs[1]) + (zs[2] + zs[3]), c, st[b]);
  }
}

// The fragment loop of a wave owning NB >= 1 blocks.  Two accumulator sets alternate
// (fragment f's products in one while the other's exp2 work is done), unrolled by two so
// that both stay in registers.
template <int D, int BPW, int NB, int NW>
__device__ inline void stats_loop(const uint16_t* kp, const UnitInfo& ui, int key_begin, int nf, uint8_t* ring,
                                  const RowRegs<D, BPW>& q, RowStat (&st)[BPW], float c) {
  using C = Qs<D, NW>;
  f32x16 A[BPW], B[BPW];
  // slot_c: the ring slot of fragment f (f % kSlots) as a compile-time constant, so the slot
  // offsets of the loads and LDS reads are immediates
  auto step = [&](auto slot_c, int f, f32x16(&nxt)[BPW], f32x16(&cur)[BPW]) {
    constexpr int kSlot = decltype(slot_c)::value;
    ring_wait<waitcnt_imm((kAhead - 1) * C::kPerWave, 0)>();
    const int fa = f + kAhead < nf ? f + kAhead : nf - 1;
    issue_fragment<D, NW>(kp, key_begin + 32 * fa, ui.L, ring + ((kSlot + kAhead) % kSlots) * C::kFragBytes);
    KeyRegs<D> k;
    read_keys<D>(ring + kSlot * C::kFragBytes, k);
    if (f == 0) {
      stats_first<D, BPW, NB>(k, q, nxt);
    } else {
      const int pkey0 = key_begin + 32 * (f - 1);
      if (pkey0 + 32 > ui.L)
        stats_step<D, BPW, NB, true>(k, q, cur, nxt, st, pkey0, ui.L, c);
      else
        stats_step<D, BPW, NB, false>(k, q, cur, nxt, st, pkey0, ui.L, c);
    }
  };
  static_assert(kSlots == 4, "the loop below walks the ring slots in order");
  for (int f = 0; f < nf; f += 4) {
    step(std::integral_constant<int, 0>{}, f, A, B);
    if (f + 1 < nf) step(std::integral_constant<int, 1>{}, f + 1, B, A);
    if (f + 2 < nf) step(std::integral_constant<int, 2>{}, f + 2, A, B);
    if (f + 3 < nf) step(std::integral_constant<int, 3>{}, f + 3, B, A);
  }
  auto drain = [&](f32x16(&last)[BPW]) {
    const int pkey0 = key_begin + 32 * (nf - 1);
    if (pkey0 + 32 > ui.L)
      stats_drain<NB, BPW, true>(last, st, pkey0, ui.L, c);
    else
      stats_drain<NB, BPW, false>(last, st, pkey0, ui.L, c);
  };
  if (nf & 1)
    drain(A);
  else
    drain(B);
}

// Tiles tile0 .. tile0+ntile-1 of one unit -> partial statistics out_m/out_z [nqb*32].
template <int D, int BPW, int NW>
__device__ void qs_stats_segment(const ScoreArgs& a, const UnitInfo& ui, int tile0, int ntile, float* out_m,
                                 float* out_z, uint8_t* ring) {
  using C = Qs<D, NW>;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint16_t* kp = a.k[ui.layer] + (static_cast<size_t>(ui.b) * a.n_kv_heads + ui.h) * a.capacity * D;
  const int key_begin = tile0 * kScoreTile;
  const int key_end = std::min(ui.L, (tile0 + ntile) * kScoreTile);
  const int nf = (key_end - key_begin + 31) / 32;
#pragma unroll
  for (int f = 0; f < kAhead; ++f)
    issue_fragment<D, NW>(kp, key_begin + 32 * (f < nf ? f : nf - 1), ui.L, ring + f * C::kFragBytes);
  RowRegs<D, BPW> q;
  load_rows<D, BPW, NW>(a, ui, q);
  const int nb = owned_blocks<NW>(ui.nqb);
  const float c = a.scale_log2;
  RowStat st[BPW];
#pragma unroll
  for (int b = 0; b < BPW; ++b) st[b] = RowStat{kNegInf, 0.f};
  if (nb == BPW) {
    stats_loop<D, BPW, BPW, NW>(kp, ui, key_begin, nf, ring, q, st, c);
  } else if (BPW == 3 && nb == 2) {
    stats_loop<D, BPW, (BPW > 2 ? 2 : 1), NW>(kp, ui, key_begin, nf, ring, q, st, c);
  } else if (nb == 1) {
    stats_loop<D, BPW, 1, NW>(kp, ui, key_begin, nf, ring, q, st, c);
  } else {   // no rows: keep the workgroup's barrier count
    for (int f = 0; f < nf; ++f) {
      ring_wait<waitcnt_imm((kAhead - 1) * C::kPerWave, 0)>();
      issue_fragment<D, NW>(kp, key_begin + 32 * (f + kAhead < nf ? f + kAhead : nf - 1), ui.L,
                            ring + ((f + kAhead) % kSlots) * C::kFragBytes);
    }
  }
  // lanes l and l ^ 32 hold the two key halves of the same row
#pragma unroll
  for (int b = 0; b < BPW; ++b) {
    if (b < nb) {
      float m = st[b].m, z = st[b].z;
      merge_stats(m, z, __shfl_xor(m, 32), __shfl_xor(z, 32));
      const int row = (wave + NW * b) * 32 + lane;
      if (lane < 32) {
        out_m[row] = m;
        out_z[row] = z;
      }
    }
  }
  __syncthreads();   // the ring is refilled by the next segment; its loads have all landed
}

// ---- kernels ----------------------------------------------------------------------------


template <int D>
constexpr size_t qs_lds_bytes() {
  return static_cast<size_t>(kSlots) * 32 * 2 * D;
}

template <int D, int BPW, int NW>
__device__ inline void qs_stats_body(const ScoreArgs& a, uint8_t* ring) {
  const int w = static_cast<int>(blockIdx.x);
  const int T = layer_tiles(a);
  Split sp;
  sp.N = static_cast<long long>(T) * a.n_layers;
  sp.G = static_cast<int>(sp.N < gridDim.x ? sp.N : gridDim.x);
  if (w >= sp.G) return;
  const bool weighted = a.paired && sp.G == static_cast<int>(gridDim.x) && (sp.G & 1) == 0 && sp.N >= 2LL * sp.G;
  sp.H = sp.G / 2;
  sp.A = weighted ? a.weights.stats_old : 1;
  sp.B = weighted ? a.weights.stats_new : 1;
  const long long c0 = sp.begin(w);
  const long long c1 = sp.begin(w + 1);
  Cursor cur = locate(a, c0, T);
  long long c = c0;
  for (;;) {
    const long long left = c1 - c;
    const int n = static_cast<int>(left < cur.nt - cur.tile ? left : cur.nt - cur.tile);
    const int w0 = sp.owner(c - cur.tile);   // slot 0 of the unit's partials
    const UnitInfo ui = unit_info(a, cur.u);
    // A workgroup past the unit's slots (which the host's sizing rules out) has nowhere to
    // put its partial; the finish pass then gives the unit NaN scores.
    if (w - w0 < a.slots) {
      const size_t o = (static_cast<size_t>(cur.u) * a.slots + (w - w0)) * a.obs_pad;
      qs_stats_segment<D, BPW, NW>(a, ui, cur.tile, n, a.part_m + o, a.part_z + o, ring);
    }
    c += n;
    if (c >= c1 || !next_unit(a, cur)) break;
  }
}

// Up to two row blocks per wave fit in 256 registers (two waves per SIMD); three take one
// wave per SIMD and its 512 registers.  With head_dim 128, 9 to 16 blocks instead take one
// workgroup of 8 waves per CU (two per SIMD, up to two blocks each).
template <int D, int BPW>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 8))) void qs_stats_kernel(const ScoreArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t ring[];
  qs_stats_body<D, BPW, kWaves>(a, ring);
}

template <int D, int BPW>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void qs_stats_kernel_wide(
    const ScoreArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t ring[];
  qs_stats_body<D, BPW, kWaves>(a, ring);
}

constexpr int kWaves8 = 8;

template <int D>
__global__ __launch_bounds__(64 * kWaves8) __attribute__((amdgpu_waves_per_eu(2, 2))) void qs_stats_kernel8(
    const ScoreArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t ring[];
  qs_stats_body<D, 2, kWaves8>(a, ring);
}

// Kernel of a row-block count class: 1, 2 or 3 blocks per wave of 4, or 8 waves (BPW 8).
template <int D, int BPW>
constexpr auto qs_kernel_of() {
  if constexpr (BPW == 8)
    return &qs_stats_kernel8<D>;
  else if constexpr (BPW == 3)
    return &qs_stats_kernel_wide<D, BPW>;
  else
    return &qs_stats_kernel<D, BPW>;
}

template <int BPW>
constexpr int threads_of() {
  return BPW == 8 ? 64 * kWaves8 : kThreads;
}

template <int D, int BPW>
hipError_t prepare() {
  static PerDeviceOnce once;
  return once_per_device(once, [] {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(qs_kernel_of<D, BPW>()),
                               hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(qs_lds_bytes<D>()));
  });
}

template <int D, int BPW>
hipError_t occupancy(int* per_cu) {
  hipError_t e = prepare<D, BPW>();
  if (e != hipSuccess) return note_hip_error(e, "score: hipFuncSetAttribute");
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, qs_kernel_of<D, BPW>(), threads_of<BPW>(),
                                                   qs_lds_bytes<D>());
  return note_hip_error(e, "score: hipOccupancyMaxActiveBlocksPerMultiprocessor");
}

template <int D, int BPW>
hipError_t launch(const ScoreArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((qs_kernel_of<D, BPW>()), dim3(grid), dim3(threads_of<BPW>()), qs_lds_bytes<D>(), s, a);
  return note_hip_error(hipGetLastError(), "score: launch score_stats");
}

}  // namespace

// Kernel class of a row count: 1, 2 or 3 blocks per wave of a 4-wave workgroup (up to 128,
// 256 or 384 padded rows), or, with head_dim 128, 8 waves for 257 to 512 rows.
static int blocks_per_wave(int head_dim, int obs_pad) {
  if (head_dim == 128 && obs_pad > kWaves * 64) return 8;
  return (obs_pad + kWaves * 32 - 1) / (kWaves * 32);
}

bool qs_stats_covers(int head_dim, int obs_pad) { return obs_pad <= (head_dim == 128 ? 512 : kQsMaxRows); }

hipError_t qs_stats_occupancy(int head_dim, int obs_pad, int* per_cu) {
  const int bpw = blocks_per_wave(head_dim, obs_pad);
  if (head_dim == 128) return bpw == 8 ? occupancy<128, 8>(per_cu) : bpw == 2 ? occupancy<128, 2>(per_cu)
                                                                              : occupancy<128, 1>(per_cu);
  return bpw == 3 ? occupancy<64, 3>(per_cu) : bpw == 2 ? occupancy<64, 2>(per_cu) : occupancy<64, 1>(per_cu);
}

hipError_t launch_qs_stats(const ScoreArgs& a, int head_dim, int grid, hipStream_t s) {
  const int bpw = blocks_per_wave(head_dim, a.obs_pad);
  if (head_dim == 128)
    return bpw == 8 ? launch<128, 8>(a, grid, s) : bpw == 2 ? launch<128, 2>(a, grid, s) : launch<128, 1>(a, grid, s);
  return bpw == 3 ? launch<64, 3>(a, grid, s) : bpw == 2 ? launch<64, 2>(a, grid, s) : launch<64, 1>(a, grid, s);
}

}  // namespace bkv
