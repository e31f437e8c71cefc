// Beacon maintenance by continual farthest-point sampling on cosine distance
// (BeaconKV page, Figure 7 caption "Continual FPS"; Abstract: beacons represent the
// global query clusters without keeping the query history; Figure 4 (a): queries are
// compared by their cosine).
//
// Pools of up to 768 rows (continual updates): one workgroup per unit, one thread per pool
// row (the workgroup is the largest pool rounded up to whole waves, so two units share a CU
// on the largest workloads); larger pools take fps_pool_kernel below.  Thread p
// holds pool row p (live beacons, then the group's new queries head-major in time order)
// in registers as packed bf16 pairs, with its inverse norm.  Once a pick is known every
// wave loads its row from the (read-only) pool source into scalar registers by scalar
// loads, and each thread takes the dot product of its row with it by v_dot2_f32_bf16 with
// the row in SGPRs: no cross-lane reduction and no per-word lane moves.  Each thread keeps
// its row's distance to the nearest chosen row; a block-wide max of (distance, lowest index
// on ties) names the next pick: a DPP max per wave, then one 64-bit LDS atomic max per wave
// of (distance key, complement of the index), read back by every thread after a barrier.
// One barrier per pick.

#include "bkv_internal.h"

namespace bkv {
namespace {

constexpr int kWaves = kFpsThreads / 64;

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef const __attribute__((address_space(4))) uint32_t* const_u32;
typedef __attribute__((ext_vector_type(16))) uint32_t u32x16;
typedef const __attribute__((address_space(4))) u32x16* const_u32x16;

__device__ inline float dot2(uint32_t x, uint32_t y, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), __builtin_bit_cast(bf16x2, y), acc, false);
}

// Max over the wave of non-negative 32-bit values: four DPP steps give every lane its
// 16-lane row's max (lane pairs i^1, i^2, then mirrors within 8 and 16 lanes), and the
// four rows meet in scalar registers.
__device__ inline unsigned wave_umax(unsigned v) {
  v = max(v, static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xB1, 0xF, 0xF, false)));   // quad_perm 1,0,3,2
  v = max(v, static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4E, 0xF, 0xF, false)));   // quad_perm 2,3,0,1
  v = max(v, static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x141, 0xF, 0xF, false)));  // row_half_mirror
  v = max(v, static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x140, 0xF, 0xF, false)));  // row_mirror
  const unsigned r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const unsigned r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return max(max(r0, r1), max(r2, r3));
}

template <int D>
__global__ __launch_bounds__(kFpsThreads) void fps_kernel(const FpsArgs a) {
  constexpr int W = D / 2;   // 32-bit words (bf16 pairs) per row
  __shared__ float inv_s[kFpsThreads];
  __shared__ unsigned long long src_s[kFpsThreads];   // address of each pool row's source
  __shared__ unsigned long long best[3];   // per pick (mod 3): max of (distance key << 32 | ~index)
  const int nthr = static_cast<int>(blockDim.x);

  const int u = blockIdx.x;
  const int per_layer = a.batch * a.n_kv_heads;
  const int layer = u / per_layer;
  const int bh = u - layer * per_layer;
  const int b = bh / a.n_kv_heads;
  const int h = bh - b * a.n_kv_heads;
  int c_in = a.nb_max > 0 ? a.n_in[layer][bh] : 0;
  c_in = c_in < 0 ? 0 : (c_in > a.nb_max ? a.nb_max : c_in);
  const int P = c_in + a.group * a.t_new;
  const uint16_t* bin = a.beacons_in[layer] + static_cast<size_t>(bh) * a.nb_max * D;
  const uint16_t* qn = a.q_new[layer];
  uint16_t* out = a.beacons_out[layer] + static_cast<size_t>(bh) * a.nb_max * D;
  const int tid = threadIdx.x;

  auto row_ptr = [&](int p) -> const uint16_t* {
    if (p < c_in) return bin + static_cast<size_t>(p) * D;
    const int qi = p - c_in;
    const int r = qi / a.t_new;
    const int t = qi - r * a.t_new;
    return qn + ((static_cast<size_t>(b) * a.n_q_heads + h * a.group + r) * a.q_len + (a.q_len - a.t_new + t)) * D;
  };

  if (P <= a.nb_max) {  // everything fits: keep the pool as is
    constexpr int kChunks = D / 8;
    for (int e = tid; e < P * kChunks; e += nthr) {
      const int p = e / kChunks;
      const int cc = e - p * kChunks;
      *reinterpret_cast<uint4*>(out + static_cast<size_t>(p) * D + cc * 8) =
          *reinterpret_cast<const uint4*>(row_ptr(p) + cc * 8);
    }
    if (tid == 0) a.n_out[layer][bh] = P;
    return;
  }

  const int p = tid;
  const bool have = p < P;
  uint32_t x[W];
  if (have) {
    const uint4* src = reinterpret_cast<const uint4*>(row_ptr(p));
    src_s[p] = reinterpret_cast<unsigned long long>(src);
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      const uint4 v = src[i];
      x[4 * i] = v.x;
      x[4 * i + 1] = v.y;
      x[4 * i + 2] = v.z;
      x[4 * i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < W; ++i) x[i] = 0u;
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < W; ++i) ss = dot2(x[i], x[i], ss);
  const float inv = 1.0f / fmaxf(sqrtf(ss), 1e-30f);
  inv_s[tid] = inv;
  if (tid == 0) best[0] = 0ull;
  __syncthreads();   // every row's inverse norm is read by index below

  float mind = 0.f;
  bool avail = have;
  int cur = 0;
  for (int t = 0; t < a.nb_max; ++t) {
    if (p == cur) {   // the pick's owner writes it out and leaves the candidates
      uint4* dst = reinterpret_cast<uint4*>(out + static_cast<size_t>(t) * D);
#pragma unroll
      for (int i = 0; i < W / 4; ++i) dst[i] = make_uint4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
      avail = false;
    }
    if (t == a.nb_max - 1) break;
    unsigned key = 0;   // distance bits + 1 (monotone for distances >= 0); 0: cannot be picked
    if ((tid & ~63) < P) {   // waves holding no pool row skip the products
      // the pick's row from its read-only source, through the scalar cache: its address is
      // one LDS word for the whole block, moved to scalar registers
      const unsigned long long sa = src_s[cur];
      const unsigned lo = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(sa));
      const unsigned hi = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(sa >> 32));
      const const_u32x16 y = (const_u32x16)((static_cast<unsigned long long>(hi) << 32) | lo);
      // all of the row's loads issued before the first product: one scalar-cache round trip
      u32x16 yr[W / 16];
#pragma unroll
      for (int i = 0; i < W / 16; ++i) yr[i] = y[i];
      float acc[2] = {0.f, 0.f};   // two chains: shorter dependency
#pragma unroll
      for (int i = 0; i < W / 2; ++i) {
        acc[0] = dot2(x[2 * i], yr[i / 8][(2 * i) % 16], acc[0]);
        acc[1] = dot2(x[2 * i + 1], yr[i / 8][(2 * i + 1) % 16], acc[1]);
      }
      const float dt = acc[0] + acc[1];
      float d = 1.0f - dt * inv * inv_s[cur];
      d = fminf(fmaxf(d, 0.f), 2.f);
      mind = t == 0 ? d : fminf(mind, d);
      key = avail ? __float_as_uint(mind) + 1u : 0u;
    }
    const unsigned wmax = wave_umax(key);
    // lowest lane holding the wave max = lowest pool index of the wave; one LDS max per
    // wave of (key, complement of the index): the largest key wins, then the lowest index
    const unsigned long long hit = __ballot(key == wmax);
    // best[(t + 1) % 3] was last read right after pick t - 2's barrier, which every thread
    // has left behind since passing pick t - 1's barrier: safe to clear for pick t + 1
    if (tid == 0) best[(t + 1) % 3] = 0ull;
    if ((tid & 63) == 0) {
      const unsigned idx = static_cast<unsigned>((tid & ~63) + __ffsll(static_cast<long long>(hit)) - 1);
      atomicMax(&best[t % 3], (static_cast<unsigned long long>(wmax) << 32) | (0xffffffffu - idx));
    }
    __syncthreads();
    const unsigned long long bw = best[t % 3];
    cur = __builtin_amdgcn_readfirstlane(static_cast<int>(0xffffffffu - static_cast<unsigned>(bw)));
  }
  if (tid == 0) a.n_out[layer][bh] = a.nb_max;
}

// Pools larger than the register-resident kernel takes (the Naive FPS of Figure 7: every
// query of the history in one pool): 1024 threads per unit, thread t handles pool rows
// t, t + 1024, ...  Each row's inverse norm and distance to its nearest chosen row sit in
// LDS (a chosen row's distance is set to -1, which no distance reaches), and each pick
// streams the rows again from their read-only sources.  Picks, distances and the tie rule
// (lowest pool index) are those of fps_kernel.
template <int D>
__global__ __launch_bounds__(kFpsThreads) void fps_pool_kernel(const FpsArgs a) {
  constexpr int W = D / 2;
  extern __shared__ float2 row_s[];   // [pool rows]: (inverse norm, distance to the chosen set)
  __shared__ unsigned best_v[2][kWaves];
  __shared__ int best_i[2][kWaves];
  const int u = blockIdx.x;
  const int per_layer = a.batch * a.n_kv_heads;
  const int layer = u / per_layer;
  const int bh = u - layer * per_layer;
  const int b = bh / a.n_kv_heads;
  const int h = bh - b * a.n_kv_heads;
  int c_in = a.nb_max > 0 ? a.n_in[layer][bh] : 0;
  c_in = c_in < 0 ? 0 : (c_in > a.nb_max ? a.nb_max : c_in);
  const int P = c_in + a.group * a.t_new;
  const uint16_t* bin = a.beacons_in[layer] + static_cast<size_t>(bh) * a.nb_max * D;
  const uint16_t* qn = a.q_new[layer];
  uint16_t* out = a.beacons_out[layer] + static_cast<size_t>(bh) * a.nb_max * D;
  const int tid = threadIdx.x;

  auto row_ptr = [&](int p) -> const uint16_t* {
    if (p < c_in) return bin + static_cast<size_t>(p) * D;
    const int qi = p - c_in;
    const int r = qi / a.t_new;
    const int t = qi - r * a.t_new;
    return qn + ((static_cast<size_t>(b) * a.n_q_heads + h * a.group + r) * a.q_len + (a.q_len - a.t_new + t)) * D;
  };

  if (P <= a.nb_max) {  // everything fits: keep the pool as is
    constexpr int kChunks = D / 8;
    for (int e = tid; e < P * kChunks; e += kFpsThreads) {
      const int p = e / kChunks;
      const int cc = e - p * kChunks;
      *reinterpret_cast<uint4*>(out + static_cast<size_t>(p) * D + cc * 8) =
          *reinterpret_cast<const uint4*>(row_ptr(p) + cc * 8);
    }
    if (tid == 0) a.n_out[layer][bh] = P;
    return;
  }

  for (int p = tid; p < P; p += kFpsThreads) {
    const uint4* src = reinterpret_cast<const uint4*>(row_ptr(p));
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      const uint4 v = src[i];
      ss = dot2(v.x, v.x, ss);
      ss = dot2(v.y, v.y, ss);
      ss = dot2(v.z, v.z, ss);
      ss = dot2(v.w, v.w, ss);
    }
    row_s[p] = make_float2(1.0f / fmaxf(sqrtf(ss), 1e-30f), 2.f);
  }
  __syncthreads();

  int cur = 0;
  for (int t = 0; t < a.nb_max; ++t) {
    if ((cur & (kFpsThreads - 1)) == tid) {   // the pick's owner writes it out and leaves the candidates
      const uint4* src = reinterpret_cast<const uint4*>(row_ptr(cur));
      uint4* dst = reinterpret_cast<uint4*>(out + static_cast<size_t>(t) * D);
#pragma unroll
      for (int i = 0; i < W / 4; ++i) dst[i] = src[i];
      row_s[cur].y = -1.f;
    }
    if (t == a.nb_max - 1) break;
    const const_u32 y = (const_u32)(row_ptr(cur));   // uniform: scalar loads
    const float ic = row_s[cur].x;
    unsigned best = 0u;   // distance bits + 1 of this thread's farthest candidate; 0: none
    int best_p = 0;
    for (int p = tid; p < P; p += kFpsThreads) {   // ascending: strict > keeps the lowest index
      const uint4* src = reinterpret_cast<const uint4*>(row_ptr(p));
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < W / 4; ++i) {
        const uint4 v = src[i];
        acc[0] = dot2(v.x, y[4 * i], acc[0]);
        acc[1] = dot2(v.y, y[4 * i + 1], acc[1]);
        acc[2] = dot2(v.z, y[4 * i + 2], acc[2]);
        acc[3] = dot2(v.w, y[4 * i + 3], acc[3]);
      }
      const float dt = (acc[0] + acc[1]) + (acc[2] + acc[3]);
      const float2 rs = row_s[p];
      float d = 1.0f - dt * rs.x * ic;
      d = fminf(fmaxf(d, 0.f), 2.f);
      if (rs.y >= 0.f) {   // still a candidate
        const float m = fminf(rs.y, d);   // the initial 2 is the largest distance
        row_s[p].y = m;
        const unsigned key = __float_as_uint(m) + 1u;
        if (key > best) {
          best = key;
          best_p = p;
        }
      }
    }
    // workgroup max of (distance, lowest pool index on ties)
    const unsigned wmax = wave_umax(best);
    const unsigned lowest = ~wave_umax(best == wmax ? ~static_cast<unsigned>(best_p) : 0u);
    if ((tid & 63) == 0) {
      best_v[t & 1][tid >> 6] = wmax;
      best_i[t & 1][tid >> 6] = static_cast<int>(lowest);
    }
    __syncthreads();
    unsigned bv = best_v[t & 1][0];
    int bi = best_i[t & 1][0];
    for (int w = 1; w < kWaves; ++w) {
      const unsigned ov = best_v[t & 1][w];
      const int oi = best_i[t & 1][w];
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    cur = __builtin_amdgcn_readfirstlane(bi);
  }
  if (tid == 0) a.n_out[layer][bh] = a.nb_max;
}

// Table 3's Initial+Recent baseline keeps the earliest queries instead: the live rows stay
// in place and the new queries fill the free slots in time order (all heads of a step, in
// head order, before the next step); once full the set never changes.  A plain copy of
// 16-byte chunks, one workgroup per unit.
template <int D>
__global__ __launch_bounds__(256) void initial_kernel(const FpsArgs a) {
  constexpr int kChunks = D / 8;
  const int u = blockIdx.x;
  const int per_layer = a.batch * a.n_kv_heads;
  const int layer = u / per_layer;
  const int bh = u - layer * per_layer;
  const int b = bh / a.n_kv_heads;
  const int h = bh - b * a.n_kv_heads;
  int c_in = a.n_in[layer][bh];
  c_in = c_in < 0 ? 0 : (c_in > a.nb_max ? a.nb_max : c_in);
  const int fresh = a.group * a.t_new;
  const int n = c_in + (fresh < a.nb_max - c_in ? fresh : a.nb_max - c_in);
  const uint16_t* bin = a.beacons_in[layer] + static_cast<size_t>(bh) * a.nb_max * D;
  uint16_t* out = a.beacons_out[layer] + static_cast<size_t>(bh) * a.nb_max * D;
  for (int e = threadIdx.x; e < n * kChunks; e += blockDim.x) {
    const int p = e / kChunks;
    const int cc = e - p * kChunks;
    const uint16_t* src;
    if (p < c_in) {
      src = bin + static_cast<size_t>(p) * D;
    } else {
      const int i = p - c_in;
      const int t = i / a.group;
      const int r = i - t * a.group;
      src = a.q_new[layer] +
            ((static_cast<size_t>(b) * a.n_q_heads + h * a.group + r) * a.q_len + (a.q_len - a.t_new + t)) * D;
    }
    *reinterpret_cast<uint4*>(out + static_cast<size_t>(p) * D + cc * 8) =
        *reinterpret_cast<const uint4*>(src + cc * 8);
  }
  if (threadIdx.x == 0) a.n_out[layer][bh] = n;
}

}  // namespace

hipError_t launch_initial(const FpsArgs& a, int n_layers, int head_dim, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>(n_layers) * a.batch * a.n_kv_heads;
  if (head_dim == 128)
    hipLaunchKernelGGL(initial_kernel<128>, dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(initial_kernel<64>, dim3(grid), dim3(256), 0, s, a);
  return note_hip_error(hipGetLastError(), "initial beacons: launch");
}

hipError_t launch_fps(const FpsArgs& a, int n_layers, int head_dim, int pool_max, hipStream_t s) {
  if (pool_max > kFpsThreads * kFpsPoolRowsPerThread) return hipErrorInvalidValue;   // rejected by the host beforehand
  const unsigned grid = static_cast<unsigned>(n_layers) * a.batch * a.n_kv_heads;
  if (pool_max > kFpsRegisterPool) {
    static PerDeviceOnce once;
    const hipError_t attr_err = once_per_device(once, [] {
      const int lds = kFpsThreads * kFpsPoolRowsPerThread * static_cast<int>(sizeof(float2));
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&fps_pool_kernel<128>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      if (e == hipSuccess)
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&fps_pool_kernel<64>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      return e;
    });
    if (attr_err != hipSuccess) return note_hip_error(attr_err, "fps: hipFuncSetAttribute");
    const size_t lds = static_cast<size_t>(pool_max) * sizeof(float2);
    if (head_dim == 128)
      hipLaunchKernelGGL(fps_pool_kernel<128>, dim3(grid), dim3(kFpsThreads), lds, s, a);
    else
      hipLaunchKernelGGL(fps_pool_kernel<64>, dim3(grid), dim3(kFpsThreads), lds, s, a);
    return note_hip_error(hipGetLastError(), "fps: launch pool kernel");
  }
  const int threads = pool_max < 64 ? 64 : (pool_max + 63) / 64 * 64;
  if (head_dim == 128)
    hipLaunchKernelGGL(fps_kernel<128>, dim3(grid), dim3(threads), 0, s, a);
  else
    hipLaunchKernelGGL(fps_kernel<64>, dim3(grid), dim3(threads), 0, s, a);
  return note_hip_error(hipGetLastError(), "fps: launch");
}

}  // namespace bkv
