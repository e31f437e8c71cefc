// Beacon maintenance by continual farthest-point sampling on cosine distance
// (BeaconKV page, Figure 7 caption "Continual FPS"; Abstract: beacons represent the
// global query clusters without keeping the query history; Figure 4 (a): cosine
// similarity between queries).
//
// One 512-thread workgroup per unit.  The pool (live beacons, then the group's new
// queries head-major in time order) is held in registers: a row is spread over D/8
// lanes, 16 bytes (8 bf16) each, and group g of D/8 lanes owns rows g, g + G, g + 2G...
// (G = 512 / (D/8) groups).  Each pick broadcasts the chosen row through LDS, every
// group updates the distance of its rows to their nearest chosen row, and a block-wide
// argmax (largest distance, lowest pool index on ties) names the next pick.
#include "bkv_internal.h"

namespace bkv {
namespace {

constexpr int kWaves = kFpsThreads / 64;

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Dot product of 8 bf16 pairs with fp32 accumulation (v_dot2_f32_bf16 consumes the
// packed pairs directly, so rows stay packed in registers).
__device__ inline float dot8(const uint4& x, const uint4& y) {
  float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x.x), __builtin_bit_cast(bf16x2, y.x), 0.f, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x.y), __builtin_bit_cast(bf16x2, y.y), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x.z), __builtin_bit_cast(bf16x2, y.z), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x.w), __builtin_bit_cast(bf16x2, y.w), s, false);
  return s;
}

template <int LPR>
__device__ inline float group_sum(float v) {
#pragma unroll
  for (int o = LPR / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <int D, int RPG>
__global__ __launch_bounds__(kFpsThreads) void fps_kernel(const FpsArgs a) {
  constexpr int LPR = D / 8;
  constexpr int GROUPS = kFpsThreads / LPR;
  __shared__ uint4 pick_row[LPR];
  __shared__ float pick_inv;
  __shared__ float wbest_v[kWaves];
  __shared__ int wbest_i[kWaves];

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
    for (int e = tid; e < P * LPR; e += kFpsThreads) {
      const int p = e / LPR;
      const int cc = e - p * LPR;
      *reinterpret_cast<uint4*>(out + static_cast<size_t>(p) * D + cc * 8) =
          *reinterpret_cast<const uint4*>(row_ptr(p) + cc * 8);
    }
    if (tid == 0) a.n_out[layer][bh] = P;
    return;
  }

  const int g = tid / LPR;
  const int c = tid - g * LPR;
  uint4 xr[RPG];
  float inv[RPG];
  float mind[RPG];
  uint32_t taken = 0;  // bit k: row k*GROUPS+g already chosen (or absent)
#pragma unroll
  for (int k = 0; k < RPG; ++k) {
    const int p = k * GROUPS + g;
    xr[k] = p < P ? *reinterpret_cast<const uint4*>(row_ptr(p) + c * 8) : make_uint4(0, 0, 0, 0);
    const float ss = group_sum<LPR>(dot8(xr[k], xr[k]));
    inv[k] = 1.0f / fmaxf(sqrtf(ss), 1e-30f);
    mind[k] = 0.f;
    if (p >= P) taken |= 1u << k;
  }

  int cur = 0;
  for (int t = 0; t < a.nb_max; ++t) {
    if (g == cur % GROUPS) {
      const int k0 = cur / GROUPS;
#pragma unroll
      for (int k = 0; k < RPG; ++k)
        if (k == k0) {
          pick_row[c] = xr[k];
          *reinterpret_cast<uint4*>(out + static_cast<size_t>(t) * D + c * 8) = xr[k];
          if (c == 0) pick_inv = inv[k];
          taken |= 1u << k;
        }
    }
    __syncthreads();
    if (t == a.nb_max - 1) break;
    const uint4 y = pick_row[c];
    const float ip = pick_inv;
    float best_v = -1.f;
    int best_i = 0x7FFFFFFF;
#pragma unroll
    for (int k = 0; k < RPG; ++k) {
      const float dt = group_sum<LPR>(dot8(xr[k], y));
      float d = 1.0f - dt * inv[k] * ip;
      d = fminf(fmaxf(d, 0.f), 2.f);
      mind[k] = t == 0 ? d : fminf(mind[k], d);
      const float v = (taken >> k) & 1u ? -1.f : mind[k];
      if (v > best_v) {  // k ascending = pool index ascending: strict > keeps the lowest
        best_v = v;
        best_i = k * GROUPS + g;
      }
    }
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) {
      const float ov = __shfl_xor(best_v, o);
      const int oi = __shfl_xor(best_i, o);
      if (ov > best_v || (ov == best_v && oi < best_i)) {
        best_v = ov;
        best_i = oi;
      }
    }
    if ((tid & 63) == 0) {
      wbest_v[tid >> 6] = best_v;
      wbest_i[tid >> 6] = best_i;
    }
    __syncthreads();
    best_v = wbest_v[0];
    best_i = wbest_i[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      const float ov = wbest_v[w];
      const int oi = wbest_i[w];
      if (ov > best_v || (ov == best_v && oi < best_i)) {
        best_v = ov;
        best_i = oi;
      }
    }
    cur = best_i;
  }
  if (tid == 0) a.n_out[layer][bh] = a.nb_max;
}

}  // namespace

hipError_t launch_fps(const FpsArgs& a, int n_layers, int head_dim, int pool_max, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>(n_layers) * a.batch * a.n_kv_heads;
  const int groups = kFpsThreads / (head_dim / 8);
  const int rpg = (pool_max + groups - 1) / groups;
#define BKV_FPS_CASE(R)                                                                   \
  if (rpg <= R) {                                                                         \
    if (head_dim == 128)                                                                  \
      hipLaunchKernelGGL((fps_kernel<128, R>), dim3(grid), dim3(kFpsThreads), 0, s, a);  \
    else                                                                                  \
      hipLaunchKernelGGL((fps_kernel<64, R>), dim3(grid), dim3(kFpsThreads), 0, s, a);   \
    return note_hip_error(hipGetLastError(), "fps: launch");                                                             \
  }
  BKV_FPS_CASE(1)
  BKV_FPS_CASE(2)
  BKV_FPS_CASE(4)
  BKV_FPS_CASE(8)
  BKV_FPS_CASE(12)
  BKV_FPS_CASE(16)
  BKV_FPS_CASE(20)
  BKV_FPS_CASE(24)
#undef BKV_FPS_CASE
  return hipErrorInvalidValue;  // pool above BKV_MAX_POOL: rejected by the host beforehand
}

}  // namespace bkv
