// One decoding step of attention over a (compacted) cache: for every sequence and query
// head, out = softmax(q . K^T / sqrt(d)) V over the sequence's valid rows.  This is what
// the compressed cache is for (BeaconKV page, Abstract and Table 4: decoding reads the
// kept KV pairs only, which is where its throughput gain comes from).
//
// Memory-bound (each K and V row is read once per step for the G query heads sharing
// it), so the kernel is built around the loads rather than the matrix units:
//   decode_partial  one workgroup per (layer, sequence, KV head, chunk of 1024 keys, or 512
//                   or 256 where 1024 would leave the launch too few workgroups to fill the
//                   chip); each wave takes a quarter of the chunk in blocks of 64 keys.
//                   Logits: lane = key, the key
//                   row in registers, the G query rows read through scalar loads as SGPR
//                   operands of v_dot2_f32_bf16.  Values: lanes 16 k + j read row k's dims
//                   8 j .. 8 j + 7, so every load instruction reads whole 256-byte rows; the
//                   weights come from LDS.  Per query a running max and sum (log2 domain)
//                   keep the chunk's partial output exact; the four waves merge in LDS.
//   decode_merge    per (sequence, query head): the chunks' partials combined and
//                   normalised.
#include "bkv_internal.h"

namespace bkv {
namespace {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef const __attribute__((address_space(4))) uint32_t* const_u32;

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr float kNegInf = -__builtin_inff();
constexpr int kValueUnroll = 4;   // value-row loads in flight per wave

__device__ inline float dot2(uint32_t x, uint32_t y, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), __builtin_bit_cast(bf16x2, y), acc, false);
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ inline float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ inline float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

template <int D, int G, int NB>
__global__ __launch_bounds__(kThreads) void decode_partial(const DecodeArgs a) {
  constexpr int W = D / 2;                 // 32-bit words per row
  constexpr int kLanesPerRow = D / 8;      // 16-byte pieces per row in the value loads
  constexpr int kRowsPerLoad = 64 / kLanesPerRow;
  __shared__ float pbuf[kWaves][G][64];
  __shared__ float m_w[kWaves][G], z_w[kWaves][G];
  __shared__ float o_w[kWaves][G][D];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int u = blockIdx.x / a.chunks;
  const int chunk = blockIdx.x - u * a.chunks;
  const int per_layer = a.batch * a.n_kv_heads;
  const int layer = u / per_layer;
  const int bh = u - layer * per_layer;
  const int b = bh / a.n_kv_heads;
  const int h = bh - b * a.n_kv_heads;
  int L = a.seq_len[b];
  L = L < 0 ? 0 : (L > a.capacity ? a.capacity : L);
  const int key_begin = chunk * (kWaves * 64 * NB);
  if (key_begin >= L) return;   // the merge reads only the chunks below L
  const uint16_t* kp = a.k[layer] + static_cast<size_t>(bh) * a.capacity * D;
  const uint16_t* vp = a.v[layer] + static_cast<size_t>(bh) * a.capacity * D;
  const uint16_t* qp = a.q[layer] + (static_cast<size_t>(b) * a.n_q_heads + h * G) * D;

  float m[G], z[G], o[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kNegInf;
    z[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[g][e] = 0.f;
  }
  const int vrow = lane / kLanesPerRow;    // row of the value load within a group of rows
  const int vcol = (lane % kLanesPerRow) * 8;

  for (int blk = 0; blk < NB; ++blk) {
    const int k0 = key_begin + (wave * NB + blk) * 64;
    if (k0 >= L) break;   // uniform across the wave
    // logits of key k0 + lane for every query of the group
    const int key = k0 + lane < L ? k0 + lane : L - 1;
    uint32_t kr[W];
    const uint4* src = reinterpret_cast<const uint4*>(kp + static_cast<size_t>(key) * D);
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      const uint4 x = src[i];
      kr[4 * i] = x.x;
      kr[4 * i + 1] = x.y;
      kr[4 * i + 2] = x.z;
      kr[4 * i + 3] = x.w;
    }
    float t[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const const_u32 qg = (const_u32)(qp + static_cast<size_t>(g) * D);   // uniform: scalar loads
      float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
      for (int i = 0; i < W; i += 2) {
        acc0 = dot2(kr[i], qg[i], acc0);
        acc1 = dot2(kr[i + 1], qg[i + 1], acc1);
      }
      t[g] = k0 + lane < L ? (acc0 + acc1) * a.scale_log2 : kNegInf;
    }
    // running softmax per query; weights of this block to LDS
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mb = wave_max(t[g]);
      const float mn = fmaxf(m[g], mb);
      const float scale = m[g] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m[g] - mn);
      const float p = __builtin_amdgcn_exp2f(t[g] - mn);
      z[g] = z[g] * scale + wave_sum(p);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[g][e] *= scale;
      m[g] = mn;
      pbuf[wave][g][lane] = p;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    // weighted value rows: lanes read whole rows, rows vrow, vrow + kRowsPerLoad, ...
#pragma unroll kValueUnroll
    for (int r0 = 0; r0 < 64; r0 += kRowsPerLoad) {
      const int j = r0 + vrow;
      int vk = k0 + j;
      vk = vk < L ? vk : L - 1;   // weight 0 past L
      const uint4 x = *reinterpret_cast<const uint4*>(vp + static_cast<size_t>(vk) * D + vcol);
      const float v8[8] = {bf16_lo(x.x), bf16_hi(x.x), bf16_lo(x.y), bf16_hi(x.y),
                           bf16_lo(x.z), bf16_hi(x.z), bf16_lo(x.w), bf16_hi(x.w)};
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float p = pbuf[wave][g][j];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[g][e] = fmaf(p, v8[e], o[g][e]);
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");   // pbuf is rewritten by the next block
  }
  // the lanes holding the same dims (lane % kLanesPerRow) add their rows' contributions
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float s = o[g][e];
#pragma unroll
      for (int off = kLanesPerRow; off < 64; off <<= 1) s += __shfl_xor(s, off);
      o[g][e] = s;
    }
    if (lane < kLanesPerRow) {
#pragma unroll
      for (int e = 0; e < 8; ++e) o_w[wave][g][vcol + e] = o[g][e];
    }
    if (lane == 0) {
      m_w[wave][g] = m[g];
      z_w[wave][g] = z[g];
    }
  }
  __syncthreads();
  // merge the four waves; partial (max, sum, unnormalised output) of the chunk
  const size_t base = (static_cast<size_t>(u) * kDecodeMaxGroup) * a.chunks + chunk;
  for (int i = threadIdx.x; i < G * D; i += kThreads) {
    const int g = i / D;
    const int d = i - g * D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, m_w[w][g]);
    float O = 0.f, Z = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = m_w[w][g] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m_w[w][g] - M);
      O = fmaf(o_w[w][g][d], f, O);
      Z = fmaf(z_w[w][g], f, Z);
    }
    const size_t slot = base + static_cast<size_t>(g) * a.chunks;
    a.part_o[slot * D + d] = O;
    if (d == 0) {
      a.part_m[slot] = M;
      a.part_z[slot] = Z;
    }
  }
}

// Waves whose block loop never ran (all of their keys past L) keep m = -inf and z = 0 and
// add nothing to the merge.
template <int D>
__global__ __launch_bounds__(D) void decode_merge(const DecodeArgs a) {
  const int per_layer = a.batch * a.n_q_heads;
  const int layer = blockIdx.x / per_layer;
  const int bq = blockIdx.x - layer * per_layer;
  const int b = bq / a.n_q_heads;
  const int hq = bq - b * a.n_q_heads;
  const int h = hq / a.group;
  const int g = hq - h * a.group;
  int L = a.seq_len[b];
  L = L < 0 ? 0 : (L > a.capacity ? a.capacity : L);
  const int n = (L + a.chunk_keys - 1) / a.chunk_keys;
  const int u = (layer * a.batch + b) * a.n_kv_heads + h;
  const size_t base = (static_cast<size_t>(u) * kDecodeMaxGroup + g) * a.chunks;
  const int d = threadIdx.x;
  float M = kNegInf;
  for (int c = 0; c < n; ++c) M = fmaxf(M, a.part_m[base + c]);
  float O = 0.f, Z = 0.f;
  for (int c = 0; c < n; ++c) {
    const float mc = a.part_m[base + c];
    const float f = mc == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mc - M);
    O = fmaf(a.part_o[(base + c) * D + d], f, O);
    Z = fmaf(a.part_z[base + c], f, Z);
  }
  a.out[layer][(static_cast<size_t>(b) * a.n_q_heads + hq) * D + d] = Z > 0.f ? O / Z : 0.f;
}

template <int D, int G>
hipError_t launch_d(const DecodeArgs& a, unsigned grid1, unsigned grid2, hipStream_t s) {
  static_assert(kDecodeMaxChunk == kWaves * 64 * 4 && kDecodeMinChunk == kWaves * 64, "1, 2 or 4 blocks per wave");
  if (a.chunk_keys == kDecodeMaxChunk)
    hipLaunchKernelGGL((decode_partial<D, G, 4>), dim3(grid1), dim3(kThreads), 0, s, a);
  else if (a.chunk_keys == kDecodeMaxChunk / 2)
    hipLaunchKernelGGL((decode_partial<D, G, 2>), dim3(grid1), dim3(kThreads), 0, s, a);
  else if (a.chunk_keys == kDecodeMinChunk)
    hipLaunchKernelGGL((decode_partial<D, G, 1>), dim3(grid1), dim3(kThreads), 0, s, a);
  else
    return note_hip_error(hipErrorInvalidValue, "decode: chunk size");
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return note_hip_error(e, "decode: launch partial");
  hipLaunchKernelGGL(decode_merge<D>, dim3(grid2), dim3(D), 0, s, a);
  return note_hip_error(hipGetLastError(), "decode: launch merge");
}

template <int D>
hipError_t launch_g(const DecodeArgs& a, unsigned grid1, unsigned grid2, hipStream_t s) {
  static_assert(kDecodeMaxGroup == 8, "one instantiation per group size");
  switch (a.group) {
    case 1: return launch_d<D, 1>(a, grid1, grid2, s);
    case 2: return launch_d<D, 2>(a, grid1, grid2, s);
    case 3: return launch_d<D, 3>(a, grid1, grid2, s);
    case 4: return launch_d<D, 4>(a, grid1, grid2, s);
    case 5: return launch_d<D, 5>(a, grid1, grid2, s);
    case 6: return launch_d<D, 6>(a, grid1, grid2, s);
    case 7: return launch_d<D, 7>(a, grid1, grid2, s);
    case 8: return launch_d<D, 8>(a, grid1, grid2, s);
    default: return note_hip_error(hipErrorInvalidValue, "decode: group size");
  }
}

}  // namespace

// One partial kernel per (head_dim, group size, blocks per wave): the per-query registers
// (running max, sum and eight output dims) and LDS scale with the group, so small groups
// run more waves, and the chunk size follows the launch size.
hipError_t launch_decode(const DecodeArgs& a, int n_layers, int head_dim, hipStream_t s) {
  const unsigned grid1 = static_cast<unsigned>(n_layers) * a.batch * a.n_kv_heads * a.chunks;
  const unsigned grid2 = static_cast<unsigned>(n_layers) * a.batch * a.n_q_heads;
  return head_dim == 128 ? launch_g<128>(a, grid1, grid2, s) : launch_g<64>(a, grid1, grid2, s);
}

}  // namespace bkv
