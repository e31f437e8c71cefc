// Top-K selection under the cache budget with the recent window always kept
// (BeaconKV page, Figure 5 (c)).
//
// One 1024-thread workgroup per unit.  The unit's scores (non-negative fp32, so their
// bit patterns order like unsigned integers) sit in registers, element j in thread
// j % 1024, slot j / 1024.  The k-th largest bit pattern T is found by a 32-step
// bisection on the bits from the top (each step one block-wide count); every score
// above T is kept and, of the scores equal to T, the lowest positions fill the rest.
// Kept positions are written in ascending order by a ballot/prefix scan over the slots.
#include "bkv_internal.h"

namespace bkv {
namespace {

constexpr int kWaves = kSelectThreads / 64;

// Block-wide sum of one int per thread.  `buf` holds kWaves ints; the caller alternates
// two buffers between consecutive calls so a single barrier per call suffices.
__device__ inline int block_sum(int x, int* buf) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) buf[wave] = x;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) s += buf[w];
  return s;
}

// Exclusive prefix of `flag` over the block in thread order, plus the block total.
__device__ inline int block_prefix(bool flag, int* buf, int& total) {
  const unsigned long long m = __ballot(flag);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int in_wave = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) buf[wave] = __popcll(m);
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int c = buf[w];
    before += w < wave ? c : 0;
    tot += c;
  }
  total = tot;
  return before + in_wave;
}

template <int EPT>
__global__ __launch_bounds__(kSelectThreads) void select_topk_kernel(const SelectArgs a) {
  __shared__ int red[4][kWaves];
  const int u = blockIdx.x;
  const int per_layer = a.batch * a.n_kv_heads;
  const int layer = u / per_layer;
  const int bh = u - layer * per_layer;
  const int b = bh / a.n_kv_heads;
  int L = a.seq_len[b];
  L = L < 0 ? 0 : (L > a.capacity ? a.capacity : L);
  int32_t* out = a.idx[layer] + static_cast<size_t>(bh) * a.budget;
  const int tid = threadIdx.x;

  if (L <= a.budget) {
    for (int r = tid; r < L; r += kSelectThreads) out[r] = r;
    if (tid == 0) a.n_kept[layer][bh] = L;
    return;
  }
  const int prefix = L - a.window;
  const int want = a.budget - a.window;  // slots filled from positions < prefix
  const float* sc = a.scores[layer] + static_cast<size_t>(bh) * a.capacity;

  uint32_t x[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int j = tid + i * kSelectThreads;
    x[i] = j < prefix ? __float_as_uint(sc[j]) : 0u;
  }

  // Largest T with count(x >= T) >= want, over positions < prefix.  Positions >= prefix
  // hold 0 and are excluded from the count explicitly.
  uint32_t T = 0;
  int buf = 0;
  if (want > 0) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = T | (1u << bit);
      int c = 0;
#pragma unroll
      for (int i = 0; i < EPT; ++i) c += (tid + i * kSelectThreads < prefix && x[i] >= cand) ? 1 : 0;
      if (block_sum(c, red[buf]) >= want) T = cand;
      buf ^= 1;
    }
  }
  // Count the strictly larger ones and the ties at T.
  int gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const bool v = tid + i * kSelectThreads < prefix;
    gt += (v && x[i] > T) ? 1 : 0;
    eq += (v && x[i] == T) ? 1 : 0;
  }
  const int n_gt = block_sum(gt, red[buf]);
  buf ^= 1;
  const int n_eq = block_sum(eq, red[buf]);
  buf ^= 1;
  const int need_eq = want > 0 ? want - n_gt : 0;   // ties at T to keep, lowest positions first
  const bool all_eq = need_eq >= n_eq;

  int eq_base = 0, sel_base = 0;
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int j = tid + i * kSelectThreads;
    if (i * kSelectThreads >= L) break;   // uniform across the block
    const bool v = j < prefix;
    const bool is_eq = want > 0 && v && x[i] == T;
    bool keep = (want > 0 && v && x[i] > T) || (j >= prefix && j < L);
    if (all_eq) {
      keep = keep || is_eq;
    } else {
      int tot;
      const int rank = eq_base + block_prefix(is_eq, red[buf], tot);
      buf ^= 1;
      eq_base += tot;
      keep = keep || (is_eq && rank < need_eq);
    }
    int tot;
    const int pos = sel_base + block_prefix(keep, red[buf], tot);
    buf ^= 1;
    sel_base += tot;
    if (keep && pos < a.budget) out[pos] = j;
  }
  if (tid == 0) a.n_kept[layer][bh] = a.budget;
}

}  // namespace

hipError_t launch_select(const SelectArgs& a, int n_layers, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>(n_layers) * a.batch * a.n_kv_heads;
  const int ept = (a.capacity + kSelectThreads - 1) / kSelectThreads;
#define BKV_SELECT_CASE(E)                                                                        \
  if (ept <= E) {                                                                                 \
    hipLaunchKernelGGL(select_topk_kernel<E>, dim3(grid), dim3(kSelectThreads), 0, s, a);      \
    return note_hip_error(hipGetLastError(), "select: launch");                                                                     \
  }
  BKV_SELECT_CASE(1)
  BKV_SELECT_CASE(2)
  BKV_SELECT_CASE(4)
  BKV_SELECT_CASE(8)
  BKV_SELECT_CASE(16)
  BKV_SELECT_CASE(32)
  BKV_SELECT_CASE(64)
#undef BKV_SELECT_CASE
  return hipErrorInvalidValue;  // capacity above 65536: rejected by the host beforehand
}

}  // namespace bkv
