// Top-K selection under the cache budget with the recent window always kept
// (BeaconKV page, Figure 5 (c)).
//
// One 1024-thread workgroup per unit.  Thread t holds positions t*EPT .. t*EPT+EPT-1 of
// the unit's scores (in registers, past 32 of them in LDS) as bit patterns (non-negative fp32 order like unsigned
// integers).  The k-th largest pattern T among the positions before the window is found
// by a most-significant-digit-first radix select: four passes over 8-bit digits, each an
// LDS histogram of the candidates that still match the digits chosen so far (built in 16
// lane-indexed copies and then folded, since the leading digits of probabilities pile up
// on a few bins), scanned by one wave.  Every score above T is kept and, of the scores equal to T, the lowest
// positions fill the remaining slots; one block-wide scan of (ties, kept) counts in
// position order gives every thread its tie rank and its output offset, so the kept
// positions come out in ascending order.
#include "bkv_internal.h"

namespace bkv {
namespace {

constexpr int kWaves = kSelectThreads / 64;
// Histogram copies indexed by lane: lanes of one wave whose digits agree (common for the
// leading digit of probabilities) add to different copies instead of queueing on one LDS
// address; the odd stride puts the copies of a bin in different banks.
constexpr int kCopies = 16;
constexpr int kCopyStride = 257;

// Exclusive prefix over the block (thread order) of a 64-bit value.  `buf` holds kWaves
// entries; one barrier.
__device__ inline unsigned long long block_exclusive_scan(unsigned long long x, unsigned long long* buf) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  unsigned long long incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned long long y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) buf[wave] = incl;
  __syncthreads();
  unsigned long long before = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) before += w < wave ? buf[w] : 0ull;
  return before + incl - x;
}

// Wave 0: given the 256-bin histogram and the number r >= 1 of elements still to take
// from the top, find the digit d with count(> d) < r <= count(>= d); store d and
// r - count(> d) in out[0], out[1].  Clears the histogram for the next pass.
__device__ inline void pick_digit(int* hist, int r, int* out) {
  const int lane = threadIdx.x & 63;
  const int4 h = *reinterpret_cast<const int4*>(hist + 4 * lane);   // bins 4l .. 4l+3
  const int tot = h.x + h.y + h.z + h.w;
  int suf = tot;   // inclusive suffix over lanes: bins >= 4l
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_down(suf, o);
    if (lane + o < 64) suf += y;
  }
  const int above = suf - tot;   // bins >= 4l + 4
  if (above < r && r <= suf) {
    int d, gt;
    if (above + h.w >= r) {
      d = 4 * lane + 3;
      gt = above;
    } else if (above + h.w + h.z >= r) {
      d = 4 * lane + 2;
      gt = above + h.w;
    } else if (above + h.w + h.z + h.y >= r) {
      d = 4 * lane + 1;
      gt = above + h.w + h.z;
    } else {
      d = 4 * lane;
      gt = above + h.w + h.z + h.y;
    }
    out[0] = d;
    out[1] = r - gt;
  }
  *reinterpret_cast<int4*>(hist + 4 * lane) = make_int4(0, 0, 0, 0);
}

// Scores a thread keeps in registers; past 32 (capacities above 32768) the rest sit in
// LDS, element i of thread t at word (i - 32) * kSelectThreads + t, so that the registers
// of 16 waves per CU stay within the register file without spilling.
template <int EPT>
struct Held {
  static constexpr int kReg = EPT > 32 ? 32 : EPT;
  static constexpr int kLds = EPT - kReg;
  uint32_t r[kReg];
  uint32_t* lds;
  __device__ uint32_t& at_lds(int i) const { return lds[(i - kReg) * kSelectThreads + threadIdx.x]; }
};

// Orders -0 as 0 (the other patterns of non-negative fp32 values order as unsigned ints).
__device__ inline uint32_t pattern(uint32_t u) { return u == 0x80000000u ? 0u : u; }

template <int EPT>
__global__ __launch_bounds__(kSelectThreads) void select_topk_kernel(const SelectArgs a) {
  __shared__ uint32_t held_lds[Held<EPT>::kLds > 0 ? Held<EPT>::kLds * kSelectThreads : 1];
  __shared__ __attribute__((aligned(16))) int hist[256];
  __shared__ int histc[kCopies * kCopyStride];
  __shared__ unsigned long long scan_buf[kWaves];
  __shared__ int pick[2];
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
  const int prefix = L - a.window;       // candidates: positions < prefix
  const int want = a.budget - a.window;  // slots filled from the candidates
  const float* sc = a.scores[layer] + static_cast<size_t>(bh) * a.capacity;
  const int j0 = tid * EPT;

  Held<EPT> x;
  x.lds = held_lds;
  constexpr int kReg = Held<EPT>::kReg;
  if (EPT % 4 == 0 && (reinterpret_cast<uintptr_t>(sc) & 15) == 0 && j0 + EPT <= prefix) {
#pragma unroll
    for (int i = 0; i < kReg; i += 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(sc + j0 + i);
      x.r[i] = pattern(v.x);
      x.r[i + 1] = pattern(v.y);
      x.r[i + 2] = pattern(v.z);
      x.r[i + 3] = pattern(v.w);
    }
#pragma unroll 2
    for (int i = kReg; i < EPT; i += 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(sc + j0 + i);
      x.at_lds(i) = pattern(v.x);
      x.at_lds(i + 1) = pattern(v.y);
      x.at_lds(i + 2) = pattern(v.z);
      x.at_lds(i + 3) = pattern(v.w);
    }
  } else {
    // Unconditional loads at clamped positions (prefix >= 1 here: L > budget >= window), so
    // that all of a thread's loads are in flight together; positions past the candidates
    // then read as 0.  A branch per element would wait for each load in turn, and the
    // thread at the candidates' end would hold up the whole workgroup at the next barrier.
#pragma unroll
    for (int i = 0; i < kReg; ++i) {
      const int j = j0 + i;
      const uint32_t v = __float_as_uint(sc[j < prefix ? j : prefix - 1]);
      x.r[i] = j < prefix ? pattern(v) : 0u;
    }
#pragma unroll 4
    for (int i = kReg; i < EPT; ++i) {
      const int j = j0 + i;
      const uint32_t v = __float_as_uint(sc[j < prefix ? j : prefix - 1]);
      x.at_lds(i) = j < prefix ? pattern(v) : 0u;
    }
  }

  // Radix select of the want-th largest pattern among the candidates.
  uint32_t T = 0;
  int need_eq = 0;   // ties at T to keep, lowest positions first
  if (want > 0) {
    if (tid < 64) *reinterpret_cast<int4*>(hist + 4 * tid) = make_int4(0, 0, 0, 0);
    for (int i = tid; i < kCopies * kCopyStride; i += kSelectThreads) histc[i] = 0;
    __syncthreads();
    int* my_copy = histc + (tid & (kCopies - 1)) * kCopyStride;
    uint32_t P = 0;
    int r = want;
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
#pragma unroll
      for (int i = 0; i < kReg; ++i) {
        const uint32_t xi = x.r[i];
        if (j0 + i < prefix && (pass == 0 || (xi >> (shift + 8)) == P)) atomicAdd(&my_copy[(xi >> shift) & 255u], 1);
      }
#pragma unroll 4
      for (int i = kReg; i < EPT; ++i) {
        const uint32_t xi = x.at_lds(i);
        if (j0 + i < prefix && (pass == 0 || (xi >> (shift + 8)) == P)) atomicAdd(&my_copy[(xi >> shift) & 255u], 1);
      }
      __syncthreads();
      if (tid < 256) {   // fold the copies (and clear them for the next pass)
        int sum = 0;
#pragma unroll
        for (int c = 0; c < kCopies; ++c) {
          sum += histc[c * kCopyStride + tid];
          histc[c * kCopyStride + tid] = 0;
        }
        hist[tid] = sum;
      }
      __syncthreads();
      if (tid < 64) pick_digit(hist, r, pick);
      __syncthreads();
      P = (P << 8) | static_cast<uint32_t>(pick[0]);
      r = pick[1];
    }
    T = P;
    need_eq = r;
  }

  // Per-thread counts in position order: ties at T, and positions kept outright
  // (candidates above T, and the window).
  int n_eq = 0, n_fixed = 0;
  auto count = [&](int j, uint32_t xi) {
    const bool cand = j < prefix;
    n_fixed += (cand ? want > 0 && xi > T : j < L) ? 1 : 0;
    n_eq += (cand && want > 0 && xi == T) ? 1 : 0;
  };
#pragma unroll
  for (int i = 0; i < kReg; ++i) count(j0 + i, x.r[i]);
#pragma unroll 4
  for (int i = kReg; i < EPT; ++i) count(j0 + i, x.at_lds(i));
  const unsigned long long before =
      block_exclusive_scan((static_cast<unsigned long long>(n_eq) << 32) | static_cast<unsigned>(n_fixed), scan_buf);
  const int eq_before = static_cast<int>(before >> 32);
  const int fixed_before = static_cast<int>(before & 0xffffffffu);
  int eq_seen = eq_before;
  int pos = fixed_before + (eq_before < need_eq ? eq_before : need_eq);
  auto write = [&](int j, uint32_t xi) {
    bool keep;
    if (j < prefix) {
      keep = want > 0 && xi > T;
      if (want > 0 && xi == T) {
        keep = eq_seen < need_eq;
        ++eq_seen;
      }
    } else {
      keep = j < L;
    }
    if (keep) {
      if (pos < a.budget) out[pos] = j;
      ++pos;
    }
  };
#pragma unroll
  for (int i = 0; i < kReg; ++i) write(j0 + i, x.r[i]);
#pragma unroll 4
  for (int i = kReg; i < EPT; ++i) write(j0 + i, x.at_lds(i));
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
