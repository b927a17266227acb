// Exact top-k building blocks shared by the top-k kernels (page "DeepSeek V4
// 深度解析", section 2, CSA step 2: each query keeps its k highest-scoring
// entries): order-preserving integer keys for fp32 / bf16 scores, scans, and
// a radix select over keys that the caller feeds through a visitor.
#pragma once

#include "common.h"

namespace csa {

// Order-preserving keys: a larger score gives a larger key; -0 is folded
// onto +0 so that they tie, as the scores compare.
__device__ __forceinline__ uint32_t order_bf16(uint32_t b) {
  if (b == 0x8000u) b = 0;
  return (b & 0x8000u) ? (~b & 0xffffu) : (b | 0x8000u);
}
__device__ __forceinline__ uint32_t order_f32(uint32_t b) {
  if (b == 0x80000000u) b = 0;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Inverse of the order-preserving map, as a float.
template <bool BF16>
__device__ __forceinline__ float key_value(uint32_t key) {
  if constexpr (BF16) {
    const uint32_t b = (key & 0x8000u) ? (key & 0x7fffu) : (~key & 0xffffu);
    return __uint_as_float(b << 16);
  } else {
    const uint32_t b = (key & 0x80000000u) ? (key & 0x7fffffffu) : ~key;
    return __uint_as_float(b);
  }
}

// Exclusive scan of v over one wave; total returned through `total`.
__device__ __forceinline__ uint32_t wave_exclusive_scan(uint32_t v, uint32_t& total) {
  const int lane = threadIdx.x & 63;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  total = __shfl(x, 63);
  return x - v;
}

// Exclusive scan of v over the block (kWaves waves, wsum: kWaves words of
// LDS); total returned through `total`.
template <int kWaves>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wsum, uint32_t& total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  __syncthreads();
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  uint32_t before = 0, tot = 0;
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t s = wsum[w];
    before += w < wave ? s : 0;
    tot += s;
  }
  total = tot;
  return before + x - v;
}

// LDS of a radix select: one 256-bin histogram per wave and their sums.
template <int NT>
struct RadixLds {
  uint32_t hist[NT / 64][256];
  uint32_t tot[256];
};

// Radix select (8-bit digits, most significant first) of the rank-th largest
// of a multiset of KBITS-bit keys.  visit(f) calls f(key) once for each key
// this thread contributes; every thread of the block calls it (the keys of
// all threads together form the multiset).  Returns the key; `remain` = how
// many keys equal to it are needed to reach rank (rank - remain keys are
// strictly greater) and, if n_equal is given, *n_equal = how many keys equal
// it.  1 <= rank <= the multiset's size.
//
// Per digit: each wave clears and fills its own histogram; after one barrier
// the threads below 256 sum them into tot; after a second every wave finds
// the digit from tot by itself (the same in every wave).  A wave's histogram
// is only read between those two barriers, and tot only after the second and
// before the next digit's first, so no other barrier is needed, also across
// calls.
template <int KBITS, int NT, typename Visit>
__device__ uint32_t radix_select_visit(RadixLds<NT>& sh, uint32_t rank, Visit visit, uint32_t& remain,
                                       uint32_t* n_equal = nullptr) {
  // one wave (its histogram is the total), or at least one thread per digit
  // to sum the waves' histograms
  static_assert(NT == 64 || (NT >= 256 && NT % 64 == 0), "radix select: 64 or at least 256 threads");
  constexpr int kWaves = NT / 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  uint32_t prefix = 0;
  remain = rank;
  for (int shift = KBITS - 8; shift >= 0; shift -= 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sh.hist[wave][lane + 64 * i] = 0;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const uint32_t hi_mask = shift + 8 >= 32 ? 0u : (~0u << (shift + 8));
    visit([&](uint32_t key) {
      if ((key & hi_mask) == prefix) atomicAdd(&sh.hist[wave][(key >> shift) & 255u], 1u);
    });
    __syncthreads();
    if constexpr (kWaves > 1) {
      if (tid < 256) {          // per-digit totals of the per-wave histograms
        uint32_t s = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s += sh.hist[w][tid];
        sh.tot[tid] = s;
      }
      __syncthreads();
    }
    const uint32_t* tot = kWaves > 1 ? sh.tot : sh.hist[0];
    // lane l owns digits 4l..4l+3; suffix counts from the top digit down
    uint32_t c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = tot[4 * lane + i];
    const uint32_t s = c[0] + c[1] + c[2] + c[3];
    uint32_t x = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_down(x, o);
      if (lane + o < 64) x += y;
    }
    uint32_t acc = x - s, dig = 0, rem = 0;
    bool found = false;
#pragma unroll
    for (int i = 3; i >= 0; --i) {
      if (acc < remain && remain <= acc + c[i]) {
        dig = 4 * lane + i;
        rem = remain - acc;
        found = true;
      }
      acc += c[i];
    }
    const uint64_t m = __ballot(found);     // exactly one lane
    const int fl = __builtin_ctzll(m);
    const uint32_t digit = (uint32_t)__shfl((int)dig, fl);
    remain = (uint32_t)__shfl((int)rem, fl);
    prefix |= digit << shift;
    // after the last digit, its bin counts the keys equal to the result
    if (shift == 0 && n_equal != nullptr) *n_equal = tot[digit];
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();        // (one wave: its histogram is cleared next)
  }
  return prefix;
}

// The same select by one wave alone, over n keys it reads from src (LDS):
// 8-bit digits, most significant first, over a 256-bin histogram of its own
// (hist, 256 words of LDS); no barrier of the workgroup.  Returns the
// rank-th largest key, 1 <= rank <= n.
template <int KBITS, typename Key>
__device__ uint32_t wave_radix_select(const Key* src, int n, uint32_t rank, uint32_t* hist) {
  const int lane = threadIdx.x & 63;
  uint32_t prefix = 0, remain = rank;
  for (int shift = KBITS - 8; shift >= 0; shift -= 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) hist[lane + 64 * i] = 0;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const uint32_t hi_mask = shift + 8 >= 32 ? 0u : (~0u << (shift + 8));
    for (int i = lane; i < n; i += 64) {
      const uint32_t key = src[i];
      if ((key & hi_mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // lane l owns digits 4l..4l+3; suffix counts from the top digit down
    uint32_t c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = hist[4 * lane + i];
    const uint32_t s = c[0] + c[1] + c[2] + c[3];
    uint32_t x = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_down(x, o);
      if (lane + o < 64) x += y;
    }
    uint32_t acc = x - s, dig = 0, rem = 0;
    bool found = false;
#pragma unroll
    for (int i = 3; i >= 0; --i) {
      if (acc < remain && remain <= acc + c[i]) {
        dig = 4 * lane + i;
        rem = remain - acc;
        found = true;
      }
      acc += c[i];
    }
    const uint64_t m = __ballot(found);     // exactly one lane
    const int fl = __builtin_ctzll(m);
    prefix |= (uint32_t)__shfl((int)dig, fl) << shift;
    remain = (uint32_t)__shfl((int)rem, fl);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();        // (the histogram is cleared again next)
  }
  return prefix;
}

}  // namespace csa
