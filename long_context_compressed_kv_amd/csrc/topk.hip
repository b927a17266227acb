// Top-k selection of the lightning-indexer scores (page "DeepSeek V4 深度解析",
// section 2, CSA step 2: each query keeps its k most relevant entries, 1024
// for Pro and 512 for Flash; the FP4 paragraph: BF16 scores make this
// selection cheaper).
//
// Exact and deterministic.  Scores are mapped to order-preserving unsigned
// keys (-0 folded onto +0).  One workgroup per query row:
//   1. radix select, 8 bits per pass from the top (2 passes for BF16 keys,
//      4 for F32): per-wave LDS histograms of the digit among the keys that
//      match the prefix found so far -> the exact k-th largest key tau, the
//      number of keys above it, and how many tau-ties are still needed;
//   2. one ordered pass: key > tau, or key == tau among the first `need`
//      ties by index; output position = (#greater before) + min(#ties
//      before, need), from a block-wide exclusive scan, so the indices come
//      out in ascending order with no sort.
// Rows with at most k candidates skip 1. and keep everything.
#include "common.h"

using namespace csa;

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kEPT = 8;                      // consecutive elements per thread per chunk
constexpr int kChunk = kThreads * kEPT;

template <bool BF16>
__device__ __forceinline__ uint32_t order_key(const void* row, int64_t j) {
  if constexpr (BF16) {
    uint32_t b = static_cast<const uint16_t*>(row)[j];
    if (b == 0x8000u) b = 0;
    return (b & 0x8000u) ? (~b & 0xffffu) : (b | 0x8000u);
  } else {
    uint32_t b = __float_as_uint(static_cast<const float*>(row)[j]);
    if (b == 0x80000000u) b = 0;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  }
}

// Inclusive scan of one int over the block; returns the exclusive prefix and
// the block total.
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

template <bool BF16>
__global__ __launch_bounds__(kThreads) void topk_kernel(const void* __restrict__ scores, int64_t ld,
                                                        BatchDev b, int m, int k,
                                                        int32_t* __restrict__ idx) {
  __shared__ uint32_t hist[kWaves][256];
  __shared__ uint32_t merged[256];
  __shared__ uint32_t wsum[kWaves];
  __shared__ uint32_t sel_digit, sel_remain;

  const int64_t q = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const QueryMeta qm = query_meta(b, q, m);
  const int64_t n = qm.n_vis < ld ? qm.n_vis : ld;    // never past the row
  const void* row = BF16 ? (const void*)(static_cast<const uint16_t*>(scores) + q * ld)
                         : (const void*)(static_cast<const float*>(scores) + q * ld);
  int32_t* out = idx + q * (int64_t)k;

  if (n <= k) {
    for (int64_t j = tid; j < k; j += kThreads) out[j] = j < n ? (int32_t)j : -1;
    return;
  }

  // ---- 1. radix select of the k-th largest key
  constexpr int kBits = BF16 ? 16 : 32;
  uint32_t prefix = 0;
  uint32_t remain = (uint32_t)k;   // how many keys still to take among those matching prefix
  for (int shift = kBits - 8; shift >= 0; shift -= 8) {
    for (int i = tid; i < kWaves * 256; i += kThreads) (&hist[0][0])[i] = 0;
    __syncthreads();
    const uint32_t hi_mask = shift + 8 >= 32 ? 0u : (~0u << (shift + 8));
    for (int64_t j = tid; j < n; j += kThreads) {
      const uint32_t key = order_key<BF16>(row, j);
      if ((key & hi_mask) == prefix) atomicAdd(&hist[wave][(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 256) {
      uint32_t c = 0;
      for (int w = 0; w < kWaves; ++w) c += hist[w][tid];
      merged[tid] = c;
    }
    __syncthreads();
    if (tid < 64) {
      // suffix sums from the top digit down: lane l owns digits 4l..4l+3
      const int lane = tid;
      const uint32_t c0 = merged[4 * lane], c1 = merged[4 * lane + 1];
      const uint32_t c2 = merged[4 * lane + 2], c3 = merged[4 * lane + 3];
      const uint32_t s = c0 + c1 + c2 + c3;
      // exclusive count of all digits above this lane's group
      uint32_t x = s;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_down(x, o);
        if (lane + o < 64) x += y;
      }
      const uint32_t above = x - s;   // keys with a digit > 4l+3
      // the selected digit d satisfies above(d) < remain <= above(d) + count(d)
      uint32_t acc = above;
      const uint32_t cs[4] = {c3, c2, c1, c0};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (acc < remain && remain <= acc + cs[i]) {
          sel_digit = 4 * lane + 3 - i;
          sel_remain = remain - acc;
        }
        acc += cs[i];
      }
    }
    __syncthreads();
    prefix |= sel_digit << shift;
    remain = sel_remain;
    __syncthreads();
  }
  const uint32_t tau = prefix;
  const uint32_t need_eq = remain;     // ties at tau still to take

  // ---- 2. ordered emission
  uint32_t base_gt = 0, base_eq = 0;
  for (int64_t c0 = 0; c0 < n; c0 += kChunk) {
    const int64_t j0 = c0 + (int64_t)tid * kEPT;
    uint32_t keys[kEPT];
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < kEPT; ++e) {
      const int64_t j = j0 + e;
      keys[e] = j < n ? order_key<BF16>(row, j) : 0u;
      const bool valid = j < n;
      gt += (valid && keys[e] > tau) ? 1u : 0u;
      eq += (valid && keys[e] == tau) ? 1u : 0u;
    }
    uint32_t total;
    const uint32_t ex = block_exclusive_scan((gt << 16) | eq, wsum, total);
    uint32_t g_before = base_gt + (ex >> 16);
    uint32_t e_before = base_eq + (ex & 0xffffu);
#pragma unroll
    for (int e = 0; e < kEPT; ++e) {
      const int64_t j = j0 + e;
      if (j >= n) break;
      if (keys[e] > tau) {
        const uint32_t pos = g_before + (e_before < need_eq ? e_before : need_eq);
        if (pos < (uint32_t)k) out[pos] = (int32_t)j;
        ++g_before;
      } else if (keys[e] == tau) {
        if (e_before < need_eq && g_before + e_before < (uint32_t)k) out[g_before + e_before] = (int32_t)j;
        ++e_before;
      }
    }
    base_gt += total >> 16;
    base_eq += total & 0xffffu;
  }
}

}  // namespace

using namespace csa_host;

extern "C" csa_status csa_topk_select(const void* scores, int32_t score_fmt, int64_t ld,
                                      const csa_batch* batch, int32_t m, int32_t k, int32_t* idx,
                                      hipStream_t stream) {
  clear_error();
  if (batch == nullptr || batch->n_req < 1 || batch->n_q < 0 || batch->q_off == nullptr ||
      batch->q_pos == nullptr || batch->kv_off == nullptr)
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_topk_select: bad batch descriptor");
  if (score_fmt != CSA_F32 && score_fmt != CSA_BF16)
    return fail(CSA_ERR_UNSUPPORTED, "csa_topk_select: scores must be F32 or BF16");
  if (k < 1 || k > 4096) return fail(CSA_ERR_INVALID_ARGUMENT, "csa_topk_select: need 1 <= k <= 4096");
  if (m < 1) return fail(CSA_ERR_INVALID_ARGUMENT, "csa_topk_select: m must be >= 1");
  if (batch->max_kv < 0 || ld < batch->max_kv)
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_topk_select: need ld >= max_kv >= 0");
  if (batch->n_q == 0) return CSA_OK;
  if (idx == nullptr || (scores == nullptr && batch->max_kv > 0))
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_topk_select: null pointer");
  if (batch->n_q > 0x7fffffff) return fail(CSA_ERR_UNSUPPORTED, "csa_topk_select: too many rows");
  // there is no entry tensor here: the kernel clamps each row's candidates to ld
  const BatchDev b{batch->n_req, batch->q_off, batch->q_pos, batch->kv_off, nullptr, nullptr,
                   (int64_t)1 << 62, 0};
  if (score_fmt == CSA_BF16)
    hipLaunchKernelGGL(topk_kernel<true>, dim3((unsigned)batch->n_q), dim3(kThreads), 0, stream,
                       scores, ld, b, m, k, idx);
  else
    hipLaunchKernelGGL(topk_kernel<false>, dim3((unsigned)batch->n_q), dim3(kThreads), 0, stream,
                       scores, ld, b, m, k, idx);
  return check_launch("csa_topk_select");
}
