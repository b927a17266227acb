// Top-k selection of the lightning-indexer scores (page "DeepSeek V4 深度解析",
// section 2, CSA step 2: each query keeps its k most relevant entries, 1024
// for Pro and 512 for Flash; the FP4 paragraph: BF16 scores make this
// selection cheaper).
//
// Exact and deterministic.  Scores are mapped to order-preserving unsigned
// keys (-0 folded onto +0); a row keeps the min(k, n) largest keys, ties
// broken by the lower index, written in ascending index order.  One
// workgroup (8 or 16 waves: many rows or few) per query row:
//   1. threshold estimate: rows longer than half the LDS candidate capacity take
//      a sample of 4096 keys (evenly spread runs of 8 or 4 consecutive keys,
//      one 16-byte load each) and use its order statistic of rank
//      ~2k*4096/n (an exact radix select over the sample in LDS), so about
//      2k keys of the row lie at or above it;
//   2. one streaming pass over the row (waves on contiguous segments, four
//      16-byte loads in flight per lane) appends every key >= the estimate,
//      with its index, to the wave's LDS segment; positions come from wave
//      prefix sums, so the candidates stay in index order and no atomics are
//      used;
//   3. exact radix select of the k-th largest key among the candidates (LDS
//      histograms), then an ordered scan writes key > tau, or key == tau among
//      the first `need` ties, at position (#greater before) + min(#ties
//      before, need).
// When the estimate misses (fewer than k candidates, or a wave segment
// overflows), the row is redone exactly over global memory with the same
// radix select and ordered scan.
#include "select_core.h"

using namespace csa;

namespace {

constexpr int kCap = 4096;                   // LDS candidates per row
constexpr int kSample = 4096;
constexpr int kU = 4;                        // 16-byte vectors in flight per lane

template <bool BF16>
__device__ __forceinline__ uint32_t key_at(const void* row, int64_t j) {
  if constexpr (BF16) return order_bf16(static_cast<const uint16_t*>(row)[j]);
  else return order_f32(__float_as_uint(static_cast<const float*>(row)[j]));
}

template <int NT>
struct Shared {
  static constexpr int kThreads = NT;
  static constexpr int kWaves = NT / 64;
  static constexpr int kBudget = kCap / kWaves;       // per wave segment
  RadixLds<NT> rx;
  uint32_t wsum[kWaves];
  uint32_t overflow;
  uint32_t cnt[kWaves];
  uint32_t cand_key[kCap];
  int32_t cand_idx[kCap];
};

// Radix select of the rank-th largest key among `count` keys produced by
// get(i) (see radix_select_visit).
template <int KBITS, int NT, typename Get>
__device__ uint32_t radix_select(Shared<NT>& sh, int64_t count, uint32_t rank, Get get, uint32_t& remain) {
  return radix_select_visit<KBITS, NT>(
      sh.rx, rank,
      [&](auto&& f) {
        for (int64_t j = threadIdx.x; j < count; j += NT) f(get(j));
      },
      remain);
}

// Ordered emission over `count` keys in index order: writes the selected
// ones' indices idx_of(i) to out[0..k).
template <int NT, typename Get, typename Idx>
__device__ void emit_ordered(Shared<NT>& sh, int64_t count, uint32_t tau, uint32_t need_eq, int k,
                             Get get, Idx idx_of, int32_t* out) {
  constexpr int kThreads = NT, kWaves = NT / 64;
  constexpr int EPT = 8;
  const int tid = threadIdx.x;
  uint32_t base_gt = 0, base_eq = 0;
  for (int64_t c0 = 0; c0 < count; c0 += (int64_t)kThreads * EPT) {
    const int64_t j0 = c0 + (int64_t)tid * EPT;
    uint32_t keys[EPT];
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int64_t j = j0 + e;
      const bool valid = j < count;
      keys[e] = valid ? get(j) : 0u;
      gt += (valid && keys[e] > tau) ? 1u : 0u;
      eq += (valid && keys[e] == tau) ? 1u : 0u;
    }
    uint32_t total;
    const uint32_t ex = block_exclusive_scan<kWaves>((gt << 16) | eq, sh.wsum, total);
    uint32_t g_before = base_gt + (ex >> 16);
    uint32_t e_before = base_eq + (ex & 0xffffu);
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int64_t j = j0 + e;
      if (j >= count) break;
      if (keys[e] > tau) {
        const uint32_t pos = g_before + (e_before < need_eq ? e_before : need_eq);
        if (pos < (uint32_t)k) out[pos] = idx_of(j);
        ++g_before;
      } else if (keys[e] == tau) {
        if (e_before < need_eq && g_before + e_before < (uint32_t)k) out[g_before + e_before] = idx_of(j);
        ++e_before;
      }
    }
    base_gt += total >> 16;
    base_eq += total & 0xffffu;
  }
}

template <bool BF16, int NT>
__global__ __launch_bounds__(NT) void topk_kernel(const void* __restrict__ scores, int64_t ld,
                                                  BatchDev b, int m, int k,
                                                  int32_t* __restrict__ idx) {
  constexpr int kThreads = NT, kWaves = NT / 64, kBudget = Shared<NT>::kBudget;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Shared<NT>& sh = *reinterpret_cast<Shared<NT>*>(smem_raw);
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int EPV = 16 / ESZ;                // elements per 16-byte vector
  constexpr int KBITS = BF16 ? 16 : 32;

  const int64_t q = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const QueryMeta qm = query_meta(b, q, m);
  const int64_t n = qm.n_vis < ld ? qm.n_vis : ld;    // never past the row
  const char* row = static_cast<const char*>(scores) + q * ld * ESZ;
  int32_t* out = idx + q * (int64_t)k;

  if (n <= k) {
    for (int64_t j = tid; j < k; j += kThreads) out[j] = j < n ? (int32_t)j : -1;
    return;
  }

  // ---- 1. threshold estimate (short rows: every key is a candidate; a
  // wave's segment then holds at most ~n/16 + 8 keys, inside its budget)
  uint32_t tau_hat = 0;
  if (n > kCap / 2) {
    // kSample keys in runs of SR consecutive ones (one 16-byte load each when
    // aligned), the runs spread evenly over the row: far fewer cache lines
    // than single scattered keys
    constexpr int SR = 16 / ESZ;
    constexpr int NRUN = kSample / SR;
    for (int r0 = tid; r0 < NRUN; r0 += kThreads) {
      const int64_t j0 = (int64_t)r0 * (n - SR) / (NRUN - 1);   // run start, j0 + SR <= n
      uint32_t ks[SR];
      if (((reinterpret_cast<uintptr_t>(row) + j0 * ESZ) & 15u) == 0) {
        const uint4 v = *reinterpret_cast<const uint4*>(row + j0 * ESZ);
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < SR; ++e) {
          if constexpr (BF16) ks[e] = order_bf16((w4[e >> 1] >> (16 * (e & 1))) & 0xffffu);
          else ks[e] = order_f32(w4[e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < SR; ++e) ks[e] = key_at<BF16>(row, j0 + e);
      }
#pragma unroll
      for (int e = 0; e < SR; ++e) sh.cand_key[r0 * SR + e] = ks[e];
    }
    __syncthreads();
    int64_t r = (2 * (int64_t)k * kSample + n - 1) / n + 8;
    if (r > kSample) r = kSample;
    uint32_t rem;
    tau_hat = radix_select<KBITS>(sh, kSample, (uint32_t)r,
                                  [&](int64_t i) { return sh.cand_key[i]; }, rem);
  }
  if (tid == 0) sh.overflow = 0;
  __syncthreads();

  // ---- 2. stream the row, keep keys >= tau_hat in index order.  A wave owns
  // a contiguous run of 16-byte vectors; each lane keeps kU of them in flight
  // (vector v0 + 64u + lane), and one packed wave scan per round places the
  // candidates of all of them.
  const float tau_f = n > kCap / 2 ? key_value<BF16>(tau_hat) : -INFINITY;
  const int64_t off = (int64_t)((reinterpret_cast<uintptr_t>(row) & 15u) / ESZ);  // row elements before its first vector boundary
  const char* vbase = row - off * ESZ;
  const int64_t nvec = (off + n + EPV - 1) / EPV;
  const int64_t per_wave = (nvec + kWaves - 1) / kWaves;
  const int64_t v_lo = wave * per_wave;
  const int64_t v_hi = v_lo + per_wave < nvec ? v_lo + per_wave : nvec;
  const char* row_end = row + n * ESZ;
  uint32_t wcount = 0;
  bool wover = false;
  for (int64_t v0 = v_lo; v0 < v_hi; v0 += 64 * kU) {
    uint4 raw[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t v = v0 + 64 * u + lane;
      const char* vp = vbase + v * 16;
      raw[u] = make_uint4(0, 0, 0, 0);
      if (v < v_hi && vp >= row && vp + 16 <= row_end) raw[u] = *reinterpret_cast<const uint4*>(vp);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      // the row's partial first and last vectors read only their in-row elements
      const int64_t v = v0 + 64 * u + lane;
      const char* vp = vbase + v * 16;
      if (v < v_hi && !(vp >= row && vp + 16 <= row_end)) {
        uint32_t t4[4] = {0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const int64_t j = v * EPV + e - off;
          if (j >= 0 && j < n) {
            uint32_t bits;
            if constexpr (BF16) bits = reinterpret_cast<const uint16_t*>(row)[j];
            else bits = __float_as_uint(reinterpret_cast<const float*>(row)[j]);
            t4[e * ESZ / 4] |= bits << (8 * ((e * ESZ) & 3));
          }
        }
        raw[u] = make_uint4(t4[0], t4[1], t4[2], t4[3]);
      }
    }
    uint32_t flags[kU], cnt01 = 0, cnt23 = 0;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t v = v0 + 64 * u + lane;
      const uint32_t w4[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
      uint32_t f = 0;
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const int64_t j = v * EPV + e - off;
        float x;
        if constexpr (BF16) x = __uint_as_float((w4[e >> 1] << (16 * (1 - (e & 1)))) & 0xffff0000u);
        else x = __uint_as_float(w4[e]);
        f |= (v < v_hi && j >= 0 && j < n && x >= tau_f) ? (1u << e) : 0u;
      }
      flags[u] = f;
      const uint32_t c = __builtin_popcount(f);
      if (u < 2) cnt01 |= c << (16 * u);
      else cnt23 |= c << (16 * (u - 2));
    }
    uint32_t tot01, tot23;
    const uint32_t ex01 = wave_exclusive_scan(cnt01, tot01);
    const uint32_t ex23 = wave_exclusive_scan(cnt23, tot23);
    const uint32_t tot[kU] = {tot01 & 0xffffu, tot01 >> 16, tot23 & 0xffffu, tot23 >> 16};
    const uint32_t ex[kU] = {ex01 & 0xffffu, ex01 >> 16, ex23 & 0xffffu, ex23 >> 16};
    const uint32_t round = tot[0] + tot[1] + tot[2] + tot[3];
    if (!wover && wcount + round <= (uint32_t)kBudget) {
      uint32_t before = wcount;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t v = v0 + 64 * u + lane;
        const uint32_t w4[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
        uint32_t slot = wave * kBudget + before + ex[u];
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          if (flags[u] & (1u << e)) {
            uint32_t key;
            if constexpr (BF16) key = order_bf16((w4[e >> 1] >> (16 * (e & 1))) & 0xffffu);
            else key = order_f32(w4[e]);
            sh.cand_key[slot] = key;
            sh.cand_idx[slot] = (int32_t)(v * EPV + e - off);
            ++slot;
          }
        }
        before += tot[u];
      }
    } else {
      wover = true;
    }
    wcount += round;
  }
  if (lane == 0) {
    sh.cnt[wave] = wover ? 0 : wcount;
    if (wover) sh.overflow = 1;
  }
  __syncthreads();
  uint32_t ccount = 0;
  for (int w = 0; w < kWaves; ++w) ccount += sh.cnt[w];

  if (!sh.overflow && ccount >= (uint32_t)k) {
    // ---- 3. exact selection among the candidates (segments in wave order)
    uint32_t segoff[kWaves + 1];
    segoff[0] = 0;
    for (int w = 0; w < kWaves; ++w) segoff[w + 1] = segoff[w] + sh.cnt[w];
    auto slot_of = [&](int64_t i) {
      int w = 0;
#pragma unroll
      for (int s = 1; s < kWaves; ++s) w += (uint32_t)i >= segoff[s] ? 1 : 0;
      return w * kBudget + (int)((uint32_t)i - segoff[w]);
    };
    uint32_t need;
    const uint32_t tau = radix_select<KBITS>(sh, ccount, (uint32_t)k,
                                             [&](int64_t i) { return sh.cand_key[slot_of(i)]; }, need);
    emit_ordered(sh, ccount, tau, need, k, [&](int64_t i) { return sh.cand_key[slot_of(i)]; },
                 [&](int64_t i) { return sh.cand_idx[slot_of(i)]; }, out);
  } else {
    // ---- exact fallback over global memory
    uint32_t need;
    const uint32_t tau = radix_select<KBITS>(sh, n, (uint32_t)k,
                                             [&](int64_t j) { return key_at<BF16>(row, j); }, need);
    emit_ordered(sh, n, tau, need, k, [&](int64_t j) { return key_at<BF16>(row, j); },
                 [&](int64_t j) { return (int32_t)j; }, out);
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
  if (ld > ((int64_t)1 << 31)) return fail(CSA_ERR_UNSUPPORTED, "csa_topk_select: rows above 2^31 scores");
  // there is no entry tensor here: the kernel clamps each row's candidates to ld
  const BatchDev b{batch->n_req, batch->q_off, batch->q_pos, batch->kv_off, nullptr, nullptr,
                   (int64_t)1 << 62, 0};
  // few rows (decode): 16 waves per row; many rows: 8, so several rows share a CU
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  const bool wide = batch->n_q < 2 * (int64_t)cus;
  const dim3 grid((unsigned)batch->n_q);
  if (score_fmt == CSA_BF16 && wide)
    hipLaunchKernelGGL((topk_kernel<true, 1024>), grid, dim3(1024), sizeof(Shared<1024>), stream, scores, ld, b, m, k, idx);
  else if (score_fmt == CSA_BF16)
    hipLaunchKernelGGL((topk_kernel<true, 512>), grid, dim3(512), sizeof(Shared<512>), stream, scores, ld, b, m, k, idx);
  else if (wide)
    hipLaunchKernelGGL((topk_kernel<false, 1024>), grid, dim3(1024), sizeof(Shared<1024>), stream, scores, ld, b, m, k, idx);
  else
    hipLaunchKernelGGL((topk_kernel<false, 512>), grid, dim3(512), sizeof(Shared<512>), stream, scores, ld, b, m, k, idx);
  return check_launch("csa_topk_select");
}
