// CSA step 1 / HCA compression (page "DeepSeek V4 深度解析", section 2, CSA
// step 1): every m raw tokens -> one entry, weights softmax(z[p] + b[s]) over
// an overlapping window of w slots, entry = sum of weighted raw rows.
//
// One workgroup (256 threads) per entry.  Threads form G = 512/D groups of
// D/2 threads; group g accumulates slots g, g+G, ... for two dims per thread,
// and the groups are summed in a fixed order, so results are deterministic.
// Memory bound: each raw row is read by w/m entries, mostly from L2.
#include "common.h"
#include "kvrow.h"

using namespace csa;

namespace {

constexpr int kThreads = 256;
constexpr int kMaxW = 1024;

template <typename T>
__device__ __forceinline__ float2 load2(const T* p);
template <>
__device__ __forceinline__ float2 load2<float>(const float* p) {
  return *reinterpret_cast<const float2*>(p);
}
template <>
__device__ __forceinline__ float2 load2<uint16_t>(const uint16_t* p) {
  const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
  return make_float2(bf16_to_f32(u & 0xffffu), bf16_to_f32(u >> 16));
}

__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
  v = is_max ? wave_max(v) : wave_sum(v);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
  return r;
}

struct OutPtrs {
  void* data;
  uint8_t* scale;
  uint16_t* rope;
  // rows: entry e_local goes to row e_local, or with a block list (a paged
  // cache) entry j = entry_begin + e_local to row blocks[j / P] * P + j % P,
  // P = 2^shift; rows outside the cache (or a negative block) are not written
  const int32_t* blocks;
  int shift;
  int64_t rows;
  int64_t entry_begin;
};

__device__ __forceinline__ int64_t out_row(const OutPtrs& o, int64_t e_local) {
  if (o.blocks == nullptr) return e_local;
  const int64_t j = o.entry_begin + e_local;
  const int64_t blk = o.blocks[j >> o.shift];
  const int64_t row = (blk << o.shift) + (j & ((1ll << o.shift) - 1));
  return blk >= 0 && row < o.rows ? row : -1;
}

// Entry i from raw rows x (positions x_pos0 .. x_pos0 + x_rows - 1) into
// row `row` of `out` (not written if row < 0); the whole workgroup calls it.
template <typename TIn, int OUTF>
__device__ __forceinline__ void compress_entry(const TIn* __restrict__ x, const float* __restrict__ z,
                                               int64_t x_pos0, int64_t x_rows, const float* __restrict__ bias,
                                               int m, int w, int64_t i, int dim, const OutPtrs& out, int64_t row) {
  __shared__ float wgt[kMaxW];
  __shared__ float red[kThreads / 64];
  __shared__ float acc_lds[2 * kThreads];

  const int64_t p0 = (i + 1) * m - w;
  const int tid = threadIdx.x;

  // softmax weights over the valid slots
  float lmax = -INFINITY;
  for (int s = tid; s < w; s += kThreads) {
    const int64_t p = p0 + s;
    const int64_t r = p - x_pos0;
    float l = -INFINITY;
    if (p >= 0 && r >= 0 && r < x_rows) l = z[r] + bias[s];
    wgt[s] = l;
    lmax = fmaxf(lmax, l);
  }
  const float mx = block_reduce(lmax, red, true);
  float lsum = 0.0f;
  for (int s = tid; s < w; s += kThreads) {
    const float l = wgt[s];
    const float e = l == -INFINITY ? 0.0f : expf(l - mx);
    wgt[s] = e;
    lsum += e;
  }
  const float sum = block_reduce(lsum, red, false);
  const float inv = sum > 0.0f ? 1.0f / sum : 0.0f;
  for (int s = tid; s < w; s += kThreads) wgt[s] *= inv;
  __syncthreads();

  // weighted sum: group g takes slots g, g+G, ...; two dims per thread
  const int tpr = dim >> 1;            // threads per row
  const int groups = kThreads / tpr;
  const int g = tid / tpr;
  const int d = (tid - g * tpr) * 2;
  // (U slots' loads in flight before their sums; a slot of weight 0, whose
  // row may not exist, reads row 0 and is skipped by a select, so the sums
  // are those of the slots in order)
  constexpr int U = 8;
  float a0 = 0.0f, a1 = 0.0f;
  int s = g;
  if (sum > 0.0f) {                     // (then some slot has a row: x_rows >= 1)
    for (; s + (U - 1) * groups < w; s += U * groups) {
      float wsv[U];
      float2 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        wsv[u] = wgt[s + u * groups];
        const int64_t r = wsv[u] != 0.0f ? p0 + s + u * groups - x_pos0 : 0;
        v[u] = load2(x + r * dim + d);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        a0 = wsv[u] != 0.0f ? fmaf(wsv[u], v[u].x, a0) : a0;
        a1 = wsv[u] != 0.0f ? fmaf(wsv[u], v[u].y, a1) : a1;
      }
    }
  }
  for (; s < w; s += groups) {
    const float ws = wgt[s];
    if (ws != 0.0f) {
      const int64_t r = p0 + s - x_pos0;
      const float2 v = load2(x + r * dim + d);
      a0 = fmaf(ws, v.x, a0);
      a1 = fmaf(ws, v.y, a1);
    }
  }
  acc_lds[2 * tid] = a0;
  acc_lds[2 * tid + 1] = a1;
  __syncthreads();
  if (g == 0) {
    for (int gg = 1; gg < groups; ++gg) {
      a0 += acc_lds[2 * (gg * tpr + tid)];
      a1 += acc_lds[2 * (gg * tpr + tid) + 1];
    }
  }

  if (OUTF == CSA_F32) {
    if (g == 0 && row >= 0)
      *reinterpret_cast<float2*>(static_cast<float*>(out.data) + row * dim + d) =
          make_float2(a0, a1);
  } else if (OUTF == CSA_BF16) {
    if (g == 0 && row >= 0)
      *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(out.data) + row * dim + d) =
          pack_bf16x2(a0, a1);
  } else {  // CSA_FP8_MIXED, dim == 512, groups == 1
    __syncthreads();
    acc_lds[d] = a0;
    acc_lds[d + 1] = a1;
    __syncthreads();
    if (tid < 64 && row >= 0) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = acc_lds[8 * tid + k];
      encode_kv_mixed_row_wave(v, static_cast<uint8_t*>(out.data) + row * 448,
                               out.scale + row * 4, out.rope + row * 64);
    }
  }
}

template <typename TIn, int OUTF>
__global__ __launch_bounds__(kThreads) void kv_compress_kernel(
    const TIn* __restrict__ x, const float* __restrict__ z, int64_t x_pos0, int64_t x_rows,
    const float* __restrict__ bias, int m, int w, int64_t entry_begin, int dim, OutPtrs out) {
  const int64_t e_local = blockIdx.x;
  compress_entry<TIn, OUTF>(x, z, x_pos0, x_rows, bias, m, w, entry_begin + e_local, dim, out,
                            out_row(out, e_local));
}

// A batch of prefill chunks (csa_batch): request r's chunk covers positions
// q_pos[r] .. q_pos[r] + T_r - 1 (T_r = q_off[r+1] - q_off[r]) and completes
// entries floor(q_pos/m) .. floor((q_pos + T_r)/m) - 1, computed from r's raw
// rows (raw_off / raw_pos) into r's cache rows (kv_off, or its blocks).
// Workgroup g takes the g-th of those entries in request order; the ones past
// the last exit.
__device__ __forceinline__ int64_t chunk_entries(const BatchDev& b, int r, int m, int64_t& first) {
  const int64_t pos = max(b.q_pos[r], (int64_t)0), T = max(b.q_off[r + 1] - b.q_off[r], (int64_t)0);
  first = pos / m;
  return (pos + T) / m - first;
}

template <typename TIn, int OUTF>
__global__ __launch_bounds__(kThreads) void kv_compress_batch_kernel(
    const TIn* __restrict__ x, const float* __restrict__ z, const float* __restrict__ bias, int m, int w,
    int dim, BatchDev b, OutPtrs out) {
  __shared__ int64_t scan[kThreads / 64];
  __shared__ int found_req;
  __shared__ int64_t found_e;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t g = blockIdx.x;
  if (tid == 0) found_req = -1;
  int64_t base = 0;
  for (int r0 = 0; r0 < b.n_req; r0 += kThreads) {
    const int r = r0 + tid;
    int64_t first = 0;
    const int64_t c = r < b.n_req ? chunk_entries(b, r, m, first) : 0;
    // inclusive scan of c over the workgroup (wave scans, then the wave totals)
    int64_t v = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int64_t u = __shfl_up(v, d);
      if (lane >= d) v += u;
    }
    __syncthreads();
    if (lane == 63) scan[wv] = v;
    __syncthreads();
    int64_t before = 0, total = 0;
#pragma unroll
    for (int k = 0; k < kThreads / 64; ++k) {
      before += k < wv ? scan[k] : 0;
      total += scan[k];
    }
    const int64_t incl = base + before + v;
    if (r < b.n_req && g >= incl - c && g < incl) {
      found_req = r;
      found_e = first + (g - (incl - c));
    }
    base += total;
    __syncthreads();
    if (found_req >= 0 || base > g) break;
  }
  const int r = found_req;
  if (r < 0) return;                               // past the batch's last entry
  const int64_t i = found_e;
  // offsets clamped to the tensors, so every access stays in bounds
  const int64_t rw0 = min(max(b.raw_off[r], (int64_t)0), b.raw_rows);
  const int64_t rw1 = min(max(b.raw_off[r + 1], rw0), b.raw_rows);
  const int64_t kv0 = b.kv_off[r], kv1 = b.kv_off[r + 1];
  int64_t row = -1;
  if (i < kv1 - kv0) {                            // the request's cache has a row for it
    if (b.pages == nullptr) {
      row = kv0 >= 0 && kv0 + i < out.rows ? kv0 + i : -1;
    } else {
      const int64_t blk = b.pages[(int64_t)r * b.page_stride + (i >> b.page_shift)];
      const int64_t pr = (blk << b.page_shift) + (i & ((1ll << b.page_shift) - 1));
      row = blk >= 0 && pr < out.rows ? pr : -1;
    }
  }
  compress_entry<TIn, OUTF>(x + rw0 * dim, z + rw0, b.raw_pos[r], rw1 - rw0, bias, m, w, i, dim, out, row);
}

// The variant with a logit and a bias per channel: z [x_rows][dim], bias
// [w][dim], one softmax per channel.  Threads hold two channels of one entry
// (512/dim entries a workgroup) and run an online softmax over the entry's
// slots in order (running maximum, sum of exponentials and weighted sum,
// fp32), so every channel is reduced in a fixed order.
template <typename TIn, int OUTF>
__global__ __launch_bounds__(kThreads) void kv_compress_channel_kernel(
    const TIn* __restrict__ x, const float* __restrict__ z, int64_t x_pos0, int64_t x_rows,
    const float* __restrict__ bias, int m, int w, int64_t entry_begin, int64_t n_entries, int dim,
    OutPtrs out) {
  __shared__ float acc_lds[2 * kThreads];
  const int tid = threadIdx.x;
  const int tpr = dim >> 1;                 // threads per entry
  const int per_wg = kThreads / tpr;
  const int g = tid / tpr;
  const int d = (tid - g * tpr) * 2;
  const int64_t e_local = (int64_t)blockIdx.x * per_wg + g;
  const bool live = e_local < n_entries;
  const int64_t i = entry_begin + e_local;
  const int64_t p0 = (i + 1) * m - w;
  float mx0 = -INFINITY, mx1 = -INFINITY, l0 = 0.0f, l1 = 0.0f, a0 = 0.0f, a1 = 0.0f;
  for (int s = 0; live && s < w; ++s) {
    const int64_t p = p0 + s;
    const int64_t r = p - x_pos0;
    if (p < 0 || r < 0 || r >= x_rows) continue;
    const float2 zz = *reinterpret_cast<const float2*>(z + r * dim + d);
    const float2 bb = *reinterpret_cast<const float2*>(bias + (int64_t)s * dim + d);
    const float2 v = load2(x + r * dim + d);
    const float g0 = zz.x + bb.x, g1 = zz.y + bb.y;
    if (g0 > mx0) {
      const float sc = expf(mx0 - g0);      // 0 while the channel is empty
      l0 *= sc;
      a0 *= sc;
      mx0 = g0;
    }
    if (g1 > mx1) {
      const float sc = expf(mx1 - g1);
      l1 *= sc;
      a1 *= sc;
      mx1 = g1;
    }
    const float e0 = expf(g0 - mx0), e1 = expf(g1 - mx1);
    l0 += e0;
    l1 += e1;
    a0 = fmaf(e0, v.x, a0);
    a1 = fmaf(e1, v.y, a1);
  }
  a0 = l0 > 0.0f ? a0 / l0 : 0.0f;
  a1 = l1 > 0.0f ? a1 / l1 : 0.0f;
  const int64_t row = live ? out_row(out, e_local) : -1;
  if (OUTF == CSA_F32) {
    if (row >= 0)
      *reinterpret_cast<float2*>(static_cast<float*>(out.data) + row * dim + d) = make_float2(a0, a1);
  } else if (OUTF == CSA_BF16) {
    if (row >= 0)
      *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(out.data) + row * dim + d) = pack_bf16x2(a0, a1);
  } else {  // CSA_FP8_MIXED, dim == 512: one entry a workgroup
    acc_lds[d] = a0;
    acc_lds[d + 1] = a1;
    __syncthreads();
    if (row >= 0 && tid < 64) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = acc_lds[8 * tid + k];
      encode_kv_mixed_row_wave(v, static_cast<uint8_t*>(out.data) + row * 448,
                               out.scale + row * 4, out.rope + row * 64);
    }
  }
}

template <typename TIn>
void launch_channel(const csa_tensor* x, const float* z, int64_t x_pos0, const float* bias, int m,
                    int w, int64_t entry_begin, int64_t n, const csa_tensor* out, hipStream_t stream,
                    const int32_t* blocks = nullptr, int shift = 0) {
  OutPtrs o{out->data, static_cast<uint8_t*>(out->scale), static_cast<uint16_t*>(out->rope), blocks,
            shift, out->rows, entry_begin};
  const TIn* xp = static_cast<const TIn*>(x->data);
  const int per_wg = kThreads / (x->dim >> 1);
  dim3 grid((unsigned)((n + per_wg - 1) / per_wg)), block(kThreads);
  switch (out->fmt) {
    case CSA_F32:
      hipLaunchKernelGGL((kv_compress_channel_kernel<TIn, CSA_F32>), grid, block, 0, stream, xp, z,
                         x_pos0, x->rows, bias, m, w, entry_begin, n, x->dim, o);
      break;
    case CSA_BF16:
      hipLaunchKernelGGL((kv_compress_channel_kernel<TIn, CSA_BF16>), grid, block, 0, stream, xp, z,
                         x_pos0, x->rows, bias, m, w, entry_begin, n, x->dim, o);
      break;
    default:
      hipLaunchKernelGGL((kv_compress_channel_kernel<TIn, CSA_FP8_MIXED>), grid, block, 0, stream,
                         xp, z, x_pos0, x->rows, bias, m, w, entry_begin, n, x->dim, o);
  }
}

template <typename TIn>
void launch(const csa_tensor* x, const float* z, int64_t x_pos0, const float* bias, int m, int w,
            int64_t entry_begin, int64_t n, const csa_tensor* out, hipStream_t stream,
            const int32_t* blocks = nullptr, int shift = 0) {
  OutPtrs o{out->data, static_cast<uint8_t*>(out->scale), static_cast<uint16_t*>(out->rope), blocks,
            shift, out->rows, entry_begin};
  const TIn* xp = static_cast<const TIn*>(x->data);
  dim3 grid((unsigned)n), block(kThreads);
  switch (out->fmt) {
    case CSA_F32:
      hipLaunchKernelGGL((kv_compress_kernel<TIn, CSA_F32>), grid, block, 0, stream, xp, z,
                         x_pos0, x->rows, bias, m, w, entry_begin, x->dim, o);
      break;
    case CSA_BF16:
      hipLaunchKernelGGL((kv_compress_kernel<TIn, CSA_BF16>), grid, block, 0, stream, xp, z,
                         x_pos0, x->rows, bias, m, w, entry_begin, x->dim, o);
      break;
    default:
      hipLaunchKernelGGL((kv_compress_kernel<TIn, CSA_FP8_MIXED>), grid, block, 0, stream, xp, z,
                         x_pos0, x->rows, bias, m, w, entry_begin, x->dim, o);
  }
}

template <typename TIn>
void launch_batch(const csa_tensor* x, const float* z, const float* bias, int m, int w,
                  const BatchDev& b, int64_t grid_n, const csa_tensor* out, hipStream_t stream) {
  OutPtrs o{out->data, static_cast<uint8_t*>(out->scale), static_cast<uint16_t*>(out->rope), nullptr,
            0, out->rows, 0};
  const TIn* xp = static_cast<const TIn*>(x->data);
  dim3 grid((unsigned)grid_n), block(kThreads);
  switch (out->fmt) {
    case CSA_F32:
      hipLaunchKernelGGL((kv_compress_batch_kernel<TIn, CSA_F32>), grid, block, 0, stream, xp, z, bias, m, w,
                         x->dim, b, o);
      break;
    case CSA_BF16:
      hipLaunchKernelGGL((kv_compress_batch_kernel<TIn, CSA_BF16>), grid, block, 0, stream, xp, z, bias, m, w,
                         x->dim, b, o);
      break;
    default:
      hipLaunchKernelGGL((kv_compress_batch_kernel<TIn, CSA_FP8_MIXED>), grid, block, 0, stream, xp, z, bias,
                         m, w, x->dim, b, o);
  }
}

}  // namespace

using namespace csa_host;

namespace {

// Checks shared by both compression calls; CSA_OK with n_entries == 0 means
// there is nothing to launch.
csa_status check_compress(const char* who, const csa_tensor* x, const float* logits, int64_t x_pos0,
                          const float* slot_bias, int32_t m, int32_t w, int64_t entry_begin,
                          int64_t n_entries, const csa_tensor* out, bool paged = false) {
  if (!fmt_valid_tensor(x) || !fmt_valid_tensor(out))
    return fail(CSA_ERR_INVALID_ARGUMENT, "%s: bad tensor descriptor", who);
  if (x->fmt != CSA_F32 && x->fmt != CSA_BF16)
    return fail(CSA_ERR_UNSUPPORTED, "%s: raw rows must be F32 or BF16", who);
  if (out->fmt != CSA_F32 && out->fmt != CSA_BF16 && out->fmt != CSA_FP8_MIXED)
    return fail(CSA_ERR_UNSUPPORTED, "%s: output must be F32, BF16 or FP8_MIXED", who);
  const int d = x->dim;
  if (out->dim != d) return fail(CSA_ERR_INVALID_ARGUMENT, "%s: dim mismatch", who);
  if (d < 16 || d > 512 || (d & (d - 1)) != 0)
    return fail(CSA_ERR_UNSUPPORTED, "%s: dim must be a power of two in [16, 512]", who);
  if (m < 1 || w < m || w > kMaxW)
    return fail(CSA_ERR_INVALID_ARGUMENT, "%s: need 1 <= m <= w <= %d", who, kMaxW);
  if (n_entries < 0 || entry_begin < 0 || (!paged && n_entries > out->rows))
    return fail(CSA_ERR_INVALID_ARGUMENT, "%s: bad entry range / output rows", who);
  if (n_entries == 0) return CSA_OK;
  if (n_entries > 0x7fffffff)
    return fail(CSA_ERR_INVALID_ARGUMENT, "%s: too many entries for one launch", who);
  if (logits == nullptr || slot_bias == nullptr)
    return fail(CSA_ERR_INVALID_ARGUMENT, "%s: null logits or biases", who);
  // every valid slot of every requested entry must be inside the raw rows
  const int64_t first = (entry_begin + 1) * m - w;
  const int64_t lo = first < 0 ? 0 : first;
  const int64_t hi = (entry_begin + n_entries) * (int64_t)m - 1;
  if (lo < x_pos0 || hi >= x_pos0 + x->rows)
    return fail(CSA_ERR_INVALID_ARGUMENT, "%s: raw rows cover positions [%lld, %lld) but entries need [%lld, %lld]", who,
                (long long)x_pos0, (long long)(x_pos0 + x->rows), (long long)lo, (long long)hi);
  return CSA_OK;
}

}  // namespace

extern "C" csa_status csa_kv_compress(const csa_tensor* x, const float* logits, int64_t x_pos0,
                                      const float* slot_bias, int32_t m, int32_t w,
                                      int64_t entry_begin, int64_t n_entries,
                                      const csa_tensor* out, hipStream_t stream) {
  clear_error();
  const csa_status st = check_compress("csa_kv_compress", x, logits, x_pos0, slot_bias, m, w,
                                       entry_begin, n_entries, out);
  if (st != CSA_OK || n_entries == 0) return st;
  if (x->fmt == CSA_F32)
    launch<float>(x, logits, x_pos0, slot_bias, m, w, entry_begin, n_entries, out, stream);
  else
    launch<uint16_t>(x, logits, x_pos0, slot_bias, m, w, entry_begin, n_entries, out, stream);
  return check_launch("csa_kv_compress");
}

extern "C" csa_status csa_kv_compress_paged(const csa_tensor* x, const float* logits, int64_t x_pos0,
                                            const float* slot_bias, int32_t m, int32_t w,
                                            int64_t entry_begin, int64_t n_entries,
                                            const int32_t* blocks, int32_t block_rows,
                                            const csa_tensor* out, hipStream_t stream) {
  clear_error();
  const csa_status st = check_compress("csa_kv_compress_paged", x, logits, x_pos0, slot_bias, m, w,
                                       entry_begin, n_entries, out, true);
  if (st != CSA_OK) return st;
  if (block_rows < 1 || block_rows > (1 << 20) || (block_rows & (block_rows - 1)) != 0)
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_kv_compress_paged: block_rows must be a power of two in [1, 2^20]");
  if (n_entries == 0) return CSA_OK;
  if (blocks == nullptr) return fail(CSA_ERR_INVALID_ARGUMENT, "csa_kv_compress_paged: null blocks");
  const int shift = __builtin_ctz((unsigned)block_rows);
  if (x->fmt == CSA_F32)
    launch<float>(x, logits, x_pos0, slot_bias, m, w, entry_begin, n_entries, out, stream, blocks, shift);
  else
    launch<uint16_t>(x, logits, x_pos0, slot_bias, m, w, entry_begin, n_entries, out, stream, blocks, shift);
  return check_launch("csa_kv_compress_paged");
}

extern "C" csa_status csa_kv_compress_channel(const csa_tensor* x, const float* logits,
                                              int64_t x_pos0, const float* slot_bias, int32_t m,
                                              int32_t w, int64_t entry_begin, int64_t n_entries,
                                              const csa_tensor* out, hipStream_t stream) {
  clear_error();
  const csa_status st = check_compress("csa_kv_compress_channel", x, logits, x_pos0, slot_bias, m,
                                       w, entry_begin, n_entries, out);
  if (st != CSA_OK || n_entries == 0) return st;
  if (x->fmt == CSA_F32)
    launch_channel<float>(x, logits, x_pos0, slot_bias, m, w, entry_begin, n_entries, out, stream);
  else
    launch_channel<uint16_t>(x, logits, x_pos0, slot_bias, m, w, entry_begin, n_entries, out, stream);
  return check_launch("csa_kv_compress_channel");
}

extern "C" csa_status csa_kv_compress_batch(const csa_tensor* x, const float* logits, const float* slot_bias,
                                            int32_t m, int32_t w, const csa_batch* batch, const csa_tensor* out,
                                            hipStream_t stream) {
  clear_error();
  const char* who = "csa_kv_compress_batch";
  if (batch == nullptr) return fail(CSA_ERR_INVALID_ARGUMENT, "%s: null batch", who);
  // the per-tensor and (m, w) checks of the single-sequence call (no entry range)
  const csa_status st = check_compress(who, x, logits, 0, slot_bias, m, w, 0, 0, out, true);
  if (st != CSA_OK) return st;
  if (batch->n_req < 0 || batch->n_q < 0) return fail(CSA_ERR_INVALID_ARGUMENT, "%s: bad batch sizes", who);
  if (batch->n_req == 0 || batch->n_q == 0) return CSA_OK;
  if (logits == nullptr || slot_bias == nullptr)
    return fail(CSA_ERR_INVALID_ARGUMENT, "%s: null logits or biases", who);
  if (batch->q_off == nullptr || batch->q_pos == nullptr || batch->kv_off == nullptr ||
      batch->raw_off == nullptr || batch->raw_pos == nullptr)
    return fail(CSA_ERR_INVALID_ARGUMENT, "%s: the batch needs q_off, q_pos, kv_off, raw_off and raw_pos", who);
  if (batch->window_ring != 0)
    return fail(CSA_ERR_UNSUPPORTED, "%s: raw rows must be stored in position order (no window ring)", who);
  BatchDev b{batch->n_req, batch->q_off, batch->q_pos, batch->kv_off, batch->raw_off, batch->raw_pos,
             out->rows, x->rows, 0};
  const csa_status pst = batch_pages(batch, b, who);
  if (pst != CSA_OK) return pst;
  // every request completes at most floor(T_r / m) + 1 entries
  const int64_t grid_n = batch->n_q / m + batch->n_req;
  if (grid_n > 0x7fffffff) return fail(CSA_ERR_INVALID_ARGUMENT, "%s: too many entries for one launch", who);
  if (x->fmt == CSA_F32)
    launch_batch<float>(x, logits, slot_bias, m, w, b, grid_n, out, stream);
  else
    launch_batch<uint16_t>(x, logits, slot_bias, m, w, b, grid_n, out, stream);
  return check_launch(who);
}
