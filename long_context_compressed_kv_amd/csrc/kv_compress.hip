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
};

template <typename TIn, int OUTF>
__global__ __launch_bounds__(kThreads) void kv_compress_kernel(
    const TIn* __restrict__ x, const float* __restrict__ z, int64_t x_pos0, int64_t x_rows,
    const float* __restrict__ bias, int m, int w, int64_t entry_begin, int dim, OutPtrs out) {
  __shared__ float wgt[kMaxW];
  __shared__ float red[kThreads / 64];
  __shared__ float acc_lds[2 * kThreads];

  const int64_t e_local = blockIdx.x;
  const int64_t i = entry_begin + e_local;
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
  float a0 = 0.0f, a1 = 0.0f;
  for (int s = g; s < w; s += groups) {
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
    if (g == 0)
      *reinterpret_cast<float2*>(static_cast<float*>(out.data) + e_local * dim + d) =
          make_float2(a0, a1);
  } else if (OUTF == CSA_BF16) {
    if (g == 0)
      *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(out.data) + e_local * dim + d) =
          pack_bf16x2(a0, a1);
  } else {  // CSA_FP8_MIXED, dim == 512, groups == 1
    __syncthreads();
    acc_lds[d] = a0;
    acc_lds[d + 1] = a1;
    __syncthreads();
    if (tid < 64) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = acc_lds[8 * tid + k];
      encode_kv_mixed_row_wave(v, static_cast<uint8_t*>(out.data) + e_local * 448,
                               out.scale + e_local * 4, out.rope + e_local * 64);
    }
  }
}

template <typename TIn>
void launch(const csa_tensor* x, const float* z, int64_t x_pos0, const float* bias, int m, int w,
            int64_t entry_begin, int64_t n, const csa_tensor* out, hipStream_t stream) {
  OutPtrs o{out->data, static_cast<uint8_t*>(out->scale), static_cast<uint16_t*>(out->rope)};
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

}  // namespace

using namespace csa_host;

extern "C" csa_status csa_kv_compress(const csa_tensor* x, const float* logits, int64_t x_pos0,
                                      const float* slot_bias, int32_t m, int32_t w,
                                      int64_t entry_begin, int64_t n_entries,
                                      const csa_tensor* out, hipStream_t stream) {
  clear_error();
  if (!fmt_valid_tensor(x) || !fmt_valid_tensor(out))
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_kv_compress: bad tensor descriptor");
  if (x->fmt != CSA_F32 && x->fmt != CSA_BF16)
    return fail(CSA_ERR_UNSUPPORTED, "csa_kv_compress: raw rows must be F32 or BF16");
  if (out->fmt != CSA_F32 && out->fmt != CSA_BF16 && out->fmt != CSA_FP8_MIXED)
    return fail(CSA_ERR_UNSUPPORTED, "csa_kv_compress: output must be F32, BF16 or FP8_MIXED");
  const int d = x->dim;
  if (out->dim != d) return fail(CSA_ERR_INVALID_ARGUMENT, "csa_kv_compress: dim mismatch");
  if (d < 16 || d > 512 || (d & (d - 1)) != 0)
    return fail(CSA_ERR_UNSUPPORTED, "csa_kv_compress: dim must be a power of two in [16, 512]");
  if (m < 1 || w < m || w > kMaxW)
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_kv_compress: need 1 <= m <= w <= %d", kMaxW);
  if (n_entries < 0 || entry_begin < 0 || n_entries > out->rows)
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_kv_compress: bad entry range / output rows");
  if (n_entries == 0) return CSA_OK;
  if (n_entries > 0x7fffffff)
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_kv_compress: too many entries for one launch");
  if (logits == nullptr || slot_bias == nullptr)
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_kv_compress: null logits or biases");
  // every valid slot of every requested entry must be inside the raw rows
  const int64_t first = (entry_begin + 1) * m - w;
  const int64_t lo = first < 0 ? 0 : first;
  const int64_t hi = (entry_begin + n_entries) * (int64_t)m - 1;
  if (lo < x_pos0 || hi >= x_pos0 + x->rows)
    return fail(CSA_ERR_INVALID_ARGUMENT,
                "csa_kv_compress: raw rows cover positions [%lld, %lld) but entries need [%lld, %lld]",
                (long long)x_pos0, (long long)(x_pos0 + x->rows), (long long)lo, (long long)hi);
  if (x->fmt == CSA_F32)
    launch<float>(x, logits, x_pos0, slot_bias, m, w, entry_begin, n_entries, out, stream);
  else
    launch<uint16_t>(x, logits, x_pos0, slot_bias, m, w, entry_begin, n_entries, out, stream);
  return check_launch("csa_kv_compress");
}
