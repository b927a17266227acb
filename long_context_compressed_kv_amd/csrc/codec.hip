// Storage-format kernels: quantise to the mixed KV / MXFP4 / bf16 formats,
// exact dequantisation, and the lossless MXFP4 -> e4m3fn regrouping.
#include "common.h"
#include "kvrow.h"

using namespace csa;

namespace {

template <typename T>
__device__ __forceinline__ float load_val(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_val<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_val<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}

// One wave per 512-dim row.
template <typename T>
__global__ __launch_bounds__(256) void quantize_kv_mixed_kernel(const T* __restrict__ src,
                                                                int64_t rows, uint8_t* nope,
                                                                uint8_t* scale, uint16_t* rope) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = load_val(src, row * 512 + 8 * lane + i);
  encode_kv_mixed_row_wave(v, nope + row * 448, scale + row * 4, rope + row * 64);
}

// One thread per MX block.
template <typename T>
__global__ __launch_bounds__(256) void quantize_mxfp4_kernel(const T* __restrict__ src,
                                                             int64_t rows, int dim,
                                                             uint8_t* codes, uint8_t* scale) {
  const int nb = dim / 32;
  const int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (blk >= rows * nb) return;
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = load_val(src, blk * 32 + i);
  encode_mxfp4_block(v, codes + blk * 16, scale + blk);
}

__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float* __restrict__ src,
                                                          int64_t n, uint16_t* dst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = (uint16_t)f32_to_bf16(src[i]);
}

// One thread per element.
__global__ __launch_bounds__(256) void dequantize_kernel(csa_tensor t, float* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= t.rows * t.dim) return;
  const int64_t r = i / t.dim;
  const int c = (int)(i % t.dim);
  float v;
  switch (t.fmt) {
    case CSA_F32:
      v = static_cast<const float*>(t.data)[i];
      break;
    case CSA_BF16:
      v = bf16_to_f32(static_cast<const uint16_t*>(t.data)[i]);
      break;
    case CSA_FP8_MIXED:
      if (c < 448) {
        const uint8_t code = static_cast<const uint8_t*>(t.data)[r * 448 + c];
        const uint8_t sc = static_cast<const uint8_t*>(t.scale)[r * 4 + c / 128];
        v = e4m3_to_f32(code) * e8m0_to_f32(sc);
      } else {
        v = bf16_to_f32(static_cast<const uint16_t*>(t.rope)[r * 64 + (c - 448)]);
      }
      break;
    default: {  // CSA_MXFP4
      const uint8_t byte = static_cast<const uint8_t*>(t.data)[r * (t.dim / 2) + c / 2];
      const uint8_t sc = static_cast<const uint8_t*>(t.scale)[r * (t.dim / 32) + c / 32];
      v = e2m1_to_f32((c & 1) ? (byte >> 4) : (byte & 15)) * e8m0_to_f32(sc);
    }
  }
  dst[i] = v;
}

// One thread per row: group exponent g = max block exponent - 6, elements
// re-encoded as e4m3fn of c * 2^(e_b - g).
__global__ __launch_bounds__(256) void mxfp4_to_fp8_kernel(csa_tensor t, uint8_t* __restrict__ fp8,
                                                           uint8_t* __restrict__ gscale,
                                                           uint8_t* __restrict__ lossless) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= t.rows) return;
  const int nb = t.dim / 32;
  const uint8_t* sc = static_cast<const uint8_t*>(t.scale) + r * nb;
  const uint8_t* cd = static_cast<const uint8_t*>(t.data) + r * (t.dim / 2);
  int emax = -1000, emin = 1000;
  for (int b = 0; b < nb; ++b) {
    const int e = (int)sc[b] - 127;
    emax = e > emax ? e : emax;
    emin = e < emin ? e : emin;
  }
  const int g = emax - 6;
  for (int b = 0; b < nb; ++b) {
    // k <= 6; below -20 every e2m1 value times 2^k rounds to a signed zero
    int k = (int)sc[b] - 127 - g;
    if (k < -20) k = -20;
    const float mul = exp2i(k);
    for (int i = 0; i < 32; ++i) {
      const uint8_t byte = cd[b * 16 + i / 2];
      const uint32_t c = (i & 1) ? (byte >> 4) : (byte & 15);
      fp8[r * t.dim + b * 32 + i] = (uint8_t)f32_to_e4m3(e2m1_to_f32(c) * mul);
    }
  }
  const int gb = g + 127;
  gscale[r] = (uint8_t)(gb < 0 ? 0 : (gb > 254 ? 254 : gb));
  lossless[r] = (emax - emin) <= 14 ? 1 : 0;
}

inline unsigned grid_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

using namespace csa_host;

extern "C" {

csa_status csa_quantize(const csa_tensor* src, const csa_tensor* dst, hipStream_t stream) {
  clear_error();
  if (!fmt_valid_tensor(src) || !fmt_valid_tensor(dst))
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_quantize: bad tensor descriptor");
  if (src->fmt != CSA_F32 && src->fmt != CSA_BF16)
    return fail(CSA_ERR_UNSUPPORTED, "csa_quantize: source must be F32 or BF16");
  if (src->rows != dst->rows || src->dim != dst->dim)
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_quantize: shape mismatch");
  const int64_t rows = src->rows;
  if (rows == 0) return CSA_OK;
  if (rows > (int64_t)1 << 40)
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_quantize: too many rows");
  switch (dst->fmt) {
    case CSA_FP8_MIXED:
      if (src->fmt == CSA_F32)
        hipLaunchKernelGGL(quantize_kv_mixed_kernel<float>, dim3(grid_for(rows, 4)), dim3(256), 0,
                           stream, (const float*)src->data, rows, (uint8_t*)dst->data,
                           (uint8_t*)dst->scale, (uint16_t*)dst->rope);
      else
        hipLaunchKernelGGL(quantize_kv_mixed_kernel<uint16_t>, dim3(grid_for(rows, 4)), dim3(256),
                           0, stream, (const uint16_t*)src->data, rows, (uint8_t*)dst->data,
                           (uint8_t*)dst->scale, (uint16_t*)dst->rope);
      break;
    case CSA_MXFP4: {
      const int64_t nblk = rows * (src->dim / 32);
      if (src->fmt == CSA_F32)
        hipLaunchKernelGGL(quantize_mxfp4_kernel<float>, dim3(grid_for(nblk, 256)), dim3(256), 0,
                           stream, (const float*)src->data, rows, src->dim, (uint8_t*)dst->data,
                           (uint8_t*)dst->scale);
      else
        hipLaunchKernelGGL(quantize_mxfp4_kernel<uint16_t>, dim3(grid_for(nblk, 256)), dim3(256),
                           0, stream, (const uint16_t*)src->data, rows, src->dim,
                           (uint8_t*)dst->data, (uint8_t*)dst->scale);
      break;
    }
    case CSA_BF16:
      if (src->fmt != CSA_F32)
        return fail(CSA_ERR_UNSUPPORTED, "csa_quantize: BF16 destination needs an F32 source");
      hipLaunchKernelGGL(f32_to_bf16_kernel, dim3(grid_for(rows * src->dim, 256)), dim3(256), 0,
                         stream, (const float*)src->data, rows * src->dim, (uint16_t*)dst->data);
      break;
    default:
      return fail(CSA_ERR_UNSUPPORTED, "csa_quantize: destination format not supported");
  }
  return check_launch("csa_quantize");
}

csa_status csa_dequantize(const csa_tensor* src, float* dst, hipStream_t stream) {
  clear_error();
  if (!fmt_valid_tensor(src) || (src->rows > 0 && dst == nullptr))
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_dequantize: bad arguments");
  const int64_t n = src->rows * src->dim;
  if (n == 0) return CSA_OK;
  hipLaunchKernelGGL(dequantize_kernel, dim3(grid_for(n, 256)), dim3(256), 0, stream, *src, dst);
  return check_launch("csa_dequantize");
}

csa_status csa_mxfp4_to_fp8(const csa_tensor* src, uint8_t* fp8, uint8_t* group_scale,
                            uint8_t* lossless, hipStream_t stream) {
  clear_error();
  if (!fmt_valid_tensor(src) || src->fmt != CSA_MXFP4)
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_mxfp4_to_fp8: source must be MXFP4");
  if (src->rows == 0) return CSA_OK;
  if (fp8 == nullptr || group_scale == nullptr || lossless == nullptr)
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_mxfp4_to_fp8: null output");
  hipLaunchKernelGGL(mxfp4_to_fp8_kernel, dim3(grid_for(src->rows, 256)), dim3(256), 0, stream,
                     *src, fp8, group_scale, lossless);
  return check_launch("csa_mxfp4_to_fp8");
}

}  // extern "C"
