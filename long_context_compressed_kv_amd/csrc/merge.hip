// Exact combination of two partial attentions over disjoint key sets by their
// log-sum-exp (the window branch and the compressed branch are attended
// together: page "DeepSeek V4 深度解析", section 2, CSA step 3).
//
// Memory bound: one wave per row, float4 per lane.
#include "common.h"

using namespace csa;

namespace {

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void swa_merge_kernel(const float* __restrict__ o_a,
                                                        const float* __restrict__ lse_a,
                                                        const float* __restrict__ o_b,
                                                        const float* __restrict__ lse_b,
                                                        int64_t rows, int dim, void* out,
                                                        float* lse_out) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const float a = lse_a[row], b = lse_b[row];
  const float mx = fmaxf(a, b);
  float wa = 0.0f, wb = 0.0f;
  if (mx != -INFINITY) {
    wa = expf(a - mx);
    wb = expf(b - mx);
  }
  const float den = wa + wb;
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  const float ca = wa * inv, cb = wb * inv;
  if (lse_out != nullptr && lane == 0) lse_out[row] = den > 0.0f ? mx + logf(den) : -INFINITY;
  for (int d = lane * 4; d < dim; d += 256) {
    const float4 x = *reinterpret_cast<const float4*>(o_a + row * dim + d);
    const float4 y = *reinterpret_cast<const float4*>(o_b + row * dim + d);
    const float r0 = ca * x.x + cb * y.x, r1 = ca * x.y + cb * y.y;
    const float r2 = ca * x.z + cb * y.z, r3 = ca * x.w + cb * y.w;
    if constexpr (OUT_BF16) {
      uint2 u;
      u.x = pack_bf16x2(r0, r1);
      u.y = pack_bf16x2(r2, r3);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + row * dim + d) = u;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(out) + row * dim + d) =
          make_float4(r0, r1, r2, r3);
    }
  }
}

}  // namespace

using namespace csa_host;

extern "C" csa_status csa_swa_merge(const float* o_a, const float* lse_a, const float* o_b,
                                    const float* lse_b, int64_t rows, int32_t dim, void* out,
                                    int32_t out_fmt, float* lse_out, hipStream_t stream) {
  clear_error();
  if (rows < 0 || dim <= 0 || dim % 4 != 0)
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_swa_merge: rows >= 0 and dim a positive multiple of 4");
  if (rows == 0) return CSA_OK;
  if (!o_a || !lse_a || !o_b || !lse_b || !out)
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_swa_merge: null pointer");
  if (out_fmt != CSA_F32 && out_fmt != CSA_BF16)
    return fail(CSA_ERR_UNSUPPORTED, "csa_swa_merge: out must be F32 or BF16");
  const int64_t blocks = (rows + 3) / 4;
  if (blocks > 0x7fffffff) return fail(CSA_ERR_INVALID_ARGUMENT, "csa_swa_merge: too many rows");
  if (out_fmt == CSA_BF16)
    hipLaunchKernelGGL(swa_merge_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, o_a,
                       lse_a, o_b, lse_b, rows, dim, out, lse_out);
  else
    hipLaunchKernelGGL(swa_merge_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, o_a,
                       lse_a, o_b, lse_b, rows, dim, out, lse_out);
  return check_launch("csa_swa_merge");
}
