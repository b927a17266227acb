// Exact combination of partial attentions over disjoint key sets by their
// log-sum-exp (the window branch and the compressed branch are attended
// together: page "DeepSeek V4 深度解析", section 2, CSA step 3):
//   M = max_p lse_p,  w_p = e^(lse_p - M),  o = sum_p w_p o_p / sum_p w_p,
//   lse = M + log(sum_p w_p).
// A part with lse = -inf contributes nothing; if all are -inf, o = 0 and
// lse = -inf.  Memory bound: one wave per row, float4 per lane, parts summed
// in a fixed order with several parts' loads in flight at once.
#include "merge.h"

using namespace csa;

namespace {

template <bool OUT_BF16, bool PART_BF16>
__global__ __launch_bounds__(256) void lse_merge_kernel(const void* __restrict__ o0,
                                                        const float* __restrict__ l0,
                                                        int64_t stride_o, int64_t stride_l,
                                                        int nparts, const int* __restrict__ cnt,
                                                        int rows_per_q, int64_t rows, int dim,
                                                        void* out, float* lse_out) {
  // the row is the same for the whole wave: held in scalar registers
  const int64_t row = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  int n = nparts;
  if (cnt != nullptr) {
    n = cnt[row / rows_per_q];
    n = n < 1 ? 1 : (n > nparts ? nparts : n);
  }
  // part p's values d .. d+3 of this row
  auto part_o = [&](int p, int d) -> float4 {
    const char* base = reinterpret_cast<const char*>(o0) + p * stride_o;
    if constexpr (PART_BF16) {
      const uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + row * dim + d);
      return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                         __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
    } else {
      return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + row * dim + d);
    }
  };
  // part p's log-sum-exp and weight are held by lane p % 64, slot p / 64
  float lv[4], w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int p = lane + 64 * j;
    lv[j] = p < n ? *(reinterpret_cast<const float*>(reinterpret_cast<const char*>(l0) + p * stride_l) + row)
                  : -INFINITY;
  }
  const float mx = wave_max(fmaxf(fmaxf(lv[0], lv[1]), fmaxf(lv[2], lv[3])));
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = (mx == -INFINITY || lv[j] == -INFINITY) ? 0.0f : expf(lv[j] - mx);
  // (with at most 64 parts the slots past the first hold 0 and add nothing)
  const float den = wave_sum(((w[0] + w[1]) + w[2]) + w[3]);
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  if (lse_out != nullptr && lane == 0) lse_out[row] = den > 0.0f ? mx + logf(den) : -INFINITY;
  // part p's weight, read from its lane into a scalar register
  auto weight = [&](int p) {
    const int j = p >> 6;
    const float v = j == 0 ? w[0] : (j == 1 ? w[1] : (j == 2 ? w[2] : w[3]));
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), p & 63));
  };
  // a part of weight 0 (lse = -inf) is skipped by a select, so its values
  // never reach the sum
  auto add = [](float& r, float wp, float x) { r = wp != 0.0f ? fmaf(wp, x, r) : r; };
  for (int d = lane * 4; d < dim; d += 256) {
    float r0 = 0.f, r1 = 0.f, r2 = 0.f, r3 = 0.f;
    int p = 0;
    // four parts' loads in flight before their sums, parts in a fixed order
    for (; p + 4 <= n; p += 4) {
      float4 x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = part_o(p + i, d);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float wp = weight(p + i);
        add(r0, wp, x[i].x);
        add(r1, wp, x[i].y);
        add(r2, wp, x[i].z);
        add(r3, wp, x[i].w);
      }
    }
    for (; p < n; ++p) {
      const float4 x = part_o(p, d);
      const float wp = weight(p);
      add(r0, wp, x.x);
      add(r1, wp, x.y);
      add(r2, wp, x.z);
      add(r3, wp, x.w);
    }
    r0 *= inv; r1 *= inv; r2 *= inv; r3 *= inv;
    if constexpr (OUT_BF16) {
      uint2 u;
      u.x = pack_bf16x2_fast(r0, r1);
      u.y = pack_bf16x2_fast(r2, r3);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + row * dim + d) = u;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(out) + row * dim + d) =
          make_float4(r0, r1, r2, r3);
    }
  }
}

}  // namespace

csa_status launch_lse_merge_bytes(const void* o0, const float* l0, int64_t stride_o_bytes,
                                  int64_t stride_l_bytes, int nparts, const int* cnt,
                                  int rows_per_q, int64_t rows, int dim, void* out, int out_fmt,
                                  float* lse_out, bool part_bf16, hipStream_t stream) {
  const int64_t blocks = (rows + 3) / 4;
  if (blocks > 0x7fffffff || nparts < 1 || nparts > 256)
    return csa_host::fail(CSA_ERR_INVALID_ARGUMENT, "merge: bad row or part count");
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, stream, o0, l0, stride_o_bytes,
                       stride_l_bytes, nparts, cnt, rows_per_q, rows, dim, out, lse_out);
  };
  if (out_fmt == CSA_BF16) {
    if (part_bf16) go(lse_merge_kernel<true, true>);
    else go(lse_merge_kernel<true, false>);
  } else {
    if (part_bf16) go(lse_merge_kernel<false, true>);
    else go(lse_merge_kernel<false, false>);
  }
  return csa_host::check_launch("lse merge");
}

csa_status launch_lse_merge(const void* o0, const float* l0, int64_t stride_o_elems,
                            int64_t stride_l_elems, int nparts, const int* cnt, int rows_per_q,
                            int64_t rows, int dim, void* out, int out_fmt, float* lse_out,
                            bool part_bf16, hipStream_t stream) {
  const int64_t vb = part_bf16 ? 2 : 4;
  return launch_lse_merge_bytes(o0, l0, stride_o_elems * vb, stride_l_elems * 4, nparts, cnt,
                                rows_per_q, rows, dim, out, out_fmt, lse_out, part_bf16, stream);
}

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
  // the two parts are addressed as base + p * (distance between them)
  const int64_t so = (int64_t)((intptr_t)o_b - (intptr_t)o_a);
  const int64_t sl = (int64_t)((intptr_t)lse_b - (intptr_t)lse_a);
  return launch_lse_merge_bytes(o_a, lse_a, so, sl, 2, nullptr, 1, rows, dim, out, out_fmt,
                                lse_out, false, stream);
}
