// Lightning indexer (page "DeepSeek V4 深度解析", section 2, CSA step 2: a
// light, low-rank relevance score of each query against every compressed
// entry; the FP4 paragraph: the indexer QK runs in FP4 and its scores are
// kept in BF16).
//
//   S[q][j] = sum_h w[q][h] * ReLU(qi[q][h] . ki[j])       (H_I = 4, d_I = 64)
//
// One MFMA tile is 32 (query, head) rows x 32 entries: rows are 8 queries x
// 4 heads, so the C layout (row = 8*(i/4) + 4*half + i%4) puts the 4 heads of
// one query in 4 consecutive registers of one lane and the ReLU + head sum
// needs no cross-lane traffic.  The entry keys are the B operand and are read
// straight from HBM in operand layout (each lane: 8 bf16 dims / 32 fp4 codes
// of one entry), so the key stream is the only large traffic: the kernel is
// HBM bound for decode and score-write bound for long prefill.
//   fp32  : v_mfma_f32_32x32x2f32, 32 per tile
//   bf16  : v_mfma_f32_32x32x16_bf16, 4 per tile
//   MXFP4 : v_mfma_scale_f32_32x32x64_f8f6f4 (e2m1 operands, e8m0 block
//           scales per lane), 1 per tile - the products and block sums are
//           exact, so this equals the lossless FP4 -> FP8 route.
#include "common.h"

using namespace csa;

namespace {

constexpr int kHI = 4;       // indexer heads
constexpr int kDI = 64;      // indexer dim
constexpr int kWaves = 4;
constexpr int kTilesPerWave = 8;
constexpr int kEntriesPerWG = kWaves * kTilesPerWave * 32;

struct IdxArgs {
  const void* qi;
  const uint8_t* qi_scale;
  const float* head_w;
  const void* ki;
  const uint8_t* ki_scale;
  BatchDev b;
  int m;
  int relu;
  int qpg;          // queries per group (8 or 1)
  int64_t n_q;
  void* scores;
  int64_t ld;
};

template <int FMT, bool SBF16>
__global__ __launch_bounds__(256) void indexer_kernel(IdxArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int rl = lane & 31;

  const int64_t q0 = (int64_t)blockIdx.y * a.qpg;
  // this lane's A row: (query q0 + rl/4, head rl%4)
  const int qa = rl >> 2, ha = rl & 3;
  const bool a_live = qa < a.qpg && q0 + qa < a.n_q;
  const int64_t qa_idx = q0 + qa;

  const QueryMeta qm = query_meta(a.b, q0, a.m);
  const int64_t kv_base = qm.kv_base;
  // entries this group scans: up to the largest n_vis of its queries
  int64_t q_hi = q0 + a.qpg - 1;
  if (q_hi >= a.n_q) q_hi = a.n_q - 1;
  const QueryMeta qm_hi = query_meta(a.b, q_hi, a.m);
  const int64_t n_scan = qm_hi.n_vis < a.ld ? qm_hi.n_vis : a.ld;   // never past a row

  // per-lane output queries: q_local = 2*(i/4) + half, i/4 = 0..3
  int64_t nvis_o[4];
  float w_o[4][kHI];
  bool live_o[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int ql = 2 * g + half;
    const int64_t qq = q0 + ql;
    live_o[g] = ql < a.qpg && qq < a.n_q;
    nvis_o[g] = live_o[g] ? query_meta(a.b, qq, a.m).n_vis : 0;
    if (nvis_o[g] > a.ld) nvis_o[g] = a.ld;
#pragma unroll
    for (int h = 0; h < kHI; ++h)
      w_o[g][h] = (live_o[g] && a.head_w != nullptr) ? a.head_w[qq * kHI + h] : 1.0f;
  }

  // A operand (queries), loaded once
  float aq_f32[kDI / 2];
  bf16x8_t aq_bf16[kDI / 16];
  i32x8_t aq_fp4{};
  int aq_scale = 127;
  const int64_t arow = qa_idx * kHI + ha;
  if constexpr (FMT == CSA_F32) {
    const float* p = static_cast<const float*>(a.qi) + arow * kDI + half;
#pragma unroll
    for (int c = 0; c < kDI / 2; ++c) aq_f32[c] = a_live ? p[2 * c] : 0.0f;
  } else if constexpr (FMT == CSA_BF16) {
    const uint16_t* p = static_cast<const uint16_t*>(a.qi) + arow * kDI + half * 8;
#pragma unroll
    for (int c = 0; c < kDI / 16; ++c) {
      const uint4 v = a_live ? *reinterpret_cast<const uint4*>(p + 16 * c) : make_uint4(0, 0, 0, 0);
      aq_bf16[c] = __builtin_bit_cast(bf16x8_t, v);
    }
  } else {
    if (a_live) {
      const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.qi) + arow * 32 + half * 16);
      aq_fp4[0] = v.x; aq_fp4[1] = v.y; aq_fp4[2] = v.z; aq_fp4[3] = v.w;
      aq_scale = a.qi_scale[arow * 2 + half];
    }
  }

  const int64_t e_wg = (int64_t)blockIdx.x * kEntriesPerWG;
  for (int t = 0; t < kTilesPerWave; ++t) {
    const int64_t e0 = e_wg + (int64_t)(t * kWaves + wave) * 32;
    if (e0 >= n_scan) break;
    const int64_t e = e0 + rl;               // this lane's entry (B column)
    const bool e_ok = e < n_scan;
    const int64_t krow = kv_base + e;
    f32x16_t acc = f32x16_t{};
    if constexpr (FMT == CSA_F32) {
      const float* p = static_cast<const float*>(a.ki) + krow * kDI + half;
#pragma unroll
      for (int c = 0; c < kDI / 2; ++c)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(aq_f32[c], e_ok ? p[2 * c] : 0.0f, acc, 0, 0, 0);
    } else if constexpr (FMT == CSA_BF16) {
      const uint16_t* p = static_cast<const uint16_t*>(a.ki) + krow * kDI + half * 8;
      uint4 kv[kDI / 16];
#pragma unroll
      for (int c = 0; c < kDI / 16; ++c)
        kv[c] = e_ok ? *reinterpret_cast<const uint4*>(p + 16 * c) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int c = 0; c < kDI / 16; ++c)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq_bf16[c], __builtin_bit_cast(bf16x8_t, kv[c]),
                                                       acc, 0, 0, 0);
    } else {
      i32x8_t bk{};
      int bscale = 127;
      if (e_ok) {
        const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.ki) + krow * 32 + half * 16);
        bk[0] = v.x; bk[1] = v.y; bk[2] = v.z; bk[3] = v.w;
        bscale = a.ki_scale[krow * 2 + half];
      }
      // cbsz = blgp = 4: both operands e2m1; opsel 0 picks scale byte 0
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aq_fp4, bk, acc, 4, 4, 0, aq_scale, 0,
                                                            bscale);
    }
    // ReLU + weighted head sum, then store
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float s = 0.0f;
#pragma unroll
      for (int h = 0; h < kHI; ++h) {
        float v = acc[4 * g + h];
        if (a.relu) v = fmaxf(v, 0.0f);
        s = fmaf(w_o[g][h], v, s);
      }
      if (live_o[g] && e < nvis_o[g]) {
        const int64_t off = (q0 + 2 * g + half) * a.ld + e;
        if constexpr (SBF16)
          static_cast<uint16_t*>(a.scores)[off] = (uint16_t)pack_bf16x2_fast(s, 0.0f);
        else
          static_cast<float*>(a.scores)[off] = s;
      }
    }
  }
}

template <int FMT>
void launch(const IdxArgs& a, bool sbf16, dim3 grid, hipStream_t s) {
  if (sbf16)
    hipLaunchKernelGGL((indexer_kernel<FMT, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((indexer_kernel<FMT, false>), grid, dim3(256), 0, s, a);
}

}  // namespace

using namespace csa_host;

extern "C" csa_status csa_indexer_score(const csa_tensor* qi, int32_t n_heads,
                                        const float* head_w, const csa_tensor* ki,
                                        const csa_batch* batch, int32_t m, int32_t relu,
                                        void* scores, int32_t score_fmt, int64_t ld,
                                        hipStream_t stream) {
  clear_error();
  if (batch == nullptr || !fmt_valid_tensor(qi) || !fmt_valid_tensor(ki, false))
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_indexer_score: bad tensor or batch");
  if (batch->n_req < 1 || batch->n_q < 0 || batch->q_off == nullptr || batch->q_pos == nullptr ||
      batch->kv_off == nullptr)
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_indexer_score: bad batch descriptor");
  if (n_heads != kHI || qi->dim != kDI || ki->dim != kDI)
    return fail(CSA_ERR_UNSUPPORTED, "csa_indexer_score: implemented for 4 heads of dim 64");
  if (qi->fmt != ki->fmt || (qi->fmt != CSA_F32 && qi->fmt != CSA_BF16 && qi->fmt != CSA_MXFP4))
    return fail(CSA_ERR_UNSUPPORTED, "csa_indexer_score: qi and ki must both be F32, BF16 or MXFP4");
  if (score_fmt != CSA_F32 && score_fmt != CSA_BF16)
    return fail(CSA_ERR_UNSUPPORTED, "csa_indexer_score: scores must be F32 or BF16");
  if (qi->rows != batch->n_q * n_heads)
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_indexer_score: qi rows must be n_q * n_heads");
  if (m < 1) return fail(CSA_ERR_INVALID_ARGUMENT, "csa_indexer_score: m must be >= 1");
  if (batch->max_kv < 0 || ld < batch->max_kv)
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_indexer_score: need ld >= max_kv >= 0");
  if (batch->n_q == 0 || batch->max_kv == 0 || ki->rows == 0) return CSA_OK;
  if (scores == nullptr) return fail(CSA_ERR_INVALID_ARGUMENT, "csa_indexer_score: null scores");

  IdxArgs a{};
  a.qi = qi->data;
  a.qi_scale = static_cast<const uint8_t*>(qi->scale);
  a.head_w = head_w;
  a.ki = ki->data;
  a.ki_scale = static_cast<const uint8_t*>(ki->scale);
  a.b = BatchDev{batch->n_req, batch->q_off, batch->q_pos, batch->kv_off, nullptr, nullptr,
                 ki->rows, 0};
  a.m = m;
  a.relu = relu ? 1 : 0;
  a.qpg = batch->n_req == 1 ? 8 : 1;
  a.n_q = batch->n_q;
  a.scores = scores;
  a.ld = ld;
  const int64_t gy = (batch->n_q + a.qpg - 1) / a.qpg;
  const int64_t gx = (batch->max_kv + kEntriesPerWG - 1) / kEntriesPerWG;
  if (gy > 65535 || gx > 0x7fffffff)
    return fail(CSA_ERR_UNSUPPORTED, "csa_indexer_score: problem too large for one launch");
  const dim3 grid((unsigned)gx, (unsigned)gy);
  const bool sb = score_fmt == CSA_BF16;
  if (qi->fmt == CSA_F32) launch<CSA_F32>(a, sb, grid, stream);
  else if (qi->fmt == CSA_BF16) launch<CSA_BF16>(a, sb, grid, stream);
  else launch<CSA_MXFP4>(a, sb, grid, stream);
  return check_launch("csa_indexer_score");
}
