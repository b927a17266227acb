// Scoring core of the lightning indexer (page "DeepSeek V4 深度解析", section
// 2, CSA step 2: a light, low-rank relevance score of each query against every
// compressed entry; the FP4 paragraph: the indexer QK runs in FP4 and its
// scores are kept in BF16), shared by the score and the fused score + select
// kernels so that both compute bit-identical scores.
//
//   S[q][j] = sum_h w[q][h] * ReLU(qi[q][h] . ki[j])       (H_I = 4, d_I = 64)
//
// One MFMA tile is 32 (query, head) rows x 32 entries: rows are 8 queries x
// 4 heads, so the C layout (row = 8*(i/4) + 4*half + i%4) puts the 4 heads of
// one query in 4 consecutive registers of one lane (register block g holds
// query 2g + half) and the ReLU + head sum needs no cross-lane traffic.  The
// entry keys are the B operand, read straight from memory in operand layout.
#pragma once

#include "common.h"

namespace csa {

constexpr int kHI = 4;       // indexer heads
constexpr int kDI = 64;      // indexer dim

// Key operand of one tile for this lane (entry e0 + rl, its half of the dims).
template <int FMT> struct KeyOp;
template <> struct KeyOp<CSA_F32> { float v[kDI / 2]; };
template <> struct KeyOp<CSA_BF16> { uint4 v[kDI / 16]; };
template <> struct KeyOp<CSA_MXFP4> { uint4 v; int scale; };

// Query operand of one 8-query group for this lane (query rl/4, head rl%4).
template <int FMT> struct QueryOp;
template <> struct QueryOp<CSA_F32> { float v[kDI / 2]; };
template <> struct QueryOp<CSA_BF16> { bf16x8_t v[kDI / 16]; };
template <> struct QueryOp<CSA_MXFP4> { i32x8_t v; int scale; };

template <int FMT>
__device__ __forceinline__ void load_key(const void* ki, const uint8_t* ki_scale, int64_t krow, bool ok, int half,
                                         KeyOp<FMT>& k) {
  if constexpr (FMT == CSA_F32) {
    const float* p = static_cast<const float*>(ki) + krow * kDI + half;
#pragma unroll
    for (int c = 0; c < kDI / 2; ++c) k.v[c] = ok ? p[2 * c] : 0.0f;
  } else if constexpr (FMT == CSA_BF16) {
    const uint16_t* p = static_cast<const uint16_t*>(ki) + krow * kDI + half * 8;
#pragma unroll
    for (int c = 0; c < kDI / 16; ++c)
      k.v[c] = ok ? *reinterpret_cast<const uint4*>(p + 16 * c) : make_uint4(0, 0, 0, 0);
  } else {
    k.v = ok ? *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(ki) + krow * 32 + half * 16)
             : make_uint4(0, 0, 0, 0);
    k.scale = ok ? ki_scale[krow * 2 + half] : 127;
  }
}

template <int FMT>
__device__ __forceinline__ void load_query(const void* qi, const uint8_t* qi_scale, int64_t arow, bool ok, int half,
                                           QueryOp<FMT>& q) {
  if constexpr (FMT == CSA_F32) {
    const float* p = static_cast<const float*>(qi) + arow * kDI + half;
#pragma unroll
    for (int c = 0; c < kDI / 2; ++c) q.v[c] = ok ? p[2 * c] : 0.0f;
  } else if constexpr (FMT == CSA_BF16) {
    const uint16_t* p = static_cast<const uint16_t*>(qi) + arow * kDI + half * 8;
#pragma unroll
    for (int c = 0; c < kDI / 16; ++c) {
      const uint4 v = ok ? *reinterpret_cast<const uint4*>(p + 16 * c) : make_uint4(0, 0, 0, 0);
      q.v[c] = __builtin_bit_cast(bf16x8_t, v);
    }
  } else {
    q.v = i32x8_t{};
    q.scale = 127;
    if (ok) {
      const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(qi) + arow * 32 + half * 16);
      q.v[0] = v.x; q.v[1] = v.y; q.v[2] = v.z; q.v[3] = v.w;
      q.scale = qi_scale[arow * 2 + half];
    }
  }
}

template <int FMT>
__device__ __forceinline__ f32x16_t tile_dots(const QueryOp<FMT>& q, const KeyOp<FMT>& k) {
  f32x16_t acc = f32x16_t{};
  if constexpr (FMT == CSA_F32) {
#pragma unroll
    for (int c = 0; c < kDI / 2; ++c) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(q.v[c], k.v[c], acc, 0, 0, 0);
  } else if constexpr (FMT == CSA_BF16) {
#pragma unroll
    for (int c = 0; c < kDI / 16; ++c)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q.v[c], __builtin_bit_cast(bf16x8_t, k.v[c]), acc, 0, 0, 0);
  } else {
    i32x8_t bk{};
    bk[0] = k.v.x; bk[1] = k.v.y; bk[2] = k.v.z; bk[3] = k.v.w;
    // cbsz = blgp = 4: both operands e2m1; opsel 0 picks scale byte 0
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(q.v, bk, acc, 4, 4, 0, q.scale, 0, k.scale);
  }
  return acc;
}


// Score of the query in register block g of a tile result: ReLU (if relu)
// of each head's dot product, weighted by hw[h] and summed over the heads.
// The ReLU is an integer max on the bit pattern: a negative float (-0
// included) is a negative int32 and becomes +0; without ReLU the floor is
// INT_MIN, which keeps every value.
__device__ __forceinline__ float head_score(const f32x16_t& acc, int g, const float* hw, int relu) {
  int lo = relu ? 0 : (int)0x80000000u;
  asm volatile("" : "+s"(lo));   // a value in a register, not a select per head
  float s = 0.0f;
#pragma unroll
  for (int h = 0; h < kHI; ++h) {
    const int b = __float_as_int(acc[4 * g + h]);
    const float v = __int_as_float(b > lo ? b : lo);
    s = fmaf(hw[h], v, s);
  }
  return s;
}

// The same with every head weight 1 (no weights given): fma(1, v, s) is
// v + s, and fma(1, v, 0) is v but for -0 (the sums can differ from
// head_score's only in the sign of a zero, which the score's key folds).
__device__ __forceinline__ float head_score_unit(const f32x16_t& acc, int g, int relu) {
  int lo = relu ? 0 : (int)0x80000000u;
  asm volatile("" : "+s"(lo));
  float v[kHI];
#pragma unroll
  for (int h = 0; h < kHI; ++h) {
    const int b = __float_as_int(acc[4 * g + h]);
    v[h] = __int_as_float(b > lo ? b : lo);
  }
  return ((v[0] + v[1]) + v[2]) + v[3];
}

}  // namespace csa
