// Wave-level encoders of one storage row (used by the quantiser and by the
// epilogue of kv_compress, so both produce the same bits).
#pragma once

#include "common.h"

namespace csa {

// One wave encodes one 512-dim row into the mixed format.  Lane l holds dims
// [8l, 8l+8) in v[0..8).  Lanes 0..55 hold the 448 e4m3 dims (16 lanes per
// 128-dim block, 8 lanes for the last, 64-dim block); lanes 56..63 hold the
// 64 bf16 RoPE dims.
__device__ __forceinline__ void encode_kv_mixed_row_wave(const float (&v)[8], uint8_t* nope_row,
                                                         uint8_t* scale_row, uint16_t* rope_row) {
  const int lane = threadIdx.x & 63;
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, __builtin_fabsf(v[i]));
  a = fmaxf(a, __shfl_xor(a, 1));
  a = fmaxf(a, __shfl_xor(a, 2));
  a = fmaxf(a, __shfl_xor(a, 4));
  const float a16 = fmaxf(a, __shfl_xor(a, 8));
  const float amax = lane < 48 ? a16 : a;          // lanes 48..55: the 64-dim block
  if (lane < 56) {
    const int e = kv_scale_exp(amax);
    const float inv = exp2i(-e);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) lo |= f32_to_e4m3(v[i] * inv) << (8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) hi |= f32_to_e4m3(v[4 + i] * inv) << (8 * i);
    uint2 packed;
    packed.x = lo;
    packed.y = hi;
    *reinterpret_cast<uint2*>(nope_row + 8 * lane) = packed;
    if ((lane & 15) == 0) scale_row[lane >> 4] = (uint8_t)(e + 127);
  } else {
    uint4 packed;
    packed.x = pack_bf16x2(v[0], v[1]);
    packed.y = pack_bf16x2(v[2], v[3]);
    packed.z = pack_bf16x2(v[4], v[5]);
    packed.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4*>(rope_row + 8 * (lane - 56)) = packed;
  }
}

// One thread encodes one MX block of 32 values into 16 code bytes + a scale.
__device__ __forceinline__ void encode_mxfp4_block(const float (&v)[32], uint8_t* codes,
                                                   uint8_t* scale) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, __builtin_fabsf(v[i]));
  const int e = mx_block_exp(amax);
  const float inv = exp2i(-e);
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) word |= f32_to_e2m1(v[8 * j + i] * inv) << (4 * i);
    w[j] = word;
  }
  *reinterpret_cast<uint4*>(codes) = make_uint4(w[0], w[1], w[2], w[3]);
  *scale = (uint8_t)(e + 127);
}

}  // namespace csa
