// Device and host helpers shared by the CSA/HCA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csa.h"

namespace csa {

constexpr int kWave = 64;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2_t;

// ---------------------------------------------------------------- bfloat16

__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// fp32 -> bf16, round to nearest-even; NaN -> quiet NaN with the sign kept.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp32 -> packed bf16 pair (low half = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return f32_to_bf16(a) | (f32_to_bf16(b) << 16);
}

// The same for finite inputs in one instruction (v_cvt_pk_bf16_f32, round to
// nearest-even); NaN payloads are not specified, so codecs use pack_bf16x2.
typedef float f32x2_v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2_fast(float a, float b) {
  const f32x2_v v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_v));
}

// ---------------------------------------------------------------- e4m3fn (OCP)

// Exact decode.  For a normal code the 7 magnitude bits placed at bits 20..26
// of a float, with 120 added to the exponent field, give (1+m/8)*2^(e-7);
// subnormal codes are m * 2^-9.  No fp32 denormal is formed on the way.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t mag = c & 0x7fu;
  float v = mag >= 8u ? __uint_as_float((mag << 20) + (120u << 23)) : (float)mag * 0x1p-9f;
  v = (c & 0x80u) ? -v : v;
  return mag == 0x7fu ? __builtin_nanf("") : v;
}

// fp32 -> e4m3fn code: round to nearest-even, saturate to +-448, NaN -> 0x7f.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t s = (u >> 24) & 0x80u;
  const float a = __builtin_fabsf(x);
  if (!(a == a)) return s | 0x7fu;
  if (a > 448.0f) return s | 0x7eu;
  if (a < 0x1p-6f) {                         // subnormal grid n * 2^-9, n in 0..8
    return s | (uint32_t)__builtin_rintf(a * 512.0f);
  }
  const uint32_t ua = __float_as_uint(a);
  const uint32_t e = (ua >> 23) - 127u + 7u;  // biased e4m3 exponent, 1..15
  const uint32_t mant = ua & 0x7fffffu;
  const uint32_t r = mant + 0x7ffffu + ((mant >> 20) & 1u);   // round to 3 bits
  uint32_t v = (e << 3) + (r >> 20);         // a carry out of the mantissa bumps e
  return s | (v > 0x7eu ? 0x7eu : v);
}

// e8m0 byte -> 2^(b-127) (b == 255 -> NaN).
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  if (b == 255u) return __builtin_nanf("");
  if (b == 0u) return 0x1p-127f;
  return __uint_as_float(b << 23);
}

// 2^e for e in [-127, 127] (exact, the result may be subnormal).
__device__ __forceinline__ float exp2i(int e) {
  return e >= -126 ? __uint_as_float((uint32_t)(e + 127) << 23)
                   : __uint_as_float(1u << (e + 149));
}

// Smallest e with amax <= 448 * 2^e, clamped to [-127, 127]; amax == 0 -> -127.
__device__ __forceinline__ int kv_scale_exp(float amax) {
  const uint32_t u = __float_as_uint(amax);
  const int be = (int)(u >> 23);
  if (amax == 0.0f || be == 0) return -127;  // zero or subnormal amax
  int e = be - 135 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// ---------------------------------------------------------------- e2m1 (OCP MX)

__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  // magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6
  const uint32_t m = c & 7u;
  const float mag = m < 2 ? 0.5f * (float)m
                          : __uint_as_float(((((m >> 1) + 126u)) << 23) | ((m & 1u) << 22));
  return (c & 8u) ? -mag : mag;
}

// value (already divided by the block scale) -> e2m1 code, nearest-even,
// saturating to +-6, sign kept.
__device__ __forceinline__ uint32_t f32_to_e2m1(float v) {
  const float a = __builtin_fabsf(v);
  uint32_t c;
  if (a <= 0.25f) c = 0;
  else if (a < 0.75f) c = 1;
  else if (a <= 1.25f) c = 2;
  else if (a < 1.75f) c = 3;
  else if (a <= 2.5f) c = 4;
  else if (a < 3.5f) c = 5;
  else if (a <= 5.0f) c = 6;
  else c = 7;
  return c | ((__float_as_uint(v) >> 28) & 8u);
}

// MX block exponent: floor(log2 amax) - 2, clamped to [-127, 127]; 0 -> -127.
__device__ __forceinline__ int mx_block_exp(float amax) {
  const uint32_t u = __float_as_uint(amax);
  const int be = (int)(u >> 23);
  if (amax == 0.0f || be == 0) return -127;
  int e = be - 127 - 2;
  return e < -127 ? -127 : e;
}

// ---------------------------------------------------------------- reductions

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Index of the request holding flat query q (q_off is nondecreasing,
// q_off[0] = 0).  Clamped to [0, n_req).  One query per request (decode)
// resolves with one pair of loads; otherwise a binary search.
__device__ __forceinline__ int find_request(const int64_t* q_off, int n_req, int64_t q) {
  if (q < n_req) {
    const int64_t a = q_off[q], b = q_off[q + 1];
    if (a <= q && q < b) return (int)q;
  }
  int lo = 0, hi = n_req - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (q_off[mid] <= q) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ int64_t clamp64(int64_t v, int64_t lo, int64_t hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

// Per-query metadata resolved from a csa_batch (device arrays), every value
// clamped to the extents of the tensors involved.
struct QueryMeta {
  int64_t t;        // absolute position of the query
  int64_t kv_base;  // first entry row of the request (paged: its first block-table slot)
  int64_t n_vis;    // visible entries
  int64_t kv_len;   // entry rows of the request
  int64_t raw_base; // first raw row of the request
  int64_t raw_pos;  // position of raw_base
  int64_t raw_len;  // raw rows of the request
};

struct BatchDev {
  int n_req;
  const int64_t* q_off;
  const int64_t* q_pos;
  const int64_t* kv_off;
  const int64_t* raw_off;
  const int64_t* raw_pos;
  int64_t kv_rows;   // rows of the entry tensor (0 if none)
  int64_t raw_rows;  // rows of the raw tensor (0 if none)
  int ring;          // raw rows of a request are a ring (position p at row p mod rows)
  // paged entries (null: contiguous): entry j of request r at row
  // pages[r * page_stride + j / 2^page_shift] * 2^page_shift + j mod 2^page_shift
  const int32_t* pages = nullptr;
  int64_t page_stride = 0;
  int page_shift = 0;
};

// Row of entry j of a request whose QueryMeta::kv_base is kv_base.  A block
// id that points outside the entry tensor gives row 0 (every read stays in
// bounds; such an entry's value is unspecified).
__device__ __forceinline__ int64_t entry_row(const BatchDev& b, int64_t kv_base, int64_t j) {
  if (b.pages == nullptr) return kv_base + j;
  const int64_t blk = b.pages[kv_base + (j >> b.page_shift)];
  const int64_t row = (blk << b.page_shift) + (j & ((1ll << b.page_shift) - 1));
  return blk >= 0 && row < b.kv_rows ? row : 0;
}

// The same for an entry that may lie past the request's entries (ok false):
// such an entry takes row 0 and reads no block table.
__device__ __forceinline__ int64_t entry_row_if(const BatchDev& b, int64_t kv_base, int64_t j, bool ok) {
  return ok ? entry_row(b, kv_base, j) : 0;
}

__device__ __forceinline__ QueryMeta query_meta(const BatchDev& b, int64_t q, int m) {
  QueryMeta r;
  const int req = find_request(b.q_off, b.n_req, q);
  // every load first (they are independent), then the arithmetic
  const bool has_kv = b.kv_off != nullptr && b.kv_rows > 0;
  const bool has_raw = b.raw_off != nullptr && b.raw_rows > 0;
  const int64_t qpos = b.q_pos[req], qoff = b.q_off[req];
  const int64_t kv0 = has_kv ? b.kv_off[req] : 0, kv1 = has_kv ? b.kv_off[req + 1] : 0;
  const int64_t rw0 = has_raw ? b.raw_off[req] : 0, rw1 = has_raw ? b.raw_off[req + 1] : 0;
  const int64_t rpos = has_raw ? b.raw_pos[req] : 0;
  r.t = qpos + (q - qoff);
  if (r.t < 0) r.t = 0;
  if (has_kv && b.pages != nullptr) {
    // paged: kv_off counts the entries, rows come from the block table
    r.kv_base = (int64_t)req * b.page_stride;
    r.kv_len = kv1 > kv0 ? kv1 - kv0 : 0;
    const int64_t cap = b.page_stride << b.page_shift;   // the request's slots in the table
    if (r.kv_len > cap) r.kv_len = cap;
    const int64_t nc = (r.t + 1) / m;
    r.n_vis = nc < r.kv_len ? nc : r.kv_len;
  } else if (has_kv) {
    const int64_t lo = clamp64(kv0, 0, b.kv_rows);
    const int64_t hi = clamp64(kv1, lo, b.kv_rows);
    r.kv_base = lo;
    r.kv_len = hi - lo;
    const int64_t nc = (r.t + 1) / m;
    r.n_vis = nc < hi - lo ? nc : hi - lo;
  } else {
    r.kv_base = 0;
    r.kv_len = 0;
    r.n_vis = 0;
  }
  if (has_raw) {
    const int64_t lo = clamp64(rw0, 0, b.raw_rows);
    const int64_t hi = clamp64(rw1, lo, b.raw_rows);
    r.raw_base = lo;
    r.raw_len = hi - lo;
    r.raw_pos = rpos;
  } else {
    r.raw_base = 0;
    r.raw_len = 0;
    r.raw_pos = 0;
  }
  return r;
}

}  // namespace csa

// ---------------------------------------------------------------- host side

namespace csa_host {

// Records `msg` as the calling thread's last error and returns `st`.
csa_status fail(csa_status st, const char* fmt, ...);
void clear_error();
csa_status check_launch(const char* what);
bool fmt_valid_tensor(const csa_tensor* t, bool need_data = true);
int64_t rows_of(const csa_tensor* t);
// Copies the paged-cache fields of `b` (kv_block_table ...) into `d` after
// checking them; `who` names the entry point in the error.
csa_status batch_pages(const csa_batch* b, csa::BatchDev& d, const char* who);

}  // namespace csa_host
