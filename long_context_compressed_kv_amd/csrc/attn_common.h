// Pieces shared by the attention kernels (page "DeepSeek V4 深度解析",
// section 2: CSA step 3 and the HCA paragraph): the call's arguments, the key
// geometry of a query (its entries, then its window rows), the source row of
// each key, LDS access helpers and the staging of one key chunk (FP8_MIXED
// entries dequantised exactly to bf16: the block scales are powers of two).
#pragma once

#include "common.h"

namespace csa_attn {

using namespace csa;

constexpr int KT = 32;           // keys per tile
constexpr int kTokMax = 16;      // query tokens per workgroup (128 rows / 8 heads)
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kStale = 8.0f;   // log2 headroom before the running max moves
constexpr int kMetaSlots = 8;    // ring of per-tile source rows and key masks
constexpr int kPartsMax = 32;    // split-K parts of one query (see split_chunk)

// Split-K parts of a query with nkeys keys: ceil(nkeys / split_keys), at
// most kPartsMax, of equal length rounded up to whole tiles (the last part
// takes the rest).  They depend on the query's own key count alone, so a
// request's parts (and the bits of its merged result) do not depend on the
// rest of the batch.  (Each part writes an fp32 partial of every head row, D
// floats: parts of a few hundred keys keep that below the keys' own bytes.)
__host__ __device__ inline int64_t split_chunk(int64_t nkeys, int split_keys) {
  if (nkeys <= 0) return KT;
  int64_t p = (nkeys + split_keys - 1) / split_keys;
  if (p > kPartsMax) p = kPartsMax;
  const int64_t c = (nkeys + p - 1) / p;
  return (c + KT - 1) / KT * KT;
}
__host__ __device__ inline int split_parts(int64_t nkeys, int split_keys) {
  if (nkeys <= 0) return 1;
  const int64_t c = split_chunk(nkeys, split_keys);
  return (int)((nkeys + c - 1) / c);
}
// Longest part of any query of at most max_keys keys: split_keys rounded up
// while ceil(n / split_keys) <= kPartsMax, else ceil(n / kPartsMax) rounded up.
__host__ __device__ inline int64_t split_chunk_max(int64_t max_keys, int split_keys) {
  const int64_t a = ((int64_t)split_keys + KT - 1) / KT * KT;
  const int64_t b = ((max_keys + kPartsMax - 1) / kPartsMax + KT - 1) / KT * KT;
  return a > b ? a : b;
}
// Most parts of any query of at most max_keys keys: a query of n keys has at
// most min(kPartsMax, ceil(n / split_keys)), which grows with n.
__host__ __device__ inline int split_parts_max(int64_t max_keys, int split_keys) {
  int64_t p = (max_keys + split_keys - 1) / split_keys;
  if (p > kPartsMax) p = kPartsMax;
  return p < 1 ? 1 : (int)p;
}

struct AttnArgs {
  const void* q;             // bf16 or fp32 rows; with fp8 queries the e4m3 codes [rows][448]
  const uint8_t* q_scale;    // fp8 queries: e8m0 block scales [rows][4]
  const uint16_t* q_rope;    // fp8 queries: bf16 RoPE dims [rows][64]
  int H;
  int64_t n_q;
  // compressed entries
  const void* kv;
  const uint8_t* kv_scale;
  const uint16_t* kv_rope;
  const int32_t* idx;
  int k;
  // raw window rows
  const void* raw;
  int window;
  BatchDev b;
  int m;
  float scale_log2;  // softmax scale * log2(e)
  void* out;
  float* lse;
  int tok;           // query tokens per workgroup
  int hg;            // heads per workgroup (a head group)
  int ngroups;       // head groups per token (H / hg)
  int nrb;           // 32-row blocks per workgroup
  int split_keys;    // 0: one workgroup per token group; else keys per split
  int max_splits;
  float* ws_o;       // [max_splits][n_q*H][D] (bf16 values when part_bf16)
  float* ws_lse;     // [max_splits][n_q*H]
  int* ws_cnt;       // [n_q] splits used per query
  int part_bf16;     // split-K partial outputs stored as bf16 (a bf16 output)
  int* ws_start;     // [n_q + 1] first work item of each query (split-K)
  int* ws_item_q;    // [n_q * max_splits] query of each work item (split-K)
  int4* ws_geo;      // [n_q][4] geometry record of each query (split-K)
  int* ws_chunk;     // (unused word of the split-K workspace layout)
  // split-K without a plan (selected keys: every query has at most
  // static_keys): chunk and splits per query fixed by the host, work item
  // i = (query i / static_splits, split i % static_splits); 0 = planned
  int static_chunk;
  int static_splits;
  int static_keys;
  int* host_splits;  // host only: where the launch reports static_splits
};

// Tile geometry shared by every thread of a workgroup.
struct Geo {
  int64_t q_first, q_last, t_first, t_last;
  int64_t kv_base, raw_base, raw_pos, kv_len;
  int64_t raw_cap;      // ring capacity of the request's raw rows (0: in order)
  int64_t wlo;          // first window position
  int nE, nkeys, key_lo, key_hi;
};

// Geometry of the token group starting at query q_first: its request, the
// entries it sees (selected or all visible) and its window, in key order
// [entries | window rows].
template <bool SPARSE>
__device__ Geo make_geo(const AttnArgs& a, int64_t q_first) {
  Geo g;
  g.q_first = q_first;
  g.q_last = g.q_first + a.tok - 1;
  if (g.q_last >= a.n_q) g.q_last = a.n_q - 1;
  const QueryMeta qm0 = query_meta(a.b, g.q_first, a.m);
  g.t_first = qm0.t;
  g.t_last = g.t_first + (g.q_last - g.q_first);
  g.kv_base = qm0.kv_base;
  g.raw_base = qm0.raw_base;
  g.raw_pos = qm0.raw_pos;
  g.kv_len = qm0.kv_len;
  g.raw_cap = a.b.ring ? qm0.raw_len : 0;
  if constexpr (SPARSE) {
    g.nE = a.kv != nullptr ? (int)(g.q_last - g.q_first + 1) * a.k : 0;
  } else {
    const int64_t nc = (g.t_last + 1) / a.m;
    g.nE = a.kv != nullptr ? (int)(nc < g.kv_len ? nc : g.kv_len) : 0;
  }
  int64_t whi = -1;
  g.wlo = 0;
  if (a.raw != nullptr && a.window > 0 && qm0.raw_len > 0) {
    g.wlo = g.t_first - a.window + 1;
    if (g.wlo < 0) g.wlo = 0;
    if (g.wlo < qm0.raw_pos) g.wlo = qm0.raw_pos;
    whi = g.t_last;
    if (g.raw_cap > 0) {
      // a ring holds the last raw_cap positions up to the group's last token
      if (g.wlo < g.t_last - g.raw_cap + 1) g.wlo = g.t_last - g.raw_cap + 1;
    } else if (whi > qm0.raw_pos + qm0.raw_len - 1) {
      whi = qm0.raw_pos + qm0.raw_len - 1;
    }
  }
  const int nW = whi >= g.wlo ? (int)(whi - g.wlo + 1) : 0;
  g.nkeys = g.nE + nW;
  g.key_lo = 0;
  g.key_hi = g.nkeys;
  return g;
}

// The geometry of a one-token group as a 64-byte record (split-K work items
// read it with one load instead of re-resolving the request).
__device__ __forceinline__ void store_geo(int4* dst, const Geo& g) {
  const int64_t v[8] = {g.t_first, g.kv_base, g.raw_base, g.raw_pos, g.kv_len, g.raw_cap, g.wlo,
                        ((int64_t)(uint32_t)g.nkeys << 32) | (uint32_t)g.nE};
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = __builtin_bit_cast(int4, make_longlong2(v[2 * i], v[2 * i + 1]));
}
__device__ __forceinline__ Geo load_geo(const int4* src, int64_t q) {
  int64_t v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const longlong2 x = __builtin_bit_cast(longlong2, src[i]);
    v[2 * i] = x.x;
    v[2 * i + 1] = x.y;
  }
  Geo g;
  g.q_first = g.q_last = q;
  g.t_first = g.t_last = v[0];
  g.kv_base = v[1];
  g.raw_base = v[2];
  g.raw_pos = v[3];
  g.kv_len = v[4];
  g.raw_cap = v[5];
  g.wlo = v[6];
  g.nE = (int)(uint32_t)v[7];
  g.nkeys = (int)(uint32_t)(v[7] >> 32);
  g.key_lo = 0;
  g.key_hi = g.nkeys;
  return g;
}


// Workgroup barrier that orders LDS only.  __syncthreads also waits for every
// outstanding global load, which would drain the prefetch of the next tile at
// each barrier inside the key loop; register uses of those loads still wait
// for them where they are consumed.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Source row of key kk, encoded: entry rows as themselves (>= 0), raw window
// rows r as -2 - r, no key as -1.  `lo` / `hi` give the range of token offsets
// g (query token t_first + g) for which the key is valid: an entry j is visible
// from the token whose position reaches (j+1)m - 1, a selected entry only to
// its owner, a window row at position p to tokens p .. p + W - 1.
template <bool SPARSE>
__device__ __forceinline__ void key_meta(const AttnArgs& a, const Geo& g, int kk, int& row,
                                         int64_t& lo, int64_t& hi) {
  row = -1;
  lo = 1;
  hi = 0;
  if (kk >= g.key_hi) return;
  if (kk < g.nE) {
    if constexpr (SPARSE) {
      const int owner = kk / a.k;
      const int slot = kk - owner * a.k;
      const int j = a.idx[(g.q_first + owner) * (int64_t)a.k + slot];
      if (j >= 0 && j < g.kv_len) {
        row = (int)entry_row(a.b, g.kv_base, j);
        lo = owner;
        hi = owner + 1;
      }
    } else {
      row = (int)entry_row(a.b, g.kv_base, kk);
      lo = (int64_t)(kk + 1) * a.m - 1 - g.t_first;
      hi = INT64_MAX;
    }
  } else {
    const int64_t p = g.wlo + (kk - g.nE);
    row = -2 - (int)(g.raw_base + (g.raw_cap > 0 ? p % g.raw_cap : p - g.raw_pos));
    lo = p - g.t_first;
    hi = lo + a.window;
  }
}

// ------------------------------------------------------------------ kernel

// bf16 key tiles are stored unpadded, [key][D], with the 16-byte chunks of row
// r permuted by j -> j ^ f(r), f(r) = 4*(r%4) + (r/4)%4.  Both reads of a
// tile then spread over all LDS banks: the logit operand (one chunk of 32
// consecutive rows per instruction; f is distinct over any 16 consecutive
// rows) and the transposed value operand (4 chunks of 8 consecutive rows).
template <int D>
__device__ __forceinline__ int swz_off(int r, int j) {
  const int f = 4 * (r & 3) + ((r >> 2) & 3);
  return r * (D * 2) + ((j ^ f) << 4);
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte LDS read through a 32-bit LDS address.
__device__ __forceinline__ uint4 lds_read_b128(const lds_u8* p) {
  const u32x4_t v = *(const __attribute__((address_space(3))) u32x4_t*)(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 64-bit transposed LDS read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane i receives element i%4 of the four 16-bit values addressed by
// lanes i/4, i/4+4, i/4+8 and i/4+12 of its group, in that order.
__device__ __forceinline__ uint2 lds_read_tr16(const lds_u8* p) {
  const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

// Dequantise 16 e4m3fn codes with a power-of-two scale into 16 bf16 (exact:
// every product has at most 4 significant bits).  v_cvt_scalef32_pk_bf16_fp8
// converts the two codes of the low half-word of its source.
__device__ __forceinline__ void fp8x16_to_bf16(const uint4 c, float s, uint4& y0, uint4& y1) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  uint32_t o[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    o[2 * q] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[q], s, false));
    o[2 * q + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[q] >> 16, s, false));
  }
  y0 = make_uint4(o[0], o[1], o[2], o[3]);
  y1 = make_uint4(o[4], o[5], o[6], o[7]);
}

// One staging slot of a bf16-compute tile: dims [d, d+16) of one key (row
// encoded as in key_meta, never -1 here).  For an FP8_MIXED entry below dim
// 448, x0 holds the 16 codes and x1.x the e8m0 scale byte (decoded only when
// stored, so a prefetch never waits on it).  Returns whether x0 holds codes.
template <int D, int KVF>
__device__ __forceinline__ bool load_slot(const AttnArgs& a, int row, int d, uint4& x0, uint4& x1) {
  if constexpr (KVF == CSA_FP8_MIXED) {
    if (row >= 0 && d < 448) {
      x0 = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.kv) + (int64_t)row * 448 + d);
      x1.x = a.kv_scale[(int64_t)row * 4 + (d >> 7)];
      return true;
    }
    const uint4* p = row >= 0
        ? reinterpret_cast<const uint4*>(a.kv_rope + (int64_t)row * 64 + (d - 448))
        : reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.raw) + (int64_t)(-2 - row) * D + d);
    x0 = p[0];
    x1 = p[1];
    return false;
  } else {
    // entries and window rows are both bf16 [rows, D]: one load through a select
    const uint16_t* base = row >= 0 ? static_cast<const uint16_t*>(a.kv) + (int64_t)row * D
                                    : static_cast<const uint16_t*>(a.raw) + (int64_t)(-2 - row) * D;
    const uint4* p = reinterpret_cast<const uint4*>(base + d);
    x0 = p[0];
    x1 = p[1];
    return false;
  }
}

// A slot's two 16-byte chunks land at lds[0] + ofs and lds[1] + ofs (swizzled
// positions in the key buffer at byte offset ofs).
__device__ __forceinline__ void store_slot(lds_u8* const* lds, int ofs, bool fp8, uint4 x0, uint4 x1) {
  if (fp8) fp8x16_to_bf16(x0, e8m0_to_f32(x1.x), x0, x1);
  *(__attribute__((address_space(3))) u32x4_t*)(lds[0] + ofs) = u32x4_t{x0.x, x0.y, x0.z, x0.w};
  *(__attribute__((address_space(3))) u32x4_t*)(lds[1] + ofs) = u32x4_t{x1.x, x1.y, x1.z, x1.w};
}

}  // namespace csa_attn

// D = 512 attention with 16 heads per wave (attn512.hip): one workgroup per
// query token (or per part of its keys); kvf BF16 | FP8_MIXED entries, outm 0
// (fp32), 1 (bf16) or 2 (split-K partials); q8: fp8 queries (FP8_MIXED
// entries), the NoPE logits on the fp8 matrix cores.
csa_status launch_attn512(const csa_attn::AttnArgs& a, int kvf, bool sparse, int outm, bool q8,
                          hipStream_t stream);
// Whether a token of at most max_keys keys (entries and window rows) fits it.
bool attn512_fits(int64_t max_keys);
// Most keys of one split-K part it takes with n_heads (64 or 128) heads.
int attn512_part_keys(int n_heads);
