// Shared-KV multi-query attention over compressed entries (selected by top-k
// for CSA, all visible for HCA) together with a sliding window of raw tokens,
// one softmax over the union (page "DeepSeek V4 深度解析", section 2: CSA step 3
// and the HCA paragraph).
//
// Work split.  A workgroup owns TOK consecutive query tokens of one request,
// i.e. TOK*H query rows (heads stacked, since all heads share the keys).  The
// rows form 32-row blocks; each block is handled by DSPLIT waves, each wave
// owning D/DSPLIT of the head dimension (partial logits are summed through
// LDS in a fixed order).  Keys are streamed in tiles of 32: the workgroup
// stages a tile into LDS twice, as K[key][d] for the logits and as
// V^T[d][key] for the value product, dequantising FP8_MIXED rows to bf16
// (exact, the scales are powers of two).  The global loads of tile t+1 are in
// flight while tile t is computed, and the source rows of a tile are resolved
// once per key, one tile ahead.
//
// Split-K (decode).  With split_keys > 0 a query's key list is cut into
// chunks of split_keys keys handled by separate workgroups (grid y); each
// writes a normalised partial output and its log-sum-exp to the workspace,
// and a combine pass merges them (the same merge as csa_swa_merge).
//
// Per tile and wave (bf16):
// Staging maps consecutive threads to consecutive groups of 4 keys at the
// same 8 dims, so the transposed V^T writes of a wave spread over the LDS
// banks and each key row is still read in 128-byte pieces.
//
//   S^T = K Q^T        v_mfma_f32_32x32x16_bf16, keys on M, queries on N;
//                      lane (q = l%32, half = l/32) gets 16 keys of query q,
//                      key = 8*(i/4) + 4*half + (i%4) for register i
//   online softmax     base 2, scale folded into the exponent; the running
//                      maximum is only raised when a tile exceeds it by more
//                      than 2^8, so the output is rarely rescaled
//   O^T += V^T P^T     same instruction, d on M; the contraction slots of both
//                      operands follow the key order above, so P never leaves
//                      registers
// fp32 inputs use v_mfma_f32_32x32x2f32 with the same structure (one key per
// lane and instruction, so V is read straight from the K layout).
#include <type_traits>

#include "common.h"
#include "merge.h"

using namespace csa;

namespace {

constexpr int KT = 32;           // keys per tile
constexpr int kRawTag = 1 << 30;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kStale = 8.0f;   // log2 headroom before the running max moves
constexpr int kMaxSplits = 64;

struct AttnArgs {
  const void* q;
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
  int nrb;           // 32-row blocks per workgroup
  int split_keys;    // 0: one workgroup per token group; else keys per split
  int max_splits;
  float* ws_o;       // [max_splits][n_q*H][D]
  float* ws_lse;     // [max_splits][n_q*H]
  int* ws_cnt;       // [n_q] splits used per query
};

// ------------------------------------------------------------------ staging

// 8 consecutive dims [d, d+8) of a key row as packed bf16.
template <int KVF>
__device__ __forceinline__ uint4 load_key8_bf16(const void* base, const uint8_t* scl,
                                                const uint16_t* rope, int64_t row, int d, int D) {
  if constexpr (KVF == CSA_BF16) {
    return *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + row * D + d);
  } else {  // CSA_FP8_MIXED, D == 512
    if (d < 448) {
      const uint2 c = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(base) + row * 448 + d);
      const float s = e8m0_to_f32(scl[row * 4 + (d >> 7)]);
      uint4 r;
      // the products are exact, so their top 16 bits are the bf16 values
      r.x = (__float_as_uint(e4m3_to_f32(c.x & 0xff) * s) >> 16) |
            (__float_as_uint(e4m3_to_f32((c.x >> 8) & 0xff) * s) & 0xffff0000u);
      r.y = (__float_as_uint(e4m3_to_f32((c.x >> 16) & 0xff) * s) >> 16) |
            (__float_as_uint(e4m3_to_f32(c.x >> 24) * s) & 0xffff0000u);
      r.z = (__float_as_uint(e4m3_to_f32(c.y & 0xff) * s) >> 16) |
            (__float_as_uint(e4m3_to_f32((c.y >> 8) & 0xff) * s) & 0xffff0000u);
      r.w = (__float_as_uint(e4m3_to_f32((c.y >> 16) & 0xff) * s) >> 16) |
            (__float_as_uint(e4m3_to_f32(c.y >> 24) * s) & 0xffff0000u);
      return r;
    }
    return *reinterpret_cast<const uint4*>(rope + row * 64 + (d - 448));
  }
}

// Tile geometry shared by every thread of a workgroup.
struct Geo {
  int64_t q_first, q_last, t_first, t_last;
  int64_t kv_base, raw_base, raw_pos, kv_len;
  int64_t nvis_first;   // visible entries of the first token (the fewest)
  int64_t wlo;          // first window position
  int nE, nkeys, key_lo, key_hi;
};

// Source row and mask tag of key kk: entry rows carry their local index
// (dense) or owning token (sparse); raw rows carry kRawTag | (p - t_first + W).
// Also whether the key is valid for every query row of the workgroup.
template <bool SPARSE>
__device__ __forceinline__ void key_meta(const AttnArgs& a, const Geo& g, int kk, int& row,
                                         int& tag, bool& all_ok) {
  row = -1;
  tag = -1;
  all_ok = false;
  if (kk >= g.key_hi) return;
  if (kk < g.nE) {
    if constexpr (SPARSE) {
      const int owner = kk / a.k;
      const int slot = kk - owner * a.k;
      const int j = a.idx[(g.q_first + owner) * (int64_t)a.k + slot];
      if (j >= 0 && j < g.kv_len) {
        row = (int)(g.kv_base + j);
        tag = owner;
        all_ok = a.tok == 1;
      }
    } else {
      row = (int)(g.kv_base + kk);
      tag = kk;
      all_ok = kk < g.nvis_first;
    }
  } else {
    const int64_t p = g.wlo + (kk - g.nE);
    row = (int)(g.raw_base + (p - g.raw_pos));
    tag = kRawTag | (int)(p - g.t_first + a.window);
    all_ok = p >= g.t_last - a.window + 1 && p <= g.t_first;
  }
}

// ------------------------------------------------------------------ kernel

template <int D, bool F32C, int KVF, bool SPARSE, int DSPLIT, int OUTM, bool PREF>
__global__ __launch_bounds__(512) void attn_kernel(AttnArgs a) {
  constexpr int DW = D / DSPLIT;                 // dims per wave
  constexpr int KSTR = F32C ? D + 4 : D + 8;     // K-layout row stride (elements)
  constexpr int VSTR = KT + 4;                   // V^T row stride (bf16 elements)
  using kelem_t = typename std::conditional<F32C, float, uint16_t>::type;
  // staging units: bf16 = 4 keys x 8 dims, fp32 = 1 key x 4 dims
  constexpr int UNITS = F32C ? KT * D / 4 : (KT / 4) * (D / 8);
  // prefetching variants run with at least 256 threads
  constexpr int UPT = PREF ? (UNITS + 255) / 256 : 1;

  extern __shared__ __align__(16) unsigned char smem[];
  kelem_t* klds = reinterpret_cast<kelem_t*>(smem);
  uint16_t* vt = reinterpret_cast<uint16_t*>(smem + KT * KSTR * sizeof(kelem_t));
  int* mrow = reinterpret_cast<int*>(smem + KT * KSTR * sizeof(kelem_t) + (F32C ? 0 : D * VSTR * 2));
  int* mtag = mrow + 2 * KT;
  int* mfull = mtag + 2 * KT;                     // [2], padded to 4 ints
  float* sx = reinterpret_cast<float*>(mfull + 4); // [nrb][DSPLIT][64][16] partial logits

  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int ql = lane & 31;
  const int rb = wave / DSPLIT;
  const int dpart = wave - rb * DSPLIT;
  const int d0 = dpart * DW;

  // ---- geometry of this workgroup's token group
  Geo g;
  g.q_first = (int64_t)blockIdx.x * a.tok;
  g.q_last = g.q_first + a.tok - 1;
  if (g.q_last >= a.n_q) g.q_last = a.n_q - 1;
  const int req = find_request(a.b.q_off, a.b.n_req, g.q_first);
  const QueryMeta qm0 = query_meta(a.b, g.q_first, a.m);
  g.t_first = qm0.t;
  g.t_last = g.t_first + (g.q_last - g.q_first);
  g.kv_base = qm0.kv_base;
  g.raw_base = qm0.raw_base;
  g.raw_pos = qm0.raw_pos;
  g.kv_len = a.b.kv_off != nullptr && a.b.kv_rows > 0
                 ? clamp64(a.b.kv_off[req + 1], qm0.kv_base, a.b.kv_rows) - qm0.kv_base
                 : 0;
  g.nvis_first = qm0.n_vis;
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
    if (whi > qm0.raw_pos + qm0.raw_len - 1) whi = qm0.raw_pos + qm0.raw_len - 1;
  }
  const int nW = whi >= g.wlo ? (int)(whi - g.wlo + 1) : 0;
  g.nkeys = g.nE + nW;

  // ---- key range of this workgroup (split-K)
  int split = 0, nsplit = 1;
  g.key_lo = 0;
  g.key_hi = g.nkeys;
  if (a.split_keys > 0) {
    int chunk = a.split_keys;
    const int need = (g.nkeys + a.max_splits - 1) / a.max_splits;
    if (need > chunk) chunk = need;
    chunk = (chunk + KT - 1) / KT * KT;
    nsplit = g.nkeys > 0 ? (g.nkeys + chunk - 1) / chunk : 1;
    split = blockIdx.y;
    if (split >= nsplit) return;                   // whole workgroup: nothing to do
    g.key_lo = split * chunk;
    g.key_hi = g.key_lo + chunk < g.nkeys ? g.key_lo + chunk : g.nkeys;
    if (split == 0 && tid == 0) a.ws_cnt[g.q_first] = nsplit;
  }

  // ---- this lane's query row
  const int row_in_wg = rb * 32 + ql;
  const int g_row = row_in_wg / a.H;
  const int h_row = row_in_wg - g_row * a.H;
  const int64_t q_row = g.q_first + g_row;
  const bool row_live = q_row <= g.q_last;
  const int64_t t_row = g.t_first + g_row;
  int64_t nvis_row = (t_row + 1) / a.m;
  if (nvis_row > g.kv_len) nvis_row = g.kv_len;
  const int64_t qrow_index = q_row * a.H + h_row;    // row of the q / out tensors

  // queries (B operand), pre-loaded for the whole key loop
  constexpr int QC = F32C ? DW / 2 : DW / 16;
  using qreg_t = typename std::conditional<F32C, float, bf16x8_t>::type;
  qreg_t qreg[QC];
  if constexpr (F32C) {
    const float* qp = static_cast<const float*>(a.q) + qrow_index * D + d0 + half;
#pragma unroll
    for (int c = 0; c < QC; ++c) qreg[c] = row_live ? qp[2 * c] : 0.0f;
  } else {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + qrow_index * D + d0 + half * 8;
#pragma unroll
    for (int c = 0; c < QC; ++c) {
      uint4 v = row_live ? *reinterpret_cast<const uint4*>(qp + 16 * c) : make_uint4(0, 0, 0, 0);
      qreg[c] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  constexpr int NDB = DW / 32;
  f32x16_t acc_o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc_o[i] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.0f;

  // ---- staging helpers
  using stage_t = typename std::conditional<F32C, float4, uint4>::type;
  constexpr int SPU = F32C ? 1 : 4;               // stage registers per unit
  stage_t stg[UPT][SPU];

  auto meta_tile = [&](int kbase, int buf) {
    if (tid < 64) {
      int row = -1, tag = -1;
      bool ok = true;
      if (tid < KT) key_meta<SPARSE>(a, g, kbase + tid, row, tag, ok);
      if (tid < KT) {
        mrow[buf * KT + tid] = row;
        mtag[buf * KT + tid] = tag;
      }
      const unsigned long long bal = __ballot(ok);
      if (tid == 0) mfull[buf] = (bal & 0xffffffffull) == 0xffffffffull ? 1 : 0;
    }
  };

  auto load_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * nthreads;
      if constexpr (F32C) {
        constexpr int UPR = D / 4;
        const int key = u / UPR;
        const int d = (u - key * UPR) * 4;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (u < UNITS) {
          const int row = mrow[buf * KT + key];
          if (row >= 0) {
            const float* src = static_cast<const float*>((mtag[buf * KT + key] & kRawTag) ? a.raw : a.kv);
            v = *reinterpret_cast<const float4*>(src + (int64_t)row * D + d);
          }
        }
        stg[i][0] = v;
      } else {
        constexpr int DG = D / 8;
        const int k4 = u & (KT / 4 - 1);          // key group fastest: V^T writes spread over banks
        const int d = (u / (KT / 4)) * 8;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint4 v = make_uint4(0, 0, 0, 0);
          if (u < UNITS) {
            const int key = k4 * 4 + j;
            const int row = mrow[buf * KT + key];
            if (row >= 0) {
              if (mtag[buf * KT + key] & kRawTag)
                v = load_key8_bf16<CSA_BF16>(a.raw, nullptr, nullptr, row, d, D);
              else
                v = load_key8_bf16<KVF>(a.kv, a.kv_scale, a.kv_rope, row, d, D);
            }
          }
          stg[i][j] = v;
        }
      }
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * nthreads;
      if (u >= UNITS) continue;
      if constexpr (F32C) {
        constexpr int UPR = D / 4;
        const int key = u / UPR;
        const int d = (u - key * UPR) * 4;
        *reinterpret_cast<float4*>(klds + key * KSTR + d) = stg[i][0];
      } else {
        constexpr int DG = D / 8;
        const int k4 = u & (KT / 4 - 1);          // key group fastest: V^T writes spread over banks
        const int d = (u / (KT / 4)) * 8;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<uint4*>(klds + (k4 * 4 + j) * KSTR + d) = stg[i][j];
        // transpose 4 keys x 8 dims into V^T rows (4 keys = 8 bytes per dim)
        const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&stg[i][0]);
        const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&stg[i][1]);
        const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&stg[i][2]);
        const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&stg[i][3]);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          uint2 lo, hi;   // dims d+2p (low halves) and d+2p+1 (high halves)
          lo.x = (w0[p] & 0xffffu) | (w1[p] << 16);
          lo.y = (w2[p] & 0xffffu) | (w3[p] << 16);
          hi.x = (w0[p] >> 16) | (w1[p] & 0xffff0000u);
          hi.y = (w2[p] >> 16) | (w3[p] & 0xffff0000u);
          *reinterpret_cast<uint2*>(vt + (d + 2 * p) * VSTR + k4 * 4) = lo;
          *reinterpret_cast<uint2*>(vt + (d + 2 * p + 1) * VSTR + k4 * 4) = hi;
        }
      }
    }
  };

  // without prefetch: every thread loads and stores units tid, tid+nthreads, ...
  auto stage_direct = [&](int buf) {
    for (int u0 = 0; u0 < UNITS; u0 += nthreads) {
      const int u = u0 + tid;
      if (u >= UNITS) break;
      if constexpr (F32C) {
        constexpr int UPR = D / 4;
        const int key = u / UPR;
        const int d = (u - key * UPR) * 4;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        const int row = mrow[buf * KT + key];
        if (row >= 0) {
          const float* src = static_cast<const float*>((mtag[buf * KT + key] & kRawTag) ? a.raw : a.kv);
          v = *reinterpret_cast<const float4*>(src + (int64_t)row * D + d);
        }
        *reinterpret_cast<float4*>(klds + key * KSTR + d) = v;
      } else {
        constexpr int DG = D / 8;
        const int k4 = u & (KT / 4 - 1);          // key group fastest: V^T writes spread over banks
        const int d = (u / (KT / 4)) * 8;
        uint4 v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = k4 * 4 + j;
          const int row = mrow[buf * KT + key];
          v[j] = make_uint4(0, 0, 0, 0);
          if (row >= 0) {
            if (mtag[buf * KT + key] & kRawTag)
              v[j] = load_key8_bf16<CSA_BF16>(a.raw, nullptr, nullptr, row, d, D);
            else
              v[j] = load_key8_bf16<KVF>(a.kv, a.kv_scale, a.kv_rope, row, d, D);
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<uint4*>(klds + (k4 * 4 + j) * KSTR + d) = v[j];
        const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&v[0]);
        const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&v[1]);
        const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&v[2]);
        const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&v[3]);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          uint2 lo, hi;
          lo.x = (w0[p] & 0xffffu) | (w1[p] << 16);
          lo.y = (w2[p] & 0xffffu) | (w3[p] << 16);
          hi.x = (w0[p] >> 16) | (w1[p] & 0xffff0000u);
          hi.y = (w2[p] >> 16) | (w3[p] & 0xffff0000u);
          *reinterpret_cast<uint2*>(vt + (d + 2 * p) * VSTR + k4 * 4) = lo;
          *reinterpret_cast<uint2*>(vt + (d + 2 * p + 1) * VSTR + k4 * 4) = hi;
        }
      }
    }
  };

  // ---- key loop: prologue resolves (and, prefetching, loads) the first tile
  const int ntiles = (g.key_hi - g.key_lo + KT - 1) / KT;
  if (ntiles > 0) {
    meta_tile(g.key_lo, 0);
    __syncthreads();
    if constexpr (PREF) load_tile(0);
  }
  for (int tile = 0; tile < ntiles; ++tile) {
    const int buf = tile & 1;
    const int kbase = g.key_lo + tile * KT;
    __syncthreads();                 // previous tile fully consumed
    if constexpr (PREF) store_tile();
    else stage_direct(buf);
    if (tile + 1 < ntiles) meta_tile(kbase + KT, buf ^ 1);
    __syncthreads();                 // tile in LDS, next tile's sources resolved
    if constexpr (PREF) {
      if (tile + 1 < ntiles) load_tile(buf ^ 1);   // in flight during the compute below
    }

    // ---- logits S^T = K Q^T (partial over this wave's dims)
    f32x16_t acc_s = f32x16_t{};
    if constexpr (F32C) {
      const float* kp = klds + ql * KSTR + d0 + half;
#pragma unroll
      for (int c = 0; c < QC; ++c)
        acc_s = __builtin_amdgcn_mfma_f32_32x32x2f32(kp[2 * c], qreg[c], acc_s, 0, 0, 0);
    } else {
      const uint16_t* kp = klds + ql * KSTR + d0 + half * 8;
#pragma unroll
      for (int c = 0; c < QC; ++c) {
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(kp + 16 * c));
        acc_s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qreg[c], acc_s, 0, 0, 0);
      }
    }
    if constexpr (DSPLIT > 1) {
      float* mine = sx + ((rb * DSPLIT + dpart) * 64 + lane) * 16;
#pragma unroll
      for (int i = 0; i < 16; i += 4)
        *reinterpret_cast<float4*>(mine + i) = make_float4(acc_s[i], acc_s[i + 1], acc_s[i + 2], acc_s[i + 3]);
      __syncthreads();
      acc_s = f32x16_t{};
#pragma unroll
      for (int p = 0; p < DSPLIT; ++p) {
        const float* part = sx + ((rb * DSPLIT + p) * 64 + lane) * 16;
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
          const float4 v = *reinterpret_cast<const float4*>(part + i);
          acc_s[i] += v.x; acc_s[i + 1] += v.y; acc_s[i + 2] += v.z; acc_s[i + 3] += v.w;
        }
      }
    }

    // ---- mask (skipped when every key of the tile is valid for every row).
    // The logits are copied out of the matrix-core result before any lane is
    // masked: masking the result vector in place miscompiled (rows kept keys
    // they had masked).
    float s[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = acc_s[i];
    if (!mfull[buf]) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 8 * (i >> 2) + 4 * half + (i & 3);
        const int tg = mtag[buf * KT + key];
        bool ok;
        if (tg < 0) ok = false;
        else if (tg & kRawTag) {
          const int rel = tg & (kRawTag - 1);
          ok = rel > g_row && rel <= g_row + a.window;
        } else if (SPARSE) ok = tg == g_row;
        else ok = tg < nvis_row;
        s[i] = ok ? s[i] : -INFINITY;
      }
    }

    // ---- online softmax (base 2, stale maximum)
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[i]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32)) * a.scale_log2;
    const bool raise = tmax > m_run + kStale || (m_run == -INFINITY && tmax != -INFINITY);
    if (__any(raise)) {
      const float m_new = raise ? tmax : m_run;
      const float alpha = m_new == m_run ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc_o[db][i] *= alpha;
      m_run = m_new;
    }
    const float nm = m_run == -INFINITY ? 0.0f : -m_run;
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(s[i], a.scale_log2, nm));
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) psum += p[i];
    l_run += psum;

    // ---- O^T += V^T P^T
    if constexpr (F32C) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const float* vp = klds + d0 + db * 32 + ql;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = 8 * (i >> 2) + 4 * half + (i & 3);
          acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vp[key * KSTR], p[i], acc_o[db], 0, 0, 0);
        }
      }
    } else {
      bf16x8_t pb[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        uint4 u;
        u.x = pack_bf16x2(p[8 * c + 0], p[8 * c + 1]);
        u.y = pack_bf16x2(p[8 * c + 2], p[8 * c + 3]);
        u.z = pack_bf16x2(p[8 * c + 4], p[8 * c + 5]);
        u.w = pack_bf16x2(p[8 * c + 6], p[8 * c + 7]);
        pb[c] = __builtin_bit_cast(bf16x8_t, u);
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const uint16_t* vp = vt + (d0 + db * 32 + ql) * VSTR + 4 * half;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          uint4 u;
          const uint2 x0 = *reinterpret_cast<const uint2*>(vp + 16 * c);
          const uint2 x1 = *reinterpret_cast<const uint2*>(vp + 16 * c + 8);
          u.x = x0.x; u.y = x0.y; u.z = x1.x; u.w = x1.y;
          acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, u),
                                                               pb[c], acc_o[db], 0, 0, 0);
        }
      }
    }
  }

  // ---- epilogue
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (!row_live) return;
  const float lse_v = l_tot > 0.0f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  const int64_t rows_total = a.n_q * a.H;
  float* lse_dst = OUTM == 2 ? a.ws_lse + split * rows_total : a.lse;
  if (lse_dst != nullptr && half == 0 && dpart == 0) lse_dst[qrow_index] = lse_v;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = d0 + db * 32 + 8 * r4 + 4 * half;
      const float o0 = acc_o[db][4 * r4 + 0] * inv, o1 = acc_o[db][4 * r4 + 1] * inv;
      const float o2 = acc_o[db][4 * r4 + 2] * inv, o3 = acc_o[db][4 * r4 + 3] * inv;
      if constexpr (OUTM == 1) {
        uint2 u;
        u.x = pack_bf16x2(o0, o1);
        u.y = pack_bf16x2(o2, o3);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + qrow_index * D + d) = u;
      } else {
        float* dst = OUTM == 2 ? a.ws_o + (split * rows_total + qrow_index) * D + d
                               : static_cast<float*>(a.out) + qrow_index * D + d;
        *reinterpret_cast<float4*>(dst) = make_float4(o0, o1, o2, o3);
      }
    }
  }
}

template <int D, bool F32C, int DSPLIT>
size_t attn_smem(int nrb);

// the same kernel without register prefetch (fewer than 256 threads)
template <int D, bool F32C, int KVF, bool SPARSE, int DSPLIT, int OUTM>
csa_status launch_attn_np(const AttnArgs& a, hipStream_t stream) {
  const size_t smem = attn_smem<D, F32C, DSPLIT>(a.nrb);
  const int threads = a.nrb * DSPLIT * 64;
  const int64_t nblk = (a.n_q + a.tok - 1) / a.tok;
  auto kern = attn_kernel<D, F32C, KVF, SPARSE, DSPLIT, OUTM, false>;
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (smem > 64 * 1024 && attr != hipSuccess)
    return csa_host::fail(CSA_ERR_HIP, "csa_sparse_mqa_attn: cannot reserve %zu B of LDS", smem);
  const unsigned gy = a.split_keys > 0 ? (unsigned)a.max_splits : 1u;
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk, gy), dim3(threads), smem, stream, a);
  return csa_host::check_launch("csa_sparse_mqa_attn");
}

template <int D, bool F32C, int DSPLIT>
size_t attn_smem(int nrb) {
  constexpr int KSTR = F32C ? D + 4 : D + 8;
  const size_t kbytes = (size_t)KT * KSTR * (F32C ? 4 : 2);
  const size_t vbytes = F32C ? 0 : (size_t)D * (KT + 4) * 2;
  const size_t meta = (4 * KT + 4) * 4;
  const size_t sxbytes = DSPLIT > 1 ? (size_t)nrb * DSPLIT * 64 * 16 * 4 : 0;
  return kbytes + vbytes + meta + sxbytes;
}

template <int D, bool F32C, int KVF, bool SPARSE, int DSPLIT, int OUTM>
csa_status launch_attn(const AttnArgs& a, hipStream_t stream) {
  const size_t smem = attn_smem<D, F32C, DSPLIT>(a.nrb);
  const int threads = a.nrb * DSPLIT * 64;
  const int64_t nblk = (a.n_q + a.tok - 1) / a.tok;
  if (nblk > 0x7fffffff) return csa_host::fail(CSA_ERR_INVALID_ARGUMENT, "attn: too many queries");
  // register prefetch of the next tile only where the registers allow it
  constexpr bool kPref = D == 128 && !F32C;
  if (kPref && threads < 256) return launch_attn_np<D, F32C, KVF, SPARSE, DSPLIT, OUTM>(a, stream);
  auto kern = attn_kernel<D, F32C, KVF, SPARSE, DSPLIT, OUTM, kPref>;
  // the kernel's LDS ceiling is raised once per instantiation, to the most any
  // launch of it can ask for (so no attribute call happens inside a captured graph)
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (smem > 64 * 1024 && attr != hipSuccess)
    return csa_host::fail(CSA_ERR_HIP, "csa_sparse_mqa_attn: cannot reserve %zu B of LDS", smem);
  const unsigned gy = a.split_keys > 0 ? (unsigned)a.max_splits : 1u;
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk, gy), dim3(threads), smem, stream, a);
  return csa_host::check_launch("csa_sparse_mqa_attn");
}

template <int D, bool F32C, int KVF, int DSPLIT>
csa_status launch_mode(const AttnArgs& a, bool sparse, int outm, hipStream_t s) {
  if (sparse) {
    if (outm == 0) return launch_attn<D, F32C, KVF, true, DSPLIT, 0>(a, s);
    if (outm == 1) return launch_attn<D, F32C, KVF, true, DSPLIT, 1>(a, s);
    return launch_attn<D, F32C, KVF, true, DSPLIT, 2>(a, s);
  }
  if (outm == 0) return launch_attn<D, F32C, KVF, false, DSPLIT, 0>(a, s);
  if (outm == 1) return launch_attn<D, F32C, KVF, false, DSPLIT, 1>(a, s);
  return launch_attn<D, F32C, KVF, false, DSPLIT, 2>(a, s);
}

int max_splits_for(int64_t max_keys, int split_keys) {
  if (split_keys <= 0) return 1;
  const int64_t chunk = ((int64_t)split_keys + KT - 1) / KT * KT;
  int64_t n = (max_keys + chunk - 1) / chunk;
  if (n < 1) n = 1;
  return n > kMaxSplits ? kMaxSplits : (int)n;
}

}  // namespace

using namespace csa_host;

extern "C" size_t csa_attn_workspace_size(int64_t n_q, int32_t n_heads, int32_t dim,
                                          int64_t max_keys, int32_t split_keys) {
  if (split_keys <= 0 || n_q <= 0 || n_heads <= 0 || dim <= 0 || max_keys < 0) return 0;
  const int ns = max_splits_for(max_keys, split_keys);
  const size_t rows = (size_t)n_q * n_heads;
  return (size_t)ns * rows * ((size_t)dim + 1) * 4 + (size_t)n_q * 4 + 256;
}

extern "C" csa_status csa_sparse_mqa_attn(const csa_tensor* q, int32_t n_heads,
                                          const csa_tensor* kv, const int32_t* idx, int32_t k,
                                          const csa_tensor* raw, int32_t window,
                                          const csa_batch* batch, int32_t m, float scale,
                                          void* out, int32_t out_fmt, float* lse,
                                          int32_t split_keys, void* workspace,
                                          size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  if (batch == nullptr || q == nullptr || !fmt_valid_tensor(q))
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_sparse_mqa_attn: bad q or batch");
  if (batch->n_q < 0 || batch->n_req < 1 || batch->q_off == nullptr || batch->q_pos == nullptr)
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_sparse_mqa_attn: bad batch descriptor");
  if (batch->n_q == 0) return CSA_OK;
  const int D = q->dim;
  const int H = n_heads;
  if (H <= 0 || q->rows != batch->n_q * H)
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_sparse_mqa_attn: q rows must be n_q * n_heads");
  if (!(H % 32 == 0 || H == 16 || H == 8))
    return fail(CSA_ERR_UNSUPPORTED, "csa_sparse_mqa_attn: n_heads must be a multiple of 32, 16 or 8");
  if (H > 128) return fail(CSA_ERR_UNSUPPORTED, "csa_sparse_mqa_attn: at most 128 heads");
  if (out == nullptr) return fail(CSA_ERR_INVALID_ARGUMENT, "csa_sparse_mqa_attn: null out");
  if (out_fmt != CSA_F32 && out_fmt != CSA_BF16)
    return fail(CSA_ERR_UNSUPPORTED, "csa_sparse_mqa_attn: out must be F32 or BF16");
  if (m < 1) return fail(CSA_ERR_INVALID_ARGUMENT, "csa_sparse_mqa_attn: m must be >= 1");
  if (!(scale > 0.0f)) return fail(CSA_ERR_INVALID_ARGUMENT, "csa_sparse_mqa_attn: scale must be > 0");
  const bool has_kv = kv != nullptr && kv->rows > 0;
  const bool has_raw = raw != nullptr && raw->rows > 0 && window > 0;
  if (has_kv) {
    if (!fmt_valid_tensor(kv) || kv->dim != D)
      return fail(CSA_ERR_INVALID_ARGUMENT, "csa_sparse_mqa_attn: bad kv tensor");
    if (batch->kv_off == nullptr)
      return fail(CSA_ERR_INVALID_ARGUMENT, "csa_sparse_mqa_attn: kv given without kv_off");
    if (kv->rows > 0x7fffffff)
      return fail(CSA_ERR_UNSUPPORTED, "csa_sparse_mqa_attn: more than 2^31 entries");
  }
  if (has_raw) {
    if (!fmt_valid_tensor(raw) || raw->dim != D || raw->fmt != q->fmt)
      return fail(CSA_ERR_INVALID_ARGUMENT, "csa_sparse_mqa_attn: raw must match q's format and dim");
    if (batch->raw_off == nullptr || batch->raw_pos == nullptr)
      return fail(CSA_ERR_INVALID_ARGUMENT, "csa_sparse_mqa_attn: raw given without raw_off/raw_pos");
    if (window > (1 << 20))
      return fail(CSA_ERR_UNSUPPORTED, "csa_sparse_mqa_attn: window too large");
    if (raw->rows > 0x7fffffff)
      return fail(CSA_ERR_UNSUPPORTED, "csa_sparse_mqa_attn: more than 2^31 raw rows");
  }
  if (window < 0) return fail(CSA_ERR_INVALID_ARGUMENT, "csa_sparse_mqa_attn: negative window");
  const bool sparse = idx != nullptr;
  if (sparse && has_kv && (k < 1 || k > 4096))
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_sparse_mqa_attn: need 1 <= k <= 4096");
  if (split_keys < 0) return fail(CSA_ERR_INVALID_ARGUMENT, "csa_sparse_mqa_attn: split_keys < 0");

  AttnArgs a{};
  a.q = q->data;
  a.H = H;
  a.n_q = batch->n_q;
  a.kv = has_kv ? kv->data : nullptr;
  a.kv_scale = has_kv ? static_cast<const uint8_t*>(kv->scale) : nullptr;
  a.kv_rope = has_kv ? static_cast<const uint16_t*>(kv->rope) : nullptr;
  a.idx = sparse ? idx : nullptr;
  a.k = sparse ? k : 0;
  a.raw = has_raw ? raw->data : nullptr;
  a.window = has_raw ? window : 0;
  a.b = BatchDev{batch->n_req, batch->q_off, batch->q_pos, has_kv ? batch->kv_off : nullptr,
                 has_raw ? batch->raw_off : nullptr, has_raw ? batch->raw_pos : nullptr,
                 has_kv ? kv->rows : 0, has_raw ? raw->rows : 0};
  a.m = m;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out = out;
  a.lse = lse;

  const bool f32c = q->fmt == CSA_F32;
  if (f32c) {
    if ((has_kv && kv->fmt != CSA_F32) || D != 128)
      return fail(CSA_ERR_UNSUPPORTED, "csa_sparse_mqa_attn: fp32 path needs F32 kv and D = 128");
  } else if (q->fmt == CSA_BF16) {
    if (has_kv && kv->fmt != CSA_BF16 && kv->fmt != CSA_FP8_MIXED)
      return fail(CSA_ERR_UNSUPPORTED, "csa_sparse_mqa_attn: bf16 path needs BF16 or FP8_MIXED kv");
    if (D != 128 && D != 512)
      return fail(CSA_ERR_UNSUPPORTED, "csa_sparse_mqa_attn: D must be 128 or 512");
    if (has_kv && kv->fmt == CSA_FP8_MIXED && D != 512)
      return fail(CSA_ERR_UNSUPPORTED, "csa_sparse_mqa_attn: FP8_MIXED kv needs D = 512");
  } else {
    return fail(CSA_ERR_UNSUPPORTED, "csa_sparse_mqa_attn: q must be F32 or BF16");
  }

  // rows per workgroup: D = 128 packs several tokens into 128 rows (when one
  // request and no split); otherwise one token's H rows (at least 32)
  const bool split = split_keys > 0;
  int rows;
  if (D == 128 && !split && batch->n_req == 1) rows = H > 128 ? H : 128;
  else rows = H < 32 ? 32 : H;
  a.tok = rows / H > 0 ? rows / H : 1;
  a.nrb = rows / 32;
  if (a.tok > 1 && batch->n_req > 1)
    return fail(CSA_ERR_UNSUPPORTED, "csa_sparse_mqa_attn: fewer than 32 heads needs a single request");
  if (split && a.tok > 1)
    return fail(CSA_ERR_UNSUPPORTED, "csa_sparse_mqa_attn: split-K needs at least 32 heads");
  int outm = out_fmt == CSA_BF16 ? 1 : 0;
  if (split) {
    const int64_t max_keys =
        (has_kv ? (sparse ? (int64_t)k : batch->max_kv) : 0) + (has_raw ? window : 0);
    a.split_keys = split_keys;
    a.max_splits = max_splits_for(max_keys, split_keys);
    const size_t need = csa_attn_workspace_size(batch->n_q, H, D, max_keys, split_keys);
    if (workspace == nullptr || workspace_bytes < need)
      return fail(CSA_ERR_WORKSPACE, "csa_sparse_mqa_attn: split-K needs %zu workspace bytes", need);
    const size_t rows_total = (size_t)batch->n_q * H;
    char* ws = static_cast<char*>(workspace);
    a.ws_o = reinterpret_cast<float*>(ws);
    a.ws_lse = reinterpret_cast<float*>(ws + (size_t)a.max_splits * rows_total * D * 4);
    a.ws_cnt = reinterpret_cast<int*>(ws + (size_t)a.max_splits * rows_total * (D + 1) * 4);
    outm = 2;
  }
  const int kvf = has_kv ? kv->fmt : (f32c ? CSA_F32 : CSA_BF16);
  csa_status st;
  if (f32c) st = launch_mode<128, true, CSA_F32, 1>(a, sparse, outm, stream);
  else if (D == 128) st = launch_mode<128, false, CSA_BF16, 1>(a, sparse, outm, stream);
  else if (kvf == CSA_FP8_MIXED) st = launch_mode<512, false, CSA_FP8_MIXED, 2>(a, sparse, outm, stream);
  else st = launch_mode<512, false, CSA_BF16, 2>(a, sparse, outm, stream);
  if (st != CSA_OK || !split) return st;
  // combine the split partials of every query row
  const size_t rows_total = (size_t)batch->n_q * H;
  return launch_lse_merge(a.ws_o, a.ws_lse, (int64_t)rows_total * D, (int64_t)rows_total,
                          a.max_splits, a.ws_cnt, H, (int64_t)rows_total, D, out, out_fmt, lse,
                          stream);
}
