// Shared-KV multi-query attention over compressed entries (selected by top-k
// for CSA, all visible for HCA) together with a sliding window of raw tokens,
// one softmax over the union (page "DeepSeek V4 深度解析", section 2: CSA step 3
// and the HCA paragraph).
//
// Work split.  A workgroup owns TOK consecutive query tokens of one request,
// i.e. TOK*H query rows (heads stacked, since all heads share the keys).  The
// rows form 32-row blocks; each block is handled by DSPLIT waves, each wave
// owning D/DSPLIT of the head dimension (partial logits are summed through
// LDS in a fixed order).  Keys are streamed in tiles of 32, staged once into
// LDS as bf16 rows (FP8_MIXED rows dequantised on the way, exactly: the
// scales are powers of two); since key = value, the same tile is the operand
// of both products, read row-wise for the logits and through transposing LDS
// reads for the values.  The source rows of a tile are resolved once per key,
// ahead of the tile, together with one 32-bit mask per query token of the keys
// that token may see (causal entries, its own selection, its window), so
// masking a logit is one bit test.  With enough waves the global loads of a
// later tile are in flight while a tile is computed: D = 128 keeps two key
// buffers in LDS (one barrier per tile), D = 512 decode one.
//
// Split-K (decode).  With split_keys > 0 a query's key list is cut into
// parts of about split_keys keys (split_chunk) handled by a persistent grid
// of workgroups; each writes a normalised partial output and
// its log-sum-exp to the workspace, and a combine pass merges a query's parts
// in order (the same merge as csa_swa_merge).  The parts follow from the
// query's own key count and split_keys alone, so a request's parts, and the
// bits of its result, do not depend on the other requests of the batch.
// Selected keys number at most k + window per query, so the work items are
// (query, split) pairs indexed statically (a query with fewer keys leaves its
// last parts empty); all visible entries vary per request, so a plan kernel
// reads the key counts and lists the items.
//
// Per tile and wave (bf16):
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
// lane and instruction, so V is read straight from a padded K layout).
#include <type_traits>

#include "attn_common.h"
#include "common.h"
#include "merge.h"

using namespace csa;
using namespace csa_attn;

namespace {

// Split-K work list.  The parts of every query (split_parts), their prefix
// sums and the query of every item, so the attention grid visits only real
// items; the geometry of every query is recorded once for the items to load.
template <bool SPARSE>
__global__ __launch_bounds__(1024) void attn_split_plan(AttnArgs a) {
  __shared__ int wsum[16];
  __shared__ int carry;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int64_t q0 = 0; q0 < a.n_q; q0 += 1024) {
    const int64_t q = q0 + tid;
    int ns = 0;
    if (q < a.n_q) {
      const Geo g = make_geo<SPARSE>(a, q);
      store_geo(a.ws_geo + q * 4, g);
      ns = split_parts(g.nkeys, a.split_keys);
      if (ns > a.max_splits) ns = a.max_splits;   // (excluded by the host's sizing)
      a.ws_cnt[q] = ns;
    }
    int x = ns;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    __syncthreads();
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int before = carry;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const int start = before + x - ns;
    if (q < a.n_q) {
      a.ws_start[q] = start;
      for (int i = 0; i < ns; ++i) a.ws_item_q[start + i] = (int)q;
    }
    __syncthreads();
    if (tid == 1023) carry = start + ns;
    __syncthreads();
  }
  if (tid == 0) a.ws_start[a.n_q] = carry;
}


template <int D, bool F32C, int KVF, bool SPARSE, int DSPLIT, int OUTM, bool PREF>
__device__ __forceinline__ void attn_body(const AttnArgs& a) {
  constexpr int DW = D / DSPLIT;                 // dims per wave
  constexpr int KSTR = D + 4;                    // fp32 K-layout row stride (elements)
  // staging units: bf16 = one key x 16 dims, fp32 = one key x 4 dims
  constexpr int UPR = F32C ? D / 4 : D / 16;     // units per key row
  constexpr int UNITS = KT * UPR;
  // prefetching variants run with at least PMIN threads
  constexpr int PMIN = D == 512 ? 512 : 256;
  constexpr int UPT = PREF ? (UNITS + PMIN - 1) / PMIN : 1;
  constexpr size_t KBYTES = F32C ? (size_t)KT * KSTR * 4 : (size_t)KT * D * 2;

  // double-buffered key tiles (at least four waves)
  constexpr bool DBUF = PREF;
  constexpr int NKB = DBUF ? 2 : 1;

  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* kb = smem;                                        // [NKB] key tiles
  // bf16 keys: the metadata also holds each key's row address
  constexpr bool ADDR = !F32C && KVF != CSA_FP8_MIXED;
  const uint16_t** maddr = reinterpret_cast<const uint16_t**>(smem + NKB * KBYTES);  // [kMetaSlots][KT]
  int* mrow = reinterpret_cast<int*>(smem + NKB * KBYTES + (ADDR ? kMetaSlots * KT * 8 : 0));  // [kMetaSlots][KT] source rows
  uint32_t* mword = reinterpret_cast<uint32_t*>(mrow + kMetaSlots * KT);  // [kMetaSlots][kTokMax] key bits
  int* mfull = reinterpret_cast<int*>(mword + kMetaSlots * kTokMax);      // [kMetaSlots]
  float* sx = reinterpret_cast<float*>(mfull + kMetaSlots); // [nrb][DSPLIT][4][64] float4 partial logits

  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int ql = lane & 31;
  const int rb = wave / DSPLIT;
  const int dpart = wave - rb * DSPLIT;
  const int d0 = dpart * DW;

  // ---- work items.  Without split-K a workgroup owns one token group (x)
  // of one head group; with split-K the grid is persistent: workgroup x takes
  // items x, x + gridDim.x, ... of the work list, for head group y.
  // (split-K is exactly the partial-output instantiation)
  constexpr bool splitk = OUTM == 2;
  const unsigned wg = blockIdx.x;
  const int hgrp = splitk ? (int)blockIdx.y : (int)(wg % (unsigned)a.ngroups);
  const bool fixed = splitk && a.static_chunk > 0;
  const int n_items = splitk ? (fixed ? (int)a.n_q * a.static_splits : a.ws_start[a.n_q]) : 1;
  for (int item = splitk ? (int)blockIdx.x : 0; item < n_items; item += splitk ? (int)gridDim.x : 1) {
  int64_t q_first;
  int split = 0;
  if (fixed) {
    q_first = item / a.static_splits;
    split = item - (int)q_first * a.static_splits;
  } else if (splitk) {
    q_first = a.ws_item_q[item];
    split = item - a.ws_start[q_first];
  } else {
    q_first = (int64_t)(wg / (unsigned)a.ngroups) * a.tok;
  }
  // ---- this lane's query row.  It follows from the group alone (its last
  // query is min(q_first + tok - 1, n_q - 1), as the geometry has it), so the
  // query loads are issued before the geometry's chain of metadata loads and
  // overlap it; a dead row loads row 0 and is zeroed by a select, so no load
  // waits behind a branch.
  const int64_t q_last = q_first + a.tok - 1 < a.n_q ? q_first + a.tok - 1 : a.n_q - 1;
  const int row_in_wg = rb * 32 + ql;
  const int g_row = row_in_wg / a.hg;
  const int h_row = hgrp * a.hg + (row_in_wg - g_row * a.hg);
  const int64_t q_row = q_first + g_row;
  const bool row_live = q_row <= q_last;
  const int64_t qrow_index = q_row * a.H + h_row;    // row of the q / out tensors
  const int64_t qrow_load = row_live ? qrow_index : 0;

  // queries (B operand), pre-loaded for the whole key loop
  constexpr int QC = F32C ? DW / 2 : DW / 16;
  using qreg_t = typename std::conditional<F32C, float, bf16x8_t>::type;
  qreg_t qreg[QC];
  if constexpr (F32C) {
    const float* qp = static_cast<const float*>(a.q) + qrow_load * D + d0 + half;
#pragma unroll
    for (int c = 0; c < QC; ++c) {
      const float v = qp[2 * c];
      qreg[c] = row_live ? v : 0.0f;
    }
  } else {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + qrow_load * D + d0 + half * 8;
#pragma unroll
    for (int c = 0; c < QC; ++c) {
      const uint4 v = *reinterpret_cast<const uint4*>(qp + 16 * c);
      qreg[c] = __builtin_bit_cast(bf16x8_t, row_live ? v : make_uint4(0, 0, 0, 0));
    }
  }

  Geo g = splitk && !fixed ? load_geo(a.ws_geo + q_first * 4, q_first) : make_geo<SPARSE>(a, q_first);
  if (splitk) {
    const int chunk = (int)split_chunk(g.nkeys, a.split_keys);
    g.key_lo = split * chunk;
    g.key_hi = g.key_lo + chunk < g.nkeys ? g.key_lo + chunk : g.nkeys;
    if (g.key_hi < g.key_lo) g.key_hi = g.key_lo;   // past this query's keys: an empty part
    lds_barrier();                 // LDS of the previous item fully consumed
  }

  constexpr int NDB = DW / 32;
  f32x16_t acc_o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc_o[i] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.0f;

  // wave 0 resolves a tile's source rows and, per query token, a 32-bit mask
  // of the keys valid for it (bit = key in tile)
  const int ntok = (int)(g.q_last - g.q_first + 1);
  // (done by wave `by`)
  auto meta_tile_by = [&](int kbase, int buf, int by) {
    if (wave == by) {
      int row = -1;
      int64_t lo = 1, hi = 0;
      if (lane < KT) key_meta<SPARSE>(a, g, kbase + lane, row, lo, hi);
      // a key without a source (past the range, or an unused selection slot)
      // reads a row that always exists and stays masked
      if (!F32C && row == -1) row = a.kv != nullptr ? 0 : -2;
      if (lane < KT) mrow[buf * KT + lane] = row;
      if constexpr (ADDR) {
        // rows are bf16 [.., D] in either tensor; -2 - r is raw row r
        const uint16_t* base = row >= 0 ? static_cast<const uint16_t*>(a.kv) + (int64_t)row * D
                                        : static_cast<const uint16_t*>(a.raw) + (int64_t)(-2 - row) * D;
        if (lane < KT) maddr[buf * KT + lane] = base;
      }
      bool full = true;
      for (int t = 0; t < a.tok; ++t) {
        const uint32_t w = (uint32_t)__ballot(t < ntok && t >= lo && t < hi);
        if (lane == 0) mword[buf * kTokMax + t] = w;
        full = full && (t >= ntok || w == 0xffffffffu);
      }
      if (lane == 0) mfull[buf] = full ? 1 : 0;
    }
  };
  auto meta_tile = [&](int kbase, int buf) { meta_tile_by(kbase, buf, 0); };

  // ---- staging: fp32 units are float4 of one key; bf16 units are 16 dims
  // of one key (32 bytes once in LDS), consecutive threads along a key row
  using stage_t = typename std::conditional<F32C, float4, uint4>::type;
  constexpr int SPU = F32C ? 1 : 2;               // stage registers per unit
  stage_t stg[UPT][SPU];
  bool sfp8[UPT];
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    sfp8[i] = false;
#pragma unroll
    for (int j = 0; j < SPU; ++j) stg[i][j] = stage_t{};
  }

  // loads one staging unit whose source row is `row`
  auto load_unit_row = [&](int row, int u, stage_t* v, bool& fp8) {
    const int key = u / UPR;
    if constexpr (F32C) {
      const int d = (u - key * UPR) * 4;
      fp8 = false;
      v[0] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (row != -1) {
        const float* src = static_cast<const float*>(row >= 0 ? a.kv : a.raw);
        const int r = row >= 0 ? row : -2 - row;
        v[0] = *reinterpret_cast<const float4*>(src + (int64_t)r * D + d);
      }
    } else {
      fp8 = load_slot<D, KVF>(a, row, (u - key * UPR) * 16, v[0], v[1]);
    }
  };
  auto load_unit = [&](int buf, int u, stage_t* v, bool& fp8) {
    load_unit_row(mrow[buf * KT + u / UPR], u, v, fp8);
  };
  // LDS destinations of a bf16 unit (tile-invariant for a given unit)
  auto unit_dst = [&](int u, lds_u8** dst) {
    const int key = u / UPR;
    const int j = (u - key * UPR) * 2;
    dst[0] = (lds_u8*)kb + swz_off<D>(key, j);
    dst[1] = (lds_u8*)kb + swz_off<D>(key, j + 1);
  };
  auto store_unit = [&](int u, const stage_t* v, bool fp8, lds_u8* const* dst, int kofs) {
    if constexpr (F32C) {
      const int key = u / UPR;
      const int d = (u - key * UPR) * 4;
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(kb + kofs) + key * KSTR + d) = v[0];
    } else {
      store_slot(dst, kofs, fp8, v[0], v[1]);
    }
  };
  // prefetching: each thread's units, and so their LDS destinations, are
  // the same every tile
  lds_u8* sdst[UPT][2];
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    sdst[i][0] = sdst[i][1] = nullptr;
    if constexpr (!F32C) {
      if (tid + i * nthreads < UNITS) unit_dst(tid + i * nthreads, sdst[i]);
    }
  }

  auto load_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * nthreads;
      if (u < UNITS) load_unit(buf, u, stg[i], sfp8[i]);
    }
  };
  // the same in two parts: source rows of this thread's units (LDS), then
  // the loads themselves
  // (for bf16 keys the row addresses instead of the rows)
  using src_t = typename std::conditional<ADDR, const uint16_t*, int>::type;
  auto tile_rows = [&](int buf, src_t* rows) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * nthreads;
      if constexpr (ADDR) rows[i] = maddr[buf * KT + (u < UNITS ? u / UPR : 0)];
      else rows[i] = u < UNITS ? mrow[buf * KT + u / UPR] : -1;
    }
  };
  auto load_tile_rows = [&](const src_t* rows) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * nthreads;
      if (u < UNITS) {
        if constexpr (ADDR) {
          // a pointer read back from LDS is generic: named global, the loads
          // stay global loads (a flat load would also count against the LDS
          // wait counter)
          typedef const __attribute__((address_space(1))) u32x4_t gu4;
          const gu4* p = (const gu4*)(uintptr_t)(rows[i] + (u % UPR) * 16);
          const u32x4_t v0 = p[0], v1 = p[1];
          stg[i][0] = make_uint4(v0[0], v0[1], v0[2], v0[3]);
          stg[i][1] = make_uint4(v1[0], v1[1], v1[2], v1[3]);
          sfp8[i] = false;
        } else {
          load_unit_row(rows[i], u, stg[i], sfp8[i]);
        }
      }
    }
  };
  auto store_tile = [&](int kofs) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * nthreads;
      if (u < UNITS) store_unit(u, stg[i], sfp8[i], sdst[i], kofs);
    }
  };
  // without prefetch: every thread stages units tid, tid+nthreads, ..., in
  // batches of SB whose loads are all issued before the first is stored
  constexpr int SB = (D == 512 && DSPLIT == 2) ? 1 : 4;   // D = 512 over two waves: no registers to spare
  auto stage_direct = [&](int buf) {
    for (int u0 = 0; u0 < UNITS; u0 += SB * nthreads) {
      stage_t v[SB][SPU] = {};
      bool fp8[SB] = {};
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        const int u = u0 + tid + i * nthreads;
        if (u < UNITS) load_unit(buf, u, v[i], fp8[i]);
      }
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        const int u = u0 + tid + i * nthreads;
        if (u < UNITS) {
          lds_u8* dst[2] = {nullptr, nullptr};
          if constexpr (!F32C) unit_dst(u, dst);
          store_unit(u, v[i], fp8[i], dst, 0);
        }
      }
    }
  };

  // Per-lane LDS byte offsets of the bf16 tile reads.  Logit operand: row ql,
  // chunk j = d0/8 + 2c + half; as d0/8 is a multiple of 16, the swizzled
  // chunk is 16*(j/16) + 2*((c%8) ^ (f/2)) + (half ^ f%2), f = f(ql).
  // Transposed value reads (see lds_read_tr16): row 16c + 8r + tk, chunk
  // 4*db' + tc (db' = d0/32 + db), swizzled to 16*(db'/4) + 4*((db'%4) ^ (tk%4))
  // + (tc ^ ((2r + tk/4) % 4)), plus the byte `sub` within it; the row terms
  // 16c and 8r and the term 16*(db'/4) are immediates.
  // The tables hold 32-bit LDS addresses with the tile's base included, so a
  // read is one instruction with an immediate offset (the base of dynamic LDS
  // is a link-time symbol the compiler cannot fold into an offset).
  lds_u8* qk_ptr[8];
  lds_u8* tr_ptr[2][4];
  {
    lds_u8* kbl = (lds_u8*)(kb);
    const int f = 4 * (ql & 3) + ((ql >> 2) & 3);
#pragma unroll
    for (int c8 = 0; c8 < 8; ++c8)
      qk_ptr[c8] = kbl + ql * (D * 2) + 32 * (c8 ^ (f >> 1)) + 16 * (half ^ (f & 1)) + (d0 >> 7) * 256;
    const int tg = lane >> 4, ts = lane & 15;
    const int tk = 4 * (tg >> 1) + (ts >> 2);
    const int tc = 2 * (tg & 1) + ((ts & 3) >> 1);
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int x = 0; x < 4; ++x)
        tr_ptr[r][x] = kbl + tk * (D * 2) + 16 * (tc ^ ((2 * r + (tk >> 2)) & 3)) + (ts & 1) * 8 +
                       (d0 >> 7) * 256 + 64 * (x ^ (tk & 3));
  }

  // The query registers are settled before the key loop: otherwise, inside
  // the loop, their loads cannot be told apart from the prefetch in flight and
  // every first use would wait for all outstanding loads.
#pragma unroll
  for (int c = 0; c < QC; ++c) asm volatile("" :: "v"(qreg[c]));

  // ---- logits of one tile, S^T = K Q^T (partial over this wave's dims and
  // summed over the waves of the row block); kofs = byte offset of the key
  // buffer
  // Keep the few per-lane offsets opaque to loop-invariant hoisting, which
  // would otherwise hold every derived address in a register of its own.
  auto launder_qk = [&]() {
    if constexpr (!F32C) {
#pragma unroll
      for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(qk_ptr[i]));
    }
  };
  auto launder_tr = [&]() {
    if constexpr (!F32C) {
#pragma unroll
      for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(tr_ptr[i >> 2][i & 3]));
    }
  };
  // bf16 operands of the two products: K chunk of logit instruction c, and
  // the V^T operand of value instruction c of dim block db
  auto read_k = [&](int c, int kofs) -> uint4 {
    return lds_read_b128(qk_ptr[c & 7] + (c >> 3) * 256 + kofs);
  };
  auto read_v = [&](int db, int c, int kofs) -> uint4 {
    const lds_u8* v0 = tr_ptr[0][db & 3] + (db >> 2) * 256 + kofs;
    const lds_u8* v1 = tr_ptr[1][db & 3] + (db >> 2) * 256 + kofs;
    const uint2 x0 = lds_read_tr16(v0 + 16 * c * (D * 2));
    const uint2 x1 = lds_read_tr16(v1 + (16 * c + 8) * (D * 2));
    return make_uint4(x0.x, x0.y, x1.x, x1.y);
  };

  auto tile_logits_with = [&](auto&& kget, int kofs) -> f32x16_t {
    f32x16_t acc_s = f32x16_t{};
    if constexpr (F32C) {
      const float* kp = reinterpret_cast<const float*>(kb + kofs) + ql * KSTR + d0 + half;
#pragma unroll
      for (int c = 0; c < QC; ++c)
        acc_s = __builtin_amdgcn_mfma_f32_32x32x2f32(kp[2 * c], qreg[c], acc_s, 0, 0, 0);
    } else {
#pragma unroll
      for (int c = 0; c < QC; ++c) {
        const uint4 k8 = kget(c);
        acc_s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, k8), qreg[c], acc_s,
                                                        0, 0, 0);
      }
    }
    if constexpr (DSPLIT > 1) {
      // [rb][wave part][register quad][lane] float4s: each access of a wave is
      // 1 KB of consecutive LDS, free of bank conflicts
      float4* mine = reinterpret_cast<float4*>(sx) + (rb * DSPLIT + dpart) * 4 * 64 + lane;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        mine[i * 64] = make_float4(acc_s[4 * i], acc_s[4 * i + 1], acc_s[4 * i + 2], acc_s[4 * i + 3]);
      lds_barrier();
      acc_s = f32x16_t{};
#pragma unroll
      for (int p = 0; p < DSPLIT; ++p) {
        const float4* part = reinterpret_cast<const float4*>(sx) + (rb * DSPLIT + p) * 4 * 64 + lane;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 v = part[i * 64];
          acc_s[4 * i] += v.x; acc_s[4 * i + 1] += v.y; acc_s[4 * i + 2] += v.z; acc_s[4 * i + 3] += v.w;
        }
      }
    }
    return acc_s;
  };
  auto tile_logits = [&](int kofs) -> f32x16_t {
    launder_qk();
    return tile_logits_with([&](int c) { return read_k(c, kofs); }, kofs);
  };

  // ---- mask, online softmax and O^T += V^T P^T for one tile whose logits are
  // acc_s; full = every key valid for every row, else mw holds this lane's
  // key bits.
  // vget(db, c) gives the V^T operand of value instruction c of dim block db.
  auto tile_softmax_pv_with = [&](const f32x16_t& acc_s, int full, uint32_t mw, auto&& vget, int kofs) {
    // mask (skipped when every key of the tile is valid for every row).  The
    // logits are copied out of the matrix-core result before any lane is
    // masked: masking the result vector in place miscompiled (rows kept keys
    // they had masked).
    float s[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = acc_s[i];
    if (!full) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        s[i] = ((mw >> (8 * (i >> 2) + (i & 3))) & 1u) ? s[i] : -INFINITY;
    }

    // online softmax (base 2, stale maximum)
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[i]);
    {
      // the other half of the wave holds the rest of each row: exchange
      // halves (lanes l and l ^ 32) without going through LDS
      const uint32_t u = __float_as_uint(tmax);
      const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
      tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * a.scale_log2;
    }
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

    // O^T += V^T P^T
    if constexpr (F32C) {
      float psum = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) psum += p[i];
      l_run += psum;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const float* vp = reinterpret_cast<const float*>(kb + kofs) + d0 + db * 32 + ql;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = 8 * (i >> 2) + 4 * half + (i & 3);
          acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vp[key * KSTR], p[i], acc_o[db], 0, 0, 0);
        }
      }
    } else {
      // contraction slot 8*half + q of instruction c holds key
      // 16c + 8*(q/4) + 4*half + q%4, the key of p[8c + q] in this lane
      bf16x8_t pb[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        uint4 u;
        u.x = pack_bf16x2_fast(p[8 * c + 0], p[8 * c + 1]);
        u.y = pack_bf16x2_fast(p[8 * c + 2], p[8 * c + 3]);
        u.z = pack_bf16x2_fast(p[8 * c + 4], p[8 * c + 5]);
        u.w = pack_bf16x2_fast(p[8 * c + 6], p[8 * c + 7]);
        pb[c] = __builtin_bit_cast(bf16x8_t, u);
      }
      // the row sum of the probabilities as rounded for the product (two per
      // dot-product instruction), so the normaliser sums the weights applied
      float psum = 0.0f;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint4 u = __builtin_bit_cast(uint4, pb[c]);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, w[j]),
                                                 __builtin_bit_cast(bf16x2_v, 0x3f803f80u), psum, false);
      }
      l_run += psum;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const uint4 u = vget(db, c);
          acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, u), pb[c],
                                                               acc_o[db], 0, 0, 0);
        }
      }
      // keep one instruction's V^T reads in flight ahead of each product
      // (left alone, the scheduler waits for every read right before its use)
      if constexpr (NDB == 4) {
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);   // LDS reads
#pragma unroll
        for (int i = 0; i < 6; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 1); // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
      }
    }
  };
  auto tile_softmax_pv = [&](const f32x16_t& acc_s, int full, uint32_t mw, int kofs) {
    launder_tr();
    tile_softmax_pv_with(acc_s, full, mw, [&](int db, int c) { return read_v(db, c, kofs); }, kofs);
  };

  // this lane's key bits of the tile in ring slot `slot`
  auto lane_mask = [&](int slot) -> uint32_t { return mword[slot * kTokMax + g_row] >> (4 * half); };

  const int ntiles = (g.key_hi - g.key_lo + KT - 1) / KT;
  if constexpr (DBUF) {
    // ---- key loop over two key buffers, one barrier per tile: during tile t
    // the workgroup stores tile t+1 (loaded during t-1) and loads tile t+2.
    // The sources of four tiles are resolved at a time, one tile per wave
    // (tiles t+4 .. t+7 during tile t, t a multiple of 4), so no wave carries
    // more than the others into a barrier; the metadata ring holds the eight
    // tiles t .. t+7.
    if (ntiles > 0) {
      if (wave < 4 && wave < ntiles) meta_tile_by(g.key_lo + wave * KT, wave, wave);
      lds_barrier();
      load_tile(0);
      store_tile(0);
      if (ntiles > 1) load_tile(1);
      lds_barrier();
    }
    int full_next = mfull[0];
    uint32_t mw_next = lane_mask(0);
    auto step = [&](int t, auto bsel) {
      constexpr int B = decltype(bsel)::value;   // buffer of tile t (= t mod 2)
      constexpr int KO = B * (int)KBYTES;
      constexpr int KS = (B ^ 1) * (int)KBYTES;
      const int full = full_next;
      const uint32_t mw = mw_next;
      const int s1 = (t + 1) & (kMetaSlots - 1);
      full_next = mfull[s1];
      mw_next = lane_mask(s1);
      src_t rows[UPT];
      tile_rows((t + 2) & (kMetaSlots - 1), rows);
      // the first key operands of this tile are in flight during the staging
      // (two: more cost the third wave per SIMD its registers)
      constexpr int KPRE = F32C ? 0 : 2;
      uint4 kr[KPRE > 0 ? KPRE : 1];
      __builtin_amdgcn_sched_barrier(0);
      launder_qk();
      if constexpr (!F32C) {
#pragma unroll
        for (int c = 0; c < KPRE; ++c) kr[c] = read_k(c, KO);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (t + 1 < ntiles) store_tile(KS);
      if (t + 2 < ntiles) load_tile_rows(rows);
      if ((t & 3) == 0 && wave < 4) {
        const int tt = t + 4 + wave;
        if (tt < ntiles) meta_tile_by(g.key_lo + tt * KT, tt & (kMetaSlots - 1), wave);
      }
      const f32x16_t sc = tile_logits_with([&](int c) { return c < KPRE ? kr[c] : read_k(c, KO); }, KO);
      tile_softmax_pv(sc, full, mw, KO);
      lds_barrier();
    };
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    for (int t = 0; t < ntiles; t += 2) {
      step(t, B0{});
      if (t + 1 >= ntiles) break;
      step(t + 1, B1{});
    }
  } else {
    // ---- key loop: prologue resolves (and, prefetching, loads) the first tile
    if (ntiles > 0) {
      meta_tile(g.key_lo, 0);
      lds_barrier();
      if constexpr (PREF) load_tile(0);
    }
    for (int tile = 0; tile < ntiles; ++tile) {
      const int buf = tile & 1;
      const int kbase = g.key_lo + tile * KT;
      lds_barrier();                 // previous tile fully consumed
      if constexpr (PREF) store_tile(0);
      else stage_direct(buf);
      if (tile + 1 < ntiles) meta_tile(kbase + KT, buf ^ 1);
      lds_barrier();                 // tile in LDS, next tile's sources resolved
      if constexpr (PREF) {
        if (tile + 1 < ntiles) load_tile(buf ^ 1);   // in flight during the compute below
      }
      tile_softmax_pv(tile_logits(0), mfull[buf], lane_mask(buf), 0);
    }
  }

  // ---- epilogue
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (row_live) {
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
        u.x = pack_bf16x2_fast(o0, o1);
        u.y = pack_bf16x2_fast(o2, o3);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + qrow_index * D + d) = u;
      } else {
        float* dst = OUTM == 2 ? a.ws_o + (split * rows_total + qrow_index) * D + d
                               : static_cast<float*>(a.out) + qrow_index * D + d;
        *reinterpret_cast<float4*>(dst) = make_float4(o0, o1, o2, o3);
      }
    }
  }
  }  // row_live
  }  // work items
}

template <int D, bool F32C, int KVF, bool SPARSE, int DSPLIT, int OUTM, bool PREF>
__global__ __launch_bounds__(512) void attn_kernel(AttnArgs a) {
  attn_body<D, F32C, KVF, SPARSE, DSPLIT, OUTM, PREF>(a);
}

// D = 128 with prefetch: registers held to three waves per SIMD, the
// occupancy its latency hiding relies on
template <int KVF, bool SPARSE, int OUTM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
void attn_kernel_d128(AttnArgs a) {
  attn_body<128, false, KVF, SPARSE, 1, OUTM, true>(a);
}

template <int D, bool F32C, int DSPLIT>
size_t attn_smem(int nrb, bool dbuf);

csa_status launch_plan(const AttnArgs& a, bool sparse, hipStream_t s) {
  if (sparse) hipLaunchKernelGGL(attn_split_plan<true>, dim3(1), dim3(1024), 0, s, a);
  else hipLaunchKernelGGL(attn_split_plan<false>, dim3(1), dim3(1024), 0, s, a);
  return csa_host::check_launch("csa_sparse_mqa_attn (split plan)");
}

// Workgroups of one launch: one per (token group, head group), or with split-K
// a persistent grid (as many as fit on the device at once, at most one per
// work item) times the head groups.
template <typename K>
dim3 attn_grid(const AttnArgs& a, K kern, int threads, size_t smem) {
  if (a.split_keys <= 0)
    return dim3((unsigned)((a.n_q + a.tok - 1) / a.tok * a.ngroups), 1u);
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, smem) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  int64_t n = (int64_t)cus * per_cu;
  const int64_t items = a.n_q * (int64_t)a.max_splits;
  if (n > items) n = items;
  return dim3((unsigned)n, (unsigned)a.ngroups);
}

// Launches one instantiation; with split-K the plan kernel runs first, its
// item target set to the persistent grid of this launch.
template <bool SPARSE, typename K>
csa_status launch_kernel(const AttnArgs& a0, K kern, int threads, size_t smem, hipStream_t stream) {
  AttnArgs a = a0;
  dim3 grid = attn_grid(a, kern, threads, smem);
  if (a.split_keys > 0 && SPARSE && a.static_keys > 0) {
    // selected keys: at most static_keys (k + window) per query, so every
    // query has the same splits of the fixed chunk and the items are indexed
    // statically
    // (a query with fewer keys has at most as many parts)
    a.static_chunk = (int)split_chunk(a.static_keys, a.split_keys);
    a.static_splits = split_parts_max(a.static_keys, a.split_keys);
    if (a.host_splits != nullptr) *a.host_splits = a.static_splits;
    const int64_t items = a.n_q * a.static_splits;
    if ((int64_t)grid.x > items) grid.x = (unsigned)items;
  } else if (a.split_keys > 0) {
    const csa_status st = launch_plan(a, SPARSE, stream);
    if (st != CSA_OK) return st;
  }
  hipLaunchKernelGGL(kern, grid, dim3(threads), smem, stream, a);
  return csa_host::check_launch("csa_sparse_mqa_attn");
}

// the same kernel without register prefetch (too few threads to share it)
template <int D, bool F32C, int KVF, bool SPARSE, int DSPLIT, int OUTM>
csa_status launch_attn_np(const AttnArgs& a, hipStream_t stream) {
  const size_t smem = attn_smem<D, F32C, DSPLIT>(a.nrb, false);
  const int threads = a.nrb * DSPLIT * 64;
  auto kern = attn_kernel<D, F32C, KVF, SPARSE, DSPLIT, OUTM, false>;
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (smem > 64 * 1024 && attr != hipSuccess)
    return csa_host::fail(CSA_ERR_HIP, "csa_sparse_mqa_attn: cannot reserve %zu B of LDS", smem);
  return launch_kernel<SPARSE>(a, kern, threads, smem, stream);
}

// LDS of one workgroup: key buffers (two when double-buffered), the metadata
// ring, and the partial-logit exchange when a row block spans several waves
template <int D, bool F32C, int DSPLIT>
size_t attn_smem(int nrb, bool dbuf) {
  const size_t kbytes = F32C ? (size_t)KT * (D + 4) * 4 : (size_t)KT * D * 2;
  const size_t meta = ((size_t)kMetaSlots * (KT + kTokMax + 1)) * 4 + (F32C ? 0 : (size_t)kMetaSlots * KT * 8);
  const size_t sxbytes = DSPLIT > 1 ? (size_t)nrb * DSPLIT * 64 * 16 * 4 : 0;
  return kbytes * (dbuf ? 2 : 1) + meta + sxbytes;
}

template <int D, bool F32C, int KVF, bool SPARSE, int DSPLIT, int OUTM>
csa_status launch_attn(const AttnArgs& a, hipStream_t stream) {
  const int threads = a.nrb * DSPLIT * 64;
  if ((a.n_q + a.tok - 1) / a.tok * a.ngroups > 0x7fffffff)
    return csa_host::fail(CSA_ERR_INVALID_ARGUMENT, "attn: too many queries");
  // register prefetch of the next tile (D = 128, bf16, or fp32 without
  // split-K, which would spill; D = 512 bf16 over four waves per row block),
  // with enough threads to share it; with one wave per row block,
  // double-buffered
  constexpr bool kPref = (D == 128 && (!F32C || OUTM != 2)) || (!F32C && DSPLIT == 4);
  if (kPref && threads < (D == 512 ? 512 : 256))
    return launch_attn_np<D, F32C, KVF, SPARSE, DSPLIT, OUTM>(a, stream);
  const size_t smem = attn_smem<D, F32C, DSPLIT>(a.nrb, kPref);
  auto kern = [] {
    if constexpr (D == 128 && !F32C && kPref && OUTM != 2) return attn_kernel_d128<KVF, SPARSE, OUTM>;
    else return attn_kernel<D, F32C, KVF, SPARSE, DSPLIT, OUTM, kPref>;
  }();
  // the kernel's LDS ceiling is raised once per instantiation, to the most any
  // launch of it can ask for (so no attribute call happens inside a captured graph)
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (smem > 64 * 1024 && attr != hipSuccess)
    return csa_host::fail(CSA_ERR_HIP, "csa_sparse_mqa_attn: cannot reserve %zu B of LDS", smem);
  return launch_kernel<SPARSE>(a, kern, threads, smem, stream);
}

// split-K only (partial outputs to the workspace)
template <int D, bool F32C, int KVF, int DSPLIT>
csa_status launch_split(const AttnArgs& a, bool sparse, hipStream_t s) {
  if (sparse) return launch_attn<D, F32C, KVF, true, DSPLIT, 2>(a, s);
  return launch_attn<D, F32C, KVF, false, DSPLIT, 2>(a, s);
}

// one pass per token group, final output (fp32 or bf16)
template <int D, bool F32C, int KVF, int DSPLIT>
csa_status launch_mode(const AttnArgs& a, bool sparse, int outm, hipStream_t s) {
  if (sparse) {
    if (outm == 0) return launch_attn<D, F32C, KVF, true, DSPLIT, 0>(a, s);
    return launch_attn<D, F32C, KVF, true, DSPLIT, 1>(a, s);
  }
  if (outm == 0) return launch_attn<D, F32C, KVF, false, DSPLIT, 0>(a, s);
  return launch_attn<D, F32C, KVF, false, DSPLIT, 1>(a, s);
}

// Most parts a query of at most max_keys keys is cut into.
int max_splits_for(int64_t max_keys, int split_keys) {
  if (split_keys <= 0) return 1;
  return split_parts_max(max_keys, split_keys);
}

}  // namespace

using namespace csa_host;

extern "C" size_t csa_attn_workspace_size(int64_t n_q, int32_t n_heads, int32_t dim,
                                          int64_t max_keys, int32_t split_keys) {
  if (split_keys <= 0 || n_q <= 0 || n_heads <= 0 || dim <= 0 || max_keys < 0) return 0;
  const int ns = max_splits_for(max_keys, split_keys);
  if (ns == 0) return 0;
  const size_t rows = (size_t)n_q * n_heads;
  // partial outputs and lse, then per query: split count, first item (+1),
  // the query of every item, and a 64-byte geometry record
  return (size_t)ns * rows * ((size_t)dim + 1) * 4 + ((size_t)n_q * (2 + (size_t)ns) + 2) * 4 + 16 +
         (size_t)n_q * 64 + 256;
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
    // (window rows are bf16 with fp8 queries)
    const int raw_fmt = q->fmt == CSA_FP8_MIXED ? (int)CSA_BF16 : (int)q->fmt;
    if (!fmt_valid_tensor(raw) || raw->dim != D || raw->fmt != raw_fmt)
      return fail(CSA_ERR_INVALID_ARGUMENT, "csa_sparse_mqa_attn: raw must match q's format and dim");
    if (batch->raw_off == nullptr || batch->raw_pos == nullptr)
      return fail(CSA_ERR_INVALID_ARGUMENT, "csa_sparse_mqa_attn: raw given without raw_off/raw_pos");
    if (batch->window_ring != 0 && batch->window_ring != 1)
      return fail(CSA_ERR_INVALID_ARGUMENT, "csa_sparse_mqa_attn: window_ring must be 0 or 1");
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
  int static_splits = 0;       // reported by a fixed split-K launch
  a.host_splits = &static_splits;
  a.q = q->data;
  a.q_scale = static_cast<const uint8_t*>(q->scale);
  a.q_rope = static_cast<const uint16_t*>(q->rope);
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
                 has_kv ? kv->rows : 0, has_raw ? raw->rows : 0, batch->window_ring};
  if (const csa_status st = batch_pages(batch, a.b, "csa_sparse_mqa_attn"); st != CSA_OK) return st;
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
  } else if (q->fmt == CSA_FP8_MIXED) {
    // fp8 queries: the 512-dim kernel only, over mixed fp8 entries (their
    // block scales are read with every tile, so the entries must be given)
    if (!has_kv || kv->fmt != CSA_FP8_MIXED)
      return fail(CSA_ERR_UNSUPPORTED, "csa_sparse_mqa_attn: fp8 queries need FP8_MIXED kv");
    if (H != 64 && H != 128)
      return fail(CSA_ERR_UNSUPPORTED, "csa_sparse_mqa_attn: fp8 queries need 64 or 128 heads");
  } else {
    return fail(CSA_ERR_UNSUPPORTED, "csa_sparse_mqa_attn: q must be F32, BF16 or FP8_MIXED");
  }

  // rows per workgroup: D = 128 packs several tokens into 128 rows (when one
  // request and no split), otherwise one token's H rows (at least 32).  D = 512
  // runs two waves per 32 rows (all heads of a token in one workgroup, so its
  // keys are staged once) or, split over keys (decode), four waves per 32 rows
  // on at most 64 heads (a head group), which leaves registers for prefetching
  const bool split = split_keys > 0;
  int rows;
  a.hg = H;
  if (D == 512 && split && H % 64 == 0) a.hg = 64;
  else if (D == 512 && split && H % 32 == 0) a.hg = 32;
  if (D == 128 && !split && batch->n_req == 1) rows = H > 128 ? H : 128;
  else rows = a.hg < 32 ? 32 : a.hg;
  a.ngroups = H / a.hg;
  a.tok = rows / a.hg > 0 ? rows / a.hg : 1;
  if (a.tok > kTokMax) return fail(CSA_ERR_UNSUPPORTED, "csa_sparse_mqa_attn: too many tokens per workgroup");
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
    a.ws_start = a.ws_cnt + batch->n_q;
    a.ws_item_q = a.ws_start + batch->n_q + 1;
    a.ws_chunk = a.ws_item_q + (size_t)batch->n_q * a.max_splits;
    const uintptr_t geo = reinterpret_cast<uintptr_t>(a.ws_chunk + 1);
    a.ws_geo = reinterpret_cast<int4*>((geo + 15) & ~(uintptr_t)15);
    if (sparse && a.tok == 1) a.static_keys = (int)max_keys;
    outm = 2;
  }
  const int kvf = has_kv ? kv->fmt : (f32c ? CSA_F32 : CSA_BF16);
  // D = 512 with 64 or 128 heads: one workgroup per token (or per part of its
  // keys with split-K), 16 heads per wave (attn512.hip).  Without a split a
  // token whose keys exceed its capacity takes the general kernel; with a
  // split the choice must not depend on the batch, so a part longer than
  // that capacity is refused instead.
  const int64_t tok_keys = (has_kv ? (sparse ? (int64_t)k : batch->max_kv) : 0) + (has_raw ? window : 0);
  const bool q8 = q->fmt == CSA_FP8_MIXED;
  const bool wide = D == 512 && !f32c && (H == 64 || H == 128);
  const int part_cap = q8 ? attn512_part_keys(128) : attn512_part_keys(H);
  if (wide && split && split_chunk_max(tok_keys, split_keys) > part_cap)
    return fail(CSA_ERR_UNSUPPORTED, "csa_sparse_mqa_attn: split parts of up to %lld keys exceed %d with %d heads",
                (long long)split_chunk_max(tok_keys, split_keys), part_cap, H);
  if (q8 && !split && !attn512_fits(tok_keys))
    return fail(CSA_ERR_UNSUPPORTED, "csa_sparse_mqa_attn: fp8 queries see at most 4096 keys each");
  const bool use512 = wide && (split || attn512_fits(tok_keys));
  // the 512-dim kernel keeps split partials in bf16 when the output is bf16
  a.part_bf16 = use512 && split && out_fmt == CSA_BF16 ? 1 : 0;
  csa_status st;
  if (use512) st = launch_attn512(a, kvf, sparse, outm, q8, stream);
  else if (f32c && split) st = launch_split<128, true, CSA_F32, 1>(a, sparse, stream);
  else if (f32c) st = launch_mode<128, true, CSA_F32, 1>(a, sparse, outm, stream);
  else if (D == 128 && split) st = launch_split<128, false, CSA_BF16, 1>(a, sparse, stream);
  else if (D == 128) st = launch_mode<128, false, CSA_BF16, 1>(a, sparse, outm, stream);
  else if (kvf == CSA_FP8_MIXED && split) st = launch_split<512, false, CSA_FP8_MIXED, 4>(a, sparse, stream);
  else if (kvf == CSA_FP8_MIXED) st = launch_mode<512, false, CSA_FP8_MIXED, 2>(a, sparse, outm, stream);
  else if (split) st = launch_split<512, false, CSA_BF16, 4>(a, sparse, stream);
  else st = launch_mode<512, false, CSA_BF16, 2>(a, sparse, outm, stream);
  if (st != CSA_OK || !split) return st;
  // combine the split partials of every query row: the parts each query
  // used (ws_cnt), or with a fixed split all of its parts, the empty ones
  // with lse = -inf
  const size_t rows_total = (size_t)batch->n_q * H;
  const bool fixed = !use512 && a.static_keys > 0;
  return launch_lse_merge(a.ws_o, a.ws_lse, (int64_t)rows_total * D, (int64_t)rows_total,
                          fixed ? static_splits : a.max_splits, fixed ? nullptr : a.ws_cnt, H,
                          (int64_t)rows_total, D, out, out_fmt, lse, a.part_bf16 != 0, stream);
}
