// Shared-KV multi-query attention over 512-dim entries (page "DeepSeek V4
// 深度解析", section 2: CSA step 3, the selected entries attended together with
// the window of raw tokens; the HCA paragraph, all visible entries): one
// softmax over the union, key = value, mixed-precision entries (RoPE dims
// BF16, the rest FP8 with power-of-two block scales, dequantised exactly).
//
// Work split.  A workgroup owns one query token and all its heads (with
// split-K, decode: one part of the token's keys, cut by split_chunk, writing
// a normalised partial output and its log-sum-exp for the merge); wave w
// owns heads 16w .. 16w+15 over all 512 dims, so no wave needs another's
// partial logits.  Keys are streamed in tiles of 32, staged once into LDS as
// bf16 rows and read by every wave for both products:
//   S^T = K Q^T   v_mfma_f32_16x16x32_bf16, 16 keys on M, the wave's 16 heads
//                 on N; lane (h = l%16, g = l/16) gets keys 4g .. 4g+3 of
//                 each 16-key half for head h
//   softmax       per head over the 4 lanes holding it (row swaps), base 2,
//                 running maximum raised lazily
//   O^T += V^T P^T  same instruction, 16 dims on M; contraction slot 8g + j
//                 holds key 4g + j (j < 4) or 16 + 4g + j - 4, so P^T is the
//                 lane's own probabilities; V^T comes from two transposing
//                 LDS reads of 4 keys each
// Pipeline: one barrier per tile.  The source rows of the token's keys are
// resolved into LDS once; each iteration reads the few it needs next with one
// LDS read per lane, an iteration ahead.  Wave w owns keys of every tile (4
// of 32 with eight waves): it copies their raw bytes (fp8 codes, RoPE dims
// and block scales of an entry, or a bf16 window row) from global memory
// straight into LDS two tiles ahead (global_load_lds, one instruction per
// key, no registers held), and one tile ahead turns them into the bf16 key
// tile, so only the barrier after that conversion joins the waves.
#include <type_traits>

#include "attn_common.h"
#include "common.h"
#include "merge.h"

using namespace csa;
using namespace csa_attn;

namespace {

constexpr int kD = 512;
constexpr int kRowS = kD * 2 + 32;     // LDS stride of a bf16 key row (1 KB + pad)
constexpr int kTileB = KT * kRowS;     // 33 KB
constexpr int kUPR = kD / 16;          // staging units (16 dims) per key row

// LDS layout: NK bf16 key tiles, NR raw tiles (RS bytes per key), their
// block scales (4 bytes per key), and the source rows of up to kMax keys of
// the token.  Three arrangements (MODE):
//   0  prefill: two key and two raw tiles, one barrier per tile; fills a CU;
//   1  decode (split-K over 64 heads): one of each, two barriers per tile, so
//      two workgroups share a CU and one's waits are covered by the other's
//      work;
//   2  fp8 queries: the logits read the fp8 codes of a tile's entries from
//      its raw tile while the key tile (bf16, for the values) is in use, so
//      one key tile and three raw tiles (copies two tiles ahead), two
//      barriers per tile; raw rows padded like key rows for the fp8 operand
//      reads of 16 consecutive rows.
template <int MODE>
struct Lay {
  static constexpr int NK = MODE == 0 ? 2 : 1;
  static constexpr int NR = MODE == 0 ? 2 : (MODE == 1 ? 1 : 3);
  static constexpr int RS = MODE == 2 ? kRowS : 1024;
  static constexpr int kMax = MODE == 1 ? 2048 : 4096;
  static constexpr int raw = NK * kTileB;
  static constexpr int scale = raw + NR * KT * RS;
  static constexpr int rows = scale + NR * KT * 4;
  static constexpr size_t smem = rows + (size_t)kMax * 4;
};
static_assert(Lay<0>::smem <= 160 * 1024, "LDS of a workgroup");
static_assert(2 * Lay<1>::smem <= 160 * 1024, "two decode workgroups per CU");
static_assert(Lay<2>::smem <= 160 * 1024, "LDS of a workgroup");

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f4_t;

// Key rows sit kRowS = 1056 bytes apart in a tile, dims in order: with the
// 32-byte pad, the logit operand reads (16 bytes of 16 consecutive rows per
// 16 lanes) and the transposed value reads (8-byte runs of 4 dims, 4 rows
// per 16 lanes) fall on distinct LDS banks, which neither an unpadded 1 KB
// stride nor a 16-byte pad achieves for the 16-byte reads.

// Copies `bytes` (16 or 4) per active lane from global memory to LDS at
// lds + lane * bytes, without registers (global_load_lds); completion is
// counted in vmcnt like a load.
__device__ __forceinline__ void dma16(uint32_t lds, const void* src) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" :: "s"(lds), "v"(src) : "memory", "m0");
}
__device__ __forceinline__ void dma4(uint32_t lds, const void* src) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" :: "s"(lds), "v"(src) : "memory", "m0");
}
// Wait until at most N of this wave's vector memory operations are in flight
// (LDS reads of copied data stay behind it: a compiler memory barrier too).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt %0" :: "n"((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8)) : "memory");
}

// DS: waves per head group; each keeps the output of 512 / DS of the dims
// (all of them compute the group's logits and softmax, the same in each)
template <int KVF, bool SPARSE, int OUTM, int NW, int MODE, int DS = 1>
__device__ __forceinline__ void attn512_body(const AttnArgs& a) {
  using L = Lay<MODE>;
  constexpr bool DEC = MODE == 1;
  constexpr bool Q8 = MODE == 2;                  // fp8 queries (entries fp8 too)
  static_assert(!Q8 || KVF == CSA_FP8_MIXED, "fp8 queries take fp8 entries");
  constexpr int KPW = KT / NW;                    // keys of a tile per wave
  constexpr bool FP8 = KVF == CSA_FP8_MIXED;
  constexpr int NDMA = KPW + (FP8 ? 1 : 0);       // copies per wave and tile
  constexpr int UPL = KPW * kUPR / 64;            // conversion units per lane
  extern __shared__ __align__(16) unsigned char smem[];
  lds_u8* kb = (lds_u8*)smem;                     // key tiles
  lds_u8* raw = (lds_u8*)(smem + L::raw);         // raw tiles
  lds_u8* rsc = (lds_u8*)(smem + L::scale);       // their block scales
  int* krow = reinterpret_cast<int*>(smem + L::rows);
  const uint32_t lds0 = (uint32_t)(uintptr_t)kb;  // LDS address of the layout

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane & 15, lg = lane >> 4;

  // one token per workgroup, or with split-K (partial outputs) one part of a
  // token: workgroup x takes part x % max_splits of token x / max_splits
  constexpr bool SPLIT = OUTM == 2;
  const int64_t q = SPLIT ? (int64_t)(blockIdx.x / (unsigned)a.max_splits) : (int64_t)blockIdx.x;
  const int split = SPLIT ? (int)(blockIdx.x - (unsigned)q * (unsigned)a.max_splits) : 0;
  constexpr int NHG = NW / DS;                    // head groups of 16 heads
  constexpr int DB = 32 / DS;                     // 16-dim output blocks per wave
  static_assert(DS == 1 || (DS == 2 && MODE == 0), "dims split over the waves of a head group");
  const int dpart = wave / NHG;                   // (uniform)
  const int head = (wave - dpart * NHG) * 16 + hl;
  const int64_t qrow = q * a.H + head;            // row of the q / out tensors

  // queries: B operand of step s (dims 32s .. 32s+31): this lane's 8 dims.
  // fp8 queries: the codes of block b (dims 128b + 32lg .. +31, zero past
  // dim 447) as the B operand of the fp8 product of block b, the head's four
  // block scales (byte b), and the RoPE dims 448 + 32s + 8lg .. +7 (s < 2) in
  // bf16
  bf16x8_t qreg[Q8 ? 1 : 16];
  i32x8_t qc[Q8 ? 4 : 1];
  bf16x8_t qrope[Q8 ? 2 : 1];
  uint32_t qsc = 0;
  auto load_q = [&]() {
    if constexpr (Q8) {
      const uint8_t* qp = static_cast<const uint8_t*>(a.q) + qrow * 448 + 32 * lg;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        qc[b] = i32x8_t{};
        if (b < 3 || lg < 2) {
          const uint4 v0 = *reinterpret_cast<const uint4*>(qp + 128 * b);
          const uint4 v1 = *reinterpret_cast<const uint4*>(qp + 128 * b + 16);
          qc[b] = i32x8_t{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w, (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
        }
      }
      qsc = *reinterpret_cast<const uint32_t*>(a.q_scale + qrow * 4);
      const uint16_t* rp = a.q_rope + qrow * 64 + 8 * lg;
#pragma unroll
      for (int s = 0; s < 2; ++s) qrope[s] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(rp + 32 * s));
    } else {
      const uint16_t* qp = static_cast<const uint16_t*>(a.q) + qrow * kD + 8 * lg;
#pragma unroll
      for (int s = 0; s < 16; ++s)
        qreg[s] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qp + 32 * s));
    }
  };
  // The loads overlap the geometry's chain of loads.  With a split over
  // selected keys every token has about k + window keys, so its parts exist
  // and are loaded for early; with a split over all visible entries most of
  // the grid's parts of short rows do not, and load nothing.
  constexpr bool EARLY_Q = !SPLIT || SPARSE;
  if constexpr (EARLY_Q) load_q();
  Geo g = make_geo<SPARSE>(a, q);
  if constexpr (SPLIT) {
    // parts from the token's own key count (split_chunk): the same whatever
    // the rest of the batch
    const int parts = split_parts(g.nkeys, a.split_keys);
    if (split >= parts) return;                   // (uniform: before any barrier)
    const int chunk = (int)split_chunk(g.nkeys, a.split_keys);
    g.key_lo = split * chunk;
    g.key_hi = g.key_lo + chunk < g.nkeys ? g.key_lo + chunk : g.nkeys;
    if (split == 0 && tid == 0) a.ws_cnt[q] = parts;
    if constexpr (!EARLY_Q) load_q();
  }
  // the geometry is the same in every lane: kept in scalar registers
  auto uni = [](int64_t v) -> int64_t {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
  };
  g.q_first = uni(g.q_first);
  g.q_last = uni(g.q_last);
  g.t_first = uni(g.t_first);
  g.t_last = uni(g.t_last);
  g.kv_base = uni(g.kv_base);
  g.raw_base = uni(g.raw_base);
  g.raw_pos = uni(g.raw_pos);
  g.kv_len = uni(g.kv_len);
  g.raw_cap = uni(g.raw_cap);
  g.wlo = uni(g.wlo);
  g.nE = __builtin_amdgcn_readfirstlane(g.nE);
  g.nkeys = __builtin_amdgcn_readfirstlane(g.nkeys);
  g.key_lo = __builtin_amdgcn_readfirstlane(g.key_lo);
  g.key_hi = __builtin_amdgcn_readfirstlane(g.key_hi);
  const int nk = g.key_hi - g.key_lo;             // at most L::kMax (host check)
  const int ntiles = (nk + KT - 1) / KT;

  // source rows of the token's keys (key_meta's encoding; a key without a
  // source, or past the last, reads a row that exists and is masked)
  const int dummy = a.kv != nullptr ? 0 : -2;
  for (int i = tid; i < ntiles * KT; i += NW * 64) {
    int row = -1;
    int64_t lo, hi;
    if (i < nk) key_meta<SPARSE>(a, g, g.key_lo + i, row, lo, hi);
    krow[i] = row;
  }
  __syncthreads();

  // Source rows an iteration needs, read one iteration ahead with one LDS
  // read per lane: lanes 0..31 the keys of tile t (its mask), lanes 32 ..
  // 32+KPW-1 this wave's keys of the tile it converts (t+1 in the prefill
  // layout, t in the others), lanes 40 .. 40+KPW-1 those of the tile it
  // copies (t+2, or t+1 in the decode layout).  Tiles past the last read row 0.
  constexpr int CONV_AHEAD = MODE == 0 ? 1 : 0;
  constexpr int COPY_AHEAD = MODE == 1 ? 1 : 2;
  // key and raw buffers of tile t
  auto kbuf = [](int t) { return MODE == 0 ? (t & 1) : 0; };
  auto rbuf = [](int t) { return MODE == 0 ? (t & 1) : (MODE == 1 ? 0 : t % 3); };
  auto meta_read = [&](int t) -> int {
    int tile = t, key = lane;
    if (lane >= 32) {
      tile = lane < 40 ? t + CONV_AHEAD : t + COPY_AHEAD;
      key = wave * KPW + (lane & 7);
    }
    const bool ok = tile < ntiles && (lane < 32 || (lane & 7) < KPW) && lane < 48;
    return krow[ok ? tile * KT + key : 0];
  };
  // per-lane parts of an fp8 entry's copy: codes (lanes 0..27), RoPE dims
  // (lanes 28..35)
  const uint8_t* f8_src = lane < 28 ? static_cast<const uint8_t*>(a.kv) + 16 * lane
                                    : reinterpret_cast<const uint8_t*>(a.kv_rope) + 16 * (lane - 28);
  const uint32_t f8_stride = lane < 28 ? 448u : 128u;
  // copies of this wave's keys of tile t into its raw tile, one
  // instruction per key (and one for the block scales); rows(j) gives the
  // source row of the wave's key j (uniform), lane l0 + j holds it in lrow
  auto dma_rows = [&](int t, auto rows, int lrow, int l0) {
    const int buf = rbuf(t);
#pragma unroll
    for (int j = 0; j < KPW; ++j) {
      const int key = wave * KPW + j;
      int row = rows(j);
      row = row == -1 ? dummy : row;
      const uint32_t dst = lds0 + L::raw + (buf * KT + key) * L::RS;
      const uint8_t* rbase = row >= 0 ? static_cast<const uint8_t*>(a.kv) + (int64_t)row * 1024
                                      : static_cast<const uint8_t*>(a.raw) + (int64_t)(-2 - row) * 1024;
      const uint8_t* src = rbase + 16 * lane;
      bool act = true;
      if constexpr (FP8) {
        if (row >= 0) {
          src = f8_src + (uint32_t)row * f8_stride;       // < 2^32: rows * 448 bytes
          act = lane < 36;
        }
      }
      if (act) dma16(dst, src);
    }
    if constexpr (FP8) {
      if (lane >= l0 && lane < l0 + KPW) {
        const int64_t r = lrow >= 0 ? lrow : 0;   // window keys copy a scale they never use
        dma4(lds0 + L::scale + (buf * KT + wave * KPW) * 4 - 4 * l0, a.kv_scale + r * 4);
      }
    }
  };
  auto dma_tile = [&](int t) {
    const int lrow = lane < KPW ? krow[t * KT + wave * KPW + lane] : 0;
    dma_rows(t, [&](int j) { return __builtin_amdgcn_readfirstlane(krow[t * KT + wave * KPW + j]); }, lrow, 0);
  };
  // this wave's keys of tile t from its raw tile into its key tile
  // rowof(kw): source row of the wave's key kw of tile t (uniform)
  auto convert_rows = [&](int t, auto rowof) {
    const int buf = rbuf(t);
    lds_u8* tile = kb + kbuf(t) * kTileB;
#pragma unroll
    for (int i = 0; i < UPL; ++i) {
      const int v = lane + 64 * i;
      const int key = wave * KPW + (v >> 5), j = v & 31;
      const lds_u8* src = raw + (buf * KT + key) * L::RS;
      int row = (lane >> 5) ? rowof(2 * i + 1) : rowof(2 * i);
      row = row == -1 ? dummy : row;             // as dma_rows copied it
      uint4 x0, x1;
      if (FP8 && row >= 0) {
        if (j < 28) {
          const uint4 c = lds_read_b128(src + 16 * j);
          const uint32_t sb = rsc[(buf * KT + key) * 4 + (j >> 3)];
          fp8x16_to_bf16(c, e8m0_to_f32(sb), x0, x1);
        } else {
          x0 = lds_read_b128(src + 448 + 32 * (j - 28));
          x1 = lds_read_b128(src + 448 + 32 * (j - 28) + 16);
        }
      } else {
        x0 = lds_read_b128(src + 32 * j);
        x1 = lds_read_b128(src + 32 * j + 16);
      }
      *(__attribute__((address_space(3))) u32x4_t*)(tile + key * kRowS + 32 * j) =
          u32x4_t{x0.x, x0.y, x0.z, x0.w};
      *(__attribute__((address_space(3))) u32x4_t*)(tile + key * kRowS + 32 * j + 16) =
          u32x4_t{x1.x, x1.y, x1.z, x1.w};
    }
  };
  auto convert_tile = [&](int t) {
    convert_rows(t, [&](int kw) { return __builtin_amdgcn_readfirstlane(krow[t * KT + wave * KPW + kw]); });
  };

  // LDS read addresses (tile 0's buffer; the other buffer is kTileB above).
  // K operand of half hk, step s = 4 sh + sl: row 16 hk + hl, logical chunk
  // 4 s + lg.  V^T operand of dim block db = 8 dh + dl, read rho: rows
  // 16 rho + 4 lg + hl / 4, dims 16 db + 4 (hl % 4) .. +3.
  // (one base each; the reads of step s and block db add constants)
  lds_u8* kptr0;
  lds_u8* vptr0;
  {
    kptr0 = kb + hl * kRowS + 16 * lg;
    const int rv = 4 * lg + (hl >> 2);
    vptr0 = kb + rv * kRowS + 8 * (hl & 3) + 32 * (dpart * DB);   // (this wave's dim blocks)
  }
  auto launder = [&]() {
    asm volatile("" : "+v"(kptr0));
    asm volatile("" : "+v"(vptr0));
  };

  f4_t acc_o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc_o[i] = f4_t{};
  float m_run = -INFINITY, l_run = 0.0f;

  if constexpr (Q8) {
#pragma unroll
    for (int b = 0; b < 4; ++b) asm volatile("" :: "v"(qc[b]));
#pragma unroll
    for (int s = 0; s < 2; ++s) asm volatile("" :: "v"(qrope[s]));
  } else {
#pragma unroll
    for (int s = 0; s < 16; ++s) asm volatile("" :: "v"(qreg[s]));
  }

  // the read addresses point into the key buffer of the tile being computed
  // (moved to the other buffer after each tile)
  constexpr int KD = 3;                          // logit steps of operand reads in flight
  auto compute = [&](int t, int meta) {
    constexpr int bofs = 0;
    launder();
    // S^T = K Q^T, two 16-key halves; the operands of step s + 2 are read
    // while step s multiplies
    f4_t s0 = f4_t{}, s1 = f4_t{};
    if constexpr (!Q8) {
      auto kread = [&](int s, uint4& k0, uint4& k1) {
        const int sl = s & 3, sh = s >> 2;
        k0 = lds_read_b128(kptr0 + 64 * sl + bofs + sh * 256);
        k1 = lds_read_b128(kptr0 + 64 * sl + bofs + sh * 256 + 16 * kRowS);
      };
      // KD steps of operand reads in flight ahead of the products
      uint4 kr[KD][2];
#pragma unroll
      for (int s = 0; s < KD; ++s) kread(s, kr[s][0], kr[s][1]);
  #pragma unroll
      for (int s = 0; s < 16; ++s) {
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kr[s % KD][0]), qreg[s], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kr[s % KD][1]), qreg[s], s1, 0, 0, 0);
        if (s + KD < 16) kread(s + KD, kr[s % KD][0], kr[s % KD][1]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * KD, 0);      // LDS reads of steps 0 .. KD-1
  #pragma unroll
      for (int i = 0; i < 16 - KD; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);    // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);    // LDS reads
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * KD, 0);
    } else {
      // fp8 queries.  A tile of entries only: the NoPE dims on the fp8
      // matrix cores, the keys' codes (row 16 hk + hl, bytes 128 b + 32 lg
      // .. +31 of block b, zero past byte 447) read from the tile's raw
      // copy, each product scaled in the instruction by the key's and the
      // head's power-of-two block scales (exact); the RoPE dims in bf16 from
      // the key tile.
      const int rb = rbuf(t);
      const lds_u8* rt = raw + rb * KT * L::RS;
      auto rope = [&](f4_t acc, int hk) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const uint4 k = lds_read_b128(kb + (16 * hk + hl) * kRowS + 2 * (448 + 32 * s + 8 * lg));
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, k), qrope[s], acc, 0, 0, 0);
        }
        return acc;
      };
      if (g.key_lo + (t + 1) * KT <= g.nE) {
#pragma unroll
        for (int hk = 0; hk < 2; ++hk) {
          const lds_u8* rowp = rt + (16 * hk + hl) * L::RS + 32 * lg;
          const uint32_t ksc =
              *(const __attribute__((address_space(3))) uint32_t*)(rsc + (rb * KT + 16 * hk + hl) * 4);
          f4_t acc = f4_t{};
          auto block = [&](auto bc) {
            constexpr int b = decltype(bc)::value;
            i32x8_t ka = i32x8_t{};
            if (b < 3 || lg < 2) {
              const uint4 x0 = lds_read_b128(rowp + 128 * b), x1 = lds_read_b128(rowp + 128 * b + 16);
              ka = i32x8_t{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
            }
            // both operands e4m3 (format 0); opsel picks block b's scale byte
            acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qc[b], acc, 0, 0, b, (int)ksc, b, (int)qsc);
          };
          block(std::integral_constant<int, 0>{});
          block(std::integral_constant<int, 1>{});
          block(std::integral_constant<int, 2>{});
          block(std::integral_constant<int, 3>{});
          acc = rope(acc, hk);
          if (hk == 0) s0 = acc;
          else s1 = acc;
        }
      } else {
        // a window key in the tile (bf16 rows): the NoPE products in bf16,
        // the query codes converted exactly; contraction slots of step j of
        // block b hold dims 128 b + 32 lg + 8 j .. +7 in both operands
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const float sc = e8m0_to_f32((qsc >> (8 * b)) & 255u);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t w0 = (uint32_t)qc[b][2 * j], w1 = (uint32_t)qc[b][2 * j + 1];
            const uint32_t o[4] = {
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, false)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0 >> 16, sc, false)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, false)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1 >> 16, sc, false))};
            const bf16x8_t qb = __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
            const int dofs = 2 * (128 * b + 32 * lg + 8 * j);
            const uint4 k0 = lds_read_b128(kb + hl * kRowS + dofs);
            const uint4 k1 = lds_read_b128(kb + (16 + hl) * kRowS + dofs);
            s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, k0), qb, s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, k1), qb, s1, 0, 0, 0);
          }
        }
        s0 = rope(s0, 0);
        s1 = rope(s1, 1);
      }
    }
    // mask: key 4 lg + i of half hk is bit 16 hk + 4 lg + i of the tile's word
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = s0[i];
      sv[4 + i] = s1[i];
    }
    const uint32_t w = (uint32_t)__ballot(lane < KT && meta != -1);
    if (w != 0xffffffffu) {
      const uint32_t mine = w >> (4 * lg);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[i] = ((mine >> i) & 1u) ? sv[i] : -INFINITY;
        sv[4 + i] = ((mine >> (16 + i)) & 1u) ? sv[4 + i] : -INFINITY;
      }
    }
    // online softmax over the 4 lanes of each head
    float tmax = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, sv[i]);
    {
      const uint32_t u = __float_as_uint(tmax);
      const auto x32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
      const float m1 = fmaxf(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
      const uint32_t v = __float_as_uint(m1);
      const auto x16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
      tmax = fmaxf(__uint_as_float(x16[0]), __uint_as_float(x16[1])) * a.scale_log2;
    }
    const bool raise = tmax > m_run + kStale || (m_run == -INFINITY && tmax != -INFINITY);
    if (__any(raise)) {
      const float m_new = raise ? tmax : m_run;
      const float alpha = m_new == m_run ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc_o[db][i] *= alpha;
      m_run = m_new;
    }
    const float nm = m_run == -INFINITY ? 0.0f : -m_run;
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(sv[i], a.scale_log2, nm));
    uint4 pu;
    pu.x = pack_bf16x2_fast(p[0], p[1]);
    pu.y = pack_bf16x2_fast(p[2], p[3]);
    pu.z = pack_bf16x2_fast(p[4], p[5]);
    pu.w = pack_bf16x2_fast(p[6], p[7]);
    // the row sum of the probabilities as rounded for the product
    {
      const uint32_t pw[4] = {pu.x, pu.y, pu.z, pu.w};
      float ps = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, pw[j]),
                                             __builtin_bit_cast(bf16x2_v, 0x3f803f80u), ps, false);
      l_run += ps;
    }
    const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pu);
    // O^T += V^T P^T over 32 dim blocks; the operands of block db + 2 are
    // read while block db multiplies
    auto vread = [&](int db) -> uint4 {
      const int dl = db & 7, dh = db >> 3;
      const uint2 v0 = lds_read_tr16(vptr0 + 32 * dl + bofs + dh * 256);
      const uint2 v1 = lds_read_tr16(vptr0 + 32 * dl + bofs + dh * 256 + 16 * kRowS);
      return make_uint4(v0.x, v0.y, v1.x, v1.y);
    };
    uint4 va = vread(0), vb = vread(1);
#pragma unroll
    for (int db = 0; db < DB; db += 2) {
      acc_o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, va), pb, acc_o[db], 0, 0, 0);
      if (db + 2 < DB) va = vread(db + 2);
      acc_o[db + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vb), pb, acc_o[db + 1], 0, 0, 0);
      if (db + 3 < DB) vb = vread(db + 3);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);      // LDS reads of blocks 0, 1
#pragma unroll
    for (int i = 0; i < DB - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);    // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);    // LDS reads
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
  };

  if constexpr (DEC) {
    // ---- decode layout, two barriers per tile: convert tile t, copy tile
    // t+1 while computing t
    if (ntiles > 0) {
      dma_tile(0);
      wait_vm<0>();
    }
    int meta = meta_read(0);
    for (int t = 0; t < ntiles; ++t) {
      convert_rows(t, [&](int kw) { return __builtin_amdgcn_readlane(meta, 32 + kw); });
      lds_barrier();                                // key tile complete, raw tile free
      if (t + 1 < ntiles)
        dma_rows(t + 1, [&](int j) { return __builtin_amdgcn_readlane(meta, 40 + j); }, meta, 40);
      const int meta_next = meta_read(t + 1);
      compute(t, meta);
      wait_vm<0>();                                 // this wave's copies of tile t+1 landed
      lds_barrier();                                // every wave done with the key tile
      meta = meta_next;
    }
  } else if constexpr (Q8) {
    // ---- fp8 queries, two barriers per tile: convert tile t, copy tile t+2
    // while computing t (three raw tiles: t's codes are read by the logits)
    if (ntiles > 0) {
      dma_tile(0);
      if (ntiles > 1) {
        dma_tile(1);
        wait_vm<NDMA>();
      } else {
        wait_vm<0>();
      }
    }
    int meta = meta_read(0);
    for (int t = 0; t < ntiles; ++t) {
      convert_rows(t, [&](int kw) { return __builtin_amdgcn_readlane(meta, 32 + kw); });
      lds_barrier();                                // key tile and every wave's raw tile t complete
      if (t + 2 < ntiles)                           // (its raw tile held t-1, consumed last tile)
        dma_rows(t + 2, [&](int j) { return __builtin_amdgcn_readlane(meta, 40 + j); }, meta, 40);
      const int meta_next = meta_read(t + 1);
      compute(t, meta);
      if (t + 2 < ntiles) wait_vm<NDMA>();          // this wave's copies of tile t+1 landed
      else wait_vm<0>();
      lds_barrier();                                // every wave done with the key tile
      meta = meta_next;
    }
  } else {
  // ---- prologue: tile 0 in LDS, tile 1 copying
  if (ntiles > 0) {
    dma_tile(0);
    if (ntiles > 1) {
      dma_tile(1);
      wait_vm<NDMA>();
    } else {
      wait_vm<0>();
    }
    convert_tile(0);
    lds_barrier();
  }
  // ---- key loop: one barrier per tile.  The upper half of the waves (one
  // per SIMD) converts its keys of tile t+1 before computing tile t, the
  // lower half after, so the two waves of a SIMD are out of phase: one
  // multiplies while the other converts or runs its softmax.
  const bool conv_first = wave >= NW / 2;           // (uniform)
  int flip = kTileB;
  int meta = meta_read(0);
  for (int t = 0; t < ntiles; ++t) {
    // copies of tile t+2 (raw tile t % 2 was converted last tile): the waves
    // that convert first issue them first, the others after their products
    // (the wait before each conversion counts them either way)
    auto dma_next = [&]() {
      if (t + 2 < ntiles)
        dma_rows(t + 2, [&](int j) { return __builtin_amdgcn_readlane(meta, 40 + j); }, meta, 40);
    };
    if (conv_first) dma_next();
    const int meta_next = meta_read(t + 1);
    // (key tile (t+1) % 2 was last read in the tile before, behind the barrier)
    auto convert_next = [&]() {
      if (t + 1 < ntiles) {
        if (t + 2 < ntiles) wait_vm<NDMA>();        // this wave's copies of tile t+1 landed
        else wait_vm<0>();
        convert_rows(t + 1, [&](int kw) { return __builtin_amdgcn_readlane(meta, 32 + kw); });
      }
    };
    if (conv_first) convert_next();
    compute(t, meta);
    kptr0 += flip;
    vptr0 += flip;
    flip = -flip;
    if (!conv_first) {
      dma_next();
      convert_next();
    }
    lds_barrier();
    meta = meta_next;
  }
  }

  // ---- epilogue: normaliser over the 4 lanes of each head
  float l_tot;
  {
    const uint32_t u = __float_as_uint(l_run);
    const auto x32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const float s1 = __uint_as_float(x32[0]) + __uint_as_float(x32[1]);
    const uint32_t v = __float_as_uint(s1);
    const auto x16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    l_tot = __uint_as_float(x16[0]) + __uint_as_float(x16[1]);
  }
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (head < a.H) {
    const float lse_v = l_tot > 0.0f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    // split-K: normalised partial output and lse of this part, [split][row]
    const int64_t prow = SPLIT ? (int64_t)split * (a.n_q * a.H) + qrow : qrow;
    float* lse_dst = SPLIT ? a.ws_lse : a.lse;
    if (lse_dst != nullptr && lg == 0 && dpart == 0) lse_dst[prow] = lse_v;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d = (dpart * DB + db) * 16 + 4 * lg;
      const float o0 = acc_o[db][0] * inv, o1 = acc_o[db][1] * inv;
      const float o2 = acc_o[db][2] * inv, o3 = acc_o[db][3] * inv;
      // (split-K partials in bf16 when the output is bf16: one more rounding
      // of each part, half the partial bytes)
      if (OUTM == 1 || (SPLIT && a.part_bf16 != 0)) {
        uint2 uo;
        uo.x = pack_bf16x2_fast(o0, o1);
        uo.y = pack_bf16x2_fast(o2, o3);
        uint16_t* dst = SPLIT ? reinterpret_cast<uint16_t*>(a.ws_o) + prow * kD + d
                              : static_cast<uint16_t*>(a.out) + qrow * kD + d;
        *reinterpret_cast<uint2*>(dst) = uo;
      } else {
        float* dst = SPLIT ? a.ws_o + prow * kD + d : static_cast<float*>(a.out) + qrow * kD + d;
        *reinterpret_cast<float4*>(dst) = make_float4(o0, o1, o2, o3);
      }
    }
  }
}

template <int KVF, bool SPARSE, int OUTM, int NW, int MODE, int DS = 1>
__global__ __launch_bounds__(NW * 64) void attn512_kernel(AttnArgs a) {
  attn512_body<KVF, SPARSE, OUTM, NW, MODE, DS>(a);
}

// decode layout (split-K, 64 heads): registers held to two waves per SIMD,
// so two workgroups fit a CU
template <int KVF, bool SPARSE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void attn512_dec_kernel(AttnArgs a) {
  attn512_body<KVF, SPARSE, 2, 4, 1>(a);
}

template <int KVF, bool SPARSE, int OUTM, int NW, bool Q8>
csa_status launch512(const AttnArgs& a, hipStream_t s) {
  // 64 heads split over selected keys (a CSA decode: every token's parts
  // exist): eight waves, two per head group each keeping half the dims, in
  // the prefill layout (one workgroup per CU); over all visible entries (HCA)
  // most of the grid's parts of short rows do not exist, and the decode
  // layout (two workgroups per CU) keeps the parts that do in one wave of
  // workgroups
  constexpr bool DSPL = OUTM == 2 && NW == 4 && !Q8 && SPARSE;
  constexpr int MODE = Q8 ? 2 : (OUTM == 2 && NW == 4 && !SPARSE ? 1 : 0);
  constexpr int NWK = DSPL ? 8 : NW;
  constexpr int DS = DSPL ? 2 : 1;
  const void* kern = MODE == 1 ? (const void*)attn512_dec_kernel<KVF, SPARSE>
                               : (const void*)attn512_kernel<KVF, SPARSE, OUTM, NWK, MODE, DS>;
  const size_t smem = Lay<MODE>::smem;
  static const hipError_t attr =
      hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)Lay<MODE>::smem);
  if (attr != hipSuccess) return csa_host::fail(CSA_ERR_HIP, "csa_sparse_mqa_attn: cannot reserve %zu B of LDS", smem);
  const int64_t blocks = OUTM == 2 ? a.n_q * a.max_splits : a.n_q;
  if constexpr (MODE == 1)
    hipLaunchKernelGGL((attn512_dec_kernel<KVF, SPARSE>), dim3((unsigned)blocks), dim3(256), smem, s, a);
  else
    hipLaunchKernelGGL((attn512_kernel<KVF, SPARSE, OUTM, NWK, MODE, DS>), dim3((unsigned)blocks), dim3(NWK * 64), smem, s, a);
  return csa_host::check_launch("csa_sparse_mqa_attn (D = 512)");
}

template <int KVF, bool SPARSE, int OUTM, bool Q8>
csa_status launch512_heads(const AttnArgs& a, hipStream_t s) {
  switch (a.H / 16) {
    case 4: return launch512<KVF, SPARSE, OUTM, 4, Q8>(a, s);
    case 8: return launch512<KVF, SPARSE, OUTM, 8, Q8>(a, s);
    default: return csa_host::fail(CSA_ERR_UNSUPPORTED, "csa_sparse_mqa_attn: this D = 512 path takes 64 or 128 heads");
  }
}

}  // namespace

// D = 512, bf16 compute, one workgroup per query token, or per part of a
// token's keys with split-K (outm 2: partial outputs to the workspace).
bool attn512_fits(int64_t max_keys) { return max_keys <= Lay<0>::kMax; }
int attn512_part_keys(int n_heads) { return n_heads == 64 ? Lay<1>::kMax : Lay<0>::kMax; }

csa_status launch_attn512(const AttnArgs& a, int kvf, bool sparse, int outm, bool q8, hipStream_t s) {
  const int64_t blocks = outm == 2 ? a.n_q * a.max_splits : a.n_q;
  if (blocks > 0x7fffffff) return csa_host::fail(CSA_ERR_UNSUPPORTED, "csa_sparse_mqa_attn: too many queries");
  auto by_out = [&](auto kvf_c, auto sparse_c, auto q8_c) -> csa_status {
    constexpr int K = decltype(kvf_c)::value;
    constexpr bool S = decltype(sparse_c)::value;
    constexpr bool Q = decltype(q8_c)::value;
    if (outm == 2) return launch512_heads<K, S, 2, Q>(a, s);
    return outm ? launch512_heads<K, S, 1, Q>(a, s) : launch512_heads<K, S, 0, Q>(a, s);
  };
  using fp8_t = std::integral_constant<int, CSA_FP8_MIXED>;
  using bf16_t = std::integral_constant<int, CSA_BF16>;
  using yes = std::true_type;
  using no = std::false_type;
  if (q8) return sparse ? by_out(fp8_t{}, yes{}, yes{}) : by_out(fp8_t{}, no{}, yes{});
  if (kvf == CSA_FP8_MIXED) return sparse ? by_out(fp8_t{}, yes{}, no{}) : by_out(fp8_t{}, no{}, no{});
  return sparse ? by_out(bf16_t{}, yes{}, no{}) : by_out(bf16_t{}, no{}, no{});
}
