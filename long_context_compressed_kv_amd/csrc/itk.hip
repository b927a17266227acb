// Fused lightning indexer + top-k (page "DeepSeek V4 深度解析", section 2,
// CSA step 2: every query scores the compressed entries with the light
// indexer and keeps the k best).  The result equals csa_indexer_score
// followed by csa_topk_select, bit for bit, but the score matrix never goes
// to memory: only a short list of candidates per query does.
//
//   1. itk_sample_kernel (groups of several queries of one request):
//      each query scores a sample of its visible entries (runs of 32
//      consecutive entries spread evenly over the row, about 40n/3k of them)
//      and takes as threshold the sample key of rank ~3k * sample / n, so that
//      about 3k entries of the row score at least as high.  Rows of at most
//      `cap` entries take every entry (threshold 0).
//   2. itk_filter_kernel: the indexer's tiles (same grid and arithmetic as
//      csa_indexer_score); an entry whose order key reaches its threshold is
//      appended, (key, index), to the query's candidate list.  Each workgroup
//      reserves its span with one atomic per query.  With one query per group
//      (decode) there is no sample: each workgroup takes as its threshold the
//      key of rank ~3k/n of its own entries (+1), and records the largest
//      such threshold of the row.
//   3. itk_select_kernel: per query, an exact radix select of the k-th
//      largest candidate key, ties resolved to the lowest indices by a radix
//      select over the tied indices, the chosen entries marked in an LDS
//      bitmap of the row and read back in index order.  Every entry left out
//      scored below its threshold, so the list holds the exact top-k unless
//      the k-th candidate key is below the row's (largest) threshold.  A row
//      where that happens, or whose candidates overflowed `cap` or fell short
//      of k (masses of equal scores), is redone there exactly from recomputed
//      scores.
// The candidates arrive in no fixed order, but every step after the filter
// depends only on the candidate set, so the output is deterministic.
#include <mutex>
#include <type_traits>

#include "indexer_core.h"
#include "select_core.h"

using namespace csa;

namespace {

constexpr int kWaves = 4;            // waves of the scoring kernels
constexpr int kTilesPerWave = 8;     // tiles per wave, several queries per group
constexpr int kBitmapMax = 1 << 20;  // longest row the select kernel takes
constexpr int kMaxWg = kBitmapMax / 1024;   // filter workgroups of a streamed row, at most

struct ItkArgs {
  const void* qi;
  const uint8_t* qi_scale;
  const float* head_w;
  const void* ki;
  const uint8_t* ki_scale;
  BatchDev b;
  int m;
  int relu;
  int qpg;            // queries per group (8 for a single request, else 1)
  int64_t n_q;
  int k;
  int cap;            // candidates kept per query
  int64_t max_n;      // rows are cut to this many entries (the batch's max_kv, at most 2^20)
  uint32_t* tau;      // [n_q] threshold keys (query groups)
  uint32_t* cnt;      // [n_q] candidates found (may exceed cap)
  uint2* cand;        // [n_q][cap] (key, entry)
  uint2* hdr;         // [n_q][kMaxWg] streaming: (count, threshold) of each filter workgroup
  int32_t* idx;       // [n_q][k] result
};

// Keys per tile batch when one query per group streams its row (as in the
// score kernel's decode mode).
template <int FMT> struct Tiling;
template <> struct Tiling<CSA_F32> { static constexpr int TB = 1, TPW = 8; };
template <> struct Tiling<CSA_BF16> { static constexpr int TB = 1, TPW = 8; };
template <> struct Tiling<CSA_MXFP4> { static constexpr int TB = 8, TPW = 16; };

template <int FMT>
constexpr int entries_per_wg(bool stream) {
  return kWaves * (stream ? Tiling<FMT>::TPW : kTilesPerWave) * 32;
}

// Order key of a score as the score kernel would store it.
template <bool SBF16>
__device__ __forceinline__ uint32_t score_key(float s) {
  if constexpr (SBF16) return order_bf16(pack_bf16x2_fast(s, 0.0f) & 0xffffu);
  else return order_f32(__float_as_uint(s));
}

// A group of queries as the score kernel forms it: its first query, the
// queries' visible counts, the A operand of this lane and the head weights of
// the lane's register blocks.
template <int FMT, int NG>
struct Group {
  int64_t qblock;
  QueryMeta qm;
  QueryOp<FMT> aq;
  int nv[NG];
  float hw[NG][kHI];
};

template <int FMT, int NG>
__device__ __forceinline__ void load_group(const ItkArgs& a, int64_t qblock, Group<FMT, NG>& gr) {
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int rl = lane & 31;
  gr.qblock = qblock;
  gr.qm = query_meta(a.b, qblock, a.m);
  const int qa = rl >> 2, ha = rl & 3;
  load_query<FMT>(a.qi, a.qi_scale, (qblock + qa) * kHI + ha, qa < a.qpg && qblock + qa < a.n_q, half, gr.aq);
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int ql = 2 * g + half;
    int v = 0;
    if (ql < a.qpg && qblock + ql < a.n_q) {
      int64_t n = (gr.qm.t + ql + 1) / a.m;
      if (n > gr.qm.kv_len) n = gr.qm.kv_len;
      if (n > a.max_n) n = a.max_n;
      v = (int)n;
    }
    gr.nv[g] = v;
#pragma unroll
    for (int h = 0; h < kHI; ++h)
      gr.hw[g][h] = (a.head_w != nullptr && v > 0) ? a.head_w[(qblock + ql) * kHI + h] : 1.0f;
  }
}

// visible entries of query q (cut to max_n, which bounds every LDS bitmap)
__device__ __forceinline__ int64_t visible(const ItkArgs& a, int64_t q) {
  const int64_t n = query_meta(a.b, q, a.m).n_vis;
  return n < a.max_n ? n : a.max_n;
}

// ------------------------------------------------------------------ 1. sample

constexpr int kSampleRun = 32;       // one tile per run

// Grid: one workgroup (8 waves) per query group.  LDS: the sample keys of the
// group's queries, [8][S] (16-bit keys for bf16 scores, S = 4096; 32-bit for
// fp32, S = 2048).  A wave loads the keys of STB runs before scoring them.
template <int FMT> struct SampleTiles { static constexpr int STB = 4; };
template <> struct SampleTiles<CSA_F32> { static constexpr int STB = 2; };
template <> struct SampleTiles<CSA_MXFP4> { static constexpr int STB = 8; };
constexpr int kSampleThreads = 512;

template <int FMT, bool SBF16>
__global__ __launch_bounds__(kSampleThreads) void itk_sample_kernel(ItkArgs a) {
  constexpr int S = SBF16 ? 4096 : 2048;
  constexpr int NRUN = S / kSampleRun;
  constexpr int NW = kSampleThreads / 64;
  static_assert(NW >= 8, "one wave per query of a group");
  constexpr int STB = SampleTiles<FMT>::STB;
  using skey_t = typename std::conditional<SBF16, uint16_t, uint32_t>::type;
  __shared__ skey_t sk[8][S];
  __shared__ RadixLds<kSampleThreads> rx;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5, rl = lane & 31;
  const int64_t qblock = (int64_t)blockIdx.x * a.qpg;
  const int nq = (int)(a.n_q - qblock < a.qpg ? a.n_q - qblock : a.qpg);

  // the group's queries see n_lo .. n_lo + a few entries; only rows longer
  // than cap are sampled, over the entries all of them see
  const int64_t n_lo = visible(a, qblock);
  const int64_t n_hi = visible(a, qblock + nq - 1);
  // runs enough that the threshold is the sample's ~40th key (a relative
  // spread of about 1/sqrt(40) in the candidate count), at least 16
  int nrun = (int)((40 * n_lo + 3 * (int64_t)a.k * kSampleRun - 1) / (3 * (int64_t)a.k * kSampleRun));
  nrun = nrun < 16 ? 16 : (nrun > NRUN ? NRUN : nrun);
  const int ns = nrun * kSampleRun;        // sample keys
  if (n_hi > a.cap) {
    Group<FMT, 4> gr;
    load_group<FMT, 4>(a, qblock, gr);
    auto run_start = [&](int r) { return (int64_t)r * (n_lo - kSampleRun) / (nrun - 1); };  // + 32 <= n_lo
    for (int r0 = wave * STB; r0 < nrun; r0 += NW * STB) {
      KeyOp<FMT> kt[STB];
#pragma unroll
      for (int tb = 0; tb < STB; ++tb)
        load_key<FMT>(a.ki, a.ki_scale,
                      entry_row_if(a.b, gr.qm.kv_base, run_start(r0 + tb) + rl, r0 + tb < nrun),
                      r0 + tb < nrun, half, kt[tb]);
#pragma unroll
      for (int tb = 0; tb < STB; ++tb) {
        const int r = r0 + tb;
        if (r >= nrun) break;
        const f32x16_t acc = tile_dots<FMT>(gr.aq, kt[tb]);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int ql = 2 * g + half;
          if (ql < nq) sk[ql][r * kSampleRun + rl] = (skey_t)score_key<SBF16>(head_score(acc, g, gr.hw[g], a.relu));
        }
      }
    }
  }
  __syncthreads();
  // wave ql selects the threshold of query ql (a group holds at most one
  // query per wave)
  const int ql = wave;
  if (ql < nq) {
    const int64_t q = qblock + ql;
    const int64_t n = visible(a, q);
    uint32_t tau = 0;
    if (n > a.cap) {
      // about 3k of the row's keys reach the sample key of this rank
      int64_t rank = (3 * (int64_t)a.k * ns + n - 1) / n;
      if (rank < 1) rank = 1;
      if (rank > ns) rank = ns;
      tau = wave_radix_select<SBF16 ? 16 : 32>(&sk[ql][0], ns, (uint32_t)rank, &rx.hist[wave][0]);
    }
    if (lane == 0) {
      a.tau[q] = tau;
      a.cnt[q] = 0;
    }
  }
}

// ------------------------------------------------------------------ 2a. filter, query groups

// The query groups of one request (prefill): the sample gave each query a
// threshold key tau.  A workgroup scores its group against GT tiles of 32
// entries per wave (kGroupTiles, or kGroupTilesShort for short rows).  Per
// lane and register block a score is the ReLU'd head sum (as the score
// kernel forms it) compared with a float floor below which no score can
// reach tau; the few that pass are staged per wave in LDS with their exact
// scores, then one atomic per query reserves the workgroup's span of the
// list and the waves copy their candidates out.
// A query whose row fits the list whole (at most cap entries, tau = 0) takes
// every visible entry at list slot = entry index instead.
//
// Staging: the two queries of a lane's register block g (lanes 0-31 query
// 2g, lanes 32-63 query 2g + 1) share one area per (wave, g), in the order
// of their lanes, the upper half's entries tagged in bit 31; a lane's slot is
// the area's count plus the passing lanes below it, all counts uniform.  An
// area takes a tile's passes while it holds fewer than kStageSlots, so 64
// more slots hold any tile's; every lane writes, a lane that does not pass
// into a slot of its own past the areas (no branch per lane).  Passes that
// find the area full are counted, not staged, and send both rows to the
// exact redo.
constexpr int kGroupTiles = 64;     // tiles per wave: 8192 entries per workgroup
// rows of at most kShortRows entries: 8 tiles per wave, so that all four
// waves of a workgroup have entries (1024 per workgroup)
constexpr int kGroupTilesShort = 8;
constexpr int64_t kShortRows = 8192;
constexpr int kStageSlots = 128;    // staged candidates per (wave, register block)
constexpr int kStageCap = kStageSlots + 64;

// A float below which a score's key cannot reach tau (taken a little low:
// a score at or above it may still fall short, and is then only an extra
// candidate).  fp32 keys: key(s) >= tau exactly when s >= the value of tau
// (-0 and +0 compare equal).  bf16 keys: a score rounds to the value v of tau
// or above only from above the midpoint below v, which lies above
// v - |v| 2^-7; 2^-120 more keeps zero and tiny values on the safe side.
template <bool SBF16>
__device__ __forceinline__ float score_floor(uint32_t tau) {
  const float v = key_value<SBF16>(tau);
  if constexpr (!SBF16) return v;
  return fmaf(-__builtin_fabsf(v), 0x1p-7f, v) - 0x1p-120f;
}

// Bytes of one entry key row and of its block scales.
template <int FMT> struct KeyRow;
template <> struct KeyRow<CSA_F32> { static constexpr int B = kDI * 4, S = 0; };
template <> struct KeyRow<CSA_BF16> { static constexpr int B = kDI * 2, S = 0; };
template <> struct KeyRow<CSA_MXFP4> { static constexpr int B = kDI / 2, S = kDI / 32; };

// The key operand of a lane whose row starts at `row` (bytes; the lane's
// half of the dims as load_key reads it) and whose scales start at `srow`.
template <int FMT>
__device__ __forceinline__ void load_key_row(const uint8_t* row, const uint8_t* srow, int half,
                                             KeyOp<FMT>& k) {
  if constexpr (FMT == CSA_F32) {
    const float* p = reinterpret_cast<const float*>(row) + half;
#pragma unroll
    for (int c = 0; c < kDI / 2; ++c) k.v[c] = p[2 * c];
  } else if constexpr (FMT == CSA_BF16) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(row) + half * 8;
#pragma unroll
    for (int c = 0; c < kDI / 16; ++c) k.v[c] = *reinterpret_cast<const uint4*>(p + 16 * c);
  } else {
    k.v = *reinterpret_cast<const uint4*>(row + half * 16);
    k.scale = srow[half];
  }
}

// Tiles are scored in pairs: both products are issued before either result
// is read, so one pair's matrix-core latency overlaps the other's vector work.
template <int FMT, bool SBF16, bool PAGED, bool HW, int GT>
__global__ __launch_bounds__(256) void itk_group_filter_kernel(ItkArgs a) {
  constexpr int QS = 8;                      // query slots of a group
  constexpr int EW = GT * 32;                // entries per wave (GT tiles)
  // staged candidates: (score bits, entry | upper half << 31); the key is
  // formed when copied out
  __shared__ uint2 stage[kWaves][4 * kStageCap + 64];
  __shared__ uint32_t wcnt[kWaves][QS];
  __shared__ uint32_t wover[kWaves][4];
  __shared__ uint32_t gbase[QS];
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, rl = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform over the wave

  const int64_t qblock = (int64_t)blockIdx.x * a.qpg;
  int64_t q_hi = qblock + a.qpg - 1;
  if (q_hi >= a.n_q) q_hi = a.n_q - 1;
  // the group's longest and shortest rows (at most 2^20 entries; uniform)
  const int n_scan = __builtin_amdgcn_readfirstlane((int)visible(a, q_hi));
  const int n_lo = __builtin_amdgcn_readfirstlane((int)visible(a, qblock));
  const int e_wg = (int)blockIdx.y * (kWaves * EW);
  if (e_wg >= n_scan) return;                // the whole workgroup: no barrier reached
  const int e_wave = e_wg + wave * EW;
  const QueryMeta qm = query_meta(a.b, qblock, a.m);
  const int64_t kv_base = qm.kv_base;

  // A operand: query rl / 4, head rl % 4 of the group
  QueryOp<FMT> aq;
  {
    const int qa = rl >> 2, ha = rl & 3;
    load_query<FMT>(a.qi, a.qi_scale, (qblock + qa) * kHI + ha, qa < a.qpg && qblock + qa < a.n_q,
                    half, aq);
  }
  // the lane's queries (2g + half): visible entries, floors, head weights,
  // and whether their rows are taken whole (at most cap entries)
  int nv[4];
  float tf[4];
  float hw[HW ? 4 : 1][kHI];
  bool whole[4];
  bool any_whole = false;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int ql = 2 * g + half;
    int v = 0;
    if (ql < a.qpg && qblock + ql < a.n_q) {
      int64_t n = (qm.t + ql + 1) / a.m;
      if (n > qm.kv_len) n = qm.kv_len;
      if (n > a.max_n) n = a.max_n;
      v = (int)n;
    }
    nv[g] = v;
    whole[g] = v > 0 && v <= a.cap;
    tf[g] = v > 0 && !whole[g] ? score_floor<SBF16>(a.tau[qblock + ql]) : INFINITY;
    any_whole = any_whole || whole[g];
    if constexpr (HW) {
#pragma unroll
      for (int h = 0; h < kHI; ++h) hw[g][h] = v > 0 ? a.head_w[(qblock + ql) * kHI + h] : 1.0f;
    }
  }
  any_whole = __any(any_whole);
  uint32_t cnt[QS];                          // candidates per query (uniform)
#pragma unroll
  for (int q = 0; q < QS; ++q) cnt[q] = 0;
  uint32_t ns[4] = {0u, 0u, 0u, 0u};         // passes per register block (uniform)
  uint32_t st[4] = {0u, 0u, 0u, 0u};         // of them staged (uniform)
  const uint32_t htag = (uint32_t)half << 31;

  // key rows: a tile wholly inside the rows is addressed from a base shared by
  // the wave plus this lane's row offset; a tile crossing the end (or a paged
  // cache) per lane, rows past the end reading zeros
  const uint8_t* kd = static_cast<const uint8_t*>(a.ki);
  const uint32_t lrow = (uint32_t)rl * KeyRow<FMT>::B, lsrow = (uint32_t)rl * KeyRow<FMT>::S;
  auto load_tile = [&](int t, KeyOp<FMT>& k) {
    const int e0 = e_wave + t * 32;
    if (!PAGED && e0 + 32 <= n_scan) {
      const int64_t r0 = kv_base + e0;
      load_key_row<FMT>(kd + r0 * KeyRow<FMT>::B + lrow, a.ki_scale + r0 * KeyRow<FMT>::S + lsrow,
                        half, k);
    } else {
      const int e = e0 + rl;
      const int64_t row = PAGED ? entry_row_if(a.b, kv_base, e, e < n_scan) : kv_base + e;
      load_key<FMT>(a.ki, a.ki_scale, row, e < n_scan, half, k);
    }
  };
  // the scores of one tile's product: the lane's four queries against its
  // entry.  WHOLE: some query of the group takes its row whole; TAIL: some
  // entry of the tile lies past a row's end (separate code, so that the
  // other tiles carry no test of it)
  auto score_tile = [&](int t, const f32x16_t& acc, auto whole_c, auto tail_c) {
    constexpr bool WHOLE = decltype(whole_c)::value;
    constexpr bool TAIL = decltype(tail_c)::value;
    const int e0 = e_wave + t * 32;          // the tile's first entry
    const int el = e0 + rl;                  // this lane's entry
    const uint32_t elt = (uint32_t)el | htag;
    auto stage_g = [&](int g, float sc, float thr) {
      const bool pass = sc >= thr;
      const uint64_t m = __ballot(pass);
      if (m != 0) {                          // (uniform)
        const uint32_t mlo = (uint32_t)m, mhi = (uint32_t)(m >> 32);
        const uint32_t pclo = __builtin_popcount(mlo), pchi = __builtin_popcount(mhi);
        if (ns[g] < (uint32_t)kStageSlots) {    // (then every pass is staged so far)
          const uint32_t slot = __builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, ns[g]));
          stage[wave][pass ? g * kStageCap + slot : 4 * kStageCap + lane] =
              make_uint2(__float_as_uint(sc), elt);
          st[g] = ns[g] + pclo + pchi;
        }
        ns[g] += pclo + pchi;
        cnt[2 * g] += pclo;
        cnt[2 * g + 1] += pchi;
      }
    };
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float sc;
      if constexpr (HW) sc = head_score(acc, g, hw[g], a.relu);
      else sc = head_score_unit(acc, g, a.relu);
      if constexpr (WHOLE) {
        if (whole[g] && el < nv[g])
          a.cand[(qblock + 2 * g + half) * (int64_t)a.cap + el] =
              make_uint2(score_key<SBF16>(sc), (uint32_t)el);
      }
      float thr = tf[g];
      if constexpr (TAIL) thr = el < nv[g] ? thr : INFINITY;
      stage_g(g, sc, thr);
    }
  };
  auto tile_live = [&](int t) { return e_wave + t * 32 < n_scan; };
  // tiles [0, t_full) lie wholly below the group's shortest row, so they need
  // no row-end test; they are scored in pairs, both products issued before
  // either is read
  int t_full = (n_lo - e_wave) / 32;
  t_full = t_full < 0 ? 0 : (t_full > GT ? GT : t_full);
  const int np_full = t_full / 2;
  auto do_pair = [&](int p, const KeyOp<FMT>* k, auto whole_c) {
    const f32x16_t acc0 = tile_dots<FMT>(aq, k[0]);
    const f32x16_t acc1 = tile_dots<FMT>(aq, k[1]);
    score_tile(2 * p, acc0, whole_c, std::false_type{});
    score_tile(2 * p + 1, acc1, whole_c, std::false_type{});
  };
  // a tile of those in contiguous rows: no test of the rows' end
  auto load_full = [&](int t, KeyOp<FMT>& k) {
    if constexpr (PAGED) {
      load_tile(t, k);
    } else {
      const int64_t r0 = kv_base + e_wave + t * 32;
      load_key_row<FMT>(kd + r0 * KeyRow<FMT>::B + lrow, a.ki_scale + r0 * KeyRow<FMT>::S + lsrow,
                        half, k);
    }
  };
  auto run = [&](auto whole_c) {
    if (np_full > 0) {
      KeyOp<FMT> ka[2], kb[2];
      load_full(0, ka[0]);
      load_full(1, ka[1]);
      for (int p = 0; p < np_full; p += 2) {
        const bool l1 = p + 1 < np_full;
        if (l1) {
          load_full(2 * p + 2, kb[0]);
          load_full(2 * p + 3, kb[1]);
        }
        do_pair(p, ka, whole_c);
        if (!l1) break;
        const bool l2 = p + 2 < np_full;
        if (l2) {
          load_full(2 * p + 4, ka[0]);
          load_full(2 * p + 5, ka[1]);
        }
        do_pair(p + 1, kb, whole_c);
        if (!l2) break;
      }
    }
    // the wave's other live tiles (at the rows' ends), one at a time
    for (int t = 2 * np_full; t < GT && tile_live(t); ++t) {
      KeyOp<FMT> kt;
      load_tile(t, kt);
      score_tile(t, tile_dots<FMT>(aq, kt), whole_c, std::true_type{});
    }
  };
  if (any_whole) run(std::true_type{});
  else run(std::false_type{});

  // the workgroup's span of each query's list: its staged candidates (a
  // (wave, register block) that staged more than its area holds sends both
  // rows to the exact redo by a count above cap), or for a row taken whole
  // its visible entries
  if (lane == 0) {
#pragma unroll
    for (int q = 0; q < QS; ++q) wcnt[wave][q] = cnt[q];
#pragma unroll
    for (int g = 0; g < 4; ++g) wover[wave][g] = ns[g] != st[g] ? 1u : 0u;
  }
  __syncthreads();
  if (tid < QS && qblock + tid < a.n_q) {
    const int64_t nv = visible(a, qblock + tid);
    uint32_t add = 0;
    if (nv > 0 && nv <= a.cap) {
      int64_t own = nv - e_wg;
      own = own < 0 ? 0 : (own > kWaves * EW ? kWaves * EW : own);
      add = (uint32_t)own;
    } else {
      bool over = false;
      for (int w = 0; w < kWaves; ++w) {
        over = over || wover[w][tid >> 1] != 0;
        add += wcnt[w][tid];
      }
      if (over) add += (uint32_t)a.cap + 1u;
    }
    gbase[tid] = add > 0 ? atomicAdd(&a.cnt[qblock + tid], add) : 0u;
  }
  __syncthreads();
  // each wave copies its areas out, query by query, in staging order
#pragma unroll
  for (int q = 0; q < QS; ++q) {
    if (qblock + q >= a.n_q) break;
    if (cnt[q] == 0) continue;               // (rows taken whole stage nothing)
    const int g = q >> 1;
    const uint32_t tag = (uint32_t)(q & 1);
    const uint32_t n = st[g];
    uint32_t base = gbase[q];
    for (int w = 0; w < wave; ++w) base += wcnt[w][q];
    uint2* list = a.cand + (qblock + q) * (int64_t)a.cap;
    for (uint32_t i0 = 0; i0 < n; i0 += 64) {
      const uint32_t i = i0 + lane;
      const uint2 c = i < n ? stage[wave][g * kStageCap + i] : make_uint2(0u, 0u);
      const bool mine = i < n && (c.y >> 31) == tag;
      const uint64_t m = __ballot(mine);
      if (mine) {
        const uint32_t slot = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                               __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (slot < (uint32_t)a.cap)
          list[slot] = make_uint2(score_key<SBF16>(__uint_as_float(c.x)), c.y & 0x7fffffffu);
      }
      base += (uint32_t)__builtin_popcountll(m);
    }
  }
}

// ------------------------------------------------------------------ 2. filter

// Grid: entry chunks and query groups, as the score kernel.  Pass 1
// scores the wave's tiles into an LDS row of keys per query of the group and
// counts the candidates per (wave, query) (streaming: after the workgroup's
// own threshold is selected from that row); one atomic per query reserves the
// workgroup's span of the list; pass 2 rescans the LDS rows and writes the
// candidates (each wave its own entries, so the reserved spans line up).
template <int FMT, bool SBF16, bool STREAM, bool PAGED>
__global__ __launch_bounds__(256) void itk_filter_kernel(ItkArgs a) {
  constexpr int TB = STREAM ? Tiling<FMT>::TB : 1;
  constexpr int TPW = STREAM ? Tiling<FMT>::TPW : kTilesPerWave;
  constexpr int NG = STREAM ? 1 : 4;
  constexpr int QS = STREAM ? 1 : 8;                   // query slots of a group
  constexpr int EW = TPW * 32;                         // entries per wave
  using skey_t = typename std::conditional<SBF16, uint16_t, uint32_t>::type;
  __shared__ skey_t lk[QS][kWaves * EW];
  __shared__ uint32_t wcnt[kWaves][QS];   // candidates per (wave, query)
  __shared__ uint32_t gbase[QS];          // the workgroup's first list slot per query
  __shared__ uint32_t stau[QS];           // the queries' thresholds
  __shared__ uint32_t send[QS];           // end of the workgroup's slots per query
  __shared__ RadixLds<256> frx;           // the workgroup's own threshold (streaming)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5, rl = lane & 31;

  // several queries per group (prefill): x = query group, y = entry chunk,
  // so the groups reading one chunk of keys run together and share it in L2;
  // streaming: x = entry chunk, y = query
  const unsigned bq = STREAM ? blockIdx.y : blockIdx.x, be = STREAM ? blockIdx.x : blockIdx.y;
  const int64_t qblock = (int64_t)bq * a.qpg;
  Group<FMT, NG> gr;
  load_group<FMT, NG>(a, qblock, gr);
  int64_t q_hi = qblock + a.qpg - 1;
  if (q_hi >= a.n_q) q_hi = a.n_q - 1;
  const int64_t n_scan = visible(a, q_hi);
  const int64_t e_wg = (int64_t)be * (kWaves * EW);
  const int e_wave = wave * EW;
  if (e_wg >= n_scan) return;            // the whole workgroup: no barrier reached

  // pass 1: keys into LDS, candidate counts per query in this lane
  uint32_t tau[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) tau[g] = !STREAM && gr.nv[g] > 0 ? a.tau[qblock + 2 * g + half] : 0u;
  uint32_t c[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) c[g] = 0;
  auto score_tile = [&](int t, const KeyOp<FMT>& k) {
    const int el = e_wave + t * 32 + rl;
    const f32x16_t acc = tile_dots<FMT>(gr.aq, k);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int ql = 2 * g + half;
      const uint32_t key = score_key<SBF16>(head_score(acc, g, gr.hw[g], a.relu));
      if (ql < QS) lk[ql][el] = (skey_t)key;
      if constexpr (!STREAM) c[g] += (e_wg + el < gr.nv[g] && key >= tau[g]) ? 1u : 0u;
    }
  };
  auto tile_live = [&](int t) { return e_wg + e_wave + t * 32 < n_scan; };
  // Paged keys (a separate instantiation, so the contiguous one keeps its
  // registers): with blocks of at least 32 entries each of this wave's tiles
  // (32 entries from a multiple of 32) lies in one block, whose id lane t
  // loads up front for tile t, so the key loads wait on no block-table read.
  const bool pre = PAGED && a.b.page_shift >= 5;
  int my_blk = -1;
  if (pre && lane < TPW && tile_live(lane))
    my_blk = a.b.pages[gr.qm.kv_base + ((e_wg + e_wave + lane * 32) >> a.b.page_shift)];
  auto key_row = [&](int t, int64_t e, bool ok) -> int64_t {
    if constexpr (!PAGED) {
      return gr.qm.kv_base + e;
    } else {
      if (pre) {
        const int64_t blk = __builtin_amdgcn_readlane(my_blk, t);
        const int64_t row = (blk << a.b.page_shift) + (e & ((1ll << a.b.page_shift) - 1));
        return ok && blk >= 0 && row < a.b.kv_rows ? row : 0;
      }
      return entry_row_if(a.b, gr.qm.kv_base, e, ok);
    }
  };
  if constexpr (STREAM) {
    constexpr int NB = TPW / TB;
    auto load_batch = [&](int b, KeyOp<FMT>* k) {
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const int64_t e = e_wg + e_wave + (b * TB + tb) * 32 + rl;
        load_key<FMT>(a.ki, a.ki_scale, key_row(b * TB + tb, e, e < n_scan), e < n_scan, half, k[tb]);
      }
    };
    auto score_batch = [&](int b, const KeyOp<FMT>* k) {
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
        if (tile_live(b * TB + tb)) score_tile(b * TB + tb, k[tb]);
    };
    if (tile_live(0)) {
      KeyOp<FMT> k0[TB], k1[TB];
      load_batch(0, k0);
      for (int b = 0; b < NB; b += 2) {
        const bool l1 = b + 1 < NB && tile_live((b + 1) * TB);
        if (l1) load_batch(b + 1, k1);
        score_batch(b, k0);
        if (!l1) break;
        const bool l2 = b + 2 < NB && tile_live((b + 2) * TB);
        if (l2) load_batch(b + 2, k0);
        score_batch(b + 1, k1);
        if (!l2) break;
      }
    }
  } else {
    // one tile at a time: occupancy hides the loads (more in flight per wave
    // measured slower)
    for (int t = 0; t < TPW; ++t) {
      if (!tile_live(t)) break;
      KeyOp<FMT> kt;
      const int64_t e = e_wg + e_wave + t * 32 + rl;
      load_key<FMT>(a.ki, a.ki_scale, key_row(t, e, e < n_scan), e < n_scan, half, kt);
      score_tile(t, kt);
    }
  }
  if constexpr (STREAM) {
    // the workgroup's own threshold: the key of rank ~3k * mine / n among its
    // mine = n_valid entries (+1 for rounding), all of them in rows of at
    // most cap entries
    __syncthreads();
    int64_t nvq = (gr.qm.t + 1) / a.m;
    if (nvq > gr.qm.kv_len) nvq = gr.qm.kv_len;
    if (nvq > a.max_n) nvq = a.max_n;
    int64_t nvalid = nvq - e_wg;
    if (nvalid > kWaves * EW) nvalid = kWaves * EW;
    uint32_t tw = 0;
    if (nvq > a.cap) {
      int64_t r = (3 * (int64_t)a.k * nvalid + nvq - 1) / nvq + 1;
      if (r < nvalid) {
        uint32_t rem;
        tw = radix_select_visit<SBF16 ? 16 : 32, 256>(
            frx, (uint32_t)r,
            [&](auto&& f) {
              for (int i = tid; i < nvalid; i += 256) f((uint32_t)lk[0][i]);
            },
            rem);
      }
    }
    uint32_t x = 0;
    for (int i = 0; i < EW; i += 64) {
      const int el = e_wave + i + lane;
      x += __builtin_popcountll(__ballot(el < nvalid && (uint32_t)lk[0][el] >= tw));
    }
    if (lane == 0) wcnt[wave][0] = x;
    __syncthreads();
    // the workgroup's region of the list: R = cap / (workgroups of the row)
    // slots from be * R; its count and threshold go to its header
    const int64_t nwg = (nvq + kWaves * EW - 1) / (kWaves * EW);
    const uint32_t reg = (uint32_t)(a.cap / nwg);
    if (tid == 0 && qblock < a.n_q) {
      uint32_t tot = 0;
      for (int w = 0; w < kWaves; ++w) tot += wcnt[w][0];
      a.hdr[qblock * kMaxWg + be] = make_uint2(tot, tw);
      gbase[0] = be * reg;
      send[0] = (be + 1) * reg;
      stau[0] = tw;
    }
    __syncthreads();
  } else {
    // sums over each half of the wave: lanes 0-31 count query 2g, lanes
    // 32-63 query 2g + 1 of register block g
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      uint32_t x = c[g];
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) x += __shfl_xor(x, o);
      const int ql = 2 * g + half;
      if (rl == 0 && ql < QS) wcnt[wave][ql] = x;
    }
    __syncthreads();
    if (tid < QS && qblock + tid < a.n_q) {
      uint32_t tot = 0;
      for (int w = 0; w < kWaves; ++w) tot += wcnt[w][tid];
      gbase[tid] = tot > 0 ? atomicAdd(&a.cnt[qblock + tid], tot) : 0u;
      send[tid] = (uint32_t)a.cap;
      stau[tid] = a.tau[qblock + tid];
    }
    __syncthreads();
  }

  // pass 2: each wave writes its entries' candidates, query by query (slots
  // past the workgroup's end are dropped; the count still records them, which
  // sends the row to the exact redo)
  for (int ql = 0; ql < QS; ++ql) {
    const int64_t q = qblock + ql;
    if (q >= a.n_q || wcnt[wave][ql] == 0) continue;   // uniform over the wave
    // visible entries of the group's query ql (consecutive positions of one
    // request, as load_group counts them)
    int64_t nvq = (gr.qm.t + ql + 1) / a.m;
    if (nvq > gr.qm.kv_len) nvq = gr.qm.kv_len;
    if (nvq > a.max_n) nvq = a.max_n;
    const uint32_t tq = stau[ql], end = send[ql];
    uint32_t base = gbase[ql];
    for (int w = 0; w < wave; ++w) base += wcnt[w][ql];
    uint2* list = a.cand + q * (int64_t)a.cap;
    for (int i = 0; i < EW; i += 64) {
      const int el = e_wave + i + lane;
      const uint32_t key = lk[ql][el];
      const bool f = e_wg + el < nvq && key >= tq;
      const uint64_t m = __ballot(f);
      if (f) {
        const uint32_t slot = base + __builtin_popcountll(m & ((1ull << lane) - 1ull));
        if (slot < end) list[slot] = make_uint2(key, (uint32_t)(e_wg + el));
      }
      base += __builtin_popcountll(m);
    }
  }
}

// ------------------------------------------------------------------ 3. select

// Selected entries of a row, marked in an LDS bitmap, written in index order
// to out[0..k): each thread owns a contiguous run of bitmap words.
template <int NT>
__device__ void emit_bitmap(const uint32_t* bm, int nwords, uint32_t* wsum, int32_t* out, int k) {
  const int tid = threadIdx.x;
  const int per = (nwords + NT - 1) / NT;
  const int w0 = tid * per;
  const int w1 = w0 + per < nwords ? w0 + per : nwords;
  uint32_t c = 0;
  for (int w = w0; w < w1; ++w) c += __builtin_popcount(bm[w]);
  uint32_t total;
  uint32_t pos = block_exclusive_scan<NT / 64>(c, wsum, total);
  for (int w = w0; w < w1; ++w) {
    uint32_t bits = bm[w];
    while (bits) {
      const int b = __builtin_ctz(bits);
      if (pos < (uint32_t)k) out[pos] = 32 * w + b;
      ++pos;
      bits &= bits - 1;
    }
  }
}

// Index of the nth (1-based) set bit of the LDS bitmap (nwords words; n at
// most the number of set bits), the same in every thread.
template <int NT>
__device__ uint32_t bitmap_nth(const uint32_t* bm, int nwords, uint32_t n, uint32_t* wsum,
                               uint32_t* found) {
  const int tid = threadIdx.x;
  const int per = (nwords + NT - 1) / NT;
  const int w0 = tid * per;
  const int w1 = w0 + per < nwords ? w0 + per : nwords;
  uint32_t c = 0;
  for (int w = w0; w < w1; ++w) c += __builtin_popcount(bm[w]);
  uint32_t total;
  uint32_t pos = block_exclusive_scan<NT / 64>(c, wsum, total);
  if (pos < n && n <= pos + c) {
    for (int w = w0; w < w1; ++w) {
      uint32_t bits = bm[w];
      const uint32_t pc = __builtin_popcount(bits);
      if (pos + pc >= n) {
        for (uint32_t i = pos + 1; i < n; ++i) bits &= bits - 1;   // drop the lower ones
        *found = 32u * w + __builtin_ctz(bits);
        break;
      }
      pos += pc;
    }
  }
  __syncthreads();
  return *found;
}

// at most this many entries tied at the k-th key are resolved through a
// short list (more: through the row's bitmap)
constexpr int kTieList = 64;
template <int NT>
struct SelectLds {
  RadixLds<NT> rx;
  uint32_t wsum[NT / 64];
  uint32_t found;
  uint32_t ntie;
  uint32_t tie[kTieList];          // the entries tied at the k-th key (few ties)
  uint32_t hcount[kMaxWg];         // streaming: the filter workgroups' counts
  uint32_t hfloor, htot, hover;    // their largest threshold, total, overflow
};

// The exact top-k of a row whose keys visit(f) produces (f(key, entry), each
// thread its share; every thread calls it): the k-th largest key tau by radix
// select, ties to the lowest entries (the needed one found in a short list
// of the tied entries, or by its rank among them in the bitmap), the chosen
// entries marked in the LDS bitmap (nwords words, cleared here) and written
// in index order to out[0..k).  The keys visited must include every key of
// the row at or above `floor`; if tau turns out below it, entries that were
// not visited could belong to the top-k: nothing is written and false is
// returned.  Always inlined: as a call, the visitor's captured state would
// go through scratch memory.
template <int KBITS, int NT, typename Visit>
__device__ __forceinline__ bool select_row(SelectLds<NT>& sh, uint32_t* bm, int nwords, int k, int32_t* out,
                           Visit visit, uint32_t floor = 0) {
  const int tid = threadIdx.x;
  uint32_t need, n_eq;
  const uint32_t tau = radix_select_visit<KBITS, NT>(
      sh.rx, (uint32_t)k, [&](auto&& f) { visit([&](uint32_t key, uint32_t) { f(key); }); }, need,
      &n_eq);
  if (tau < floor) return false;          // the same in every thread
  for (int w = tid; w < nwords; w += NT) bm[w] = 0;
  // of the entries tied at tau only the need lowest are kept: mark the tied
  // ones, find the need-th set bit of the row, start the bitmap again
  uint32_t iota = 0xffffffffu;
  if (need < n_eq && n_eq <= (uint32_t)kTieList) {
    // few entries tie at tau: their indices into a short list, and the
    // need-th lowest is the one with need - 1 lower ones (entries are distinct)
    if (tid == 0) sh.ntie = 0;
    __syncthreads();
    visit([&](uint32_t key, uint32_t e) {
      if (key == tau) {
        const uint32_t j = atomicAdd(&sh.ntie, 1u);
        if (j < (uint32_t)kTieList) sh.tie[j] = e;
      }
    });
    __syncthreads();
    if (tid < 64) {
      const uint32_t mine = (uint32_t)tid < n_eq ? sh.tie[tid] : 0xffffffffu;
      uint32_t below = 0;
      for (uint32_t j = 0; j < n_eq; ++j) below += sh.tie[j] < mine ? 1u : 0u;
      if ((uint32_t)tid < n_eq && below == need - 1) sh.found = mine;
    }
    __syncthreads();
    iota = sh.found;
  } else if (need < n_eq) {
    __syncthreads();
    visit([&](uint32_t key, uint32_t e) {
      if (key == tau) atomicOr(&bm[e >> 5], 1u << (e & 31));
    });
    __syncthreads();
    iota = bitmap_nth<NT>(bm, nwords, need, sh.wsum, &sh.found);
    for (int w = tid; w < nwords; w += NT) bm[w] = 0;
  }
  __syncthreads();
  visit([&](uint32_t key, uint32_t e) {
    if (key > tau || (key == tau && e <= iota)) atomicOr(&bm[e >> 5], 1u << (e & 31));
  });
  __syncthreads();
  emit_bitmap<NT>(bm, nwords, sh.wsum, out, k);
  return true;
}

// Grid: one workgroup per query.  A list of at most CPT * NT candidates is
// read once into registers (CPT per thread); a longer one is read from memory
// at every pass.  A row whose list overflowed or fell short of k is redone
// here exactly: its keys are recomputed tile by tile for every pass (the query
// in its group's slot, so the arithmetic is the score kernel's).
template <int FMT, bool SBF16, int NT, int CPT>
__global__ __launch_bounds__(NT) void itk_select_kernel(ItkArgs a) {
  constexpr int KBITS = SBF16 ? 16 : 32;
  constexpr int NW = NT / 64;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  SelectLds<NT>& sh = *reinterpret_cast<SelectLds<NT>*>(smem_raw);
  uint32_t* bm = reinterpret_cast<uint32_t*>(smem_raw + sizeof(SelectLds<NT>));
  const int tid = threadIdx.x;
  const int64_t q = blockIdx.x;
  const int64_t n = visible(a, q);
  int32_t* out = a.idx + q * (int64_t)a.k;
  if (n <= a.k) {
    for (int64_t j = tid; j < a.k; j += NT) out[j] = j < n ? (int32_t)j : -1;
    return;
  }
  const int nwords = (int)((n + 31) / 32);
  const bool streamed = a.qpg == 1;
  uint32_t c, floor, reg = 0;
  int64_t nwg = 0;
  if (streamed) {
    // the filter workgroups' headers: counts (each within its region of
    // reg = cap / nwg slots), the largest threshold
    nwg = (n + entries_per_wg<FMT>(true) - 1) / entries_per_wg<FMT>(true);
    reg = (uint32_t)(a.cap / nwg);
    if (tid == 0) {
      sh.hfloor = 0;
      sh.htot = 0;
      sh.hover = 0;
    }
    __syncthreads();
    uint32_t fl = 0, tot = 0, ov = 0;
    for (int64_t w = tid; w < nwg; w += NT) {
      const uint2 h = a.hdr[q * kMaxWg + w];
      sh.hcount[w] = h.x;
      fl = h.y > fl ? h.y : fl;
      tot += h.x;
      ov |= h.x > reg ? 1u : 0u;
    }
    // reduced within each wave first: atomics of every thread on one LDS
    // word serialise
    if ((int64_t)(tid & ~63) < nwg) {
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const uint32_t f2 = __shfl_xor(fl, o);
        fl = f2 > fl ? f2 : fl;
        tot += __shfl_xor(tot, o);
        ov |= __shfl_xor(ov, o);
      }
      if ((tid & 63) == 0) {
        atomicMax(&sh.hfloor, fl);
        atomicAdd(&sh.htot, tot);
        atomicOr(&sh.hover, ov);
      }
    }
    __syncthreads();
    c = sh.hover ? (uint32_t)a.cap + 1 : sh.htot;
    floor = sh.hfloor;
  } else {
    c = a.cnt[q];
    floor = a.tau[q];
  }
  auto redo = [&]() {
    // the exact redo over the whole row
    const int lane = tid & 63, wave = tid >> 6, half = lane >> 5, rl = lane & 31;
    const int64_t qblock = q / a.qpg * a.qpg;
    const int slot = (int)(q - qblock);
    Group<FMT, 4> gr;
    load_group<FMT, 4>(a, qblock, gr);
    const int gs = slot >> 1;             // register block of the query
    const bool mine = (slot & 1) == half; // lanes of the query's half
    select_row<KBITS, NT>(sh, bm, nwords, a.k, out, [&](auto&& f) {
      for (int64_t t0 = (int64_t)wave * 32; t0 < n; t0 += NW * 32) {
        const int64_t e = t0 + rl;
        KeyOp<FMT> kt;
        load_key<FMT>(a.ki, a.ki_scale, entry_row_if(a.b, gr.qm.kv_base, e, e < n), e < n, half, kt);
        const f32x16_t acc = tile_dots<FMT>(gr.aq, kt);
        float s = 0.0f;
#pragma unroll
        for (int g = 0; g < 4; ++g)
          if (g == gs) s = head_score(acc, g, gr.hw[g], a.relu);
        if (mine && e < n) f(score_key<SBF16>(s), (uint32_t)e);
      }
    });
  };
  if (c > (uint32_t)a.cap || c < (uint32_t)a.k) {
    redo();
    return;
  }
  const uint2* list = a.cand + q * (int64_t)a.cap;
  // slot i holds a candidate: below c (query groups), or within the count of
  // its workgroup's region (streaming)
  const uint32_t span = streamed ? (uint32_t)(nwg * reg) : c;
  auto live = [&](uint32_t i) {
    if (!streamed) return i < c;
    if (i >= span) return false;
    const uint32_t w = i / reg;
    return i - w * reg < sh.hcount[w];
  };
  if (span <= (uint32_t)(CPT * NT)) {
    uint2 cr[CPT];
    bool lv[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const uint32_t i = tid + j * NT;
      lv[j] = live(i);
      cr[j] = lv[j] ? list[i] : make_uint2(0, 0);
    }
    if (!select_row<KBITS, NT>(sh, bm, nwords, a.k, out, [&](auto&& f) {
#pragma unroll
          for (int j = 0; j < CPT; ++j)
            if (lv[j]) f(cr[j].x, cr[j].y);
        }, floor))
      redo();
  } else {
    if (!select_row<KBITS, NT>(sh, bm, nwords, a.k, out, [&](auto&& f) {
          for (uint32_t i = tid; i < span; i += NT) {
            if (!live(i)) continue;
            const uint2 ce = list[i];
            f(ce.x, ce.y);
          }
        }, floor))
      redo();
  }
}

// (by default the list of k <= 1024 fits the registers: 6k slots)
template <int FMT, bool SBF16, int NT, int CPT = 6144 / NT>
csa_status launch_select(const ItkArgs& a, size_t bm_bytes, hipStream_t s) {
  auto kern = itk_select_kernel<FMT, SBF16, NT, CPT>;
  const size_t lds = sizeof(SelectLds<NT>) + bm_bytes;
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (lds > 64 * 1024 && attr != hipSuccess)
    return csa_host::fail(CSA_ERR_HIP, "csa_indexer_topk: cannot reserve %zu B of LDS", lds);
  hipLaunchKernelGGL(kern, dim3((unsigned)a.n_q), dim3(NT), lds, s, a);
  return csa_host::check_launch("csa_indexer_topk (select)");
}

template <int FMT, bool SBF16>
csa_status launch_all(const ItkArgs& a, int64_t max_kv, hipStream_t s) {
  const int64_t groups = (a.n_q + a.qpg - 1) / a.qpg;
  const bool stream = a.qpg == 1;
  // query groups: the sample sets the thresholds and clears the counts;
  // streaming needs neither (each workgroup writes its own header)
  csa_status st = CSA_OK;
  if (!stream) {
    hipLaunchKernelGGL((itk_sample_kernel<FMT, SBF16>), dim3((unsigned)groups), dim3(kSampleThreads), 0, s, a);
    st = csa_host::check_launch("csa_indexer_topk (sample)");
  }
  if (st != CSA_OK) return st;
  const bool paged = a.b.pages != nullptr;
  if (stream) {
    const int64_t epw = entries_per_wg<FMT>(true);
    const dim3 fgrid((unsigned)((max_kv + epw - 1) / epw), (unsigned)groups);
    if (paged) hipLaunchKernelGGL((itk_filter_kernel<FMT, SBF16, true, true>), fgrid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((itk_filter_kernel<FMT, SBF16, true, false>), fgrid, dim3(256), 0, s, a);
  } else {
    const bool hw = a.head_w != nullptr;
    auto go = [&](auto gt_c) {
      constexpr int GT = decltype(gt_c)::value;
      const int64_t epw = kWaves * GT * 32;
      const dim3 fgrid((unsigned)groups, (unsigned)((max_kv + epw - 1) / epw));
      if (paged && hw) hipLaunchKernelGGL((itk_group_filter_kernel<FMT, SBF16, true, true, GT>), fgrid, dim3(256), 0, s, a);
      else if (paged) hipLaunchKernelGGL((itk_group_filter_kernel<FMT, SBF16, true, false, GT>), fgrid, dim3(256), 0, s, a);
      else if (hw) hipLaunchKernelGGL((itk_group_filter_kernel<FMT, SBF16, false, true, GT>), fgrid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((itk_group_filter_kernel<FMT, SBF16, false, false, GT>), fgrid, dim3(256), 0, s, a);
    };
    if (max_kv <= kShortRows) go(std::integral_constant<int, kGroupTilesShort>{});
    else go(std::integral_constant<int, kGroupTiles>{});
  }
  st = csa_host::check_launch("csa_indexer_topk (filter)");
  if (st != CSA_OK) return st;
  const size_t bm_bytes = (size_t)((max_kv < kBitmapMax ? max_kv : kBitmapMax) + 31) / 32 * 4;
  // few rows (decode): 16 waves per row; many: 8, so several rows share a CU
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  if (a.n_q < 2 * (int64_t)cus) {
    // fp32 indexer queries and keys: the exact redo's fp32 query group does
    // not fit the 128 registers of a 1024-lane workgroup, so 8 waves a row
    if constexpr (FMT == CSA_F32) return launch_select<FMT, SBF16, 512>(a, bm_bytes, s);
    else return launch_select<FMT, SBF16, 1024>(a, bm_bytes, s);
  }
  // many short rows (at most 1024 entries, so every entry is a candidate and
  // the list fits one wave's registers): one wave a row, whose barriers cost
  // next to nothing, and four times the rows resident
  if (max_kv <= 1024 && a.qpg > 1) return launch_select<FMT, SBF16, 64, 16>(a, bm_bytes, s);
  return launch_select<FMT, SBF16, 512>(a, bm_bytes, s);
}

// candidates kept per query: the thresholds aim at about 3k.  A multiple of
// the largest filter chunk (2048 entries), so that a row of at most cap
// entries gives every filter workgroup a region of a whole chunk.
int64_t cap_for(int32_t k) {
  int64_t c = 6 * (int64_t)k;
  c = c > 4096 ? c : 4096;
  return (c + 2047) / 2048 * 2048;
}

}  // namespace

using namespace csa_host;

extern "C" size_t csa_indexer_topk_workspace_size(int64_t n_q, int32_t k) {
  if (n_q <= 0 || k < 1) return 0;
  // tau and cnt per query, then the candidate lists (16-byte aligned), then
  // the streaming filter's workgroup headers
  const size_t head = ((size_t)n_q * 2 * 4 + 15) / 16 * 16;
  return head + (size_t)n_q * (size_t)cap_for(k) * 8 + (size_t)n_q * kMaxWg * 8;
}

namespace {

// Checks the arguments of csa_indexer_topk (all but the workspace) on the
// host; `who` names the entry point in the error.
csa_status itk_check(const csa_tensor* qi, int32_t n_heads, const csa_tensor* ki,
                     const csa_batch* batch, int32_t m, int32_t score_fmt, int32_t k,
                     const int32_t* idx, const char* who) {
  if (batch == nullptr || !fmt_valid_tensor(qi) || !fmt_valid_tensor(ki, false))
    return fail(CSA_ERR_INVALID_ARGUMENT, "%s: bad tensor or batch", who);
  if (batch->n_req < 1 || batch->n_q < 0 || batch->q_off == nullptr || batch->q_pos == nullptr ||
      batch->kv_off == nullptr)
    return fail(CSA_ERR_INVALID_ARGUMENT, "%s: bad batch descriptor", who);
  if (n_heads != kHI || qi->dim != kDI || ki->dim != kDI)
    return fail(CSA_ERR_UNSUPPORTED, "%s: implemented for 4 heads of dim 64", who);
  if (qi->fmt != ki->fmt || (qi->fmt != CSA_F32 && qi->fmt != CSA_BF16 && qi->fmt != CSA_MXFP4))
    return fail(CSA_ERR_UNSUPPORTED, "%s: qi and ki must both be F32, BF16 or MXFP4", who);
  if (score_fmt != CSA_F32 && score_fmt != CSA_BF16)
    return fail(CSA_ERR_UNSUPPORTED, "%s: scores must be F32 or BF16", who);
  if (qi->rows != batch->n_q * n_heads)
    return fail(CSA_ERR_INVALID_ARGUMENT, "%s: qi rows must be n_q * n_heads", who);
  if (m < 1) return fail(CSA_ERR_INVALID_ARGUMENT, "%s: m must be >= 1", who);
  if (k < 1 || k > 4096) return fail(CSA_ERR_INVALID_ARGUMENT, "%s: need 1 <= k <= 4096", who);
  if (batch->max_kv < 0) return fail(CSA_ERR_INVALID_ARGUMENT, "%s: max_kv < 0", who);
  if (batch->max_kv > kBitmapMax) return fail(CSA_ERR_UNSUPPORTED, "%s: rows above 2^20 entries", who);
  if (batch->n_q > 0x7fffffff) return fail(CSA_ERR_UNSUPPORTED, "%s: too many queries", who);
  if (batch->n_q > 0 && idx == nullptr) return fail(CSA_ERR_INVALID_ARGUMENT, "%s: null idx", who);
  return CSA_OK;
}

// Launches the three kernels of csa_indexer_topk with the candidate lists in
// `ws` (already checked: large enough and 16-byte aligned).
csa_status itk_launch(const csa_tensor* qi, int32_t n_heads, const float* head_w,
                      const csa_tensor* ki, const csa_batch* batch, int32_t m, int32_t relu,
                      int32_t score_fmt, int32_t k, int32_t* idx, char* ws, const char* who,
                      hipStream_t stream) {
  (void)n_heads;
  ItkArgs a{};
  a.qi = qi->data;
  a.qi_scale = static_cast<const uint8_t*>(qi->scale);
  a.head_w = head_w;
  a.ki = ki->data;
  a.ki_scale = static_cast<const uint8_t*>(ki->scale);
  a.b = BatchDev{batch->n_req, batch->q_off, batch->q_pos, batch->kv_off, nullptr, nullptr, ki->rows, 0};
  if (const csa_status st = batch_pages(batch, a.b, who); st != CSA_OK) return st;
  a.m = m;
  a.relu = relu ? 1 : 0;
  a.qpg = batch->n_req == 1 ? 8 : 1;
  a.n_q = batch->n_q;
  a.k = k;
  a.cap = (int)cap_for(k);
  a.tau = reinterpret_cast<uint32_t*>(ws);
  a.cnt = a.tau + batch->n_q;
  a.cand = reinterpret_cast<uint2*>(ws + ((size_t)batch->n_q * 2 * 4 + 15) / 16 * 16);
  a.hdr = a.cand + (size_t)batch->n_q * a.cap;
  a.idx = idx;
  const int64_t groups = (batch->n_q + a.qpg - 1) / a.qpg;
  const int64_t max_kv = batch->max_kv < ki->rows ? batch->max_kv : ki->rows;
  a.max_n = max_kv;
  // (grid y: the queries when streaming; else the entry chunks, at most 1024)
  if (groups > 0x7fffffff || (a.qpg == 1 && groups > 65535))
    return fail(CSA_ERR_UNSUPPORTED, "%s: problem too large for one launch", who);
  const bool sb = score_fmt == CSA_BF16;
  if (qi->fmt == CSA_F32) return sb ? launch_all<CSA_F32, true>(a, max_kv, stream) : launch_all<CSA_F32, false>(a, max_kv, stream);
  if (qi->fmt == CSA_BF16) return sb ? launch_all<CSA_BF16, true>(a, max_kv, stream) : launch_all<CSA_BF16, false>(a, max_kv, stream);
  return sb ? launch_all<CSA_MXFP4, true>(a, max_kv, stream) : launch_all<CSA_MXFP4, false>(a, max_kv, stream);
}

}  // namespace

extern "C" csa_status csa_indexer_topk(const csa_tensor* qi, int32_t n_heads, const float* head_w,
                                       const csa_tensor* ki, const csa_batch* batch, int32_t m,
                                       int32_t relu, int32_t score_fmt, int32_t k, int32_t* idx,
                                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  if (const csa_status st = itk_check(qi, n_heads, ki, batch, m, score_fmt, k, idx, "csa_indexer_topk");
      st != CSA_OK)
    return st;
  if (batch->n_q == 0) return CSA_OK;
  const size_t need = csa_indexer_topk_workspace_size(batch->n_q, k);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(CSA_ERR_WORKSPACE, "csa_indexer_topk: needs %zu workspace bytes", need);
  if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_indexer_topk: workspace must be 16-byte aligned");
  return itk_launch(qi, n_heads, head_w, ki, batch, m, relu, score_fmt, k, idx,
                    static_cast<char*>(workspace), "csa_indexer_topk", stream);
}


// ------------------------------------------------------------------ no allocation

// csa_indexer_topk_noalloc keeps the candidate lists in this file-scope
// device array instead of a caller workspace: one copy per GPU, held until
// the process ends.  Host code never passes the array's name to a kernel
// (on the host it is only a handle); it uses the device address that
// hipGetSymbolAddress returns for the current GPU.
namespace {

constexpr size_t kNoAllocScratch = 16u << 20;
__device__ __align__(256) unsigned char scratch[kNoAllocScratch];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current GPU, resolved once per device.
csa_status scratch_ptr(char** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(CSA_ERR_HIP, "csa_indexer_topk_noalloc: no current device (or more than %d)",
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(CSA_ERR_HIP, "csa_indexer_topk_noalloc: hipGetSymbolAddress failed (%s)",
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<char*>(g_scratch_ptr[dev]);
  return CSA_OK;
}

}  // namespace

extern "C" size_t csa_indexer_topk_noalloc_max_bytes(void) { return kNoAllocScratch; }

extern "C" csa_status csa_indexer_topk_noalloc(const csa_tensor* qi, int32_t n_heads,
                                               const float* head_w, const csa_tensor* ki,
                                               const csa_batch* batch, int32_t m, int32_t relu,
                                               int32_t score_fmt, int32_t k, int32_t* idx,
                                               hipStream_t stream) {
  clear_error();
  if (const csa_status st = itk_check(qi, n_heads, ki, batch, m, score_fmt, k, idx,
                                      "csa_indexer_topk_noalloc");
      st != CSA_OK)
    return st;
  if (batch->n_q == 0) return CSA_OK;
  const size_t need = csa_indexer_topk_workspace_size(batch->n_q, k);
  if (need > kNoAllocScratch)
    return fail(CSA_ERR_WORKSPACE,
                "csa_indexer_topk_noalloc: %lld queries at k = %d need %zu bytes of candidate "
                "lists, above the %zu-byte static scratch (use csa_indexer_topk)",
                (long long)batch->n_q, k, need, kNoAllocScratch);
  char* ws = nullptr;
  if (const csa_status st = scratch_ptr(&ws); st != CSA_OK) return st;
  return itk_launch(qi, n_heads, head_w, ki, batch, m, relu, score_fmt, k, idx, ws,
                    "csa_indexer_topk_noalloc", stream);
}
