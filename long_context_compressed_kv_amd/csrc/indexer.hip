// Lightning indexer scores (page "DeepSeek V4 深度解析", section 2, CSA step
// 2; the scoring arithmetic is in indexer_core.h).  For decode a wave keeps
// several key tiles in flight.  The key stream is the only large read: the
// kernel is HBM bound for decode and score-write bound for long prefill.
//   fp32  : v_mfma_f32_32x32x2f32, 32 per tile
//   bf16  : v_mfma_f32_32x32x16_bf16, 4 per tile
//   MXFP4 : v_mfma_scale_f32_32x32x64_f8f6f4 (e2m1 operands, e8m0 block
//           scales per lane), 1 per tile - the products and block sums are
//           exact, so this equals the lossless FP4 -> FP8 route.
#include <type_traits>

#include "indexer_core.h"

using namespace csa;

namespace {

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
  int vec_out;      // score rows start 16-byte aligned: stage and write vectors
};

// Tiles whose keys one wave loads before computing any of them when the
// kernel streams keys (one query per request, decode).  A prefill instead
// keeps one tile in flight and relies on occupancy, its cost being the score
// writes.
template <int FMT> struct Tiling;
// TPW = tiles per wave when streaming (each wave reads 16 to 32 KB of keys);
// batches of TB tiles are double-buffered.
template <> struct Tiling<CSA_F32> { static constexpr int TB = 1, TPW = 8; };
template <> struct Tiling<CSA_BF16> { static constexpr int TB = 1, TPW = 8; };
template <> struct Tiling<CSA_MXFP4> { static constexpr int TB = 8, TPW = 16; };

// entries per workgroup
template <int FMT>
constexpr int entries_per_wg(bool stream) {
  return kWaves * (stream ? Tiling<FMT>::TPW : kTilesPerWave) * 32;
}

// Grid: x = chunks of kEntriesPerWG entries, y = groups of qpg queries
// (qpg = 8 for a single request, else 1); neighbouring workgroups stream
// neighbouring key chunks.  Wave w scores the contiguous
// entries [w*256, w*256 + 256) of its chunk, one 32-entry tile at a time.
// A prefill (STREAM false) stages the chunk's 8 x 1024 scores in LDS and
// writes every query row out in 16-byte vectors (when rows are 16-byte
// aligned); decode stores each score directly.
template <int FMT, bool SBF16, bool STREAM>
__global__ __launch_bounds__(256) void indexer_kernel(IdxArgs a) {
  constexpr int TB = Tiling<FMT>::TB;
  using score_t = typename std::conditional<SBF16, uint16_t, float>::type;
  constexpr int VEC = 16 / (int)sizeof(score_t);      // scores per 16-byte vector
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int rl = lane & 31;

  const int64_t qblock = (int64_t)blockIdx.y * a.qpg;
  const QueryMeta qm = query_meta(a.b, qblock, a.m);
  const int64_t kv_base = qm.kv_base;
  // entries this group scans: up to the largest n_vis of its queries
  int64_t q_hi = qblock + a.qpg - 1;
  if (q_hi >= a.n_q) q_hi = a.n_q - 1;
  const QueryMeta qm_hi = query_meta(a.b, q_hi, a.m);
  const int64_t n_scan = qm_hi.n_vis < a.ld ? qm_hi.n_vis : a.ld;   // never past a row

  // visible entries of query ql of the group (one request, consecutive
  // positions); 0 past the batch
  auto nvis_of = [&](int ql) -> int {
    const int64_t qq = qblock + ql;
    if (ql >= a.qpg || qq >= a.n_q) return 0;
    int64_t v = (qm.t + ql + 1) / a.m;
    if (v > qm.kv_len) v = qm.kv_len;
    if (v > a.ld) v = a.ld;
    return (int)v;
  };

  // A operand (queries): this lane's row is (query rl/4, head rl%4)
  QueryOp<FMT> aq;
  const int qa = rl >> 2, ha = rl & 3;
  load_query<FMT>(a.qi, a.qi_scale, (qblock + qa) * kHI + ha, qa < a.qpg && qblock + qa < a.n_q, half, aq);

  // this lane's output queries: 2g + half for register block g
  // (streaming, a group is one query: only block 0 of the lower half has one)
  constexpr int NG = STREAM ? 1 : 4;
  int nv[NG];
  float hw[NG][kHI];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int ql = 2 * g + half;
    nv[g] = nvis_of(ql);
#pragma unroll
    for (int h = 0; h < kHI; ++h)
      hw[g][h] = (a.head_w != nullptr && nv[g] > 0) ? a.head_w[(qblock + ql) * kHI + h] : 1.0f;
  }

  constexpr int TPW = STREAM ? Tiling<FMT>::TPW : kTilesPerWave;
  const int64_t e_wg = (int64_t)blockIdx.x * entries_per_wg<FMT>(STREAM);
  const int e_wave = wave * (TPW * 32);                // first entry of this wave in the chunk

  // scores of tile t (keys k, this lane's entry e_wave + 32t + rl of the
  // chunk) for this lane's queries
  auto score_tile = [&](int t, const KeyOp<FMT>& k, score_t* stage, bool staged) {
    const int el = e_wave + t * 32 + rl;               // entry within the chunk
    const int64_t e = e_wg + el;                       // this lane's entry (B column)
    const f32x16_t acc = tile_dots<FMT>(aq, k);
    // ReLU + weighted head sum; register block g holds the 4 heads of
    // query 2g + half
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (e >= nv[g]) continue;                        // also covers queries past the batch
      const float s = head_score(acc, g, hw[g], a.relu);
      score_t o;
      if constexpr (SBF16) o = (uint16_t)pack_bf16x2_fast(s, 0.0f);
      else o = s;
      if (staged) stage[(2 * g + half) * kEntriesPerWG + el] = o;
      else static_cast<score_t*>(a.scores)[(qblock + 2 * g + half) * a.ld + e] = o;
    }
  };

  if constexpr (STREAM) {
    // batches of TB tiles, the keys of batch b+1 in flight while batch b is
    // scored
    constexpr int NB = TPW / TB;
    auto batch_live = [&](int b) { return e_wg + e_wave + b * TB * 32 < n_scan; };
    auto load_batch = [&](int b, KeyOp<FMT>* k) {
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const int64_t e = e_wg + e_wave + (b * TB + tb) * 32 + rl;
        load_key<FMT>(a.ki, a.ki_scale, entry_row_if(a.b, kv_base, e, e < n_scan), e < n_scan, half, k[tb]);
      }
    };
    auto score_batch = [&](int b, const KeyOp<FMT>* k) {
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        if (e_wg + e_wave + (b * TB + tb) * 32 >= n_scan) break;
        score_tile(b * TB + tb, k[tb], nullptr, false);
      }
    };
    if (!batch_live(0)) return;
    KeyOp<FMT> k0[TB], k1[TB];
    load_batch(0, k0);
    for (int b = 0; b < NB; b += 2) {
      const bool l1 = b + 1 < NB && batch_live(b + 1);
      if (l1) load_batch(b + 1, k1);
      score_batch(b, k0);
      if (!l1) break;
      const bool l2 = b + 2 < NB && batch_live(b + 2);
      if (l2) load_batch(b + 2, k0);
      score_batch(b + 1, k1);
      if (!l2) break;
    }
    return;
  }

  const bool staged = !STREAM && a.vec_out;
  score_t* stage = nullptr;
  if constexpr (!STREAM) {
    __shared__ __align__(16) score_t sc[8 * kEntriesPerWG];
    stage = sc;
  }
  // prefill: one tile at a time, occupancy hides the loads
  for (int t = 0; t < kTilesPerWave; ++t) {
    if (e_wg + e_wave + t * 32 >= n_scan) break;
    KeyOp<FMT> kt;
    const int64_t e = e_wg + e_wave + t * 32 + rl;
    load_key<FMT>(a.ki, a.ki_scale, entry_row_if(a.b, kv_base, e, e < n_scan), e < n_scan, half, kt);
    score_tile(t, kt, stage, staged);
  }
  if constexpr (!STREAM) {
    if (!staged) return;
    __syncthreads();
    // every query row of the chunk in 16-byte vectors; a vector that crosses
    // the query's visible end is written element by element
    constexpr int VPR = kEntriesPerWG / VEC;          // vectors per query row
    for (int i = threadIdx.x; i < 8 * VPR; i += 256) {
      const int ql = i / VPR;
      const int el = (i - ql * VPR) * VEC;
      const int nvq = nvis_of(ql);
      const int64_t e = e_wg + el;
      if (e >= nvq) continue;
      score_t* dst = static_cast<score_t*>(a.scores) + (qblock + ql) * a.ld + e;
      const score_t* src = stage + ql * kEntriesPerWG + el;
      if (e + VEC <= nvq) {
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
      } else {
        for (int j = 0; j < VEC && e + j < nvq; ++j) dst[j] = src[j];
      }
    }
  }
}

template <int FMT>
void launch(const IdxArgs& a, bool sbf16, dim3 grid, hipStream_t s) {
  if (a.qpg == 8 && sbf16) hipLaunchKernelGGL((indexer_kernel<FMT, true, false>), grid, dim3(256), 0, s, a);
  else if (a.qpg == 8) hipLaunchKernelGGL((indexer_kernel<FMT, false, false>), grid, dim3(256), 0, s, a);
  else if (sbf16) hipLaunchKernelGGL((indexer_kernel<FMT, true, true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((indexer_kernel<FMT, false, true>), grid, dim3(256), 0, s, a);
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
  if (const csa_status st = batch_pages(batch, a.b, "csa_indexer_score"); st != CSA_OK) return st;
  a.m = m;
  a.relu = relu ? 1 : 0;
  a.qpg = batch->n_req == 1 ? 8 : 1;
  a.n_q = batch->n_q;
  a.scores = scores;
  a.ld = ld;
  const int64_t gy = (batch->n_q + a.qpg - 1) / a.qpg;
  const int esz = score_fmt == CSA_BF16 ? 2 : 4;
  a.vec_out = (reinterpret_cast<uintptr_t>(scores) % 16 == 0) && ((ld * esz) % 16 == 0) ? 1 : 0;
  // (the kernel streams keys when one query per request: qpg == 1)
  const bool streams = a.qpg != 8;
  const int epw = qi->fmt == CSA_F32    ? entries_per_wg<CSA_F32>(streams)
                  : qi->fmt == CSA_BF16 ? entries_per_wg<CSA_BF16>(streams)
                                        : entries_per_wg<CSA_MXFP4>(streams);
  const int64_t gx = (batch->max_kv + epw - 1) / epw;
  if (gy > 65535 || gx > 0x7fffffff)
    return fail(CSA_ERR_UNSUPPORTED, "csa_indexer_score: problem too large for one launch");
  const dim3 grid((unsigned)gx, (unsigned)gy);
  const bool sb = score_fmt == CSA_BF16;
  if (qi->fmt == CSA_F32) launch<CSA_F32>(a, sb, grid, stream);
  else if (qi->fmt == CSA_BF16) launch<CSA_BF16>(a, sb, grid, stream);
  else launch<CSA_MXFP4>(a, sb, grid, stream);
  return check_launch("csa_indexer_score");
}
