// Decode-time compression through a per-request state (page "DeepSeek V4
// 深度解析", section 4, the paragraph on KV-cache management for the hybrid
// attention: a fixed per-request state holds the window and the tail of
// tokens not yet compressed; finished entries go to the compressed cache).
//
// Each call appends one raw token to every request of a batch.  With w <= 2m
// a position lies in the windows of at most two entries (its own block's and
// the next block's), so the state of a request is two open entries, each an
// online softmax over the entry's slots so far: the running maximum of the
// logits, the running sum of their exponentials and the correspondingly
// weighted sum of the raw rows, all fp32, kept in the slot given by the
// entry's parity.  Entry i's slot is reset at the first valid position of its
// window, max(0, (i+1)m - w), and the entry is finished (divided by the sum
// and stored in the cache format) when position (i+1)m - 1 arrives.  The raw
// token can also be written to a per-request ring of window rows.
//
// One wave per request; lane l holds dims [l*dim/64, (l+1)*dim/64).
#include "common.h"
#include "kvrow.h"

using namespace csa;

namespace {

constexpr int kHead = 4;   // floats before an open entry's weighted row: max, sum, 2 unused

struct AppendArgs {
  const void* x;          // [n_req, dim] F32 or BF16
  const float* logits;    // [n_req]
  const float* bias;      // [w]
  int m, w, dim;
  int n_req;
  const int64_t* pos;     // [n_req]
  float* state;           // [n_req][2][dim + kHead]
  const int64_t* entry_off;
  const int32_t* pages;   // or a block table: entry i of r at row pages[r*page_stride + i/P]*P + i%P
  int64_t page_stride;
  int page_shift;         // P = 2^page_shift
  void* cache;            // entry rows (F32 / BF16 / mixed nope codes)
  uint8_t* cache_scale;
  uint16_t* cache_rope;
  int64_t cache_rows;
  void* window;           // ring rows (F32 / BF16), or null
  const int64_t* window_off;
  int64_t window_rows_total;
  int window_rows;        // ring capacity per request
};

template <int XF, int OUTF, int WF>
__global__ __launch_bounds__(64) void kv_append_kernel(AppendArgs a) {
  const int r = blockIdx.x;
  const int lane = threadIdx.x;
  const int64_t p = a.pos[r];
  if (p < 0) return;
  const int vpl = a.dim >> 6;
  const int d0 = lane * vpl;

  float xv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    xv[j] = 0.0f;
    if (j < vpl) {
      if constexpr (XF == CSA_F32) xv[j] = static_cast<const float*>(a.x)[(int64_t)r * a.dim + d0 + j];
      else xv[j] = bf16_to_f32(static_cast<const uint16_t*>(a.x)[(int64_t)r * a.dim + d0 + j]);
    }
  }
  const float z = a.logits[r];
  const int64_t m = a.m, w = a.w;

  // the (at most two) entries whose window [(i+1)m - w, (i+1)m - 1] holds p
  // are i_lo = ceil((p + 1) / m) - 1 .. i_hi <= i_lo + 1; both slots and both
  // biases are loaded at once, then each entry is updated
  const int64_t i_lo = (p + m) / m - 1;
  const int64_t i_hi = (p + w) / m - 1;
  float mx[2], l[2], acc[2][8], lg[2];
  bool fresh[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int64_t i = i_lo + e;
    const int64_t start = (i + 1) * m - w;
    fresh[e] = p == (start > 0 ? start : 0);    // the entry's first valid slot
    const bool live = i <= i_hi;
    const float* st = a.state + ((int64_t)r * 2 + (i & 1)) * (a.dim + kHead);
    mx[e] = live && !fresh[e] ? st[0] : -INFINITY;
    l[e] = live && !fresh[e] ? st[1] : 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[e][j] = live && !fresh[e] && j < vpl ? st[kHead + d0 + j] : 0.0f;
    lg[e] = live ? z + a.bias[p - start] : 0.0f;
  }
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int64_t i = i_lo + e;
    if (i > i_hi) break;
    // online softmax: raise the maximum first, then add this slot's weight
    if (lg[e] > mx[e]) {
      const float sc = expf(mx[e] - lg[e]);   // 0 when the entry was empty
      l[e] *= sc;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[e][j] *= sc;
      mx[e] = lg[e];
    }
    const float ew = expf(lg[e] - mx[e]);
    l[e] += ew;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[e][j] = fmaf(ew, xv[j], acc[e][j]);

    if (p == (i + 1) * m - 1) {
      // the entry is complete
      const float inv = l[e] > 0.0f ? 1.0f / l[e] : 0.0f;
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = acc[e][j] * inv;
      int64_t row = -1;
      if (a.pages == nullptr) {
        row = a.entry_off[r] + i;
      } else if ((i >> a.page_shift) < a.page_stride) {
        const int64_t blk = a.pages[(int64_t)r * a.page_stride + (i >> a.page_shift)];
        row = blk < 0 ? -1 : (blk << a.page_shift) + (i & ((1ll << a.page_shift) - 1));
      }
      if (row < 0 || row >= a.cache_rows) continue;   // metadata outside the cache: not written
      if constexpr (OUTF == CSA_F32) {
        float* dst = static_cast<float*>(a.cache) + row * a.dim + d0;
        for (int j = 0; j < vpl; ++j) dst[j] = v[j];
      } else if constexpr (OUTF == CSA_BF16) {
        uint16_t* dst = static_cast<uint16_t*>(a.cache) + row * a.dim + d0;
        for (int j = 0; j < vpl; ++j) dst[j] = (uint16_t)f32_to_bf16(v[j]);
      } else {   // mixed format, dim 512: eight dims per lane
        encode_kv_mixed_row_wave(v, static_cast<uint8_t*>(a.cache) + row * 448, a.cache_scale + row * 4,
                                 a.cache_rope + row * 64);
      }
    } else {
      float* st = a.state + ((int64_t)r * 2 + (i & 1)) * (a.dim + kHead);
      if (lane == 0) {
        st[0] = mx[e];
        st[1] = l[e];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < vpl) st[kHead + d0 + j] = acc[e][j];
    }
  }

  if constexpr (WF >= 0) {
    const int64_t row = a.window_off[r] + p % a.window_rows;
    if (row >= 0 && row < a.window_rows_total) {
      if constexpr (WF == CSA_F32) {
        float* dst = static_cast<float*>(a.window) + row * a.dim + d0;
        for (int j = 0; j < vpl; ++j) dst[j] = xv[j];
      } else {
        uint16_t* dst = static_cast<uint16_t*>(a.window) + row * a.dim + d0;
        for (int j = 0; j < vpl; ++j) dst[j] = (uint16_t)f32_to_bf16(xv[j]);
      }
    }
  }
}

template <int XF, int OUTF>
void launch_out(const AppendArgs& a, int wf, hipStream_t s) {
  const dim3 grid((unsigned)a.n_req), block(64);
  if (wf == CSA_F32) hipLaunchKernelGGL((kv_append_kernel<XF, OUTF, CSA_F32>), grid, block, 0, s, a);
  else if (wf == CSA_BF16) hipLaunchKernelGGL((kv_append_kernel<XF, OUTF, CSA_BF16>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((kv_append_kernel<XF, OUTF, -1>), grid, block, 0, s, a);
}

template <int XF>
void launch_in(const AppendArgs& a, int outf, int wf, hipStream_t s) {
  if (outf == CSA_F32) launch_out<XF, CSA_F32>(a, wf, s);
  else if (outf == CSA_BF16) launch_out<XF, CSA_BF16>(a, wf, s);
  else launch_out<XF, CSA_FP8_MIXED>(a, wf, s);
}

}  // namespace

using namespace csa_host;

extern "C" size_t csa_kv_append_state_size(int64_t n_req, int32_t dim) {
  if (n_req <= 0 || dim <= 0) return 0;
  return (size_t)n_req * 2 * ((size_t)dim + kHead) * sizeof(float);
}

extern "C" csa_status csa_kv_compress_append(const csa_tensor* x, const float* logits,
                                             const float* slot_bias, int32_t m, int32_t w,
                                             const int64_t* pos, float* state,
                                             const int64_t* entry_off, const int32_t* block_table,
                                             int64_t block_stride, int32_t block_rows,
                                             const csa_tensor* cache, const csa_tensor* window,
                                             const int64_t* window_off, int32_t window_rows,
                                             hipStream_t stream) {
  clear_error();
  if (!fmt_valid_tensor(x) || !fmt_valid_tensor(cache))
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_kv_compress_append: bad tensor descriptor");
  if (x->fmt != CSA_F32 && x->fmt != CSA_BF16)
    return fail(CSA_ERR_UNSUPPORTED, "csa_kv_compress_append: raw rows must be F32 or BF16");
  if (cache->fmt != CSA_F32 && cache->fmt != CSA_BF16 && cache->fmt != CSA_FP8_MIXED)
    return fail(CSA_ERR_UNSUPPORTED, "csa_kv_compress_append: cache must be F32, BF16 or FP8_MIXED");
  const int d = x->dim;
  if (cache->dim != d) return fail(CSA_ERR_INVALID_ARGUMENT, "csa_kv_compress_append: dim mismatch");
  if (d != 64 && d != 128 && d != 256 && d != 512)
    return fail(CSA_ERR_UNSUPPORTED, "csa_kv_compress_append: dim must be 64, 128, 256 or 512");
  if (m < 1 || w < m || w > 2 * m || w > 1024)
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_kv_compress_append: need 1 <= m <= w <= min(2m, 1024)");
  const int64_t n_req = x->rows;
  if (n_req > 0x7fffffff)
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_kv_compress_append: too many requests");
  if (window != nullptr) {
    if (!fmt_valid_tensor(window) || (window->fmt != CSA_F32 && window->fmt != CSA_BF16) ||
        window->dim != d)
      return fail(CSA_ERR_INVALID_ARGUMENT, "csa_kv_compress_append: window must be F32 or BF16 rows of dim");
    if (window_off == nullptr || window_rows < 1)
      return fail(CSA_ERR_INVALID_ARGUMENT, "csa_kv_compress_append: window needs window_off and window_rows >= 1");
  }
  if (block_table != nullptr &&
      (block_stride < 1 || block_rows < 1 || block_rows > (1 << 20) || (block_rows & (block_rows - 1)) != 0))
    return fail(CSA_ERR_INVALID_ARGUMENT,
                "csa_kv_compress_append: block_table needs block_stride >= 1 and block_rows a power of two in [1, 2^20]");
  if (n_req == 0) return CSA_OK;
  if (logits == nullptr || slot_bias == nullptr || pos == nullptr || state == nullptr ||
      (entry_off == nullptr && block_table == nullptr))
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_kv_compress_append: null pointer");
  AppendArgs a{};
  a.x = x->data;
  a.logits = logits;
  a.bias = slot_bias;
  a.m = m;
  a.w = w;
  a.dim = d;
  a.n_req = (int)n_req;
  a.pos = pos;
  a.state = state;
  a.entry_off = entry_off;
  a.pages = block_table;
  a.page_stride = block_table != nullptr ? block_stride : 0;
  a.page_shift = block_table != nullptr ? __builtin_ctz((unsigned)block_rows) : 0;
  a.cache = cache->data;
  a.cache_scale = static_cast<uint8_t*>(cache->scale);
  a.cache_rope = static_cast<uint16_t*>(cache->rope);
  a.cache_rows = cache->rows;
  a.window = window != nullptr ? window->data : nullptr;
  a.window_off = window_off;
  a.window_rows_total = window != nullptr ? window->rows : 0;
  a.window_rows = window_rows;
  const int wf = window != nullptr ? window->fmt : -1;
  if (x->fmt == CSA_F32) launch_in<CSA_F32>(a, cache->fmt, wf, stream);
  else launch_in<CSA_BF16>(a, cache->fmt, wf, stream);
  return check_launch("csa_kv_compress_append");
}
