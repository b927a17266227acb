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
// (exact, the scales are powers of two).
//
// Per tile and wave (bf16):
//   S^T = K Q^T        v_mfma_f32_32x32x16_bf16, keys on M, queries on N;
//                      lane (q = l%32, half = l/32) gets 16 keys of query q,
//                      key = 8*(i/4) + 4*half + (i%4) for register i
//   online softmax     per query, max/sum across the two halves by lane swap
//   O^T += V^T P^T     same instruction, d on M; the contraction slots of both
//                      operands follow the key order above, so P never leaves
//                      registers
// fp32 inputs use v_mfma_f32_32x32x2f32 with the same structure (one key per
// lane and instruction, so V is read straight from the K layout).
#include "common.h"

using namespace csa;

namespace {

constexpr int KT = 32;           // keys per tile
constexpr int kRawTag = 1 << 30;
constexpr float kLn2 = 0.69314718055994530942f;

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

// Where key kk of the workgroup's key list comes from.
struct KeySrc {
  int64_t row;  // row of the source tensor, -1 = no key (stage zeros)
  bool raw;     // raw tensor (else entry tensor)
  int tag;      // mask tag, -1 = never valid
};

template <bool SPARSE>
__device__ __forceinline__ KeySrc key_source(const AttnArgs& a, int kk, int nE, int64_t q_first,
                                             const QueryMeta& qm, int64_t kv_len, int64_t wlo,
                                             int64_t t_first, int nkeys) {
  KeySrc s{-1, false, -1};
  if (kk >= nkeys) return s;
  if (kk < nE) {
    if constexpr (SPARSE) {
      const int owner = kk / a.k;
      const int slot = kk - owner * a.k;
      const int j = a.idx[(q_first + owner) * (int64_t)a.k + slot];
      if (j >= 0 && j < kv_len) {
        s.row = qm.kv_base + j;
        s.tag = owner;
      }
    } else {
      s.row = qm.kv_base + kk;
      s.tag = kk;
    }
  } else {
    const int64_t p = wlo + (kk - nE);
    s.row = qm.raw_base + (p - qm.raw_pos);
    s.raw = true;
    s.tag = kRawTag | (int)(p - t_first + a.window);
  }
  return s;
}

// ------------------------------------------------------------------ kernel

template <int D, bool F32C, int KVF, bool SPARSE, int DSPLIT, bool OUT_BF16>
__global__ __launch_bounds__(512) void attn_kernel(AttnArgs a) {
  constexpr int DW = D / DSPLIT;                 // dims per wave
  constexpr int KSTR = F32C ? D + 4 : D + 8;     // K-layout row stride (elements)
  constexpr int VSTR = KT + 4;                   // V^T row stride (bf16 elements)
  using kelem_t = typename std::conditional<F32C, float, uint16_t>::type;

  extern __shared__ __align__(16) unsigned char smem[];
  kelem_t* klds = reinterpret_cast<kelem_t*>(smem);
  uint16_t* vt = reinterpret_cast<uint16_t*>(smem + KT * KSTR * sizeof(kelem_t));
  int* tags = reinterpret_cast<int*>(smem + KT * KSTR * sizeof(kelem_t) +
                                     (F32C ? 0 : D * VSTR * 2));
  float* sx = reinterpret_cast<float*>(tags + KT);   // [nrb][DSPLIT][64][16] partial logits

  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int ql = lane & 31;
  const int rb = wave / DSPLIT;
  const int dpart = wave - rb * DSPLIT;
  const int d0 = dpart * DW;

  const int64_t q_first = (int64_t)blockIdx.x * a.tok;
  int64_t q_last = q_first + a.tok - 1;
  if (q_last >= a.n_q) q_last = a.n_q - 1;
  const QueryMeta qm0 = query_meta(a.b, q_first, a.m);
  const int64_t t_first = qm0.t;
  const int64_t t_last = t_first + (q_last - q_first);
  const int64_t kv_len = a.b.kv_off != nullptr && a.b.kv_rows > 0
                             ? (clamp64(a.b.kv_off[find_request(a.b.q_off, a.b.n_req, q_first) + 1],
                                        qm0.kv_base, a.b.kv_rows) - qm0.kv_base)
                             : 0;

  // key list: [entries | window]
  int nE;
  if constexpr (SPARSE) {
    nE = a.kv != nullptr ? (int)(q_last - q_first + 1) * a.k : 0;
  } else {
    const int64_t nc = (t_last + 1) / a.m;
    nE = a.kv != nullptr ? (int)(nc < kv_len ? nc : kv_len) : 0;
  }
  int64_t wlo = 0, whi = -1;
  if (a.raw != nullptr && a.window > 0 && qm0.raw_len > 0) {
    wlo = t_first - a.window + 1;
    if (wlo < 0) wlo = 0;
    if (wlo < qm0.raw_pos) wlo = qm0.raw_pos;
    whi = t_last;
    if (whi > qm0.raw_pos + qm0.raw_len - 1) whi = qm0.raw_pos + qm0.raw_len - 1;
  }
  const int nW = whi >= wlo ? (int)(whi - wlo + 1) : 0;
  const int nkeys = nE + nW;

  // this lane's query row
  const int row_in_wg = rb * 32 + ql;
  const int g_row = row_in_wg / a.H;
  const int h_row = row_in_wg - g_row * a.H;
  const int64_t q_row = q_first + g_row;
  const bool row_live = q_row <= q_last;
  const int64_t t_row = t_first + g_row;
  int64_t nvis_row = (t_row + 1) / a.m;
  if (nvis_row > kv_len) nvis_row = kv_len;
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

  const int ntiles = (nkeys + KT - 1) / KT;
  for (int tile = 0; tile < ntiles; ++tile) {
    const int kbase = tile * KT;
    __syncthreads();   // previous tile fully consumed
    // ---- stage
    if constexpr (F32C) {
      constexpr int UPR = D / 4;                // float4 units per key row
      for (int u = tid; u < KT * UPR; u += nthreads) {
        const int key = u / UPR;
        const int d = (u - key * UPR) * 4;
        const KeySrc s = key_source<SPARSE>(a, kbase + key, nE, q_first, qm0, kv_len, wlo,
                                            t_first, nkeys);
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (s.row >= 0) {
          const float* src = static_cast<const float*>(s.raw ? a.raw : a.kv);
          v = *reinterpret_cast<const float4*>(src + s.row * D + d);
        }
        *reinterpret_cast<float4*>(klds + key * KSTR + d) = v;
        if (d == 0) tags[key] = s.tag;
      }
    } else {
      constexpr int DG = D / 8;                 // 8-dim groups per row
      for (int u = tid; u < (KT / 4) * DG; u += nthreads) {
        const int k4 = u / DG;
        const int d = (u - k4 * DG) * 8;
        uint4 v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = k4 * 4 + j;
          const KeySrc s = key_source<SPARSE>(a, kbase + key, nE, q_first, qm0, kv_len, wlo,
                                              t_first, nkeys);
          v[j] = make_uint4(0, 0, 0, 0);
          if (s.row >= 0) {
            if (s.raw)
              v[j] = load_key8_bf16<CSA_BF16>(a.raw, nullptr, nullptr, s.row, d, D);
            else
              v[j] = load_key8_bf16<KVF>(a.kv, a.kv_scale, a.kv_rope, s.row, d, D);
          }
          *reinterpret_cast<uint4*>(klds + key * KSTR + d) = v[j];
          if (d == 0) tags[key] = s.tag;
        }
        // transpose 4 keys x 8 dims into V^T rows (4 keys = 8 bytes per dim)
        const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&v[0]);
        const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&v[1]);
        const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&v[2]);
        const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&v[3]);
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
    __syncthreads();

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
      for (int i = 0; i < 16; ++i) mine[i] = acc_s[i];
      __syncthreads();
      acc_s = f32x16_t{};
#pragma unroll
      for (int p = 0; p < DSPLIT; ++p) {
        const float* part = sx + ((rb * DSPLIT + p) * 64 + lane) * 16;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc_s[i] += part[i];
      }
    }

    // ---- mask + online softmax (base 2)
    float s[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = 8 * (i >> 2) + 4 * half + (i & 3);
      const int tg = tags[key];
      bool ok;
      if (tg < 0) ok = false;
      else if (tg & kRawTag) {
        const int rel = tg & (kRawTag - 1);
        ok = rel > g_row && rel <= g_row + a.window;
      } else if (SPARSE) ok = tg == g_row;
      else ok = tg < nvis_row;
      s[i] = ok ? acc_s[i] * a.scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, s[i]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    float alpha = 1.0f;
    float p[16];
    if (m_new == -INFINITY) {
#pragma unroll
      for (int i = 0; i < 16; ++i) p[i] = 0.0f;
    } else {
      alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(s[i] - m_new);
    }
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) psum += p[i];
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc_o[db][i] *= alpha;

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
  if (a.lse != nullptr && half == 0 && dpart == 0)
    a.lse[qrow_index] = l_tot > 0.0f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = d0 + db * 32 + 8 * r4 + 4 * half;
      const float o0 = acc_o[db][4 * r4 + 0] * inv, o1 = acc_o[db][4 * r4 + 1] * inv;
      const float o2 = acc_o[db][4 * r4 + 2] * inv, o3 = acc_o[db][4 * r4 + 3] * inv;
      if constexpr (OUT_BF16) {
        uint2 u;
        u.x = pack_bf16x2(o0, o1);
        u.y = pack_bf16x2(o2, o3);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + qrow_index * D + d) = u;
      } else {
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + qrow_index * D + d) =
            make_float4(o0, o1, o2, o3);
      }
    }
  }
}

template <int D, bool F32C, int KVF, bool SPARSE, int DSPLIT>
csa_status launch_attn(const AttnArgs& a, bool out_bf16, hipStream_t stream) {
  constexpr int KSTR = F32C ? D + 4 : D + 8;
  const size_t kbytes = (size_t)KT * KSTR * (F32C ? 4 : 2);
  const size_t vbytes = F32C ? 0 : (size_t)D * (KT + 4) * 2;
  const size_t sxbytes = DSPLIT > 1 ? (size_t)a.nrb * DSPLIT * 64 * 16 * 4 : 0;
  const size_t smem = kbytes + vbytes + KT * 4 + sxbytes;
  const int threads = a.nrb * DSPLIT * 64;
  const int64_t nblk = (a.n_q + a.tok - 1) / a.tok;
  if (nblk > 0x7fffffff) return csa_host::fail(CSA_ERR_INVALID_ARGUMENT, "attn: too many queries");
  auto kern = out_bf16 ? attn_kernel<D, F32C, KVF, SPARSE, DSPLIT, true>
                       : attn_kernel<D, F32C, KVF, SPARSE, DSPLIT, false>;
  if (smem > 64 * 1024 &&
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)smem) != hipSuccess)
    return csa_host::fail(CSA_ERR_HIP, "csa_sparse_mqa_attn: cannot reserve %zu B of LDS", smem);
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(threads), smem, stream, a);
  return csa_host::check_launch("csa_sparse_mqa_attn");
}

template <int D, bool F32C, int KVF, int DSPLIT>
csa_status launch_mode(const AttnArgs& a, bool sparse, bool out_bf16, hipStream_t s) {
  return sparse ? launch_attn<D, F32C, KVF, true, DSPLIT>(a, out_bf16, s)
                : launch_attn<D, F32C, KVF, false, DSPLIT>(a, out_bf16, s);
}

}  // namespace

using namespace csa_host;

extern "C" csa_status csa_sparse_mqa_attn(const csa_tensor* q, int32_t n_heads,
                                          const csa_tensor* kv, const int32_t* idx, int32_t k,
                                          const csa_tensor* raw, int32_t window,
                                          const csa_batch* batch, int32_t m, float scale,
                                          void* out, int32_t out_fmt, float* lse,
                                          hipStream_t stream) {
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
  if (H > 128 && !(H % 128 == 0))
    return fail(CSA_ERR_UNSUPPORTED, "csa_sparse_mqa_attn: n_heads above 128 must be a multiple of 128");
  if (out == nullptr) return fail(CSA_ERR_INVALID_ARGUMENT, "csa_sparse_mqa_attn: null out");
  if (out_fmt != CSA_F32 && out_fmt != CSA_BF16)
    return fail(CSA_ERR_UNSUPPORTED, "csa_sparse_mqa_attn: out must be F32 or BF16");
  if (m < 1) return fail(CSA_ERR_INVALID_ARGUMENT, "csa_sparse_mqa_attn: m must be >= 1");
  const bool has_kv = kv != nullptr && kv->rows > 0;
  const bool has_raw = raw != nullptr && raw->rows > 0 && window > 0;
  if (has_kv) {
    if (!fmt_valid_tensor(kv) || kv->dim != D)
      return fail(CSA_ERR_INVALID_ARGUMENT, "csa_sparse_mqa_attn: bad kv tensor");
    if (batch->kv_off == nullptr)
      return fail(CSA_ERR_INVALID_ARGUMENT, "csa_sparse_mqa_attn: kv given without kv_off");
  }
  if (has_raw) {
    if (!fmt_valid_tensor(raw) || raw->dim != D || raw->fmt != q->fmt)
      return fail(CSA_ERR_INVALID_ARGUMENT, "csa_sparse_mqa_attn: raw must match q's format and dim");
    if (batch->raw_off == nullptr || batch->raw_pos == nullptr)
      return fail(CSA_ERR_INVALID_ARGUMENT, "csa_sparse_mqa_attn: raw given without raw_off/raw_pos");
    if (window > (1 << 20))
      return fail(CSA_ERR_UNSUPPORTED, "csa_sparse_mqa_attn: window too large");
  }
  if (window < 0) return fail(CSA_ERR_INVALID_ARGUMENT, "csa_sparse_mqa_attn: negative window");
  const bool sparse = idx != nullptr;
  if (sparse && has_kv && (k < 1 || k > 4096))
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_sparse_mqa_attn: need 1 <= k <= 4096");

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

  // rows per workgroup: 128 for D = 128 (several tokens when H < 128);
  // one token (H rows, at least 32) for D = 512
  int rows = D == 128 ? (H > 128 ? H : 128) : (H < 32 ? 32 : H);
  if (D == 512 && H > 128) return fail(CSA_ERR_UNSUPPORTED, "csa_sparse_mqa_attn: D = 512 needs n_heads <= 128");
  if (D == 128 && H > 128) rows = H;
  if (rows > 256) return fail(CSA_ERR_UNSUPPORTED, "csa_sparse_mqa_attn: too many heads");
  a.tok = rows / H > 0 ? rows / H : 1;
  a.nrb = rows / 32;
  if (a.tok > 1 && batch->n_req > 1)
    return fail(CSA_ERR_UNSUPPORTED, "csa_sparse_mqa_attn: n_heads < 32 (D=512) or < 128 (D=128) needs a single request");
  const bool ob = out_fmt == CSA_BF16;
  const int kvf = has_kv ? kv->fmt : (f32c ? CSA_F32 : CSA_BF16);
  if (f32c) return launch_mode<128, true, CSA_F32, 1>(a, sparse, ob, stream);
  if (D == 128) return launch_mode<128, false, CSA_BF16, 1>(a, sparse, ob, stream);
  if (kvf == CSA_FP8_MIXED) return launch_mode<512, false, CSA_FP8_MIXED, 2>(a, sparse, ob, stream);
  return launch_mode<512, false, CSA_BF16, 2>(a, sparse, ob, stream);
}
