// The projections around the path (page "DeepSeek V4 深度解析", section 2, the
// HCA paragraph: CSA and HCA both project their outputs in groups to cut
// compute; page "wmrh.cn/news/726125", "V4 改进一": the output side projected
// in groups, and the MLA passage before it: a low-rank query side, the
// key/value up-projections absorbed into the query and output projections).
// The pages give neither sizes nor formulas: these are plain projections
// y = x W^T (W stored [out, in]) of bf16 operands with fp32 accumulation on
// the matrix cores, batched over groups, and the grouped output projection as
// two launches of them.
//
// Tiles of 128 x 128 outputs over 64-deep slices of K.  Four waves each own
// a 64 x 64 quarter as 2 x 2 blocks of v_mfma_f32_32x32x16_bf16 (rows of x on
// M, rows of W on N, so both operands are K-contiguous rows).  Each slice of x
// and W (16 KB each) is copied from global memory straight into LDS
// (global_load_lds, 1 KB per instruction, no registers held), slice k+1
// copying while slice k multiplies, one barrier per slice.  An LDS row holds
// a row's 64 values (128 bytes) with its 16-byte chunks permuted by
// chunk ^ (row % 8); the permutation is made on the copy side (each lane
// fetches the chunk that belongs at its LDS position), so the operand reads,
// 16 bytes of 32 consecutive rows, meet every bank once per 8 lanes.  Two
// workgroups share a CU (64 KB of LDS each).
#include "common.h"

using namespace csa;

namespace {

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kSlice = kBM * kBK * 2;            // bytes of one operand slice
constexpr size_t kSmemGemm = 2 * 2 * kSlice;     // two slices of x and W

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;

struct GemmArgs {
  const uint16_t* x;
  const uint16_t* w;
  void* y;
  int64_t ldx, ldw, ldy;      // row strides (elements)
  int64_t sx, sw, sy;         // batch strides (elements)
  int M, N, K;
  int tiles_m, tiles_n;
};

// 16 bytes per lane from global memory to LDS at lds + 16 * lane (counted in
// vmcnt like a load).
__device__ __forceinline__ void copy16(uint32_t lds, const void* src) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" :: "s"(lds), "v"(src) : "memory", "m0");
}
__device__ __forceinline__ void wait_copies() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}
__device__ __forceinline__ void lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  extern __shared__ __align__(16) unsigned char smem[];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_u8*)smem;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // tile of this workgroup: consecutive workgroups sit on different XCDs, so
  // the index is first regrouped per XCD, then walked in bands of 8 tile rows
  // (neighbours share rows of x or W in their XCD's L2)
  unsigned pid = blockIdx.x;
  const unsigned nb = gridDim.x;
  if (nb % 8u == 0u) pid = (pid % 8u) * (nb / 8u) + pid / 8u;
  const int band = (int)(pid / (unsigned)(8 * g.tiles_n));
  const int first_m = band * 8;
  const int band_m = g.tiles_m - first_m < 8 ? g.tiles_m - first_m : 8;
  const int in_band = (int)(pid - (unsigned)band * (unsigned)(8 * g.tiles_n));
  const int tm = first_m + in_band % band_m;
  const int tn = in_band / band_m;
  const int row0 = tm * kBM, col0 = tn * kBN;

  const int64_t b = blockIdx.y;
  const uint16_t* x = g.x + b * g.sx;
  const uint16_t* w = g.w + b * g.sw;

  // copy sources: instruction j of this wave fills LDS chunks
  // p = (4 wave + j) 64 + lane, i.e. row p / 8 and physical chunk p % 8,
  // which holds logical chunk (p % 8) ^ (row % 8); rows past the matrix read
  // its last row (their outputs are never stored)
  const uint16_t* xs[4];
  const uint16_t* ws[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int p = (4 * wave + j) * 64 + lane;
    const int r = p >> 3;
    const int c = (p & 7) ^ (r & 7);
    const int xr = row0 + r < g.M ? row0 + r : g.M - 1;
    const int wr = col0 + r < g.N ? col0 + r : g.N - 1;
    xs[j] = x + (int64_t)xr * g.ldx + 8 * c;
    ws[j] = w + (int64_t)wr * g.ldw + 8 * c;
  }
  auto copy_slice = [&](int kt, int buf) {
    const uint32_t base = lds0 + buf * 2 * kSlice;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      copy16(__builtin_amdgcn_readfirstlane(base + (4 * wave + j) * 1024), xs[j] + kt * kBK);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      copy16(__builtin_amdgcn_readfirstlane(base + kSlice + (4 * wave + j) * 1024), ws[j] + kt * kBK);
  };

  // operand reads: block i of this wave's rows of x (j of W): row
  // 32 i + lane % 32 of its quarter; step s reads logical chunk
  // 2 s + lane / 32 (k = 16 s + 8 (lane / 32) .. + 7), at physical chunk
  // (2 s + lane / 32) ^ (lane % 8), since the quarter's rows start at
  // multiples of 8
  const int wm = wave >> 1, wn = wave & 1;
  const lds_u8* sm = (const lds_u8*)smem;
  uint32_t xoff[2], woff[2], coff[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    xoff[i] = (uint32_t)(wm * 64 + i * 32 + (lane & 31)) * 128;
    woff[i] = (uint32_t)kSlice + (uint32_t)(wn * 64 + i * 32 + (lane & 31)) * 128;
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) coff[s] = (uint32_t)(((2 * s + (lane >> 5)) ^ (lane & 7)) * 16);

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

  auto read16 = [&](uint32_t ofs) -> bf16x8_t {
    const u32x4_t v = *(const __attribute__((address_space(3))) u32x4_t*)(sm + ofs);
    return __builtin_bit_cast(bf16x8_t, v);
  };
  auto multiply = [&](int buf) {
    const uint32_t base = (uint32_t)(buf * 2 * kSlice);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8_t a[2], bw[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = read16(base + xoff[i] + coff[s]);
        bw[i] = read16(base + woff[i] + coff[s]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bw[j], acc[i][j], 0, 0, 0);
    }
  };

  const int nk = g.K / kBK;
  copy_slice(0, 0);
  wait_copies();
  lds_sync();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) copy_slice(kt + 1, (kt + 1) & 1);   // its buffer was read last slice
    multiply(kt & 1);
    wait_copies();                                         // this wave's copies of slice kt+1
    lds_sync();                                            // everyone's, and slice kt consumed
  }

  // C block (i, j): lane holds column lane % 32, rows 8 (r / 4) + 4 (lane / 32) + r % 4
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = col0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < g.M && col < g.N) {
          const int64_t at = b * g.sy + (int64_t)row * g.ldy + col;
          if constexpr (OUT_BF16)
            static_cast<uint16_t*>(g.y)[at] = (uint16_t)f32_to_bf16(acc[i][j][r]);
          else
            static_cast<float*>(g.y)[at] = acc[i][j][r];
        }
      }
    }
}

csa_status launch_gemm(const GemmArgs& a, int batch, int out_fmt, hipStream_t s) {
  const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
  if (tiles > 0x7fffffff) return csa_host::fail(CSA_ERR_UNSUPPORTED, "csa_linear: too many output tiles");
  const dim3 grid((unsigned)tiles, (unsigned)batch);
  if (out_fmt == CSA_BF16) {
    static const hipError_t attr = hipFuncSetAttribute((const void*)gemm_kernel<true>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSmemGemm);
    if (attr != hipSuccess) return csa_host::fail(CSA_ERR_HIP, "csa_linear: cannot reserve LDS");
    hipLaunchKernelGGL(gemm_kernel<true>, grid, dim3(256), kSmemGemm, s, a);
  } else {
    static const hipError_t attr = hipFuncSetAttribute((const void*)gemm_kernel<false>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSmemGemm);
    if (attr != hipSuccess) return csa_host::fail(CSA_ERR_HIP, "csa_linear: cannot reserve LDS");
    hipLaunchKernelGGL(gemm_kernel<false>, grid, dim3(256), kSmemGemm, s, a);
  }
  return csa_host::check_launch("csa_linear");
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Host checks shared by both entry points (what = the call's name).
csa_status check_linear(const char* what, const void* x, int64_t ldx, int64_t sx, const void* w,
                        int64_t ldw, int64_t sw, const void* y, int32_t y_fmt, int64_t ldy,
                        int64_t sy, int64_t M, int64_t N, int64_t K, int32_t batch) {
  using csa_host::fail;
  if (M < 0 || N < 0 || K <= 0 || batch < 1)
    return fail(CSA_ERR_INVALID_ARGUMENT, "%s: need M, N >= 0, K > 0, batch >= 1", what);
  if (M > 0x7fffffff || N > 0x7fffffff || K > 0x7fffffff || batch > 65535)
    return fail(CSA_ERR_UNSUPPORTED, "%s: sizes beyond 2^31 (batch beyond 65535)", what);
  if (K % kBK != 0) return fail(CSA_ERR_UNSUPPORTED, "%s: K must be a multiple of 64", what);
  if (y_fmt != CSA_F32 && y_fmt != CSA_BF16)
    return fail(CSA_ERR_UNSUPPORTED, "%s: y must be F32 or BF16", what);
  if (M == 0 || N == 0) return CSA_OK;
  if (x == nullptr || w == nullptr || y == nullptr) return fail(CSA_ERR_INVALID_ARGUMENT, "%s: null pointer", what);
  if (ldx < K || ldw < K || ldy < N)
    return fail(CSA_ERR_INVALID_ARGUMENT, "%s: leading dimensions must cover the rows", what);
  if (sx < 0 || sw < 0 || sy < 0) return fail(CSA_ERR_INVALID_ARGUMENT, "%s: negative batch stride", what);
  if (!aligned16(x) || !aligned16(w) || ldx % 8 != 0 || ldw % 8 != 0 || sx % 8 != 0 || sw % 8 != 0)
    return fail(CSA_ERR_INVALID_ARGUMENT, "%s: x and w rows must start on 16-byte boundaries", what);
  return CSA_OK;
}

GemmArgs make_args(const void* x, int64_t ldx, int64_t sx, const void* w, int64_t ldw, int64_t sw,
                   void* y, int64_t ldy, int64_t sy, int64_t M, int64_t N, int64_t K) {
  GemmArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.w = static_cast<const uint16_t*>(w);
  a.y = y;
  a.ldx = ldx; a.ldw = ldw; a.ldy = ldy;
  a.sx = sx; a.sw = sw; a.sy = sy;
  a.M = (int)M; a.N = (int)N; a.K = (int)K;
  a.tiles_m = (int)((M + kBM - 1) / kBM);
  a.tiles_n = (int)((N + kBN - 1) / kBN);
  return a;
}

}  // namespace

using namespace csa_host;

extern "C" csa_status csa_linear(const void* x, int64_t ldx, int64_t x_bstride, const void* w,
                                 int64_t ldw, int64_t w_bstride, void* y, int32_t y_fmt,
                                 int64_t ldy, int64_t y_bstride, int64_t M, int64_t N, int64_t K,
                                 int32_t batch, hipStream_t stream) {
  clear_error();
  if (const csa_status st = check_linear("csa_linear", x, ldx, x_bstride, w, ldw, w_bstride, y, y_fmt, ldy,
                                         y_bstride, M, N, K, batch);
      st != CSA_OK || M == 0 || N == 0)
    return st;
  const GemmArgs a = make_args(x, ldx, x_bstride, w, ldw, w_bstride, y, ldy, y_bstride, M, N, K);
  return launch_gemm(a, batch, y_fmt, stream);
}

extern "C" size_t csa_grouped_out_proj_workspace_size(int64_t n_q, int32_t groups, int32_t d_group) {
  if (n_q <= 0 || groups <= 0 || d_group <= 0) return 0;
  return (size_t)n_q * (size_t)groups * (size_t)d_group * 2 + 256;
}

extern "C" csa_status csa_grouped_out_proj(const void* o, int64_t n_q, int32_t n_heads, int32_t dim,
                                           int32_t groups, const void* w_group, int32_t d_group,
                                           const void* w_out, int32_t d_model, void* out,
                                           int32_t out_fmt, void* workspace, size_t workspace_bytes,
                                           hipStream_t stream) {
  clear_error();
  if (n_q < 0 || n_heads <= 0 || dim <= 0 || groups <= 0 || d_group <= 0 || d_model <= 0)
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_grouped_out_proj: sizes must be positive");
  if (n_heads % groups != 0)
    return fail(CSA_ERR_INVALID_ARGUMENT, "csa_grouped_out_proj: groups must divide the heads");
  const int64_t kg = (int64_t)(n_heads / groups) * dim;   // inputs of one group
  const int64_t mid = (int64_t)groups * d_group;           // concatenated group outputs
  if (kg % kBK != 0 || mid % kBK != 0)
    return fail(CSA_ERR_UNSUPPORTED,
                "csa_grouped_out_proj: (heads / groups) * dim and groups * d_group must be multiples of 64");
  if (out_fmt != CSA_F32 && out_fmt != CSA_BF16)
    return fail(CSA_ERR_UNSUPPORTED, "csa_grouped_out_proj: out must be F32 or BF16");
  if (n_q == 0) return CSA_OK;
  const size_t need = csa_grouped_out_proj_workspace_size(n_q, groups, d_group);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(CSA_ERR_WORKSPACE, "csa_grouped_out_proj: needs %zu workspace bytes", need);
  // the bf16 group results [n_q][groups * d_group], 256-byte aligned
  void* tmp = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(workspace) + 255) & ~(uintptr_t)255);
  if (static_cast<char*>(tmp) + (size_t)n_q * mid * 2 > static_cast<char*>(workspace) + workspace_bytes)
    return fail(CSA_ERR_WORKSPACE, "csa_grouped_out_proj: needs %zu workspace bytes", need);
  // group g: heads g H/G .. of every row (row stride H dim), its weight, and
  // columns g d_group .. of the group results
  csa_status st = check_linear("csa_grouped_out_proj", o, (int64_t)n_heads * dim, kg, w_group, kg,
                               (int64_t)d_group * kg, tmp, CSA_BF16, mid, d_group, n_q, d_group, kg, groups);
  if (st != CSA_OK) return st;
  st = check_linear("csa_grouped_out_proj", tmp, mid, 0, w_out, mid, 0, out, out_fmt, d_model, 0, n_q,
                    d_model, mid, 1);
  if (st != CSA_OK) return st;
  const GemmArgs g1 = make_args(o, (int64_t)n_heads * dim, kg, w_group, kg, (int64_t)d_group * kg, tmp,
                                mid, d_group, n_q, d_group, kg);
  st = launch_gemm(g1, groups, CSA_BF16, stream);
  if (st != CSA_OK) return st;
  const GemmArgs g2 = make_args(tmp, mid, 0, w_out, mid, 0, out, d_model, 0, n_q, d_model, mid);
  return launch_gemm(g2, 1, out_fmt, stream);
}
