// n-way log-sum-exp merge of partial attentions (used by csa_swa_merge and by
// the split-K combine of csa_sparse_mqa_attn).
#pragma once

#include "common.h"

// Part p of row r: output at o0 + p*stride_o_bytes (bytes) + r*dim values
// (float, or bf16 when part_bf16), its log-sum-exp at l0 + p*stride_l_bytes +
// r floats.  Row r merges cnt[r/rows_per_q] parts (clamped to [1, nparts]) or
// `nparts` when cnt is null.  nparts <= 256.
csa_status launch_lse_merge(const void* o0, const float* l0, int64_t stride_o_elems,
                            int64_t stride_l_elems, int nparts, const int* cnt, int rows_per_q,
                            int64_t rows, int dim, void* out, int out_fmt, float* lse_out,
                            bool part_bf16, hipStream_t stream);
csa_status launch_lse_merge_bytes(const void* o0, const float* l0, int64_t stride_o_bytes,
                                  int64_t stride_l_bytes, int nparts, const int* cnt,
                                  int rows_per_q, int64_t rows, int dim, void* out, int out_fmt,
                                  float* lse_out, bool part_bf16, hipStream_t stream);
