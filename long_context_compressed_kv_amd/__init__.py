"""MI355X (gfx950) implementation of the CSA / HCA compressed-attention path.

The compute lives in libcsa.so (hand-written HIP, C ABI in include/csa.h);
`ops` is its Python binding.  Importing the package does not load the
library; the first call does, and fails loudly if it has not been built.
"""
from . import ops  # noqa: F401
from .ops import (KV, Batch, F32, BF16, FP8_MIXED, MXFP4, kv_compress, indexer_score,  # noqa: F401
                  topk_select, sparse_mqa_attn, swa_merge, quantize, dequantize, mxfp4_to_fp8)
