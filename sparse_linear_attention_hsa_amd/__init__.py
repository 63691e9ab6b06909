"""MI355X-native (gfx950) Hybrid Sparse Attention decode step over a paged KV cache.

The compute lives in libhsa_attn.so (HIP kernels behind the C ABI declared in
include/hsa_attn.h).  Python entry points with the same names as the C calls
are in `sparse_linear_attention_hsa_amd.ops`; `sparse_linear_attention_hsa_amd.step.HsaStep`
chains the six stages over device buffers.  Build with
`python -m sparse_linear_attention_hsa_amd.build`.
"""
from ._lib import (HSA_BF16, HSA_F32, HSA_LIN_PROJ_ONLY, HSA_LIN_REUSE_PROJ, HSA_MAX_KBLOCKS,  # noqa: F401
                   HSA_MAX_PAGES, Geom, HsaError)
