"""ctypes binding of libhsa_attn.so (the C ABI declared in include/hsa_attn.h).

Argument marshalling only: every step of the HSA path runs in the library's
HIP kernels.  There is no fallback -- if the built library is missing the
import fails loudly.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhsa_attn.so")

HSA_F32, HSA_BF16 = 0, 1
HSA_LIN_REUSE_PROJ, HSA_LIN_PROJ_ONLY, HSA_LIN_HISTORY_PROJ, HSA_LIN_CHUNK_PROJ = 1, 2, 4, 8
HSA_MAX_PAGES = 128
HSA_MAX_BANK_PAGES = 8192
HSA_MAX_KBLOCKS = 2048
HSA_MAX_ROWS = 4096
HSA_MAX_CHUNKS = 4096
HSA_MAX_EMBED = 65536
HSA_MAX_INTRA_SPLIT = 4
HSA_NOALLOC_SCRATCH_BYTES = 16 << 20

RC_NAMES = {0: "HSA_OK", 1: "HSA_ERR_NULL_ARG", 2: "HSA_ERR_BAD_SHAPE", 3: "HSA_ERR_BAD_DTYPE",
            4: "HSA_ERR_BAD_PARAM", 5: "HSA_ERR_WORKSPACE", 6: "HSA_ERR_HIP"}

# Every function the header declares, with its ctypes signature.
_vp, _i32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t


class Geom(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("frame_h", ctypes.c_int32), ("frame_w", ctypes.c_int32),
                ("frames_per_page", ctypes.c_int32), ("query_frames", ctypes.c_int32),
                ("tile_t", ctypes.c_int32), ("tile_h", ctypes.c_int32), ("tile_w", ctypes.c_int32),
                ("n_sel_pages", ctypes.c_int32), ("rank", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("intra_split", ctypes.c_int32)]


_GP = ctypes.POINTER(Geom)
SIGNATURES = {
    "hsa_score_pages": (_i32, [_GP, _vp, ctypes.POINTER(_vp), _vp, _i32, _vp, _vp, _vp, _sz, _vp]),
    "hsa_score_chunk_pages": (_i32, [_GP, _vp, ctypes.POINTER(_vp), _vp, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _sz,
                                     _vp]),
    "hsa_score_pages_devtab": (_i32, [_GP, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _sz, _vp]),
    "hsa_score_chunk_pages_devtab": (_i32, [_GP, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _sz, _vp]),
    "hsa_gather_active_devtab": (_i32, [_GP, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "hsa_retrieve_chunks": (_i32, [_vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp]),
    "hsa_gather_pages": (_i32, [_GP, ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i32, _vp, _vp, _vp, _vp, _vp]),
    "hsa_gather_active": (_i32, [_GP, ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _vp]),
    "hsa_gather_chunk": (_i32, [_GP, _vp, _vp, _vp, _vp, _vp, _vp]),
    "hsa_linear_branch": (_i32, [_GP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _sz, _vp]),
    "hsa_page_prepare": (_i32, [_GP, _vp, _vp, _vp, _vp, _vp, _vp]),
    "hsa_chunk_page_count": (_i32, [_GP]),
    "hsa_chunk_prepare": (_i32, [_GP, _vp, _vp, ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.POINTER(_vp), _vp]),
    "hsa_gather_block_means": (_i32, [_GP, ctypes.POINTER(_vp), _i32, _vp, _vp, _vp]),
    "hsa_linear_branch_paged": (_i32, [_GP, _vp, ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i32, _vp, _vp, _vp, _vp,
                                       _vp, _vp, _i32, _vp, _sz, _vp]),
    "hsa_sparse_attn_paged": (_i32, [_GP, _vp, ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i32, _vp, _vp, _vp, _vp,
                                     _vp, _sz, _vp, _vp, _vp]),
    "hsa_gather_block_means_devtab": (_i32, [_GP, _vp, _i32, _vp, _vp, _vp]),
    "hsa_linear_branch_paged_devtab": (_i32, [_GP, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _sz,
                                              _vp]),
    "hsa_sparse_attn_paged_devtab": (_i32, [_GP, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp, _vp, _vp]),
    "hsa_block_select": (_i32, [_GP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "hsa_block_select_noalloc": (_i32, [_GP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "hsa_sparse_attn": (_i32, [_GP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "hsa_sparse_attn_timed": (_i32, [_GP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp, _vp, _vp]),
    "hsa_fuse": (_i32, [_GP, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "hsa_workspace_bytes": (_sz, [_GP, _i32]),
    "hsa_linear_workspace_bytes": (_sz, [_GP]),
    "hsa_geom_check": (_i32, [_GP]),
    "hsa_rc_string": (ctypes.c_char_p, [_i32]),
    "hsa_abi_version": (_i32, []),
    "hsa_tier_create": (_vp, [_i32, _i32, _i32]),
    "hsa_tier_destroy": (None, [_vp]),
    "hsa_tier_seed": (_i32, [_vp, _vp, _i32, _i32, _vp]),
    "hsa_tier_request": (_i32, [_vp, _vp, _i32, _vp, _vp, _i32, _vp]),
    "hsa_tier_locate": (_i32, [_vp, _i32, _vp, _vp]),
    "hsa_tier_stats": (_i32, [_vp, _vp]),
    "hsa_probe_mfma_bf16": (_i32, [_i32, _i32, _vp, _vp, _vp, _vp]),
    "hsa_probe_hbm_copy": (_i32, [_vp, _vp, _sz, _vp, _vp, _vp]),
}


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    # torch ships its own HIP runtime under the same soname; load it first so
    # the library binds to the runtime that owns torch's streams and memory.
    import torch  # noqa: F401
    if not os.path.exists(path):
        raise ImportError(
            f"HSA HIP library not built: {path} is missing "
            "(run `python -m sparse_linear_attention_hsa_amd.build` or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_LIB = None


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        _LIB = load()
    return _LIB


class HsaError(RuntimeError):
    def __init__(self, fn: str, rc: int):
        super().__init__(f"{fn} failed: {lib().hsa_rc_string(rc).decode()}")
        self.rc = rc


def check(fn: str, rc: int) -> None:
    if rc != 0:
        raise HsaError(fn, rc)
