"""Python entry points of the HSA library, one per C-ABI call (same names).

Tensors are torch tensors on the GPU (torch is used only for device memory
and streams); each function forwards raw pointers and the current HIP stream
to libhsa_attn.so and raises HsaError on a non-zero return code.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

from ._lib import HSA_BF16, HSA_F32, Geom, check, lib

_DTYPES = {torch.float32: HSA_F32, torch.bfloat16: HSA_BF16}


def make_geom(n_heads, head_dim, frame_h, frame_w, frames_per_page, query_frames, tile,
              n_sel_pages, rank, dtype, intra_split: int = 0) -> Geom:
    dt = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else {"f32": HSA_F32, "bf16": HSA_BF16}[dtype]
    return Geom(n_heads, head_dim, frame_h, frame_w, frames_per_page, query_frames,
                tile[0], tile[1], tile[2], n_sel_pages, rank, dt, intra_split)


@dataclass(frozen=True)
class Dims:
    """Buffer sizes implied by a geometry (mirrors the library's own derivation)."""
    H: int
    d: int
    Lp: int
    Lq: int
    B: int
    Kp: int
    L: int
    nKB: int
    nQB: int
    r: int
    dtype: torch.dtype
    split: int = 0   # intra_split
    Bk: int = 0      # tokens per key block
    Lh: int = 0      # keys of the retrieved pages
    nKBh: int = 0    # B-token history tiles
    nC: int = 0      # selection candidates (row length of blk_mass)

    @staticmethod
    def of(g: Geom) -> "Dims":
        tpf = g.frame_h * g.frame_w
        B = g.tile_t * g.tile_h * g.tile_w
        Lp, Lq = tpf * g.frames_per_page, tpf * g.query_frames
        s = int(g.intra_split)
        Bk = B // s if s else B
        Lh = Lp * g.n_sel_pages
        L = Lh + (Lq if s else 0)
        nKB = L // Bk
        nC = Lh // B + Lq // Bk if s else nKB
        return Dims(g.n_heads, g.head_dim, Lp, Lq, B, g.n_sel_pages, L, nKB, Lq // B, g.rank,
                    torch.bfloat16 if g.dtype == HSA_BF16 else torch.float32, s, Bk, Lh, Lh // B, nC)


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("HSA buffers must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _s(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _table(pages: Sequence[Optional[torch.Tensor]]):
    arr = (ctypes.c_void_p * len(pages))()
    for i, t in enumerate(pages):
        arr[i] = None if t is None else t.data_ptr()
    return arr


class DeviceTable:
    """A page pointer table in device memory (the *_devtab calls): entry j is
    page j's device address, 0 for a page without one.  Holds the pages so
    their memory stays alive.  Built once per bank (one host-to-device copy),
    not per step."""

    def __init__(self, pages: Sequence[Optional[torch.Tensor]], device="cuda"):
        self.pages = list(pages)
        ptrs = [0 if t is None else t.data_ptr() for t in self.pages]
        self.ptrs = torch.tensor(ptrs, dtype=torch.int64).to(device)

    def __len__(self) -> int:
        return len(self.pages)


def hsa_workspace_bytes(geom: Geom, n_pages: int) -> int:
    return int(lib().hsa_workspace_bytes(ctypes.byref(geom), n_pages))


def hsa_linear_workspace_bytes(geom: Geom) -> int:
    return int(lib().hsa_linear_workspace_bytes(ctypes.byref(geom)))


def hsa_geom_check(geom: Geom) -> int:
    return int(lib().hsa_geom_check(ctypes.byref(geom)))


def hsa_score_pages(geom, q, pages_k, page_kmean, scores, sel_pages, ws, stream=None):
    """pages_k: a list of page tensors (host table) or a DeviceTable."""
    if isinstance(pages_k, DeviceTable):
        check("hsa_score_pages_devtab", lib().hsa_score_pages_devtab(
            ctypes.byref(geom), _p(q), _p(pages_k.ptrs), _p(page_kmean), len(pages_k), _p(scores), _p(sel_pages),
            _p(ws), ws.numel() * ws.element_size(), _s(stream)))
        return
    check("hsa_score_pages", lib().hsa_score_pages(
        ctypes.byref(geom), _p(q), _table(pages_k), _p(page_kmean), len(pages_k), _p(scores), _p(sel_pages),
        _p(ws), ws.numel() * ws.element_size(), _s(stream)))


def hsa_retrieve_chunks(prompt, chunk_prompts, k_chunks, sims, sel_chunks, stream=None):
    """prompt [E] and chunk_prompts [C][E] float32 device tensors."""
    n_chunks, emb_dim = chunk_prompts.shape
    check("hsa_retrieve_chunks", lib().hsa_retrieve_chunks(
        _p(prompt), _p(chunk_prompts), n_chunks, emb_dim, k_chunks, _p(sims), _p(sel_chunks), _s(stream)))


def hsa_score_chunk_pages(geom, q, pages_k, page_kmean, page_chunk, sel_chunks, scores, sel_pages, ws,
                          stream=None):
    if isinstance(pages_k, DeviceTable):
        check("hsa_score_chunk_pages_devtab", lib().hsa_score_chunk_pages_devtab(
            ctypes.byref(geom), _p(q), _p(pages_k.ptrs), _p(page_kmean), len(pages_k), _p(page_chunk),
            _p(sel_chunks), sel_chunks.numel(), _p(scores), _p(sel_pages), _p(ws), ws.numel() * ws.element_size(),
            _s(stream)))
        return
    check("hsa_score_chunk_pages", lib().hsa_score_chunk_pages(
        ctypes.byref(geom), _p(q), _table(pages_k), _p(page_kmean), len(pages_k), _p(page_chunk),
        _p(sel_chunks), sel_chunks.numel(), _p(scores), _p(sel_pages), _p(ws), ws.numel() * ws.element_size(),
        _s(stream)))


def hsa_gather_pages(geom, pages_k, pages_v, sel_pages, k_act, v_act, kblk_mean=None, stream=None):
    if isinstance(pages_k, DeviceTable):
        return hsa_gather_active(geom, pages_k, pages_v, sel_pages, None, None, k_act, v_act, kblk_mean, stream)
    check("hsa_gather_pages", lib().hsa_gather_pages(
        ctypes.byref(geom), _table(pages_k), _table(pages_v), len(pages_k), _p(sel_pages), _p(k_act), _p(v_act),
        _p(kblk_mean), _s(stream)))


def hsa_gather_active(geom, pages_k, pages_v, sel_pages, k_cur, v_cur, k_act, v_act, kblk_mean=None,
                      stream=None):
    """k_cur / v_cur: the chunk's own [Lq][H][d] keys and values (None
    without intra-chunk keys).  pages_k / pages_v: lists (host tables) or
    DeviceTables."""
    if isinstance(pages_k, DeviceTable):
        check("hsa_gather_active_devtab", lib().hsa_gather_active_devtab(
            ctypes.byref(geom), _p(pages_k.ptrs), _p(pages_v.ptrs), len(pages_k), _p(sel_pages), _p(k_cur),
            _p(v_cur), _p(k_act), _p(v_act), _p(kblk_mean), _s(stream)))
        return
    check("hsa_gather_active", lib().hsa_gather_active(
        ctypes.byref(geom), _table(pages_k), _table(pages_v), len(pages_k), _p(sel_pages), _p(k_cur), _p(v_cur),
        _p(k_act), _p(v_act), _p(kblk_mean), _s(stream)))


def hsa_gather_chunk(geom, k_cur, v_cur, k_act, v_act, kblk_mean=None, stream=None):
    """Rewrite only the chunk's part of the active K/V and its key-block means."""
    check("hsa_gather_chunk", lib().hsa_gather_chunk(
        ctypes.byref(geom), _p(k_cur), _p(v_cur), _p(k_act), _p(v_act), _p(kblk_mean), _s(stream)))


def hsa_linear_branch(geom, q, k_act, v_act, e_k, e_v, k_proj, v_proj, o_lin, flags, ws, stream=None):
    check("hsa_linear_branch", lib().hsa_linear_branch(
        ctypes.byref(geom), _p(q), _p(k_act), _p(v_act), _p(e_k), _p(e_v), _p(k_proj), _p(v_proj), _p(o_lin),
        flags, _p(ws), 0 if ws is None else ws.numel() * ws.element_size(), _s(stream)))


def hsa_page_prepare(geom, k_page, v_page, k_out, v_out, blk_mean=None, stream=None):
    check("hsa_page_prepare", lib().hsa_page_prepare(
        ctypes.byref(geom), _p(k_page), _p(v_page), _p(k_out), _p(v_out), _p(blk_mean), _s(stream)))


def hsa_chunk_page_count(geom) -> int:
    return int(lib().hsa_chunk_page_count(ctypes.byref(geom)))


def hsa_chunk_prepare(geom, k_cur, v_cur, k_out, v_out, blk_mean=None, stream=None):
    check("hsa_chunk_prepare", lib().hsa_chunk_prepare(
        ctypes.byref(geom), _p(k_cur), _p(v_cur), _table(k_out), _table(v_out),
        None if blk_mean is None else _table(blk_mean), _s(stream)))


def hsa_gather_block_means(geom, page_blk_mean, sel_pages, kblk_mean, stream=None):
    """page_blk_mean: a list of per-page block-mean tensors (host table) or a DeviceTable."""
    if isinstance(page_blk_mean, DeviceTable):
        check("hsa_gather_block_means_devtab", lib().hsa_gather_block_means_devtab(
            ctypes.byref(geom), _p(page_blk_mean.ptrs), len(page_blk_mean), _p(sel_pages), _p(kblk_mean), _s(stream)))
        return
    check("hsa_gather_block_means", lib().hsa_gather_block_means(
        ctypes.byref(geom), _table(page_blk_mean), len(page_blk_mean), _p(sel_pages), _p(kblk_mean), _s(stream)))


def hsa_linear_branch_paged(geom, q, pages_k, pages_v, sel_pages, e_k, e_v, k_proj, v_proj, o_lin, flags, ws,
                            stream=None):
    """pages_k, pages_v: lists of laid-out page tensors (host tables) or DeviceTables."""
    if isinstance(pages_k, DeviceTable):
        check("hsa_linear_branch_paged_devtab", lib().hsa_linear_branch_paged_devtab(
            ctypes.byref(geom), _p(q), _p(pages_k.ptrs), _p(pages_v.ptrs), len(pages_k), _p(sel_pages), _p(e_k),
            _p(e_v), _p(k_proj), _p(v_proj), _p(o_lin), flags, _p(ws),
            0 if ws is None else ws.numel() * ws.element_size(), _s(stream)))
        return
    check("hsa_linear_branch_paged", lib().hsa_linear_branch_paged(
        ctypes.byref(geom), _p(q), _table(pages_k), _table(pages_v), len(pages_k), _p(sel_pages), _p(e_k), _p(e_v),
        _p(k_proj), _p(v_proj), _p(o_lin), flags, _p(ws), 0 if ws is None else ws.numel() * ws.element_size(),
        _s(stream)))


def hsa_sparse_attn_paged(geom, q, pages_k, pages_v, sel_pages, blk_count, blk_idx, o_sp, ws, events=None,
                          stream=None):
    """events: optional (begin, end) torch.cuda.Event pair (enable_timing=True)
    recorded around the attention kernel alone."""
    handles = _event_handles(events, stream) if events is not None else (None, None)
    if isinstance(pages_k, DeviceTable):
        check("hsa_sparse_attn_paged_devtab", lib().hsa_sparse_attn_paged_devtab(
            ctypes.byref(geom), _p(q), _p(pages_k.ptrs), _p(pages_v.ptrs), len(pages_k), _p(sel_pages),
            _p(blk_count), _p(blk_idx), _p(o_sp), _p(ws), ws.numel() * ws.element_size(), _s(stream), handles[0],
            handles[1]))
        return
    check("hsa_sparse_attn_paged", lib().hsa_sparse_attn_paged(
        ctypes.byref(geom), _p(q), _table(pages_k), _table(pages_v), len(pages_k), _p(sel_pages), _p(blk_count),
        _p(blk_idx), _p(o_sp), _p(ws), ws.numel() * ws.element_size(), _s(stream), handles[0], handles[1]))


def hsa_block_select(geom, q, k_act, kblk_mean, tau, blk_count, blk_idx, blk_mass, ws, stream=None):
    check("hsa_block_select", lib().hsa_block_select(
        ctypes.byref(geom), _p(q), _p(k_act), _p(kblk_mean), _p(tau), _p(blk_count), _p(blk_idx), _p(blk_mass),
        _p(ws), ws.numel() * ws.element_size(), _s(stream)))


def hsa_block_select_noalloc(geom, q, k_act, kblk_mean, tau, blk_count, blk_idx, blk_mass, stream=None):
    """hsa_block_select with the library's own device scratch instead of a workspace."""
    check("hsa_block_select_noalloc", lib().hsa_block_select_noalloc(
        ctypes.byref(geom), _p(q), _p(k_act), _p(kblk_mean), _p(tau), _p(blk_count), _p(blk_idx), _p(blk_mass),
        _s(stream)))


def hsa_sparse_attn(geom, q, k_act, v_act, blk_count, blk_idx, o_sp, ws, stream=None):
    check("hsa_sparse_attn", lib().hsa_sparse_attn(
        ctypes.byref(geom), _p(q), _p(k_act), _p(v_act), _p(blk_count), _p(blk_idx), _p(o_sp),
        _p(ws), ws.numel() * ws.element_size(), _s(stream)))


def hsa_sparse_attn_timed(geom, q, k_act, v_act, blk_count, blk_idx, o_sp, ws, ev_begin, ev_end, stream=None):
    """hsa_sparse_attn that also records two torch.cuda.Event objects (created
    with enable_timing=True) around the attention kernel alone."""
    handles = _event_handles((ev_begin, ev_end), stream)
    check("hsa_sparse_attn_timed", lib().hsa_sparse_attn_timed(
        ctypes.byref(geom), _p(q), _p(k_act), _p(v_act), _p(blk_count), _p(blk_idx), _p(o_sp),
        _p(ws), ws.numel() * ws.element_size(), _s(stream), handles[0], handles[1]))


def _event_handles(events, stream):
    handles = []
    for ev in events:
        if ev is None:
            handles.append(None)
            continue
        if not ev.cuda_event:  # torch creates the underlying event on first use
            ev.record(torch.cuda.current_stream() if stream is None else stream)
        handles.append(ctypes.c_void_p(ev.cuda_event))
    return handles


def hsa_probe_mfma_bf16(n_workgroups, iters, out, ev_begin, ev_end, stream=None):
    """The matrix-core rate probe (a measurement helper, not part of the
    step): out is a float32 device tensor of n_workgroups * 512 values."""
    if out.numel() < n_workgroups * 512 or out.dtype != torch.float32:
        raise ValueError("out must hold n_workgroups * 512 float32 values")
    h = _event_handles((ev_begin, ev_end), stream)
    check("hsa_probe_mfma_bf16", lib().hsa_probe_mfma_bf16(n_workgroups, iters, _p(out), _s(stream), h[0], h[1]))


def hsa_probe_hbm_copy(src, dst, ev_begin, ev_end, stream=None):
    """The HBM stream-copy probe (a measurement helper, not part of the step):
    copies src into dst (same byte size, contiguous device tensors)."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("src and dst must have the same byte size")
    h = _event_handles((ev_begin, ev_end), stream)
    check("hsa_probe_hbm_copy", lib().hsa_probe_hbm_copy(_p(src), _p(dst), n, _s(stream), h[0], h[1]))


def hsa_fuse(geom, x, w_g, gate_override, o_lin, o_sp, out, stream=None):
    check("hsa_fuse", lib().hsa_fuse(
        ctypes.byref(geom), _p(x), _p(w_g), _p(gate_override), _p(o_lin), _p(o_sp), _p(out), _s(stream)))
