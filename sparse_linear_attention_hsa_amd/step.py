"""One HSA decode step (one layer, one denoising step) over device buffers.

Holds the intermediate buffers of the six stages (allocated once with torch)
and issues the six C-ABI calls:

    score_pages -> gather_pages -+-> linear_branch ---------------------+-> fuse
                                 +-> block_select -> sparse_attn ------+

The linear branch reads only the gathered K/V and the queries, and its
output meets the sparse branch's only in the gated sum (WorldAttention
paper, section 3.3 "Hybrid Sparse Attention", paragraph on the gated fusion
of the two branches).  By default it therefore runs on a side stream (default priority)
with a workspace of its own, beside block selection and the sparse branch,
and the fusion waits for both; run(..., concurrent=False) issues all six
calls in order on one stream.  The two schedules give bit-identical results.

Nothing here computes: every stage runs in the library's HIP kernels, and the
selections never leave the device.
"""
from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import ops
from ._lib import HSA_LIN_REUSE_PROJ, HSA_MAX_PAGES
from .ops import Dims, Geom


class HsaStep:
    def __init__(self, geom: Geom, n_pages: int, device: str = "cuda"):
        self.geom = geom
        self.n_pages = n_pages
        self.s = s = Dims.of(geom)
        dev = torch.device(device)
        f32, i32, dt = torch.float32, torch.int32, s.dtype
        self.page_kmean = torch.empty(n_pages, s.H, s.d, dtype=f32, device=dev)
        self.scores = torch.empty(n_pages, dtype=f32, device=dev)
        # pages read in place with intra-chunk keys: the selected pages, then
        # the table indices of the chunk's page-format buffers (one array;
        # sel_pages is its head, which scoring writes)
        self.n_chunk_pages = ops.hsa_chunk_page_count(geom)
        self.sel_ext = torch.empty(s.Kp + self.n_chunk_pages, dtype=i32, device=dev)
        self.sel_pages = self.sel_ext[:s.Kp]
        self._sel_tail_base: Optional[int] = None
        self._chunk_bufs = None
        self._devtabs = None  # (key, device tables) of the last paged bank
        self.k_act = torch.empty(s.H, s.L, s.d, dtype=dt, device=dev)
        self.v_act = torch.empty(s.H, s.L // 16, s.d, 16, dtype=dt, device=dev)
        self.kblk_mean = torch.empty(s.H, s.nKB, s.d, dtype=f32, device=dev)
        self.k_proj = torch.empty(s.H, s.r, s.d, dtype=f32, device=dev)
        self.v_proj = torch.empty(s.H, s.d, s.r, dtype=f32, device=dev)
        self.o_lin = torch.empty(s.Lq, s.H, s.d, dtype=f32, device=dev)
        self.blk_count = torch.empty(s.H, s.nQB, dtype=i32, device=dev)
        self.blk_idx = torch.empty(s.H, s.nQB, s.nKB, dtype=i32, device=dev)
        self.blk_mass = torch.empty(s.H, s.nQB, s.nC, dtype=f32, device=dev)
        self.o_sp = torch.empty(s.Lq, s.H, s.d, dtype=f32, device=dev)
        self.out = torch.empty(s.Lq, s.H, s.d, dtype=dt, device=dev)
        nbytes = ops.hsa_workspace_bytes(geom, n_pages)
        if nbytes == 0:
            raise ValueError("invalid geometry")
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        # the linear branch's own workspace and stream, so that it can run
        # beside block selection and the sparse branch
        self.ws_lin = torch.empty(ops.hsa_linear_workspace_bytes(geom), dtype=torch.uint8, device=dev)
        self.side = torch.cuda.Stream(device=dev)
        # prompt-level retrieval outputs (sized on first use)
        self.chunk_sims: Optional[torch.Tensor] = None
        self.sel_chunks: Optional[torch.Tensor] = None
        self._null_table: Optional[ops.DeviceTable] = None

    # individual stages --------------------------------------------------
    def score(self, q, pages_k, stream=None, use_cache: bool = False):
        """use_cache: score every page from the page index (page_kmean,
        filled by index_pages) instead of reading its keys.  pages_k: a list
        of page tensors, or an ops.DeviceTable (banks beyond HSA_MAX_PAGES)."""
        pages = self.no_pages() if use_cache else pages_k
        ops.hsa_score_pages(self.geom, q, pages, self.page_kmean, self.scores, self.sel_pages, self.ws, stream)

    def no_pages(self):
        """A page table of NULL entries (every page scored from the page
        index): a host list, or a device table for banks beyond HSA_MAX_PAGES."""
        if self.n_pages <= HSA_MAX_PAGES:
            return [None] * self.n_pages
        if self._null_table is None:
            self._null_table = ops.DeviceTable([None] * self.n_pages, self.k_act.device)
        return self._null_table

    def retrieve(self, q, pages_k, chunks, stream=None):
        """Stage 1 and page scoring inside the retrieved chunks (WorldAttention
        paper, section 3.2, "Stage 1: prompt-level retrieval"; section 4.5,
        candidate chunks).  chunks = (prompt [E], chunk_prompts [C][E] float32,
        page_chunk [P] int32, k_chunks), all device tensors but k_chunks."""
        prompt, chunk_prompts, page_chunk, k_chunks = chunks
        n_chunks = chunk_prompts.shape[0]
        if self.chunk_sims is None or self.chunk_sims.numel() != n_chunks or self.sel_chunks.numel() != k_chunks:
            self.chunk_sims = torch.empty(n_chunks, dtype=torch.float32, device=q.device)
            self.sel_chunks = torch.empty(k_chunks, dtype=torch.int32, device=q.device)
        ops.hsa_retrieve_chunks(prompt, chunk_prompts, k_chunks, self.chunk_sims, self.sel_chunks, stream)
        ops.hsa_score_chunk_pages(self.geom, q, pages_k, self.page_kmean, page_chunk, self.sel_chunks, self.scores,
                                  self.sel_pages, self.ws, stream)

    def index_pages(self, q, pages_k: Sequence[torch.Tensor], stream=None):
        """Build the page index: every page's mean key (WorldAttention paper,
        section 3.2, the page index built from the keys), as it would be kept
        when a page is written.  Runs one scoring call over the pages."""
        ops.hsa_score_pages(self.geom, q, pages_k, self.page_kmean, self.scores, self.sel_pages, self.ws, stream)

    def gather(self, pages_k, pages_v, stream=None, k_cur=None, v_cur=None):
        """k_cur / v_cur: the chunk's own keys and values [Lq][H][d], which
        follow the pages when the geometry has intra-chunk keys."""
        if self.geom.intra_split:
            ops.hsa_gather_active(self.geom, pages_k, pages_v, self.sel_pages, k_cur, v_cur, self.k_act, self.v_act,
                                  self.kblk_mean, stream)
        else:
            ops.hsa_gather_pages(self.geom, pages_k, pages_v, self.sel_pages, self.k_act, self.v_act,
                                 self.kblk_mean, stream)

    def linear(self, q, e_k, e_v, flags: int = 0, stream=None, ws=None):
        ws = self.ws if ws is None else ws
        if flags & HSA_LIN_REUSE_PROJ:
            ops.hsa_linear_branch(self.geom, q, None, None, None, None, self.k_proj, self.v_proj, self.o_lin,
                                  flags, ws, stream)
        else:
            ops.hsa_linear_branch(self.geom, q, self.k_act, self.v_act, e_k, e_v, self.k_proj, self.v_proj,
                                  self.o_lin, flags, ws, stream)

    def select(self, q, tau, use_kblk_mean: bool = True, stream=None):
        ops.hsa_block_select(self.geom, q, self.k_act, self.kblk_mean if use_kblk_mean else None, tau,
                             self.blk_count, self.blk_idx, self.blk_mass, self.ws, stream)

    def sparse(self, q, stream=None, kernel_events=None):
        if kernel_events is None:
            ops.hsa_sparse_attn(self.geom, q, self.k_act, self.v_act, self.blk_count, self.blk_idx, self.o_sp,
                                self.ws, stream)
        else:
            ops.hsa_sparse_attn_timed(self.geom, q, self.k_act, self.v_act, self.blk_count, self.blk_idx,
                                      self.o_sp, self.ws, kernel_events[0], kernel_events[1], stream)

    def fuse(self, x, w_g, stream=None):
        ops.hsa_fuse(self.geom, x, w_g, None, self.o_lin, self.o_sp, self.out, stream)

    # pages read in place ------------------------------------------------
    def prepare_pages(self, pages_k, pages_v, stream=None):
        """Lay out every page once, as when it is written: K [H][Lp][d], V
        [H][Lp/16][d][16] and the block means [H][Lp/B][d] (the layouts the
        kernels read, over one page).  Returns (k_pages, v_pages, blk_means)."""
        ks, vs, ms = [], [], []
        for pk, pv in zip(pages_k, pages_v):
            ko, vo, mo = self._page_buffers()
            ops.hsa_page_prepare(self.geom, pk, pv, ko, vo, mo, stream)
            ks.append(ko)
            vs.append(vo)
            ms.append(mo)
        return ks, vs, ms

    def _page_buffers(self):
        s, dev = self.s, self.k_act.device
        return (torch.empty(s.H, s.Lp, s.d, dtype=s.dtype, device=dev),
                torch.empty(s.H, s.Lp // 16, s.d, 16, dtype=s.dtype, device=dev),
                torch.empty(s.H, s.Lp // s.Bk, s.d, dtype=torch.float32, device=dev))

    def paged_inputs(self, prepared, k_cur=None, v_cur=None, stream=None, device_tables: Optional[bool] = None):
        """Page tables and selection list of a paged step.  With intra-chunk
        keys the chunk's own keys and values are laid out into page-format
        buffers (kept from step to step), appended to the tables, and their
        table indices follow the selected pages in sel_ext.  device_tables:
        the tables in device memory (built once per bank and kept), which
        banks beyond HSA_MAX_PAGES need; by default only for those.  Returns
        (k_pages, v_pages, blk_means, sel)."""
        kp, vp, bm, sel = self._paged_lists(prepared, k_cur, v_cur, stream)
        if device_tables is None:
            device_tables = len(kp) > HSA_MAX_PAGES
        if not device_tables:
            return kp, vp, bm, sel
        key = (id(prepared[0]), len(kp))
        if self._devtabs is None or self._devtabs[0] != key:
            self._devtabs = (key, (ops.DeviceTable(kp), ops.DeviceTable(vp), ops.DeviceTable(bm)))
        dk, dv, dm = self._devtabs[1]
        return dk, dv, dm, sel

    def _paged_lists(self, prepared, k_cur, v_cur, stream):
        kp, vp, bm = prepared
        if not self.n_chunk_pages:
            return kp, vp, bm, self.sel_ext
        if k_cur is None or v_cur is None:
            raise ValueError("this geometry has intra-chunk keys: pass k_cur and v_cur")
        if self._chunk_bufs is None:
            self._chunk_bufs = [self._page_buffers() for _ in range(self.n_chunk_pages)]
        ck, cv, cm = (list(t) for t in zip(*self._chunk_bufs))
        ops.hsa_chunk_prepare(self.geom, k_cur, v_cur, ck, cv, cm, stream)
        if self._sel_tail_base != len(kp):  # the chunk buffers' table indices
            tail = torch.arange(len(kp), len(kp) + self.n_chunk_pages, dtype=torch.int32)
            self.sel_ext[self.s.Kp:].copy_(tail)
            self._sel_tail_base = len(kp)
        return list(kp) + ck, list(vp) + cv, list(bm) + cm, self.sel_ext

    def run_paged(self, q, prepared, e_k, e_v, w_g, x, tau, stream=None, concurrent: bool = True,
                  kernel_events=None, k_cur=None, v_cur=None, device_tables: Optional[bool] = None):
        """The step over laid-out pages, with no active-buffer copy: scoring
        from the page index (index_pages ran before), the selected pages' block
        means, the linear branch (side stream) and the sparse branch reading
        the pages in place, then the fusion.  k_cur, v_cur: the chunk's own
        keys and values (geometries with intra-chunk keys), laid out into
        page-format buffers first.  device_tables: see paged_inputs."""
        main = torch.cuda.current_stream() if stream is None else stream
        self.score(q, None, main, use_cache=True)
        kp, vp, bm, sel = self.paged_inputs(prepared, k_cur, v_cur, main, device_tables)
        ops.hsa_gather_block_means(self.geom, bm, sel, self.kblk_mean, main)
        side = self.side if concurrent else main
        if concurrent:
            scored = torch.cuda.Event()
            scored.record(main)
            self.side.wait_event(scored)
        ops.hsa_linear_branch_paged(self.geom, q, kp, vp, sel, e_k, e_v, self.k_proj, self.v_proj,
                                    self.o_lin, 0, self.ws_lin if concurrent else self.ws, side)
        if concurrent:
            linear_done = torch.cuda.Event()
            linear_done.record(side)
        ops.hsa_block_select(self.geom, q, None, self.kblk_mean, tau, self.blk_count, self.blk_idx, self.blk_mass,
                             self.ws, main)
        ops.hsa_sparse_attn_paged(self.geom, q, kp, vp, sel, self.blk_count, self.blk_idx, self.o_sp,
                                  self.ws, kernel_events, main)
        if concurrent:
            main.wait_event(linear_done)
        self.fuse(x, w_g, main)
        return self.out

    # the whole step -----------------------------------------------------
    def run(self, q, pages_k, pages_v, e_k, e_v, w_g, x, tau, stream=None, concurrent: bool = True,
            indexed: bool = False, chunks=None, k_cur=None, v_cur=None):
        """indexed: score from the page index (index_pages ran before) rather
        than from the pages' keys; the gather still copies the pages.
        chunks: run prompt-level retrieval first and score only the pages of
        the retrieved chunks (see retrieve).
        k_cur, v_cur: the chunk's own keys and values (geometries with
        intra-chunk keys)."""
        main = torch.cuda.current_stream() if stream is None else stream
        if chunks is not None:
            self.retrieve(q, self.no_pages() if indexed else pages_k, chunks, main)
        else:
            self.score(q, pages_k, main, use_cache=indexed)
        self.gather(pages_k, pages_v, main, k_cur, v_cur)
        if concurrent:
            gathered = torch.cuda.Event()
            gathered.record(main)
            self.side.wait_event(gathered)
            self.linear(q, e_k, e_v, 0, self.side, ws=self.ws_lin)
            linear_done = torch.cuda.Event()
            linear_done.record(self.side)
        else:
            self.linear(q, e_k, e_v, 0, main)
        self.select(q, tau, True, main)
        self.sparse(q, main)
        if concurrent:
            main.wait_event(linear_done)
        self.fuse(x, w_g, main)
        return self.out
