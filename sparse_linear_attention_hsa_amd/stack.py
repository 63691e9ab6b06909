"""The per-chunk schedule of a layer stack: several layers x several
denoising steps over one query chunk.

WorldAttention paper, section 3.2 ("Active KV construction": the retrieved
pages form the active KV of the chunk) and the structured summary's
weaknesses discussion (prefetch pages from pinned host memory): for each
layer the page scoring, the gather and the linear-branch projection depend
only on the chunk, so they run once, in the first denoising step, and every
later step reuses them (HSA_LIN_REUSE_PROJ); the linear attention, block
selection, sparse branch and fusion run every step, on that step's Q and X.

With intra-chunk keys (section 3.3, "Inter- and intra-chunk sparse
granularity") the chunk's own keys and values change with every denoising
step while the retrieved history does not: the first step gathers the
history and projects it alone (HSA_LIN_HISTORY_PROJ), and every step writes
its own keys into the chunk's part of the active buffer (hsa_gather_chunk)
and projects only them, added to the history's projection
(HSA_LIN_CHUNK_PROJ).

Pages that are not resident in device memory live in pinned host memory.
Their mean keys were taken while they were resident (the page index), so
scoring reads the cached mean instead of the page (a NULL page pointer).
Before a layer's gather, its non-resident pages are copied into one of
n_slots device staging slots on a side stream: the copies for the next
n_slots-1 layers are in flight while a layer computes, and a slot is
refilled only after the gather that last read it.  The schedule prefetches
every non-resident page of the coming layers (the host never sees a
selection).

As in a single step, each layer-step's linear branch runs on a side stream
(default priority, its own workspace) beside block selection and the sparse
branch, and the fusion waits for it; the next linear branch waits for that
fusion, which is the last reader of the shared per-step O_lin buffer.

Nothing here computes: every stage runs in the library's HIP kernels; this
module only orders the calls, the copies and the stream events.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import torch

from . import ops
from ._lib import HSA_LIN_CHUNK_PROJ, HSA_LIN_HISTORY_PROJ, HSA_LIN_REUSE_PROJ
from .ops import Dims, Geom


@dataclass
class LayerInputs:
    """Device tensors of one layer (pages may be None where host-resident)."""
    pages_k: List[Optional[torch.Tensor]]
    pages_v: List[Optional[torch.Tensor]]
    host_k: Dict[int, torch.Tensor]       # page id -> pinned host tensor [Lp][H][d]
    host_v: Dict[int, torch.Tensor]
    e_k: torch.Tensor
    e_v: torch.Tensor
    w_g: torch.Tensor
    tau: torch.Tensor
    page_kmean: torch.Tensor              # [P][H][d] f32, filled while every page was resident
    q: List[torch.Tensor] = field(default_factory=list)   # per step [Lq][H][d]
    x: List[torch.Tensor] = field(default_factory=list)   # per step [Lq][D]
    k_cur: List[torch.Tensor] = field(default_factory=list)  # per step [Lq][H][d] (intra-chunk keys)
    v_cur: List[torch.Tensor] = field(default_factory=list)


class _LayerState:
    """What a layer keeps from the first step of a chunk to the last."""

    def __init__(self, s: Dims, n_pages: int, dev):
        f32, i32, dt = torch.float32, torch.int32, s.dtype
        self.scores = torch.empty(n_pages, dtype=f32, device=dev)
        self.sel_pages = torch.empty(s.Kp, dtype=i32, device=dev)
        self.k_act = torch.empty(s.H, s.L, s.d, dtype=dt, device=dev)
        self.v_act = torch.empty(s.H, s.L // 16, s.d, 16, dtype=dt, device=dev)
        self.kblk_mean = torch.empty(s.H, s.nKB, s.d, dtype=f32, device=dev)
        self.k_proj = torch.empty(s.H, s.r, s.d, dtype=f32, device=dev)
        self.v_proj = torch.empty(s.H, s.d, s.r, dtype=f32, device=dev)


class HsaStack:
    def __init__(self, geom: Geom, n_pages: int, n_layers: int, max_host_pages: int, n_slots: int = 4,
                 device: str = "cuda"):
        self.geom = geom
        self.n_pages = n_pages
        self.n_layers = n_layers
        self.s = s = Dims.of(geom)
        dev = torch.device(device)
        f32, i32 = torch.float32, torch.int32
        self.layers = [_LayerState(s, n_pages, dev) for _ in range(n_layers)]
        # per-step buffers, shared by the layers (one step runs at a time)
        self.o_lin = torch.empty(s.Lq, s.H, s.d, dtype=f32, device=dev)
        self.o_sp = torch.empty(s.Lq, s.H, s.d, dtype=f32, device=dev)
        self.blk_count = torch.empty(s.H, s.nQB, dtype=i32, device=dev)
        self.blk_idx = torch.empty(s.H, s.nQB, s.nKB, dtype=i32, device=dev)
        nbytes = ops.hsa_workspace_bytes(geom, n_pages)
        if nbytes == 0:
            raise ValueError("invalid geometry")
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.ws_lin = torch.empty(ops.hsa_linear_workspace_bytes(geom), dtype=torch.uint8, device=dev)
        self.side = torch.cuda.Stream(device=dev)  # default priority
        # staging slots for the non-resident pages of the coming layers
        if n_slots < 2:
            raise ValueError("at least two staging slots")
        self.n_slots = n_slots
        self.max_host = max_host_pages
        shape = (max(1, max_host_pages), s.Lp, s.H, s.d)
        self.stage_k = [torch.empty(shape, dtype=s.dtype, device=dev) for _ in range(n_slots)]
        self.stage_v = [torch.empty(shape, dtype=s.dtype, device=dev) for _ in range(n_slots)]
        self.copy_stream = torch.cuda.Stream(device=dev)  # default priority
        self.scratch_out = torch.empty(s.Lq, s.H, s.d, dtype=s.dtype, device=dev)

    # ------------------------------------------------------------------
    def _prefetch(self, l: int, inp: LayerInputs, last_reader: List[Optional[torch.cuda.Event]],
                  copy_done: List[Optional[torch.cuda.Event]]) -> None:
        """Copy layer l's non-resident pages into staging slot l % n_slots (side
        stream), after the last gather that read that slot."""
        ids = sorted(inp.host_k)
        if not ids:
            copy_done[l] = None
            return
        if len(ids) > self.max_host:
            raise ValueError(f"layer {l} has {len(ids)} non-resident pages, more than {self.max_host}")
        slot = l % self.n_slots
        with torch.cuda.stream(self.copy_stream):
            if last_reader[slot] is not None:
                self.copy_stream.wait_event(last_reader[slot])
            for n, j in enumerate(ids):
                self.stage_k[slot][n].copy_(inp.host_k[j], non_blocking=True)
                self.stage_v[slot][n].copy_(inp.host_v[j], non_blocking=True)
            ev = torch.cuda.Event()
            ev.record(self.copy_stream)
        copy_done[l] = ev

    def _staged_tables(self, l: int, inp: LayerInputs):
        """Page tables of layer l with the staging slot in place of non-resident pages."""
        pk, pv = list(inp.pages_k), list(inp.pages_v)
        for n, j in enumerate(sorted(inp.host_k)):
            pk[j] = self.stage_k[l % self.n_slots][n]
            pv[j] = self.stage_v[l % self.n_slots][n]
        return pk, pv

    def run_chunk(self, inputs: Sequence[LayerInputs], n_steps: int,
                  outputs: Dict[Tuple[int, int], torch.Tensor],
                  probe: Optional[Callable[[int, int], None]] = None, concurrent: bool = True) -> None:
        """All layers x n_steps, ending on the current stream.  outputs[(layer, step)]
        is a [Lq][H][d] tensor of the element type for every pair the caller
        wants.  probe(layer, step), if given, is called after each layer-step
        has been enqueued (to copy out the per-step buffers, in stream order).
        concurrent=False issues every call on the current stream."""
        g, ws = self.geom, self.ws
        L = self.n_layers
        intra = bool(g.intra_split)
        stream = torch.cuda.current_stream()
        side = self.side if concurrent else stream
        ws_lin = self.ws_lin if concurrent else ws
        fused: Optional[torch.cuda.Event] = None  # the last fusion (last reader of O_lin)
        copy_done: List[Optional[torch.cuda.Event]] = [None] * L
        last_reader: List[Optional[torch.cuda.Event]] = [None] * self.n_slots  # per staging slot
        issued = 0  # layers whose prefetch has been issued
        for step in range(n_steps):
            for l in range(L):
                inp, st = inputs[l], self.layers[l]
                q, x = inp.q[step], inp.x[step]
                if step == 0:
                    # keep the copies of the next n_slots-1 layers in flight; the slot
                    # of layer l+n_slots-1 was last read by layer l-1's gather
                    while issued < L and issued < l + self.n_slots:
                        self._prefetch(issued, inputs[issued], last_reader, copy_done)
                        issued += 1
                    # scoring: non-resident pages come from the cached means
                    ops.hsa_score_pages(g, q, inp.pages_k, inp.page_kmean, st.scores, st.sel_pages, ws)
                    if copy_done[l] is not None:
                        stream.wait_event(copy_done[l])
                    pk, pv = self._staged_tables(l, inp)
                    if intra:
                        ops.hsa_gather_active(g, pk, pv, st.sel_pages, inp.k_cur[0], inp.v_cur[0], st.k_act,
                                              st.v_act, st.kblk_mean)
                    else:
                        ops.hsa_gather_pages(g, pk, pv, st.sel_pages, st.k_act, st.v_act, st.kblk_mean)
                    if inp.host_k:
                        ev = torch.cuda.Event()
                        ev.record(stream)
                        last_reader[l % self.n_slots] = ev
                elif intra:
                    # this step's own keys into the chunk's part of the active buffer
                    ops.hsa_gather_chunk(g, inp.k_cur[step], inp.v_cur[step], st.k_act, st.v_act, st.kblk_mean)
                if concurrent:
                    # the linear branch needs this layer's gathered K/V (or its
                    # projections) and a free O_lin
                    ready = torch.cuda.Event()
                    ready.record(stream)
                    side.wait_event(ready)
                    if fused is not None:
                        side.wait_event(fused)
                if intra:
                    if step == 0:  # the history's projection, kept for every step
                        ops.hsa_linear_branch(g, None, st.k_act, st.v_act, inp.e_k, inp.e_v, st.k_proj, st.v_proj,
                                              None, HSA_LIN_HISTORY_PROJ, ws_lin, side)
                    ops.hsa_linear_branch(g, q, st.k_act, st.v_act, inp.e_k, inp.e_v, st.k_proj, st.v_proj,
                                          self.o_lin, HSA_LIN_CHUNK_PROJ, ws_lin, side)
                elif step == 0:
                    ops.hsa_linear_branch(g, q, st.k_act, st.v_act, inp.e_k, inp.e_v, st.k_proj, st.v_proj,
                                          self.o_lin, 0, ws_lin, side)
                else:
                    ops.hsa_linear_branch(g, q, None, None, None, None, st.k_proj, st.v_proj, self.o_lin,
                                          HSA_LIN_REUSE_PROJ, ws_lin, side)
                if concurrent:
                    linear_done = torch.cuda.Event()
                    linear_done.record(side)
                ops.hsa_block_select(g, q, st.k_act, st.kblk_mean, inp.tau, self.blk_count, self.blk_idx, None, ws)
                ops.hsa_sparse_attn(g, q, st.k_act, st.v_act, self.blk_count, self.blk_idx, self.o_sp, ws)
                if concurrent:
                    stream.wait_event(linear_done)
                out = outputs.get((l, step), self.scratch_out)
                ops.hsa_fuse(g, x, inp.w_g, None, self.o_lin, self.o_sp, out)
                if probe is not None:
                    probe(l, step)
                if concurrent:
                    # after the probe's copies too: they also read O_lin
                    fused = torch.cuda.Event()
                    fused.record(stream)


def make_layer_inputs(geom: Geom, pages_k: List[torch.Tensor], pages_v: List[torch.Tensor], host_ids: Sequence[int],
                      e_k, e_v, w_g, tau, qs: List[torch.Tensor], xs: List[torch.Tensor],
                      k_cur: Sequence[torch.Tensor] = (), v_cur: Sequence[torch.Tensor] = ()) -> LayerInputs:
    """Set up one layer: index every page (its mean key, through the library's
    scoring call) while all pages are resident, then move the pages in
    host_ids to pinned host memory and drop their device copies."""
    s = Dims.of(geom)
    n_pages = len(pages_k)
    dev = pages_k[0].device
    kmean = torch.empty(n_pages, s.H, s.d, dtype=torch.float32, device=dev)
    scores = torch.empty(n_pages, dtype=torch.float32, device=dev)
    sel = torch.empty(s.Kp, dtype=torch.int32, device=dev)
    ws = torch.empty(ops.hsa_workspace_bytes(geom, n_pages), dtype=torch.uint8, device=dev)
    ops.hsa_score_pages(geom, qs[0], pages_k, kmean, scores, sel, ws)
    torch.cuda.current_stream().synchronize()
    del ws
    pk, pv = list(pages_k), list(pages_v)
    host_k, host_v = {}, {}
    for j in host_ids:
        host_k[int(j)] = torch.empty(pk[j].shape, dtype=pk[j].dtype, pin_memory=True)
        host_v[int(j)] = torch.empty(pv[j].shape, dtype=pv[j].dtype, pin_memory=True)
        host_k[int(j)].copy_(pk[j])
        host_v[int(j)].copy_(pv[j])
        pk[j] = None
        pv[j] = None
    return LayerInputs(pages_k=pk, pages_v=pv, host_k=host_k, host_v=host_v, e_k=e_k, e_v=e_v, w_g=w_g, tau=tau,
                       page_kmean=kmean, q=list(qs), x=list(xs), k_cur=list(k_cur), v_cur=list(v_cur))
