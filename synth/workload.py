"""Seeded synthetic inputs for the HSA decode step.

This module draws random tensors and plants known structure in them; it
computes no step of the attention method.  Both the CPU oracle and the GPU
path consume exactly what it returns.

Every tensor comes from its own stream,
    numpy SeedSequence([cfg.seed, tensor_id, layer, page, step]),
so any page of any layer can be regenerated alone (long histories stream).
Floating-point values are drawn in float32; for bf16 workloads each tensor
is rounded to bfloat16 (round to nearest even, torch's CPU cast) and the
oracle reads the rounded values.

Planted structure (all in tile-major token order):
  * retrieval: a seeded target page set T (|T| = n_sel_pages).  Per head a
    unit direction w_h; pages in T get key mean mu_norm*w_h, other pages get
    mu_norm times a unit vector orthogonal to w_h; every query token gets
    q_shift*w_h.  The mean-query/mean-key score then ranks T first.
  * "rank8": per head an orthonormal basis U_h (d x 8, orthogonal to w_h);
    each key block b adds U_h a_b and each query block i adds U_h c_i with
    a_b, c_i ~ N(0, s^2 I_8), centred over the page (resp. the chunk) so the
    page and chunk means are unchanged.  Pooled block logits then spread out
    and block mass concentrates.
  * "imbalance": heads [0, uniform_heads) have iid keys and queries only;
    the other heads get the retrieval planting plus, for every query block,
    hot_per_row distinct hot key blocks inside T (disjoint across query
    blocks) that share a random direction g with the query block, scaled by
    hot_scale.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional

import numpy as np

from .configs import Config

TID = dict(q=1, k=2, v=3, x=4, ek=5, ev=6, wg=7, mu=8, struct=9, tau=10, hot=11, host=12, prompt=13,
           kcur=14, vcur=15)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    out = r.view(np.float32)
    nan = np.isnan(a)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Exact bfloat16 bit patterns (uint16) of values that are already bf16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _orthonormal(rng: np.random.Generator, d: int, k: int, avoid: Optional[np.ndarray] = None) -> np.ndarray:
    """d x k orthonormal columns, orthogonal to `avoid` (a unit vector) when given."""
    cols = rng.standard_normal((d, k + (1 if avoid is not None else 0)))
    if avoid is not None:
        cols[:, 0] = avoid
    q, _ = np.linalg.qr(cols)
    if avoid is not None:
        q = q[:, 1:]
    return q


@dataclass
class Plant:
    target_pages: np.ndarray        # sorted page ids of T
    w: np.ndarray                   # [H][d]
    U: np.ndarray                   # [H][d][8]
    hot: Optional[np.ndarray]       # [H][nQB][hot_per_row] active key-block ids (imbalance) or None


class Workload:
    """Deterministic inputs of one layer of one configuration."""

    def __init__(self, cfg: Config, layer: int = 0):
        cfg.check()
        self.cfg = cfg
        self.layer = layer
        self.plant = self._plant()

    # ------------------------------------------------------------------ rng
    def rng(self, tid: str, page: int = 0, step: int = 0) -> np.random.Generator:
        ss = np.random.SeedSequence([self.cfg.seed, TID[tid], self.layer, page, step])
        return np.random.default_rng(ss)

    def _finish(self, a: np.ndarray) -> np.ndarray:
        a = a.astype(np.float32, copy=False)
        return round_bf16(a) if self.cfg.dtype == "bf16" else a

    # ------------------------------------------------------------ structure
    def _structured_heads(self) -> np.ndarray:
        c = self.cfg
        if c.structure == "imbalance":
            return np.arange(c.uniform_heads, c.n_heads)
        return np.arange(c.n_heads)

    def _plant(self) -> Plant:
        c = self.cfg
        r = self.rng("struct")
        T = np.sort(r.choice(c.n_pages, size=c.n_sel_pages, replace=False))
        w = np.zeros((c.n_heads, c.head_dim))
        U = np.zeros((c.n_heads, c.head_dim, 8))
        for h in range(c.n_heads):
            v = r.standard_normal(c.head_dim)
            w[h] = v / np.linalg.norm(v)
            U[h] = _orthonormal(r, c.head_dim, 8, avoid=w[h])
        hot = None
        if c.structure == "imbalance":
            rh = self.rng("hot")
            need = c.n_qblocks * c.hot_per_row
            assert need <= c.n_kblocks, "hot blocks must be disjoint across query blocks"
            hot = np.zeros((c.n_heads, c.n_qblocks, c.hot_per_row), dtype=np.int64)
            for h in range(c.n_heads):
                perm = rh.permutation(c.n_kblocks)[:need]
                hot[h] = perm.reshape(c.n_qblocks, c.hot_per_row)
        return Plant(T, w, U, hot)

    def _hot_dirs(self) -> np.ndarray:
        """[H][nQB][d] shared directions g of the imbalance planting."""
        c = self.cfg
        return self.rng("hot", page=1).standard_normal((c.n_heads, c.n_qblocks, c.head_dim))

    # -------------------------------------------------------------- tensors
    def q(self, step: int = 0) -> np.ndarray:
        """Queries [Lq][H][d] of the current chunk."""
        c = self.cfg
        q = self.rng("q", step=step).standard_normal((c.query_tokens, c.n_heads, c.head_dim), dtype=np.float32)
        heads = self._structured_heads()
        q[:, heads, :] += (c.q_shift * self.plant.w[heads]).astype(np.float32)
        if c.structure == "rank8":
            rs = self.rng("struct", page=10_000, step=step)
            coef = rs.normal(0.0, c.struct_scale, size=(c.n_heads, c.n_qblocks, 8))
            coef -= coef.mean(axis=1, keepdims=True)
            add = np.einsum("hdk,hik->ihd", self.plant.U, coef)          # [nQB][H][d]
            # every token of query block i gets add[i] (in place, block by block)
            q.reshape(c.n_qblocks, c.block, c.n_heads, c.head_dim)[...] += add.astype(np.float32)[:, None]
        elif c.structure == "imbalance":
            g = self._hot_dirs()                                          # [H][nQB][d]
            for h in heads:
                q[:, h, :] += np.repeat(c.hot_scale * g[h], c.block, axis=0).astype(np.float32)
        return self._finish(q)

    def page_k(self, j: int) -> np.ndarray:
        """Keys [Lp][H][d] of history page j."""
        c = self.cfg
        k = self.rng("k", page=j).standard_normal((c.page_tokens, c.n_heads, c.head_dim), dtype=np.float32)
        heads = self._structured_heads()
        rm = self.rng("mu", page=j)
        in_T = j in set(self.plant.target_pages.tolist())
        for h in heads:
            if in_T:
                mu = c.mu_norm * self.plant.w[h]
            else:
                v = rm.standard_normal(c.head_dim)
                v -= v.dot(self.plant.w[h]) * self.plant.w[h]
                mu = c.mu_norm * v / np.linalg.norm(v)
            k[:, h, :] += mu.astype(np.float32)
        if c.structure == "rank8":
            rs = self.rng("struct", page=1 + j)
            coef = rs.normal(0.0, c.struct_scale, size=(c.n_heads, c.blocks_per_page, 8))
            coef -= coef.mean(axis=1, keepdims=True)
            add = np.einsum("hdk,hbk->bhd", self.plant.U, coef)
            # every token of key block b gets add[b] (in place, block by block)
            k.reshape(c.blocks_per_page, c.block, c.n_heads, c.head_dim)[...] += add.astype(np.float32)[:, None]
        elif c.structure == "imbalance" and in_T:
            slot = int(np.searchsorted(self.plant.target_pages, j))
            g = self._hot_dirs()
            bpp = c.blocks_per_page
            for h in heads:
                for i in range(c.n_qblocks):
                    for b in self.plant.hot[h, i]:
                        if b // bpp == slot:
                            lb = int(b % bpp)
                            k[lb * c.block:(lb + 1) * c.block, h, :] += (c.hot_scale * g[h, i]).astype(np.float32)
        return self._finish(k)

    def page_v(self, j: int) -> np.ndarray:
        """Values [Lp][H][d] of history page j."""
        c = self.cfg
        v = self.rng("v", page=j).standard_normal((c.page_tokens, c.n_heads, c.head_dim), dtype=np.float32)
        return self._finish(v)

    def k_cur(self, step: int = 0) -> np.ndarray:
        """The chunk's own keys [Lq][H][d] (joined to the history with
        intra_split): N(0, 1), plus the planted direction at mu_norm on the
        structured heads (the chunk is its own most relevant context), plus,
        for the rank-8 structure, the rank-8 code of the query tile each token
        belongs to (a query block finds its own tile's keys)."""
        c = self.cfg
        k = self.rng("kcur", step=step).standard_normal((c.query_tokens, c.n_heads, c.head_dim), dtype=np.float32)
        heads = self._structured_heads()
        k[:, heads, :] += (c.mu_norm * self.plant.w[heads]).astype(np.float32)
        if c.structure == "rank8":
            rs = self.rng("struct", page=10_000, step=step)  # the queries' coefficients
            coef = rs.normal(0.0, c.struct_scale, size=(c.n_heads, c.n_qblocks, 8))
            coef -= coef.mean(axis=1, keepdims=True)
            add = np.einsum("hdk,hik->ihd", self.plant.U, coef)          # [nQB][H][d]
            k.reshape(c.n_qblocks, c.block, c.n_heads, c.head_dim)[...] += add.astype(np.float32)[:, None]
        return self._finish(k)

    def v_cur(self, step: int = 0) -> np.ndarray:
        """The chunk's own values [Lq][H][d], N(0, 1)."""
        c = self.cfg
        v = self.rng("vcur", step=step).standard_normal((c.query_tokens, c.n_heads, c.head_dim), dtype=np.float32)
        return self._finish(v)

    def x(self, step: int = 0) -> np.ndarray:
        """Gate input [Lq][D] (the layer's hidden states of the current chunk)."""
        c = self.cfg
        return self._finish(self.rng("x", step=step).standard_normal((c.query_tokens, c.model_dim), dtype=np.float32))

    def e_k(self) -> np.ndarray:
        """Sequence projection for keys, [r][L], entries N(0, variance 1/L)."""
        c = self.cfg
        e = self.rng("ek").standard_normal((c.rank, c.active_tokens), dtype=np.float32) / np.float32(np.sqrt(c.active_tokens))
        return self._finish(e)

    def e_v(self) -> np.ndarray:
        """Sequence projection for values, [r][L], entries N(0, variance 1/L)."""
        c = self.cfg
        e = self.rng("ev").standard_normal((c.rank, c.active_tokens), dtype=np.float32) / np.float32(np.sqrt(c.active_tokens))
        return self._finish(e)

    def w_g(self) -> np.ndarray:
        """Gate weights [2H][D] (row c produces gate column c), entries N(0, std 0.02)."""
        c = self.cfg
        return self._finish(self.rng("wg").normal(0.0, 0.02, size=(2 * c.n_heads, c.model_dim)).astype(np.float32))

    def tau(self) -> np.ndarray:
        """Per-head mass thresholds tau_h (float32)."""
        c = self.cfg
        if c.tau:
            assert len(c.tau) == c.n_heads
            return np.asarray(c.tau, dtype=np.float32)
        lo, hi = c.tau_range
        return self.rng("tau").uniform(lo, hi, size=c.n_heads).astype(np.float32)

    def host_pages(self) -> np.ndarray:
        """Page ids that start in pinned host memory (stack config), seeded."""
        c = self.cfg
        n = int(round(c.host_page_frac * c.n_sel_pages))
        if n == 0:
            return np.zeros(0, dtype=np.int64)
        return np.sort(self.rng("host").choice(self.plant.target_pages, size=n, replace=False))

    # ------------------------------------------------------------ bundles
    def small_inputs(self, step: int = 0) -> Dict[str, np.ndarray]:
        d = dict(q=self.q(step), x=self.x(step), e_k=self.e_k(), e_v=self.e_v(),
                 w_g=self.w_g(), tau=self.tau())
        if self.cfg.intra_split:
            d.update(k_cur=self.k_cur(step), v_cur=self.v_cur(step))
        return d

    def pages(self):
        return [self.page_k(j) for j in range(self.cfg.n_pages)], [self.page_v(j) for j in range(self.cfg.n_pages)]


def layer_arrays(cfg: Config, layer: int, n_steps: int, workers: int = 8) -> Dict[str, object]:
    """All inputs of one layer of a stack, as float32 arrays: pages (generated
    on a thread pool), the layer's projections, gate weights and thresholds,
    the per-step queries and gate inputs, and with intra_split the per-step
    keys and values of the chunk itself."""
    from concurrent.futures import ThreadPoolExecutor
    w = Workload(cfg, layer)
    with ThreadPoolExecutor(max(1, workers)) as ex:
        pk = list(ex.map(w.page_k, range(cfg.n_pages)))
        pv = list(ex.map(w.page_v, range(cfg.n_pages)))
        qs = list(ex.map(w.q, range(n_steps)))
        xs = list(ex.map(w.x, range(n_steps)))
        kc = list(ex.map(w.k_cur, range(n_steps))) if cfg.intra_split else []
        vc = list(ex.map(w.v_cur, range(n_steps))) if cfg.intra_split else []
    return dict(pages_k=pk, pages_v=pv, e_k=w.e_k(), e_v=w.e_v(), w_g=w.w_g(), tau=w.tau(), q=qs, x=xs,
                k_cur=kc, v_cur=vc, target_pages=w.plant.target_pages)


def chunk_prompts(cfg: Config, pages_per_chunk: int, emb_dim: int = 512, noise: float = 0.5, layer: int = 0):
    """Prompt-level retrieval inputs for a layer's history: pages are grouped
    into chunks of pages_per_chunk consecutive ids (the last one may be
    shorter), every previous chunk gets a seeded N(0, 1) prompt embedding, and
    the current prompt is the embedding of the chunk holding the first target
    page plus N(0, noise^2) noise.  Returns (page_chunk [P] int32,
    current [E] float32, previous [C][E] float32, that chunk's id)."""
    n_chunks = -(-cfg.n_pages // pages_per_chunk)
    page_chunk = (np.arange(cfg.n_pages) // pages_per_chunk).astype(np.int32)
    w = Workload(cfg, layer)
    target = int(page_chunk[int(w.plant.target_pages[0])])
    r = w.rng("prompt")
    prev = r.standard_normal((n_chunks, emb_dim)).astype(np.float32)
    cur = (prev[target] + noise * r.standard_normal(emb_dim)).astype(np.float32)
    return page_chunk, cur, prev, target


def chunk_prompt_sequence(cfg: Config, pages_per_chunk: int, n: int, emb_dim: int = 512, noise: float = 0.5):
    """Prompts of n generated chunks over one history: as chunk_prompts, but
    the t-th prompt is the embedding of history chunk targets[t] plus noise,
    with targets a seeded walk that never repeats the previous chunk.
    Returns (page_chunk [P] int32, prompts [n][E], previous [C][E], targets)."""
    page_chunk, _, prev, first = chunk_prompts(cfg, pages_per_chunk, emb_dim, noise)
    r = Workload(cfg).rng("prompt", page=1)
    n_chunks = len(prev)
    targets = [first]
    for _ in range(n - 1):
        step = int(r.integers(1, n_chunks)) if n_chunks > 1 else 0
        targets.append((targets[-1] + step) % n_chunks)
    prompts = np.stack([prev[c] + noise * r.standard_normal(emb_dim) for c in targets]).astype(np.float32)
    return page_chunk, prompts, prev, np.asarray(targets)


def stack_host_pages(cfg: Config) -> List[np.ndarray]:
    """Per layer, the page ids that start in pinned host memory (layer stack).

    A seeded round(host_page_frac * layers * n_sel_pages) of the
    (layer, target page) pairs are chosen over the whole stack (for the
    30-layer stack: 36 of 120); the target pages are the ones the planted
    retrieval structure makes the scoring select."""
    n_pairs = cfg.layers * cfg.n_sel_pages
    n_host = int(round(cfg.host_page_frac * n_pairs))
    targets = [Workload(cfg, layer).plant.target_pages for layer in range(cfg.layers)]
    rng = np.random.default_rng(np.random.SeedSequence([cfg.seed, TID["host"], 1_000_000]))
    pick = np.sort(rng.choice(n_pairs, size=n_host, replace=False)) if n_host else np.zeros(0, np.int64)
    out = [[] for _ in range(cfg.layers)]
    for p in pick:
        layer, slot = divmod(int(p), cfg.n_sel_pages)
        out[layer].append(int(targets[layer][slot]))
    return [np.asarray(sorted(v), dtype=np.int64) for v in out]
