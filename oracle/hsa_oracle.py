"""CPU oracle of the HSA decode step -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package's smoke check and the benchmark's CPU-baseline leg
may import this module.  It shares no code with the GPU path (the HIP
library): it is a plain, slow, float64 NumPy restatement of what the method
computes, written from these pages:

  [WA]  "WorldAttention: An Efficient Attention Architecture for Interactive
        Video World Models", paper full text (paperpeel.com/paper/2609.34606)
  [SUM] the structured Chinese summary of the same paper
        (paper.rainbus.top/paper/2609.34606), method steps (1)-(6)

Steps, in the pages' order:
  stage 1           [WA §3.2 "Stage 1: prompt-level retrieval"; §4.5 ablation
                     of candidate chunks; SUM step (2)]: cosine similarity of
                     prompt embeddings, top-k chunks; then S1 over the pages
                     of those chunks with the page budget split evenly.
  S1 page scoring   [WA §3.2 "Stage 2: page-level retrieval", score equation;
                     SUM step (3)]: alpha_j = mean_h( Qbar_h . Kbar_{j,h} ) / sqrt(d_k),
                     top-K_p pages.
  S2 active KV      [WA §3.2 "Active KV construction"; SUM step (4)]: the
                     selected pages concatenated, ascending page id.
  S3 linear branch  [WA §3.3 "Linear branch", output equation; SUM
                     prerequisites, linear attention]: Ktil = E_K K,
                     Vtil = E_V V (E given as [r][L]); O_lin = softmax(Q Ktil^T/sqrt d) Vtil.
  S4 block selection[WA §3.3 "Head-level sparsity adaptation"; appendix A.1.2;
                     SUM step (5)]: mean-pooled blocks, pooled softmax mass per
                     (head, query block); the smallest set of key blocks whose
                     mass reaches tau_h.
  S5 sparse branch  [WA §3.3 "Sparse branch"; appendix A.1.3]: exact softmax
                     attention restricted to the tokens of the selected blocks.
  intra-chunk keys  [WA §3.3 "Inter- and intra-chunk sparse granularity"]:
                     the chunk's own tokens follow the history in the active
                     sequence; the history is selected in B-token tiles, the
                     chunk in finer b_intra-token blocks, under one softmax.
  S6 fusion         [WA §3.3 "Gated fusion of two branches"; SUM step (6)]:
                     G = X W, sigmoid gates per (token, head) and branch,
                     O = O_lin * g_lin + O_sp * g_sp.

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):
  * head averaging of the page score (Qbar has one vector per head);
  * ties in any top-k go to the lower index; selections are emitted in
    ascending index order;
  * blocks are contiguous B-token ranges of the tile-major sequence; pooling
    is the mean; the mass is the softmax of pooled logits with the same
    1/sqrt(d) scale; "exceeds" is read as >=, tau_h >= 1 keeps every block,
    and at least one block is always kept;
  * one E_K and one E_V per layer shared by all heads; two independent
    sigmoid gates, W given as [2H][D] (row c -> gate column c), no bias.

Selections at near-ties are flagged (gap < TIE_EPS); there several answers
are valid and `valid_page_selection` / `valid_block_selection` decide
validity instead of equality.
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np

TIE_EPS = 1e-5

# --------------------------------------------------------------------------
# O1 -- token order.  [WA appendix A.1.3]: each contiguous group of B tokens
# of the flattened sequence is one (C_t, C_h, C_w) cube of the (T, H, W)
# latent volume.  The cube order and the order inside a cube are not given
# (the formula is missing from the page); reading: cubes in raster order of
# the cube grid, tokens raster order inside the cube.
# --------------------------------------------------------------------------


def tile_major_index(f: int, y: int, x: int, frame_h: int, frame_w: int,
                     tile: Tuple[int, int, int]) -> int:
    ct, ch, cw = tile
    gh, gw = frame_h // ch, frame_w // cw
    b = ct * ch * cw
    cube = ((f // ct) * gh + y // ch) * gw + x // cw
    inner = ((f % ct) * ch + y % ch) * cw + x % cw
    return cube * b + inner


def raster_to_tile_major(n_frames: int, frame_h: int, frame_w: int,
                         tile: Tuple[int, int, int]) -> np.ndarray:
    """perm[raster_index] = tile-major index, for a volume of n_frames frames."""
    out = np.empty(n_frames * frame_h * frame_w, dtype=np.int64)
    i = 0
    for f in range(n_frames):
        for y in range(frame_h):
            for x in range(frame_w):
                out[i] = tile_major_index(f, y, x, frame_h, frame_w, tile)
                i += 1
    return out


# --------------------------------------------------------------------------
# S1 -- page scoring.  [WA §3.2 Stage 2, score equation; SUM step (3)]
# --------------------------------------------------------------------------


def mean_over_tokens(t: np.ndarray) -> np.ndarray:
    """[N][H][d] -> [H][d]: the average over the N tokens (float64)."""
    return np.asarray(t, dtype=np.float64).mean(axis=0)


def page_scores(qbar: np.ndarray, kbars: np.ndarray) -> np.ndarray:
    """qbar [H][d], kbars [P][H][d] -> alpha [P].

    alpha_j = (1/H) sum_h qbar_h . kbar_{j,h} / sqrt(d)  (head-averaged reading).
    """
    H, d = qbar.shape
    dots = np.einsum("hd,phd->ph", qbar.astype(np.float64), kbars.astype(np.float64))
    return dots.mean(axis=1) / math.sqrt(d)


def nan_as_neginf(vals) -> np.ndarray:
    v = np.asarray(vals, dtype=np.float64)
    return np.where(np.isnan(v), -np.inf, v)


def top_k_lower_index(vals: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Order by (value descending, index ascending); return (order, top-k ascending).
    Reading: a NaN value ranks as -inf (below every number, equal values by index)."""
    v = nan_as_neginf(vals)
    idx = np.arange(len(v))
    order = np.lexsort((idx, -v))
    return order, np.sort(order[:k])


def select_pages(alpha: np.ndarray, k: int) -> Tuple[np.ndarray, bool]:
    """Top-k pages (ascending ids) and whether the k-th/(k+1)-th gap is a near-tie."""
    order, sel = top_k_lower_index(alpha, k)
    tie = False
    if k < len(alpha):
        tie = bool(alpha[order[k - 1]] - alpha[order[k]] < TIE_EPS)
    return sel, tie


def valid_page_selection(alpha: np.ndarray, sel: Sequence[int], k: int) -> bool:
    sel = np.asarray(sel)
    if len(sel) != k or len(set(sel.tolist())) != k:
        return False
    if np.any(sel < 0) or np.any(sel >= len(alpha)):
        return False
    rest = np.setdiff1d(np.arange(len(alpha)), sel)
    if len(rest) == 0:
        return True
    return bool(alpha[sel].min() >= alpha[rest].max() - TIE_EPS)


def score_and_select(q: np.ndarray, pages_k: Sequence[np.ndarray], k: int):
    qbar = mean_over_tokens(q)
    kbars = np.stack([mean_over_tokens(p) for p in pages_k])
    alpha = page_scores(qbar, kbars)
    sel, tie = select_pages(alpha, k)
    return dict(qbar=qbar, kbars=kbars, alpha=alpha, sel=sel, tie=tie)


# --------------------------------------------------------------------------
# Stage 1 -- prompt-level retrieval, and page retrieval inside the chosen
# chunks.  [WA §3.2 "Stage 1: prompt-level retrieval" (cosine similarity of
# the current prompt embedding with the previous chunks' prompt embeddings,
# top-1 chunk) and "Stage 2: page-level retrieval" (the pages of the
# retrieved chunks are scored); §4.5 ablation of prompt-level candidate
# chunks (Top-2 takes two pages from each chunk, Top-4 one page from each,
# under the same four-page budget); SUM step (2)]
# Readings: a zero embedding has similarity 0 with every embedding; the
# budget K_p is split evenly over the chosen chunks (K_p divisible by their
# number); a chosen chunk with fewer pages than its share gives its slots to
# the best remaining pages of the chosen chunks, then to the lowest ids.
# --------------------------------------------------------------------------


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    na, nb = math.sqrt(float(a @ a)), math.sqrt(float(b @ b))
    if na == 0.0 or nb == 0.0:
        return 0.0
    return float(a @ b) / (na * nb)


def prompt_retrieval(e_cur: np.ndarray, e_past: np.ndarray, k: int):
    """Cosine similarity of the current prompt embedding [E] with every past
    chunk's [C][E]; the top-k chunks (ascending ids) and a near-tie flag."""
    sims = np.array([cosine(e_cur, e) for e in np.asarray(e_past)])
    sel, tie = select_pages(sims, k)
    return dict(sims=sims, sel=sel, tie=tie)


def select_pages_in_chunks(alpha: np.ndarray, page_chunk: Sequence[int], sel_chunks: Sequence[int], k_p: int):
    """Pages of the chosen chunks: from each chosen chunk its K_p / n best
    pages (by alpha, ties to the lower id); slots a short chunk leaves go to
    the best other pages of the chosen chunks, then to the lowest page ids.
    Returns (ascending page ids, near-tie flag)."""
    alpha = np.asarray(alpha, dtype=np.float64)
    page_chunk = np.asarray(page_chunk)
    chosen = set(int(c) for c in sel_chunks)
    n = len(chosen)
    assert k_p % n == 0, "the page budget is split evenly over the chosen chunks"
    share = k_p // n
    P = len(alpha)
    cand = np.array([int(page_chunk[j]) in chosen for j in range(P)])
    in_share = np.zeros(P, dtype=bool)
    tie = False
    for ch in sorted(chosen):
        ids = np.flatnonzero(page_chunk == ch)
        order, _ = top_k_lower_index(alpha[ids], min(share, len(ids)))
        in_share[ids[order[:share]]] = True
        if len(ids) > share and alpha[ids[order[share - 1]]] - alpha[ids[order[share]]] < TIE_EPS:
            tie = True
    # tiers: within a chunk's share, other pages of the chosen chunks, the rest
    tier = np.where(in_share, 0, np.where(cand, 1, 2))
    key_alpha = np.where(cand, nan_as_neginf(alpha), -np.inf)
    order = sorted(range(P), key=lambda j: (tier[j], -key_alpha[j], j))
    sel = np.sort(np.array(order[:k_p], dtype=np.int64))
    n_in = int(in_share.sum())
    if n_in < k_p < P and tier[order[k_p - 1]] == 1 == tier[order[k_p]]:
        tie = tie or bool(key_alpha[order[k_p - 1]] - key_alpha[order[k_p]] < TIE_EPS)
    return sel, tie


def score_chunk_pages(q: np.ndarray, pages_k: Sequence[np.ndarray], page_chunk: Sequence[int],
                      sel_chunks: Sequence[int], k_p: int):
    """Stage 2 over the chosen chunks only: alpha for their pages (-inf for
    every other page, whose keys are not read), then the per-chunk budget."""
    chosen = set(int(c) for c in sel_chunks)
    qbar = mean_over_tokens(q)
    alpha = np.full(len(pages_k), -np.inf)
    for j, p in enumerate(pages_k):
        if int(page_chunk[j]) in chosen:
            alpha[j] = page_scores(qbar, mean_over_tokens(p)[None])[0]
    sel, tie = select_pages_in_chunks(alpha, page_chunk, sel_chunks, k_p)
    return dict(alpha=alpha, sel=sel, tie=tie)


# --------------------------------------------------------------------------
# S2 -- active KV.  [WA §3.2 "Active KV construction"; SUM step (4)]
# --------------------------------------------------------------------------


def gather_active(pages: Sequence[np.ndarray], sel: Sequence[int]) -> np.ndarray:
    """Concatenate the selected pages ([Lp][H][d] each), ascending id -> [H][L][d]."""
    cat = np.concatenate([np.asarray(pages[j]) for j in sel], axis=0)   # [L][H][d]
    return np.ascontiguousarray(cat.transpose(1, 0, 2))


# --------------------------------------------------------------------------
# S3 -- linear branch.  [WA §3.3 "Linear branch", output equation;
# SUM prerequisites, Linformer projection E_K^T K with r << L]
# --------------------------------------------------------------------------


def project(e: np.ndarray, act: np.ndarray) -> np.ndarray:
    """e [r][L], act [H][L][d] -> [H][r][d]: the sequence-axis projection per head
    (one matrix product E @ act_h per head)."""
    e = np.asarray(e, dtype=np.float64)
    return np.stack([e @ np.asarray(a, dtype=np.float64) for a in act])


def softmax_rows(s: np.ndarray) -> np.ndarray:
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    return p / p.sum(axis=-1, keepdims=True)


def linear_attention(q: np.ndarray, ktil: np.ndarray, vtil: np.ndarray) -> np.ndarray:
    """q [Lq][H][d], ktil/vtil [H][r][d] -> O_lin [Lq][H][d]."""
    Lq, H, d = q.shape
    out = np.empty((Lq, H, d))
    for h in range(H):
        s = q[:, h, :].astype(np.float64) @ ktil[h].T / math.sqrt(d)
        out[:, h, :] = softmax_rows(s) @ vtil[h]
    return out


def linear_branch(q, k_act, v_act, e_k, e_v):
    ktil = project(e_k, k_act)
    vtil = project(e_v, v_act)
    return dict(ktil=ktil, vtil=vtil, o_lin=linear_attention(q, ktil, vtil))


# --------------------------------------------------------------------------
# S4 -- head-adaptive block selection.  [WA §3.3 "Head-level sparsity
# adaptation"; appendix A.1.2 (cheap coarse estimate of where the mass is);
# SUM step (5), pooled coarse selection]
# --------------------------------------------------------------------------


def block_means(t: np.ndarray, b: int) -> np.ndarray:
    """[H][N][d] -> [H][N/b][d]: mean of each contiguous b-token block."""
    H, N, d = t.shape
    return np.asarray(t, dtype=np.float64).reshape(H, N // b, b, d).mean(axis=2)


def pooled_mass(qbar_i: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """qbar_i [d], kbar [nKB][d] -> softmax over key blocks of qbar_i.kbar_j/sqrt(d)."""
    d = qbar_i.shape[0]
    s = kbar.astype(np.float64) @ qbar_i.astype(np.float64) / math.sqrt(d)
    return softmax_rows(s[None, :])[0]


def select_blocks(m: np.ndarray, tau: float) -> Tuple[np.ndarray, bool]:
    """Smallest mass-ordered prefix whose cumulative mass reaches tau (ascending ids), tie flag."""
    n_all = len(m)
    order, _ = top_k_lower_index(m, n_all)
    c = np.cumsum(m[order])
    tau = float(tau)
    if tau >= 1.0:
        n = n_all
    else:
        hit = np.nonzero(c >= tau)[0]
        n = int(hit[0]) + 1 if len(hit) else n_all
    sel = np.sort(order[:n])
    flag = False
    if tau < 1.0:
        if n < n_all and m[order[n - 1]] - m[order[n]] < TIE_EPS:
            flag = True
        if abs(c[n - 1] - tau) < TIE_EPS:
            flag = True
        if n >= 2 and abs(c[n - 2] - tau) < TIE_EPS:
            flag = True
    return sel, flag


def valid_block_selection(m: np.ndarray, sel: Sequence[int], tau: float) -> bool:
    sel = np.asarray(sel)
    n_all = len(m)
    if len(sel) == 0 or len(set(sel.tolist())) != len(sel):
        return False
    if np.any(sel < 0) or np.any(sel >= n_all):
        return False
    if float(tau) >= 1.0:
        return len(sel) == n_all
    rest = np.setdiff1d(np.arange(n_all), sel)
    if len(rest) and m[sel].min() < m[rest].max() - TIE_EPS:
        return False
    tot = m[sel].sum()
    if tot < tau - TIE_EPS:
        return False
    return bool(tot - m[sel].min() < tau + TIE_EPS)


def block_selection(q: np.ndarray, k_act: np.ndarray, tau: Sequence[float], b: int):
    """q [Lq][H][d], k_act [H][L][d] -> per (h, i) selections, masses and tie flags."""
    qb = block_means(np.asarray(q).transpose(1, 0, 2), b)     # [H][nQB][d]
    kb = block_means(k_act, b)                                 # [H][nKB][d]
    H, nqb, _ = qb.shape
    nkb = kb.shape[1]
    mass = np.empty((H, nqb, nkb))
    sel: List[List[np.ndarray]] = []
    flags = np.zeros((H, nqb), dtype=bool)
    for h in range(H):
        row = []
        for i in range(nqb):
            mass[h, i] = pooled_mass(qb[h, i], kb[h])
            s, f = select_blocks(mass[h, i], tau[h])
            row.append(s)
            flags[h, i] = f
        sel.append(row)
    counts = np.array([[len(s) for s in r] for r in sel], dtype=np.int64)
    return dict(qbar=qb, kbar=kb, mass=mass, sel=sel, counts=counts, flags=flags)


# --------------------------------------------------------------------------
# S5 -- block-sparse attention.  [WA §3.3 "Sparse branch"; appendix A.1.3]
# Given the selection this has a plain definition: softmax attention over
# exactly the tokens of the selected key blocks (computed two-pass here).
# --------------------------------------------------------------------------


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Plain softmax attention: q [n][d], k/v [m][d] -> [n][d] (float64)."""
    d = q.shape[-1]
    s = q.astype(np.float64) @ k.astype(np.float64).T / math.sqrt(d)
    mx = s.max(axis=1, keepdims=True)
    p = np.exp(s - mx)
    return (p @ v.astype(np.float64)) / p.sum(axis=1, keepdims=True)


def sparse_row(q_i: np.ndarray, k_h: np.ndarray, v_h: np.ndarray, blocks: Sequence[int], b: int) -> np.ndarray:
    idx = np.concatenate([np.arange(j * b, (j + 1) * b) for j in blocks])
    return attention(q_i, k_h[idx], v_h[idx])


def sparse_attention(q, k_act, v_act, sel, b):
    """q [Lq][H][d]; sel[h][i] block ids -> O_sp [Lq][H][d]."""
    Lq, H, d = q.shape
    out = np.empty((Lq, H, d))
    for h in range(H):
        for i in range(Lq // b):
            out[i * b:(i + 1) * b, h, :] = sparse_row(q[i * b:(i + 1) * b, h, :], k_act[h], v_act[h], sel[h][i], b)
    return out


# --------------------------------------------------------------------------
# Intra-chunk keys.  [WA §3.3 "Inter- and intra-chunk sparse granularity"]:
# the current chunk's own tokens take part in the block-sparse attention
# beside the retrieved history, through the same interface, with a finer
# partition than the history (the page: 128-token (4,8,4) cubes for the
# history, 64-token (4,4,4) cubes inside the chunk, i.e. half a history cube).
# Readings: the chunk's keys follow the history keys in the active sequence;
# the history keeps its B-token tiles as selection candidates and the chunk
# is cut into b_intra-token blocks (b_intra divides B); every candidate is
# pooled by the mean over its own tokens and one softmax runs over all of
# them; the linear branch projects the whole active sequence.
# --------------------------------------------------------------------------


def key_parts(l_hist: int, b_hist: int, l_chunk: int, b_intra: int) -> List[Tuple[int, int]]:
    """(first token, length) of every selection candidate: the history's
    b_hist-token tiles, then the chunk's b_intra-token blocks."""
    return ([(j * b_hist, b_hist) for j in range(l_hist // b_hist)] +
            [(l_hist + i * b_intra, b_intra) for i in range(l_chunk // b_intra)])


def part_means(t: np.ndarray, parts: Sequence[Tuple[int, int]]) -> np.ndarray:
    """[H][N][d] -> [H][len(parts)][d]: the mean key of every candidate."""
    t = np.asarray(t, dtype=np.float64)
    return np.stack([t[:, a:a + n, :].mean(axis=1) for a, n in parts], axis=1)


def block_selection_parts(q: np.ndarray, k_act: np.ndarray, tau: Sequence[float], b: int,
                          parts: Sequence[Tuple[int, int]]):
    """As block_selection, over the given candidates (query blocks stay b tokens)."""
    qb = block_means(np.asarray(q).transpose(1, 0, 2), b)     # [H][nQB][d]
    kb = part_means(k_act, parts)                              # [H][nC][d]
    H, nqb, _ = qb.shape
    mass = np.empty((H, nqb, kb.shape[1]))
    sel: List[List[np.ndarray]] = []
    flags = np.zeros((H, nqb), dtype=bool)
    for h in range(H):
        row = []
        for i in range(nqb):
            mass[h, i] = pooled_mass(qb[h, i], kb[h])
            s_, f = select_blocks(mass[h, i], tau[h])
            row.append(s_)
            flags[h, i] = f
        sel.append(row)
    counts = np.array([[len(x) for x in r] for r in sel], dtype=np.int64)
    return dict(qbar=qb, kbar=kb, mass=mass, sel=sel, counts=counts, flags=flags)


def sparse_row_parts(q_i, k_h, v_h, cands: Sequence[int], parts) -> np.ndarray:
    """One query block over exactly the tokens of its selected candidates."""
    idx = np.concatenate([np.arange(parts[j][0], parts[j][0] + parts[j][1]) for j in cands])
    return attention(q_i, k_h[idx], v_h[idx])


def sparse_attention_parts(q, k_act, v_act, sel, b, parts):
    """q [Lq][H][d]; sel[h][i] candidate ids -> O_sp [Lq][H][d]."""
    Lq, H, d = q.shape
    out = np.empty((Lq, H, d))
    for h in range(H):
        for i in range(Lq // b):
            out[i * b:(i + 1) * b, h, :] = sparse_row_parts(q[i * b:(i + 1) * b, h, :], k_act[h], v_act[h],
                                                            sel[h][i], parts)
    return out


# --------------------------------------------------------------------------
# S6 -- gated fusion.  [WA §3.3 "Gated fusion of two branches"; SUM step (6)]
# --------------------------------------------------------------------------


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def gates(x: np.ndarray, w_g: np.ndarray, n_heads: int) -> Tuple[np.ndarray, np.ndarray]:
    """x [Lq][D], w_g [2H][D] -> (g_lin, g_sp), each [Lq][H]."""
    g = x.astype(np.float64) @ w_g.astype(np.float64).T
    s = sigmoid(g)
    return s[:, :n_heads], s[:, n_heads:]


def fuse_with(g_lin, g_sp, o_lin, o_sp):
    return o_lin * g_lin[:, :, None] + o_sp * g_sp[:, :, None]


def fuse(x, w_g, o_lin, o_sp):
    gl, gs = gates(x, w_g, o_lin.shape[1])
    return fuse_with(gl, gs, o_lin, o_sp)


# --------------------------------------------------------------------------
# Whole step (one layer, one denoising step)
# --------------------------------------------------------------------------


def hsa_step(q, pages_k, pages_v, e_k, e_v, w_g, x, tau, n_sel_pages, block,
             sel_pages=None, block_sel=None, k_cur=None, v_cur=None, b_intra=None) -> Dict[str, object]:
    """Run S1..S6.  `sel_pages` / `block_sel` override the selections (used to
    re-run the downstream stages with another valid selection at a tie).
    With `k_cur`, `v_cur` ([Lq][H][d]) and `b_intra`, the chunk's own keys
    join the history (intra-chunk keys); `block_sel` then lists candidates
    of `key_parts`."""
    q = np.asarray(q, dtype=np.float64)
    sc = score_and_select(q, pages_k, n_sel_pages)
    sp = np.asarray(sc["sel"] if sel_pages is None else sel_pages)
    k_act = gather_active([np.asarray(p, np.float64) for p in pages_k], sp)
    v_act = gather_active([np.asarray(p, np.float64) for p in pages_v], sp)
    parts = None
    if k_cur is not None:
        l_hist = k_act.shape[1]
        k_act = np.concatenate([k_act, np.asarray(k_cur, np.float64).transpose(1, 0, 2)], axis=1)
        v_act = np.concatenate([v_act, np.asarray(v_cur, np.float64).transpose(1, 0, 2)], axis=1)
        parts = key_parts(l_hist, block, q.shape[0], b_intra)
    lin = linear_branch(q, k_act, v_act, e_k, e_v)
    if parts is None:
        bs = block_selection(q, k_act, tau, block)
        bsel = bs["sel"] if block_sel is None else block_sel
        o_sp = sparse_attention(q, k_act, v_act, bsel, block)
    else:
        bs = block_selection_parts(q, k_act, tau, block, parts)
        bsel = bs["sel"] if block_sel is None else block_sel
        o_sp = sparse_attention_parts(q, k_act, v_act, bsel, block, parts)
    out = fuse(x, w_g, lin["o_lin"], o_sp)
    return dict(score=sc, sel_pages=sp, k_act=k_act, v_act=v_act, lin=lin,
                blocks=bs, block_sel=bsel, o_sp=o_sp, out=out, parts=parts)
