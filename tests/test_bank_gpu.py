"""Page banks beyond the 128 pages of a host page table: scoring and gather
through page tables in device memory (WorldAttention paper, section 3.2: the
whole history stays retrievable, scored from a page index built from the
keys), against the float64 oracle.

  * device tables give the host-table results bit for bit (C0, M1, M2, an
    intra-chunk geometry, and prompt-level retrieval);
  * a 300-page bank: the page index, scoring from it and from the pages,
    the gather and the whole step, and chunk-restricted scoring;
  * the largest bank (8,192 pages) scored from a page index alone, with
    exact three-way ties at the K_p boundary, NaN means and pages with
    neither keys nor a cached mean, with and without a chunk filter.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import hsa_oracle as orc
from sparse_linear_attention_hsa_amd import ops
from sparse_linear_attention_hsa_amd._lib import HSA_MAX_BANK_PAGES
from sparse_linear_attention_hsa_amd.ops import DeviceTable
from synth import C0, M1, M2, M3, chunk_prompts, with_

from gpu_harness import Run, assert_close, check_block_selection, geom_of, gpu_block_lists, host

pytestmark = pytest.mark.gpu


def _tables(r: Run):
    return DeviceTable(r.pk), DeviceTable(r.pv)


@pytest.mark.parametrize("cfg", [C0, M1, M2, with_(M1, name="m1_intra2", intra_split=2)], ids=lambda c: c.name)
def test_device_tables_equal_host_tables(cfg):
    print(f"\n[bank] {cfg.name}: device vs host page tables", flush=True)
    r = Run(cfg)
    st = r.step
    names = ("scores", "sel_pages", "page_kmean", "k_act", "v_act", "kblk_mean", "out")
    r.run(concurrent=False)
    a = {k: getattr(st, k).clone() for k in names}
    kt, vt = _tables(r)
    st.run(r.q, kt, vt, r.e_k, r.e_v, r.w_g, r.x, r.tau, concurrent=False, k_cur=r.k_cur, v_cur=r.v_cur)
    torch.cuda.synchronize()
    for k in names:
        assert torch.equal(a[k], getattr(st, k)), k
    # prompt-level retrieval over the same pages
    page_chunk, cur, prev, _ = chunk_prompts(cfg, 2)
    chunks = (torch.from_numpy(cur).cuda(), torch.from_numpy(prev).cuda(), torch.from_numpy(page_chunk).cuda(), 1)
    st.retrieve(r.q, r.pk, chunks)
    torch.cuda.synchronize()
    want = (st.scores.clone(), st.sel_pages.clone())
    st.retrieve(r.q, kt, chunks)
    torch.cuda.synchronize()
    assert torch.equal(want[0], st.scores) and torch.equal(want[1], st.sel_pages)


def test_bank_of_300_pages():
    cfg = with_(M1, name="m1_bank300", n_pages=300, seed=2301)
    print(f"\n[bank] {cfg.name}: {cfg.n_pages} pages, K_p={cfg.n_sel_pages}", flush=True)
    r = Run(cfg)
    st = r.step
    kt, vt = _tables(r)
    # the page index from the pages, then scoring from it alone (NULL table)
    st.index_pages(r.q, kt)
    torch.cuda.synchronize()
    scan = (st.scores.clone(), st.sel_pages.clone())
    sc = orc.score_and_select(r.np["q"], r.pk_np, cfg.n_sel_pages)
    np.testing.assert_allclose(host(st.page_kmean), sc["kbars"], rtol=0, atol=2e-5)
    np.testing.assert_allclose(host(st.scores), sc["alpha"], rtol=0, atol=2e-5)
    st.score(r.q, None, use_cache=True)
    torch.cuda.synchronize()
    assert torch.equal(scan[0], st.scores) and torch.equal(scan[1], st.sel_pages)
    gsel = host(st.sel_pages).astype(np.int64)
    if not np.array_equal(gsel, sc["sel"]):
        assert sc["tie"] and orc.valid_page_selection(sc["alpha"], gsel, cfg.n_sel_pages)
    assert set(sc["sel"].tolist()) == set(r.w.plant.target_pages.tolist())
    # the whole step over device tables (scoring from the index)
    st.run(r.q, kt, vt, r.e_k, r.e_v, r.w_g, r.x, r.tau, indexed=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(st.k_act), orc.gather_active(r.pk_np, gsel))
    lists, _, _ = gpu_block_lists(st)
    ref = r.oracle(sel_pages=gsel)
    check_block_selection(ref["blocks"], lists, r.np["tau"])
    ref = r.oracle(sel_pages=gsel, block_sel=lists)
    assert_close("o_sp", host(st.o_sp), ref["o_sp"], cfg)
    assert_close("o_lin", host(st.o_lin), ref["lin"]["o_lin"], cfg)
    assert_close("out", host(st.out), ref["out"], cfg)
    # chunk-restricted scoring: 30 chunks of 10 pages, top-3 chunks, one page each
    page_chunk, cur, prev, _ = chunk_prompts(cfg, 10)
    chunks = (torch.from_numpy(cur).cuda(), torch.from_numpy(prev).cuda(), torch.from_numpy(page_chunk).cuda(), 3)
    st.retrieve(r.q, st.no_pages(), chunks)
    torch.cuda.synchronize()
    ref = orc.prompt_retrieval(cur, prev, 3)
    gch = host(st.sel_chunks).astype(np.int64)
    if not np.array_equal(gch, ref["sel"]):
        assert ref["tie"] and orc.valid_page_selection(ref["sims"], gch, 3)
    scc = orc.score_chunk_pages(r.np["q"], r.pk_np, page_chunk, gch, cfg.n_sel_pages)
    s = host(st.scores)
    cand = np.isfinite(scc["alpha"])
    np.testing.assert_allclose(s[cand], scc["alpha"][cand], rtol=0, atol=2e-5)
    assert np.all(np.isneginf(s[~cand]))
    psel = host(st.sel_pages).astype(np.int64)
    assert psel.tolist() == scc["sel"].tolist() or scc["tie"]


def _ties_and_nans(kbar, qbar, k_p, page_chunk=None):
    """Plant an exact three-way tie where it decides the selection, and a NaN
    mean on the best page.  Without chunks: two far-away copies of the page
    ranked K_p-th after the NaN page drops out.  With chunks: two copies, in
    the same chunk, of the best page of the second-best page's chunk (three
    pages for that chunk's two-page share).  Returns (tied pages, NaN page)."""
    n = kbar.shape[0]
    alpha = orc.page_scores(qbar, kbar.astype(np.float64))
    order, _ = orc.top_k_lower_index(alpha, n)
    nan_page = int(order[0])
    if page_chunk is None:
        a = int(order[k_p])  # K_p-th best once order[0] is NaN
        twins = [j for j in (a - 1000, a + 1000, a + 2000) if 0 <= j < n][:2]
    else:
        c0 = int(page_chunk[order[1]])
        ids = [j for j in np.flatnonzero(page_chunk == c0).tolist() if j != nan_page]
        a = max(ids, key=lambda j: (alpha[j], -j))
        twins = [j for j in ids if j != a][:2]
    for j in twins:
        kbar[j] = kbar[a]
    kbar[nan_page, 0, 5] = np.nan
    return sorted([a] + twins), nan_page


@pytest.mark.parametrize("chunked", [False, True], ids=["plain", "chunks"])
def test_largest_bank_from_the_page_index(chunked):
    cfg = M3  # K_p = 8
    n_pages = HSA_MAX_BANK_PAGES
    rng = np.random.default_rng(8192)
    r = Run(with_(cfg, n_pages=cfg.n_sel_pages))  # only its queries and geometry are used
    kbar = rng.standard_normal((n_pages, cfg.n_heads, cfg.head_dim)).astype(np.float32)
    qbar = orc.mean_over_tokens(r.np["q"])
    page_chunk = (np.arange(n_pages) // 64).astype(np.int32) if chunked else None
    tied, nan_page = _ties_and_nans(kbar, qbar, cfg.n_sel_pages, page_chunk)
    print(f"\n[bank] {n_pages} pages from the page index (K_p={cfg.n_sel_pages}, chunked={chunked}); exact tie of "
          f"pages {tied}, NaN mean at page {nan_page}", flush=True)
    geom = geom_of(cfg)
    ws = torch.empty(ops.hsa_workspace_bytes(geom, n_pages), dtype=torch.uint8, device="cuda")
    page_kmean = torch.from_numpy(kbar).cuda()
    scores = torch.empty(n_pages, dtype=torch.float32, device="cuda")
    sel = torch.empty(cfg.n_sel_pages, dtype=torch.int32, device="cuda")
    table = DeviceTable([None] * n_pages)
    alpha = orc.page_scores(qbar, kbar.astype(np.float64))
    if not chunked:
        ops.hsa_score_pages(geom, r.q, table, page_kmean, scores, sel, ws)
        torch.cuda.synchronize()
        want, tie = orc.select_pages(alpha, cfg.n_sel_pages)
    else:
        chosen = []
        for c in (int(page_chunk[tied[0]]), int(page_chunk[nan_page]), 3, 77, 101, 5):
            if c not in chosen and len(chosen) < 4:
                chosen.append(c)
        chosen = np.array(sorted(chosen), dtype=np.int32)
        ops.hsa_score_chunk_pages(geom, r.q, table, page_kmean, torch.from_numpy(page_chunk).cuda(),
                                  torch.from_numpy(chosen).cuda(), scores, sel, ws)
        torch.cuda.synchronize()
        alpha = np.where(np.isin(page_chunk, chosen), alpha, -np.inf)
        want, tie = orc.select_pages_in_chunks(alpha, page_chunk, chosen, cfg.n_sel_pages)
    s = host(scores)
    fin = np.isfinite(alpha)
    np.testing.assert_allclose(s[fin], alpha[fin], rtol=0, atol=2e-5)
    assert np.all(np.isneginf(s[~fin]))
    assert np.isneginf(s[nan_page]) and s[tied[0]] == s[tied[1]] == s[tied[2]]
    assert tie, "the planted exact tie decides the selection"
    got = host(sel).astype(np.int64)
    assert got.tolist() == np.asarray(want).tolist(), (got, want)
    # one slot for the three (plain), or a two-page share (chunks): the lowest ids
    n_in = 2 if chunked else 1
    assert [j for j in tied if j in got.tolist()] == tied[:n_in]
    # with neither keys nor a cached mean every page scores -inf: the lowest ids
    ops.hsa_score_pages(geom, r.q, table, None, scores, sel, ws)
    torch.cuda.synchronize()
    assert np.all(np.isneginf(host(scores)))
    assert host(sel).tolist() == list(range(cfg.n_sel_pages))
