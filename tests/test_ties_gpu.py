"""Exact ties and NaN inputs on the GPU, against the float64 oracle.

Near-ties (a gap below the oracle's tie threshold) may be broken either way,
and the parity tests accept any valid answer there.  An exact tie has one
answer: both sides compute bitwise-equal values for equal inputs, and the
lower id wins (WorldAttention paper, section 3.2, top-K_p page retrieval;
section 3.3, block selection by cumulative mass; the order of equal values
is a reading: ascending id).  These tests build exact ties on purpose and
require the oracle's pick element for element:

  * two pages with identical keys and values at the K_p boundary;
  * a head whose keys are one constant vector, so every block has the same
    pooled mass and each row keeps the lowest-id blocks;
  * a page whose keys hold a NaN: its score is reported as -inf and it is
    never preferred to a page with a number for a score;
  * prompt embeddings with a NaN (similarity -inf) or all zeros (similarity 0
    with every chunk, so the lowest chunk id wins).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import hsa_oracle as orc
from synth import M1, chunk_prompts

from gpu_harness import Run, assert_close, check_block_selection, dev, gpu_block_lists, host

pytestmark = pytest.mark.gpu


def _set_page(r: Run, j: int, k: np.ndarray, v: np.ndarray):
    r.pk_np[j], r.pv_np[j] = k, v
    r.pk[j], r.pv[j] = dev(k, r.cfg), dev(v, r.cfg)


def _order(r: Run):
    sc = orc.score_and_select(r.np["q"], r.pk_np, r.cfg.n_sel_pages)
    order, _ = orc.top_k_lower_index(sc["alpha"], len(sc["alpha"]))
    return sc, order


def _step_matches_oracle(r: Run, exact_pages: bool):
    """Whole step against the oracle on the GPU's page and block selection
    (each first checked against the oracle's)."""
    st, cfg = r.step, r.cfg
    ref = r.oracle()
    gsel = host(st.sel_pages).astype(np.int64)
    if exact_pages:
        assert gsel.tolist() == ref["score"]["sel"].tolist()
    else:
        assert orc.valid_page_selection(ref["score"]["alpha"], gsel, cfg.n_sel_pages)
    lists, _, _ = gpu_block_lists(st)
    ref = r.oracle(sel_pages=gsel)
    check_block_selection(ref["blocks"], lists, r.np["tau"])
    ref = r.oracle(sel_pages=gsel, block_sel=lists)
    assert_close("o_sp", host(st.o_sp), ref["o_sp"], cfg)
    assert_close("o_lin", host(st.o_lin), ref["lin"]["o_lin"], cfg)
    assert_close("out", host(st.out), ref["out"], cfg)


@pytest.mark.parametrize("which", ["kth_into_next", "next_into_kth"])
def test_identical_pages_tie_to_the_lower_id(which):
    cfg = M1
    r = Run(cfg)
    _, order = _order(r)
    a, b = int(order[cfg.n_sel_pages - 1]), int(order[cfg.n_sel_pages])
    src, dst = (a, b) if which == "kth_into_next" else (b, a)
    print(f"\n[ties] {cfg.name}: page {src} copied into page {dst} at the K_p boundary", flush=True)
    _set_page(r, dst, r.pk_np[src].copy(), r.pv_np[src].copy())
    sc, _ = _order(r)
    assert sc["alpha"][a] == sc["alpha"][b] and sc["tie"]
    assert min(a, b) in sc["sel"] and max(a, b) not in sc["sel"]
    st = r.run()
    s = host(st.scores)
    assert s[a] == s[b], "identical pages must score identically"
    _step_matches_oracle(r, exact_pages=True)
    # the same from the page index
    st.index_pages(r.q, r.pk)
    r.run(indexed=True)
    assert host(st.sel_pages).astype(np.int64).tolist() == sc["sel"].tolist()


def test_constant_key_head_keeps_the_lowest_blocks():
    cfg = M1
    r = Run(cfg)
    c = r.pk_np[0][0, 0, :].copy()  # a bf16-representable vector
    for j in range(cfg.n_pages):
        k = r.pk_np[j].copy()
        k[:, 0, :] = c
        _set_page(r, j, k, r.pv_np[j])
    tau0 = float(r.np["tau"][0])
    n_keep = int(np.ceil(tau0 * cfg.n_kblocks - 1e-9))
    print(f"\n[ties] {cfg.name}: head 0 keys constant, tau {tau0}, {cfg.n_kblocks} blocks -> "
          f"blocks 0..{n_keep - 1} in every row", flush=True)
    st = r.run()
    gsel = host(st.sel_pages).astype(np.int64)
    ref = r.oracle(sel_pages=gsel)
    m = ref["blocks"]["mass"][0]
    assert np.all(m == m[0, 0]), "uniform pooled mass under constant keys"
    lists, _, _ = gpu_block_lists(st)
    for i in range(cfg.n_qblocks):
        assert ref["blocks"]["sel"][0][i].tolist() == list(range(n_keep))
        assert lists[0][i].tolist() == list(range(n_keep)), f"head 0 row {i}: {lists[0][i].tolist()}"
    _step_matches_oracle(r, exact_pages=False)


def test_nan_page_is_never_selected():
    cfg = M1
    r = Run(cfg)
    _, order = _order(r)
    best = int(order[0])
    k = r.pk_np[best].copy()
    k[5, 1, 3] = np.nan
    _set_page(r, best, k, r.pv_np[best])
    print(f"\n[ties] {cfg.name}: a NaN in the keys of page {best}, the best-scoring page", flush=True)
    sc, _ = _order(r)
    assert np.isnan(sc["alpha"][best]) and best not in sc["sel"]
    st = r.run()
    s = host(st.scores)
    assert np.isneginf(s[best])
    fin = np.isfinite(sc["alpha"])
    np.testing.assert_allclose(s[fin], sc["alpha"][fin], rtol=0, atol=2e-5)
    _step_matches_oracle(r, exact_pages=not sc["tie"])
    assert np.all(np.isfinite(host(st.out)))
    # from the page index: the NaN mean scores -inf as well
    st.index_pages(r.q, r.pk)
    r.run(indexed=True)
    assert np.isneginf(host(st.scores)[best])
    assert best not in host(st.sel_pages).tolist()


def test_more_nan_pages_than_spare_ones():
    """K_p = 3 of 6 pages with four NaN pages: the two finite pages, then the
    lowest-id NaN page (scoring and top-K_p only)."""
    cfg = M1
    r = Run(cfg)
    nan_pages = [0, 2, 3, 5]
    for j in nan_pages:
        k = r.pk_np[j].copy()
        k[j, 2, 7] = np.nan
        _set_page(r, j, k, r.pv_np[j])
    sc, _ = _order(r)
    assert sc["sel"].tolist() == [0, 1, 4]
    st = r.step
    from sparse_linear_attention_hsa_amd import ops
    ops.hsa_score_pages(st.geom, r.q, r.pk, st.page_kmean, st.scores, st.sel_pages, st.ws)
    torch.cuda.synchronize()
    s = host(st.scores)
    assert np.all(np.isneginf(s[nan_pages]))
    assert host(st.sel_pages).astype(np.int64).tolist() == [0, 1, 4]


def test_nan_and_zero_prompt_embeddings():
    cfg = M1
    r = Run(cfg)
    st = r.step
    page_chunk, cur, prev, target = chunk_prompts(cfg, 2)
    prev = prev.copy()
    prev[target, 5] = np.nan
    zero = (target + 1) % len(prev)
    prev[zero] = 0.0
    print(f"\n[ties] {cfg.name}: NaN in the embedding of chunk {target}, zero embedding for chunk {zero}",
          flush=True)
    chunk_t = torch.from_numpy(prev).cuda()
    page_chunk_t = torch.from_numpy(page_chunk).cuda()
    # a noisy prompt: the NaN chunk ranks last, the zero chunk has similarity 0
    ref = orc.prompt_retrieval(cur, prev, 1)
    st.retrieve(r.q, r.pk, (torch.from_numpy(cur).cuda(), chunk_t, page_chunk_t, 1))
    torch.cuda.synchronize()
    sims = host(st.chunk_sims)
    assert np.isnan(ref["sims"][target]) and np.isneginf(sims[target])
    assert ref["sims"][zero] == 0.0 and sims[zero] == 0.0
    rest = [i for i in range(len(prev)) if i not in (target, zero)]
    np.testing.assert_allclose(sims[rest], ref["sims"][rest], rtol=0, atol=1e-5)
    assert target not in ref["sel"]
    assert host(st.sel_chunks).astype(np.int64).tolist() == ref["sel"].tolist()
    # a zero prompt: similarity 0 with every chunk (the NaN one too), so chunk 0 wins
    zp = np.zeros_like(cur)
    ref = orc.prompt_retrieval(zp, prev, 1)
    assert np.all(ref["sims"] == 0.0) and ref["sel"].tolist() == [0]
    st.retrieve(r.q, r.pk, (torch.from_numpy(zp).cuda(), chunk_t, page_chunk_t, 1))
    torch.cuda.synchronize()
    assert np.all(host(st.chunk_sims) == 0.0)
    assert host(st.sel_chunks).astype(np.int64).tolist() == [0]
