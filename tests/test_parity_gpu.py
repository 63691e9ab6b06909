"""Parity of the HIP path (through the C ABI) with the float64 CPU oracle,
stage by stage, on seeded workloads that span several tiles, ragged tails,
split rows and near-ties."""
import numpy as np
import pytest
import torch

from oracle import hsa_oracle as orc
from synth import C0, M1, M2, M3, M4, M5, chunk_prompts, with_

from gpu_harness import (TOL, Run, assert_close, check_block_selection, gpu_block_lists, host, untile_v)

pytestmark = pytest.mark.gpu

SMALL = [C0, M1, M2, M3, M4, M5]


@pytest.fixture(scope="module", params=SMALL, ids=lambda c: c.name)
def ran(request):
    cfg = request.param
    print(f"\n[parity] config={cfg.name}", flush=True)
    r = Run(cfg)
    r.run()
    return r


def test_page_scores_and_selection(ran):
    st, cfg = ran.step, ran.cfg
    ref = ran.oracle()["score"]
    np.testing.assert_allclose(host(st.scores), ref["alpha"], rtol=0, atol=2e-5)
    np.testing.assert_allclose(host(st.page_kmean), ref["kbars"], rtol=0, atol=2e-5)
    sel = st.sel_pages.cpu().numpy()
    if ref["tie"]:
        assert orc.valid_page_selection(ref["alpha"], sel, cfg.n_sel_pages)
    else:
        assert sel.tolist() == ref["sel"].tolist()


def test_gather_is_bit_exact(ran):
    st, cfg = ran.step, ran.cfg
    sel = st.sel_pages.cpu().numpy()
    want_k = orc.gather_active(ran.pk_np, sel)
    want_v = orc.gather_active(ran.pv_np, sel)
    assert np.array_equal(host(st.k_act), want_k)
    assert np.array_equal(untile_v(host(st.v_act)), want_v)
    np.testing.assert_allclose(host(st.kblk_mean), orc.block_means(want_k, cfg.block), rtol=0, atol=2e-5)


def test_linear_branch(ran):
    st, cfg = ran.step, ran.cfg
    ref = ran.oracle(sel_pages=st.sel_pages.cpu().numpy())
    lin = ref["lin"]
    # projections are float32 sums of products of the inputs (exact in float32 for bf16 inputs)
    proj_tol = (2e-4, 1e-5)
    assert_close("k_proj", host(st.k_proj), lin["ktil"], cfg, proj_tol)
    assert_close("v_proj", host(st.v_proj).transpose(0, 2, 1), lin["vtil"], cfg, proj_tol)
    assert_close("o_lin", host(st.o_lin), lin["o_lin"], cfg)


def test_block_selection(ran):
    st, cfg = ran.step, ran.cfg
    ref = ran.oracle(sel_pages=st.sel_pages.cpu().numpy())
    lists, cnt, idx = gpu_block_lists(st)
    check_block_selection(ref["blocks"], lists, ran.np["tau"])
    # padding after the count
    for h in range(cfg.n_heads):
        for i in range(cfg.n_qblocks):
            assert np.all(idx[h, i, cnt[h, i]:] == -1)
    np.testing.assert_allclose(host(st.blk_mass), ref["blocks"]["mass"], rtol=0, atol=1e-5)


def test_sparse_branch_and_fuse(ran):
    st, cfg = ran.step, ran.cfg
    lists, _, _ = gpu_block_lists(st)
    ref = ran.oracle(sel_pages=st.sel_pages.cpu().numpy(), block_sel=lists)
    assert_close("o_sp", host(st.o_sp), ref["o_sp"], cfg)
    assert_close("out", host(st.out), ref["out"], cfg)


def test_bitwise_reproducible(ran):
    st = ran.step
    a = [t.clone() for t in (st.out, st.o_sp, st.o_lin, st.blk_idx, st.scores)]
    ran.run()
    for x, y in zip(a, (st.out, st.o_sp, st.o_lin, st.blk_idx, st.scores)):
        assert torch.equal(x, y)


def test_side_stream_schedule_matches_in_order(ran):
    """The step's default schedule (linear branch on a side stream beside block
    selection and the sparse branch) equals the six calls in order on one
    stream, bit for bit."""
    st = ran.step
    names = ("out", "o_sp", "o_lin", "k_proj", "v_proj", "blk_count", "blk_idx", "sel_pages")
    ran.run(concurrent=True)
    a = {k: getattr(st, k).clone() for k in names}
    ran.run(concurrent=False)
    for k in names:
        assert torch.equal(a[k], getattr(st, k)), k


def test_page_index_scoring_matches_page_scan(ran):
    """Scoring every page from the page index (mean keys kept from an earlier
    pass over the pages) gives the scores, the selection and the step's
    outputs of scoring from the pages themselves, bit for bit."""
    st = ran.step
    names = ("scores", "sel_pages", "out", "o_sp", "o_lin", "blk_count", "blk_idx")
    ran.run()
    a = {k: getattr(st, k).clone() for k in names}
    st.page_kmean.fill_(float("nan"))  # nothing left over from the run above
    st.index_pages(ran.q, ran.pk)
    ran.run(indexed=True)
    for k in names:
        assert torch.equal(a[k], getattr(st, k)), k


def _chunk_cases(cfg):
    """(pages per chunk, k) pairs: chunks of 2 pages (short chunks for K_p > 2)
    and of K_p pages, every k that divides K_p and fits the chunk count."""
    out = []
    for ppc in sorted({2, cfg.n_sel_pages}):
        n_chunks = -(-cfg.n_pages // ppc)
        out += [(ppc, k) for k in range(1, cfg.n_sel_pages + 1) if cfg.n_sel_pages % k == 0 and k <= n_chunks]
    return out


def _valid_chunk_pages(alpha, page_chunk, chunks, k_p, sel):
    """A selection that differs from the oracle's only inside near-ties: in
    every chosen chunk, no unchosen page scores above a chosen one."""
    sel = set(int(j) for j in sel)
    if len(sel) != k_p:
        return False
    for ch in chunks:
        ids = [j for j in range(len(alpha)) if page_chunk[j] == ch]
        chosen = [alpha[j] for j in ids if j in sel]
        rest = [alpha[j] for j in ids if j not in sel]
        if chosen and rest and min(chosen) < max(rest) - orc.TIE_EPS:
            return False
    return True


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_prompt_retrieval_and_chunk_pages(cfg):
    """Stage 1 (cosine top-k chunks) and page scoring inside the chosen chunks
    against the oracle, for every chunk size and k of _chunk_cases; then the
    whole step on the retrieved pages."""
    r = Run(cfg)
    st = r.step
    q_np = r.np["q"]
    for ppc, k in _chunk_cases(cfg):
        page_chunk, cur, prev, _ = chunk_prompts(cfg, ppc)
        print(f"  pages per chunk {ppc}, k {k}", flush=True)
        chunks = (torch.from_numpy(cur).cuda(), torch.from_numpy(prev).cuda(),
                  torch.from_numpy(page_chunk).cuda(), k)
        st.retrieve(r.q, r.pk, chunks)
        torch.cuda.synchronize()
        ref = orc.prompt_retrieval(cur, prev, k)
        np.testing.assert_allclose(host(st.chunk_sims), ref["sims"], rtol=0, atol=1e-5)
        gsel = host(st.sel_chunks).astype(np.int64)
        if not np.array_equal(gsel, ref["sel"]):
            assert ref["tie"] and orc.valid_page_selection(ref["sims"], gsel, k)
        sc = orc.score_chunk_pages(q_np, r.pk_np, page_chunk, gsel, cfg.n_sel_pages)
        scores = host(st.scores)
        cand = np.isfinite(sc["alpha"])
        np.testing.assert_allclose(scores[cand], sc["alpha"][cand], rtol=0, atol=2e-5)
        assert np.all(np.isneginf(scores[~cand]))
        psel = host(st.sel_pages).astype(np.int64)
        if not np.array_equal(psel, sc["sel"]):
            assert sc["tie"] and _valid_chunk_pages(sc["alpha"], page_chunk, gsel, cfg.n_sel_pages, psel)
        # the same from the page index, every page pointer NULL: bit for bit
        st.index_pages(r.q, r.pk)
        st.retrieve(r.q, [None] * cfg.n_pages, chunks)
        torch.cuda.synchronize()
        assert np.array_equal(host(st.scores), scores) and np.array_equal(host(st.sel_pages), psel)
    # the whole step with retrieval (last case), against the oracle on its pages
    r.step.run(r.q, r.pk, r.pv, r.e_k, r.e_v, r.w_g, r.x, r.tau, chunks=chunks)
    torch.cuda.synchronize()
    lists, _, _ = gpu_block_lists(st)
    ref = r.oracle(sel_pages=st.sel_pages.cpu().numpy(), block_sel=lists)
    assert_close("out", host(st.out), ref["out"], cfg)


# --------------------------------------------------------------- special cases
@pytest.mark.parametrize("cfg", [C0, M1], ids=lambda c: c.name)
def test_tau_one_gives_dense_attention(cfg):
    """tau_h = 1 keeps every block, and the sparse branch is then plain softmax attention."""
    r = Run(cfg, tau=np.ones(cfg.n_heads))
    st = r.run()
    assert np.all(st.blk_count.cpu().numpy() == cfg.n_kblocks)
    q = r.np["q"].astype(np.float64)
    k = host(st.k_act)
    v = untile_v(host(st.v_act))
    o = host(st.o_sp)
    for h in range(cfg.n_heads):
        assert_close("dense", o[:, h, :], orc.attention(q[:, h, :], k[h], v[h]), cfg)


@pytest.mark.parametrize("cfg", [C0, M2], ids=lambda c: c.name)
def test_gate_override_selects_one_branch(cfg):
    r = Run(cfg)
    st = r.run()
    Lq, H = cfg.query_tokens, cfg.n_heads
    from sparse_linear_attention_hsa_amd import ops
    for gl, gs in ((1.0, 0.0), (0.0, 1.0)):
        gates = torch.empty(Lq, 2 * H, dtype=torch.float32, device="cuda")
        gates[:, :H] = gl
        gates[:, H:] = gs
        ops.hsa_fuse(st.geom, None, None, gates, st.o_lin, st.o_sp, st.out)
        torch.cuda.synchronize()
        want = host(st.o_lin) if gl == 1.0 else host(st.o_sp)
        # exact up to the final rounding to the element type
        tol = (8e-3, 4e-3) if cfg.dtype == "bf16" else (1e-7, 1e-7)
        assert_close("gate", host(st.out), want, cfg, tol)


def test_single_block_rows():
    """tau tiny: every row keeps exactly its argmax block."""
    cfg = M1
    r = Run(cfg, tau=np.full(cfg.n_heads, 1e-6))
    st = r.run()
    assert np.all(st.blk_count.cpu().numpy() == 1)
    lists, _, _ = gpu_block_lists(st)
    ref = r.oracle(sel_pages=st.sel_pages.cpu().numpy())
    check_block_selection(ref["blocks"], lists, r.np["tau"])
    ref2 = r.oracle(sel_pages=st.sel_pages.cpu().numpy(), block_sel=lists)
    assert_close("o_sp", host(st.o_sp), ref2["o_sp"], cfg)


def test_all_pages_retrieved():
    """K_p = number of pages: every page is selected, in order."""
    cfg = with_(M2, n_pages=3, n_sel_pages=3)
    r = Run(cfg)
    st = r.run()
    assert st.sel_pages.cpu().numpy().tolist() == [0, 1, 2]
    ref = r.oracle(sel_pages=np.arange(3))
    assert_close("o_lin", host(st.o_lin), ref["lin"]["o_lin"], cfg)


def test_non_resident_page_scored_from_cached_mean():
    """A NULL page pointer is scored from the cached page mean."""
    cfg = M1
    r = Run(cfg)
    st = r.run()
    cached = st.page_kmean.clone()
    scores = st.scores.clone()
    sel = st.sel_pages.clone()
    pk = list(r.pk)
    pk[1] = None
    pk[4] = None
    from sparse_linear_attention_hsa_amd import ops
    st.scores.zero_()
    ops.hsa_score_pages(st.geom, r.q, pk, st.page_kmean, st.scores, st.sel_pages, st.ws)
    torch.cuda.synchronize()
    assert torch.equal(st.page_kmean, cached)
    assert torch.equal(st.scores, scores)
    assert torch.equal(st.sel_pages, sel)


def test_graph_replays_match_eager():
    """The step (side-stream schedule) captured into a HIP graph: every replay,
    with eager steps and synchronisations between replays, equals the eager
    step bit for bit (the library records no memset in a captured step)."""
    r = Run(M1)
    st = r.step
    names = ("out", "o_sp", "o_lin", "blk_count", "blk_idx", "sel_pages", "k_proj")
    r.run()
    ref = {k: getattr(st, k).clone() for k in names}
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run(r.q, r.pk, r.pv, r.e_k, r.e_v, r.w_g, r.x, r.tau)
    for rep in range(3):
        for k in names:
            getattr(st, k).zero_()
        g.replay()
        torch.cuda.synchronize()
        for k in names:
            assert torch.equal(getattr(st, k), ref[k]), f"replay {rep}: {k}"
        r.run()  # eager work between replays
        torch.cuda.synchronize()
