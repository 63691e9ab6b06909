"""Intra-chunk keys (WorldAttention paper, section 3.3, inter- and intra-chunk
sparse granularity): the chunk's own tokens follow the retrieved pages in the
active buffer, the history is selected in B-token tiles and the chunk in
finer B/s-token key blocks, under one pooled softmax.  Parity of the HIP path
(through the C ABI) with the float64 oracle, stage by stage."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import hsa_oracle as orc
from synth import M1, M2, M3, M4, M5

from gpu_harness import (Run, assert_close, candidates_of, gpu_block_lists, host, key_blocks_of, untile_v)

pytestmark = pytest.mark.gpu

INTRA = [replace(M1, name="m1_intra2", intra_split=2),            # 96-token tiles, 48-token chunk blocks
         replace(M2, name="m2_intra3_ragged", intra_split=3),     # d = 64, 48 -> 16
         replace(M3, name="m3_intra2_long_rows", intra_split=2),  # split rows
         replace(M4, name="m4_intra3_f32", intra_split=3),        # float32
         replace(M5, name="m5_intra2_imbalance", intra_split=2),
         replace(M1, name="m1_intra1", intra_split=1)]            # chunk blocks as large as the tiles


@pytest.fixture(scope="module", params=INTRA, ids=lambda c: c.name)
def ran(request):
    cfg = request.param
    print(f"\n[intra] config={cfg.name} Lh={cfg.history_tokens} Lq={cfg.query_tokens} B={cfg.block} "
          f"Bk={cfg.key_block} nKB={cfg.n_key_blocks} nC={cfg.n_candidates}", flush=True)
    r = Run(cfg)
    r.run()
    return r


def _grp(cfg):
    return cfg.block // cfg.key_block


def test_gather_appends_the_chunk(ran):
    st, cfg = ran.step, ran.cfg
    sel = st.sel_pages.cpu().numpy()
    want_k = np.concatenate([orc.gather_active(ran.pk_np, sel), ran.np["k_cur"].transpose(1, 0, 2)], axis=1)
    want_v = np.concatenate([orc.gather_active(ran.pv_np, sel), ran.np["v_cur"].transpose(1, 0, 2)], axis=1)
    assert np.array_equal(host(st.k_act), want_k)
    assert np.array_equal(untile_v(host(st.v_act)), want_v)
    np.testing.assert_allclose(host(st.kblk_mean), orc.block_means(want_k, cfg.key_block), rtol=0, atol=2e-5)


def _check_selection(ref_blocks, st, cfg, tau):
    lists, cnt, idx = gpu_block_lists(st)
    grp, nt = _grp(cfg), cfg.n_kblocks
    differ = 0
    for h in range(cfg.n_heads):
        for i in range(cfg.n_qblocks):
            assert np.all(idx[h, i, cnt[h, i]:] == -1)
            got = candidates_of(lists[h][i], nt, grp)
            assert got is not None, f"a history tile listed incompletely (h={h}, i={i})"
            want = ref_blocks["sel"][h][i]
            if np.array_equal(got, want):
                assert np.array_equal(lists[h][i], key_blocks_of(want, nt, grp))
                continue
            assert ref_blocks["flags"][h, i], f"selection differs at unflagged row (h={h}, i={i})"
            assert orc.valid_block_selection(ref_blocks["mass"][h, i], got, tau[h])
            differ += 1
    return lists, differ


def test_block_selection_over_both_granularities(ran):
    st, cfg = ran.step, ran.cfg
    ref = ran.oracle(sel_pages=st.sel_pages.cpu().numpy())
    _check_selection(ref["blocks"], st, cfg, ran.np["tau"])
    np.testing.assert_allclose(host(st.blk_mass), ref["blocks"]["mass"], rtol=0, atol=1e-5)
    # the chunk takes part: some row keeps a block of its own tokens
    _, cnt, idx = gpu_block_lists(st)
    assert np.any(idx >= _grp(cfg) * cfg.n_kblocks)


def test_block_selection_pooled_from_k_act(ran):
    """Without the gather's key-block means the candidates are pooled from the
    active keys directly; same selection (up to flagged near-ties)."""
    st, cfg = ran.step, ran.cfg
    ref = ran.oracle(sel_pages=st.sel_pages.cpu().numpy())
    st.select(ran.q, ran.tau, use_kblk_mean=False)
    torch.cuda.synchronize()
    _check_selection(ref["blocks"], st, cfg, ran.np["tau"])
    np.testing.assert_allclose(host(st.blk_mass), ref["blocks"]["mass"], rtol=0, atol=1e-5)
    st.select(ran.q, ran.tau)  # restore the step's own selection
    torch.cuda.synchronize()


def test_linear_branch_over_the_joined_keys(ran):
    st, cfg = ran.step, ran.cfg
    lin = ran.oracle(sel_pages=st.sel_pages.cpu().numpy())["lin"]
    proj_tol = (2e-4, 1e-5)
    assert_close("k_proj", host(st.k_proj), lin["ktil"], cfg, proj_tol)
    assert_close("v_proj", host(st.v_proj).transpose(0, 2, 1), lin["vtil"], cfg, proj_tol)
    assert_close("o_lin", host(st.o_lin), lin["o_lin"], cfg)


def test_sparse_branch_and_fuse(ran):
    st, cfg = ran.step, ran.cfg
    lists, _, _ = gpu_block_lists(st)
    grp, nt = _grp(cfg), cfg.n_kblocks
    cands = [[candidates_of(lists[h][i], nt, grp) for i in range(cfg.n_qblocks)] for h in range(cfg.n_heads)]
    ref = ran.oracle(sel_pages=st.sel_pages.cpu().numpy(), block_sel=cands)
    assert_close("o_sp", host(st.o_sp), ref["o_sp"], cfg)
    assert_close("out", host(st.out), ref["out"], cfg)


def test_tau_one_is_dense_over_history_and_chunk():
    cfg = replace(M2, name="m2_intra3_dense", intra_split=3)
    r = Run(cfg, tau=np.ones(cfg.n_heads))
    st = r.run()
    assert np.all(st.blk_count.cpu().numpy() == cfg.n_key_blocks)
    ref = r.oracle(sel_pages=st.sel_pages.cpu().numpy())
    assert_close("o_sp", host(st.o_sp), ref["o_sp"], cfg)


def test_intra_graph_replays_match_eager():
    """The step with intra-chunk keys captured into a HIP graph: every replay,
    with eager steps between replays, equals the eager step bit for bit."""
    cfg = INTRA[0]
    r = Run(cfg)
    st = r.run()
    names = ("out", "o_sp", "o_lin", "blk_count", "blk_idx", "k_act", "kblk_mean")
    ref = {k: getattr(st, k).clone() for k in names}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run(r.q, r.pk, r.pv, r.e_k, r.e_v, r.w_g, r.x, r.tau, k_cur=r.k_cur, v_cur=r.v_cur)
    for rep in range(3):
        for k in names:
            getattr(st, k).zero_()
        g.replay()
        torch.cuda.synchronize()
        for k in names:
            assert torch.equal(getattr(st, k), ref[k]), f"replay {rep}: {k}"
        r.run()
        torch.cuda.synchronize()


def test_chunk_gather_rewrites_only_the_chunk(ran):
    """hsa_gather_chunk with another step's keys equals the whole gather with
    them, bit for bit, and leaves the history part as it was."""
    from sparse_linear_attention_hsa_amd import ops
    st, cfg = ran.step, ran.cfg
    k2 = torch.flip(ran.k_cur, dims=[0]).contiguous()  # other keys and values for the chunk
    v2 = torch.flip(ran.v_cur, dims=[0]).contiguous()
    ran.run()
    hist = st.k_act[:, :cfg.history_tokens].clone()
    ops.hsa_gather_chunk(st.geom, k2, v2, st.k_act, st.v_act, st.kblk_mean)
    torch.cuda.synchronize()
    got = [t.clone() for t in (st.k_act, st.v_act, st.kblk_mean)]
    assert torch.equal(got[0][:, :cfg.history_tokens], hist)
    st.gather(ran.pk, ran.pv, k_cur=k2, v_cur=v2)
    torch.cuda.synchronize()
    for a, b in zip(got, (st.k_act, st.v_act, st.kblk_mean)):
        assert torch.equal(a, b)


def test_history_and_chunk_projections_add_up(ran):
    """HSA_LIN_HISTORY_PROJ then HSA_LIN_CHUNK_PROJ gives the linear branch of
    the whole sequence: the history's projection against the oracle's over
    the history keys, O_lin against the oracle and against the single call
    (the sums differ only in order), and the history projection unchanged."""
    from sparse_linear_attention_hsa_amd import ops
    from sparse_linear_attention_hsa_amd._lib import HSA_LIN_CHUNK_PROJ, HSA_LIN_HISTORY_PROJ
    st, cfg = ran.step, ran.cfg
    ran.run(concurrent=False)
    full = st.o_lin.clone()
    kh, vh = torch.empty_like(st.k_proj), torch.empty_like(st.v_proj)
    ops.hsa_linear_branch(st.geom, None, st.k_act, st.v_act, ran.e_k, ran.e_v, kh, vh, None, HSA_LIN_HISTORY_PROJ,
                          st.ws)
    torch.cuda.synchronize()
    kh0, vh0 = kh.clone(), vh.clone()
    st.o_lin.zero_()
    ops.hsa_linear_branch(st.geom, ran.q, st.k_act, st.v_act, ran.e_k, ran.e_v, kh, vh, st.o_lin,
                          HSA_LIN_CHUNK_PROJ, st.ws)
    torch.cuda.synchronize()
    assert torch.equal(kh, kh0) and torch.equal(vh, vh0)
    sel = st.sel_pages.cpu().numpy()
    k_hist, v_hist = orc.gather_active(ran.pk_np, sel), orc.gather_active(ran.pv_np, sel)
    lh = cfg.history_tokens
    proj_tol = (2e-4, 1e-5)
    assert_close("history K~", host(kh), orc.project(ran.np["e_k"][:, :lh], k_hist), cfg, proj_tol)
    assert_close("history V~", host(vh).transpose(0, 2, 1), orc.project(ran.np["e_v"][:, :lh], v_hist), cfg,
                 proj_tol)
    ref = ran.oracle(sel_pages=sel)
    assert_close("o_lin", host(st.o_lin), ref["lin"]["o_lin"], cfg)
    f32 = cfg.dtype == "f32"
    # The two call patterns sum the projection's fp32 slice partials in
    # different groupings.  For bf16, K~ reaches the products as a bf16 high
    # part plus the bf16 rounding of the rest (about 16 significant bits), so
    # a regrouped sum can move K~ by one unit of the low part (2^-17
    # relative).  With the peaked heads of the imbalance workload that moves a
    # logit by about 1e-3 and an output element by up to about 6e-3; the
    # relative-L2 bound stays tight.
    assert_close("o_lin vs one call", host(st.o_lin), host(full), cfg, (1e-5, 1e-6) if f32 else (1e-2, 2e-4))
