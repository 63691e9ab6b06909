"""Pages read in place (no active-buffer copy): every page laid out once in the
kernels' layouts (hsa_page_prepare), then the step scores from the page index,
takes the selected pages' block means and runs the linear and sparse branches
straight from the pages.  Active key t is token t % Lp of page sel[t / Lp], so
every result must equal the active-buffer path's bit for bit; the laid-out
pages are checked against the oracle's index relation and block means, and the
outputs against the oracle."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import hsa_oracle as orc
from synth import C0, CONFIGS, M1, M2, M3, M4, M5

from gpu_harness import Run, assert_close, host, untile_v

pytestmark = pytest.mark.gpu

NAMES = ("out", "o_sp", "o_lin", "k_proj", "v_proj", "blk_count", "blk_idx", "blk_mass", "kblk_mean", "sel_pages",
         "scores")


def _both(cfg):
    r = Run(cfg)
    st = r.step
    st.index_pages(r.q, r.pk)  # the page index, as kept when pages are written
    prepared = st.prepare_pages(r.pk, r.pv)
    r.run()
    want = {k: getattr(st, k).clone() for k in NAMES}
    st.run_paged(r.q, prepared, r.e_k, r.e_v, r.w_g, r.x, r.tau)
    torch.cuda.synchronize()
    return r, st, prepared, want


@pytest.mark.parametrize("cfg", [C0, M1, M2, M3, M4, M5], ids=lambda c: c.name)
def test_paged_step_equals_gathered_step(cfg):
    print(f"\n[paged] config={cfg.name}", flush=True)
    r, st, (kp, vp, bm), want = _both(cfg)
    for k in NAMES:
        assert torch.equal(getattr(st, k), want[k]), k
    # the laid-out pages: the index relation, bit-exact, and the block means
    for j in range(cfg.n_pages):
        assert np.array_equal(host(kp[j]), r.pk_np[j].transpose(1, 0, 2)), f"k page {j}"
        assert np.array_equal(untile_v(host(vp[j])), r.pv_np[j].transpose(1, 0, 2)), f"v page {j}"
        np.testing.assert_allclose(host(bm[j]), orc.block_means(r.pk_np[j].transpose(1, 0, 2), cfg.block),
                                   rtol=0, atol=2e-5)
    ref = r.oracle(sel_pages=st.sel_pages.cpu().numpy())
    if not ref["blocks"]["flags"].any():
        assert_close("out", host(st.out), ref["out"], cfg)


def test_paged_step_in_order_and_repeated():
    """The in-order schedule and a second paged step give the same bits."""
    r, st, prepared, want = _both(M1)
    st.run_paged(r.q, prepared, r.e_k, r.e_v, r.w_g, r.x, r.tau, concurrent=False)
    torch.cuda.synchronize()
    for k in NAMES:
        assert torch.equal(getattr(st, k), want[k]), k


@pytest.mark.parametrize("name", ["c1_full", "c3_head_imbalance"])
def test_paged_full_size_equals_gathered(name):
    cfg = CONFIGS[name]
    print(f"\n[paged full size] {cfg.name}", flush=True)
    r, st, prepared, want = _both(cfg)
    for k in NAMES:
        assert torch.equal(getattr(st, k), want[k]), k
    del r, st, prepared
    torch.cuda.empty_cache()


def test_paged_graph_replays_match_eager():
    """The paged step captured into a HIP graph: every replay, with eager
    paged steps between replays, equals the eager step bit for bit."""
    r, st, prepared, want = _both(M1)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run_paged(r.q, prepared, r.e_k, r.e_v, r.w_g, r.x, r.tau)
    for rep in range(3):
        for k in NAMES:
            getattr(st, k).zero_()
        g.replay()
        torch.cuda.synchronize()
        for k in NAMES:
            assert torch.equal(getattr(st, k), want[k]), f"replay {rep}: {k}"
        st.run_paged(r.q, prepared, r.e_k, r.e_v, r.w_g, r.x, r.tau)  # eager work between replays
        torch.cuda.synchronize()


# Intra-chunk keys over pages read in place (paper section 3.3, "Inter- and
# intra-chunk sparse granularity"): the chunk's own keys and values are laid
# out into ceil(Lq / Lp) page-format buffers each step and follow the
# selected pages in the selection list, so the paged step must again equal
# the gathered step (with the chunk in the active buffer) bit for bit.
INTRA = [replace(M1, name="m1_intra2", intra_split=2),
         replace(M2, name="m2_intra3_ragged", intra_split=3),      # Lp = 144: a 32-token step spans page and chunk
         replace(M3, name="m3_intra2_long_rows", intra_split=2),
         replace(M4, name="m4_intra3_f32", intra_split=3),
         replace(M5, name="m5_intra2_lq_eq_lp", intra_split=2),    # the chunk fills its one buffer
         replace(M1, name="m1_intra2_two_chunk_pages", intra_split=2, frames_per_page=2, query_frames=4)]


def _both_intra(cfg, concurrent=True):
    r = Run(cfg)
    st = r.step
    st.index_pages(r.q, r.pk)
    prepared = st.prepare_pages(r.pk, r.pv)
    r.run()
    want = {k: getattr(st, k).clone() for k in NAMES}
    st.run_paged(r.q, prepared, r.e_k, r.e_v, r.w_g, r.x, r.tau, concurrent=concurrent, k_cur=r.k_cur,
                 v_cur=r.v_cur)
    torch.cuda.synchronize()
    return r, st, prepared, want


@pytest.mark.parametrize("cfg", INTRA, ids=lambda c: c.name)
def test_paged_intra_step_equals_gathered_intra_step(cfg):
    nc = -(-cfg.query_tokens // cfg.page_tokens)
    print(f"\n[paged intra] config={cfg.name} Lp={cfg.page_tokens} Lq={cfg.query_tokens} chunk buffers={nc}",
          flush=True)
    r, st, (kp, vp, bm), want = _both_intra(cfg)
    assert st.n_chunk_pages == nc
    for k in NAMES:
        assert torch.equal(getattr(st, k), want[k]), k
    # the selection list: the selected pages, then the chunk buffers' table indices
    assert st.sel_ext[cfg.n_sel_pages:].tolist() == list(range(cfg.n_pages, cfg.n_pages + nc))
    # the chunk's buffers: the index relation, bit-exact, and the key-block means
    kc = r.np["k_cur"].transpose(1, 0, 2)
    vc = r.np["v_cur"].transpose(1, 0, 2)
    Lp, Bk = cfg.page_tokens, cfg.key_block
    for j, (ck, cv, cm) in enumerate(st._chunk_bufs):
        n = min(Lp, cfg.query_tokens - j * Lp)
        part_k, part_v = kc[:, j * Lp:j * Lp + n], vc[:, j * Lp:j * Lp + n]
        assert np.array_equal(host(ck)[:, :n], part_k), f"chunk k buffer {j}"
        assert np.array_equal(untile_v(host(cv))[:, :n], part_v), f"chunk v buffer {j}"
        np.testing.assert_allclose(host(cm)[:, :n // Bk], orc.block_means(part_k, Bk), rtol=0, atol=2e-5)
    # a laid-out page keeps its key-block means at the chunk's block size
    np.testing.assert_allclose(host(bm[0]), orc.block_means(r.pk_np[0].transpose(1, 0, 2), Bk), rtol=0, atol=2e-5)
    ref = r.oracle(sel_pages=st.sel_pages.cpu().numpy())
    if not ref["blocks"]["flags"].any():
        assert_close("out", host(st.out), ref["out"], cfg)


def test_paged_intra_in_order_and_repeated():
    """In order on one stream, then a second concurrent paged step reusing the
    chunk's buffers: the same bits."""
    r, st, prepared, want = _both_intra(INTRA[1], concurrent=False)
    for k in NAMES:
        assert torch.equal(getattr(st, k), want[k]), k
    st.run_paged(r.q, prepared, r.e_k, r.e_v, r.w_g, r.x, r.tau, k_cur=r.k_cur, v_cur=r.v_cur)
    torch.cuda.synchronize()
    for k in NAMES:
        assert torch.equal(getattr(st, k), want[k]), k


def test_paged_intra_needs_the_chunk():
    r = Run(INTRA[0])
    prepared = r.step.prepare_pages(r.pk, r.pv)
    with pytest.raises(ValueError):
        r.step.run_paged(r.q, prepared, r.e_k, r.e_v, r.w_g, r.x, r.tau)


def test_paged_intra_full_size_equals_gathered():
    cfg = replace(CONFIGS["c1_full"], name="c1_intra2", intra_split=2)
    print(f"\n[paged intra full size] {cfg.name}", flush=True)
    r, st, prepared, want = _both_intra(cfg)
    for k in NAMES:
        assert torch.equal(getattr(st, k), want[k]), k
    del r, st, prepared
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cfg", [INTRA[0], INTRA[1], INTRA[5]], ids=lambda c: c.name)
def test_paged_intra_history_and_chunk_projections(cfg):
    """The projection split into the history's part (kept across denoising
    steps) and the chunk's part, over pages read in place, equals the same
    split over the active buffer bit for bit."""
    from sparse_linear_attention_hsa_amd import ops
    from sparse_linear_attention_hsa_amd._lib import HSA_LIN_CHUNK_PROJ, HSA_LIN_HISTORY_PROJ
    print(f"\n[paged intra split projection] config={cfg.name}", flush=True)
    r, st, prepared, _ = _both_intra(cfg)  # st.k_act / v_act hold the gathered active buffer
    kp, vp, _, sel = st.paged_inputs(prepared, r.k_cur, r.v_cur)

    def gathered(flags, kh, vh, o):
        ops.hsa_linear_branch(st.geom, None if o is None else r.q, st.k_act, st.v_act, r.e_k, r.e_v, kh, vh, o,
                              flags, st.ws)

    def paged(flags, kh, vh, o):
        ops.hsa_linear_branch_paged(st.geom, None if o is None else r.q, kp, vp, sel, r.e_k, r.e_v, kh, vh, o,
                                    flags, st.ws)

    got = {}
    for name, call in (("gathered", gathered), ("paged", paged)):
        kh, vh, o = torch.empty_like(st.k_proj), torch.empty_like(st.v_proj), torch.empty_like(st.o_lin)
        call(HSA_LIN_HISTORY_PROJ, kh, vh, None)
        call(HSA_LIN_CHUNK_PROJ, kh, vh, o)
        torch.cuda.synchronize()
        got[name] = (kh, vh, o)
    for what, a, b in zip(("history K~", "history V~", "O_lin"), got["gathered"], got["paged"]):
        assert torch.equal(a, b), what


# Page tables in device memory (the *_devtab calls), which banks beyond
# HSA_MAX_PAGES need: the same bits as host tables; a 300-page bank read in
# place equals the gathered step over the same bank; a selected page with no
# laid-out buffer reads as zeros, as the gather of a missing page writes.
@pytest.mark.parametrize("cfg", [C0, M1, INTRA[1]], ids=lambda c: c.name)
def test_paged_device_tables_equal_host_tables(cfg):
    print(f"\n[paged devtab] config={cfg.name}", flush=True)
    r = Run(cfg)
    st = r.step
    st.index_pages(r.q, r.pk)
    prepared = st.prepare_pages(r.pk, r.pv)
    st.run_paged(r.q, prepared, r.e_k, r.e_v, r.w_g, r.x, r.tau, k_cur=r.k_cur, v_cur=r.v_cur, device_tables=False)
    torch.cuda.synchronize()
    want = {k: getattr(st, k).clone() for k in NAMES}
    st.run_paged(r.q, prepared, r.e_k, r.e_v, r.w_g, r.x, r.tau, k_cur=r.k_cur, v_cur=r.v_cur, device_tables=True)
    torch.cuda.synchronize()
    for k in NAMES:
        assert torch.equal(getattr(st, k), want[k]), k


def test_paged_bank_of_300_pages():
    from sparse_linear_attention_hsa_amd.ops import DeviceTable
    from synth import with_
    cfg = with_(M1, name="m1_bank300", n_pages=300, seed=2301)
    print(f"\n[paged devtab] {cfg.name}: {cfg.n_pages} pages read in place", flush=True)
    r = Run(cfg)
    st = r.step
    kt, vt = DeviceTable(r.pk), DeviceTable(r.pv)
    st.index_pages(r.q, kt)
    st.run(r.q, kt, vt, r.e_k, r.e_v, r.w_g, r.x, r.tau, indexed=True)
    torch.cuda.synchronize()
    want = {k: getattr(st, k).clone() for k in NAMES}
    prepared = st.prepare_pages(r.pk, r.pv)
    st.run_paged(r.q, prepared, r.e_k, r.e_v, r.w_g, r.x, r.tau)  # device tables by default beyond 128 pages
    torch.cuda.synchronize()
    assert st._devtabs is not None and len(st._devtabs[1][0]) == cfg.n_pages
    for k in NAMES:
        assert torch.equal(getattr(st, k), want[k]), k


def test_paged_missing_page_reads_as_zeros():
    from sparse_linear_attention_hsa_amd.ops import DeviceTable
    cfg = M1
    r = Run(cfg)
    st = r.step
    st.index_pages(r.q, r.pk)  # the index still scores the page, so it is selected
    r.run(indexed=True)
    j = int(st.sel_pages[0])
    print(f"\n[paged devtab] {cfg.name}: selected page {j} without a buffer", flush=True)
    pk = [None if i == j else t for i, t in enumerate(r.pk)]
    pv = [None if i == j else t for i, t in enumerate(r.pv)]
    st.run(r.q, DeviceTable(pk), DeviceTable(pv), r.e_k, r.e_v, r.w_g, r.x, r.tau, indexed=True)
    torch.cuda.synchronize()
    assert int(st.sel_pages[0]) == j and not torch.any(st.k_act[:, :cfg.page_tokens].float() != 0)
    want = {k: getattr(st, k).clone() for k in NAMES}
    kp, vp, bm = st.prepare_pages(r.pk, r.pv)
    kp[j] = vp[j] = bm[j] = None
    st.run_paged(r.q, (kp, vp, bm), r.e_k, r.e_v, r.w_g, r.x, r.tau, device_tables=True)
    torch.cuda.synchronize()
    for k in NAMES:
        assert torch.equal(getattr(st, k), want[k]), k
