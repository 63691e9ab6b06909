"""Pages read in place (no active-buffer copy): every page laid out once in the
kernels' layouts (hsa_page_prepare), then the step scores from the page index,
takes the selected pages' block means and runs the linear and sparse branches
straight from the pages.  Active key t is token t % Lp of page sel[t / Lp], so
every result must equal the active-buffer path's bit for bit; the laid-out
pages are checked against the oracle's index relation and block means, and the
outputs against the oracle."""
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
