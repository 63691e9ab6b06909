"""Parity at full size, in the launch configuration the benchmark times.

For the three single-layer workloads at their real shapes (12 heads, d=128,
49,920 retrieved keys, 6,240 queries, B=96, r=256), the HIP step runs
exactly as bench.py runs it, and is checked against the float64 oracle:

  * page scores, and the page selection (exact, or valid at a flagged tie);
  * the gathered active K/V, bit-exact, and the block means;
  * the projections K~ and V~ (full), every one of the 780 block-selection
    rows (exact, or valid at a flagged tie);
  * the whole output tensors: the linear branch O_lin, the sparse branch
    O_sp (every query block of every head, over the selected blocks) and the
    fused output, element by element.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import hsa_oracle as orc
from synth import CONFIGS

from gpu_harness import (TOL, Run, assert_close, check_block_selection, gpu_block_lists, host, untile_v)

pytestmark = pytest.mark.gpu

# Projections: bf16 products accumulate exactly in fp32 over L terms.
PROJ_TOL = (2e-4, 1e-5)
# Page scores: fp32 means of bf16 values against float64 (absolute, as for the
# small workloads; scores are O(0.1)).
SCORE_ATOL = 2e-5


@pytest.mark.parametrize("name", ["c1_full", "c3_head_imbalance", "c2_long_history"])
def test_full_size_step(name):
    cfg = CONFIGS[name]
    print(f"\n[full-size parity] {name}: H={cfg.n_heads} d={cfg.head_dim} P={cfg.n_pages} "
          f"L={cfg.active_tokens} Lq={cfg.query_tokens} B={cfg.block} r={cfg.rank}", flush=True)
    r = Run(cfg)
    st = r.run()
    s = r.np
    H, d, B, Lq = cfg.n_heads, cfg.head_dim, cfg.block, cfg.query_tokens

    # S1 -- scores and selection
    sc = orc.score_and_select(s["q"], r.pk_np, cfg.n_sel_pages)
    np.testing.assert_allclose(host(st.scores), sc["alpha"], rtol=0, atol=SCORE_ATOL)
    gpu_sel = host(st.sel_pages).astype(np.int64)
    if not np.array_equal(gpu_sel, sc["sel"]):
        assert sc["tie"], f"page selection {gpu_sel} != {sc['sel']} without a flagged tie"
        assert orc.valid_page_selection(sc["alpha"], gpu_sel, cfg.n_sel_pages)
    sel = gpu_sel

    # S2 -- gathered K/V bit-exact, per head (the oracle's index relation)
    k_act_gpu = st.k_act.float().cpu().numpy()
    v_act_gpu = untile_v(st.v_act.float().cpu().numpy())
    for h in range(H):
        want_k = np.concatenate([r.pk_np[j][:, h, :] for j in sel], axis=0)
        want_v = np.concatenate([r.pv_np[j][:, h, :] for j in sel], axis=0)
        assert np.array_equal(k_act_gpu[h], want_k), f"k_act head {h} differs"
        assert np.array_equal(v_act_gpu[h], want_v), f"v_act head {h} differs"
    k_act = orc.gather_active(r.pk_np, sel)
    v_act = orc.gather_active(r.pv_np, sel)
    kb_ref = orc.block_means(k_act, B)
    assert_close("block means", host(st.kblk_mean), kb_ref, cfg, tol=(1e-5, 1e-6))

    # S3 -- projections over the whole sequence
    lin = dict(ktil=orc.project(s["e_k"], k_act), vtil=orc.project(s["e_v"], v_act))
    assert_close("k_proj", host(st.k_proj), lin["ktil"], cfg, tol=PROJ_TOL)
    assert_close("v_proj", host(st.v_proj).transpose(0, 2, 1), lin["vtil"], cfg, tol=PROJ_TOL)

    # S4 -- every selection row
    bs = orc.block_selection(s["q"], k_act, s["tau"], B)
    gl, cnt, _ = gpu_block_lists(st)
    differ = check_block_selection(bs, gl, s["tau"])
    print(f"  selected pairs {int(cnt.sum())} of {cnt.size * cfg.n_kblocks}; "
          f"flagged rows {int(bs['flags'].sum())}, differing at ties {differ}", flush=True)

    # S5, S3 output, S6 -- whole tensors
    o_sp_ref = orc.sparse_attention(s["q"], k_act, v_act, gl, B)
    assert_close("o_sp", host(st.o_sp), o_sp_ref, cfg)
    o_lin_ref = orc.linear_attention(s["q"], lin["ktil"], lin["vtil"])
    assert_close("o_lin", host(st.o_lin), o_lin_ref, cfg)
    out_ref = orc.fuse(s["x"], s["w_g"], o_lin_ref, o_sp_ref)
    mx, rl2 = assert_close("fused output", host(st.out), out_ref, cfg)
    print(f"  fused output over all {Lq} x {H} x {d}: max-abs {mx:.2e}, rel-L2 {rl2:.2e}", flush=True)
    del r, st
    torch.cuda.empty_cache()
