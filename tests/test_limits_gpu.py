"""The largest geometry the block selection and the sparse plan accept, on
the GPU against the float64 oracle, whole tensors.

32 heads x 128 query blocks = 4,096 selection rows (HSA_MAX_ROWS) over 2,048
key blocks (HSA_MAX_KBLOCKS: 16-token blocks of 32,768 retrieved keys), with
the largest rank (256).  Segments of 32 one-granule blocks then give the
sparse plan its largest shape: up to 64 segments per row (2,048 / 32) and
2,048 (head, segment) pairs.  With blocks this small many rows are near-ties
of the pooled selection (several sets pass the threshold within rounding), so
the selection is checked exactly on the other rows and for validity on those;
the attention is then compared on the GPU's (valid) selection.
"""
import ctypes

import numpy as np
import pytest

from oracle import hsa_oracle as orc
from sparse_linear_attention_hsa_amd import _lib
from synth import Config

from gpu_harness import Run, assert_close, check_block_selection, geom_of, gpu_block_lists, host

pytestmark = pytest.mark.gpu

LIM = Config(name="limits", n_heads=32, head_dim=64, frame_h=8, frame_w=16, frames_per_page=16, query_frames=16,
             tile=(1, 4, 4), n_pages=16, n_sel_pages=16, rank=256, dtype="bf16", structure="rank8", seed=4096)


def test_largest_selection_and_plan_geometry():
    cfg = LIM
    assert cfg.n_heads * cfg.n_qblocks == _lib.HSA_MAX_ROWS and cfg.n_key_blocks == _lib.HSA_MAX_KBLOCKS
    assert _lib.lib().hsa_geom_check(ctypes.byref(geom_of(cfg))) == 0
    print(f"\n[limits] {cfg.n_heads * cfg.n_qblocks} rows x {cfg.n_key_blocks} key blocks, rank {cfg.rank}",
          flush=True)
    r = Run(cfg)
    st = r.run()
    q, s = r.np["q"], r.np
    # S1, S2
    sc = orc.score_and_select(q, r.pk_np, cfg.n_sel_pages)
    np.testing.assert_allclose(host(st.scores), sc["alpha"], rtol=0, atol=2e-5)
    sel = host(st.sel_pages).astype(np.int64)
    assert np.array_equal(sel, sc["sel"]) or (sc["tie"] and orc.valid_page_selection(sc["alpha"], sel, cfg.n_sel_pages))
    k_act, v_act = orc.gather_active(r.pk_np, sel), orc.gather_active(r.pv_np, sel)
    assert np.array_equal(host(st.k_act), k_act)
    # S4, every row
    lists, cnt, _ = gpu_block_lists(st)
    bs = orc.block_selection(q, k_act, s["tau"], cfg.block)
    differ = check_block_selection(bs, lists, s["tau"])
    print(f"[limits] selection: {int(bs['flags'].sum())} near-tie rows, {differ} with another valid set; "
          f"longest row {int(cnt.max())} blocks", flush=True)
    assert cnt.max() > 32 * 32  # a row the plan cuts into more than 32 segments
    # S3, S5, S6 as whole tensors
    lin = orc.linear_branch(q, k_act, v_act, s["e_k"], s["e_v"])
    assert_close("o_lin", host(st.o_lin), lin["o_lin"], cfg)
    o_sp = orc.sparse_attention(q, k_act, v_act, lists, cfg.block)
    assert_close("o_sp", host(st.o_sp), o_sp, cfg)
    assert_close("out", host(st.out), orc.fuse(s["x"], s["w_g"], lin["o_lin"], o_sp), cfg)
