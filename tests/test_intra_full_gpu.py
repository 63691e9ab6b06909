"""Intra-chunk keys at full size, in the launch configuration the benchmark
times (bench.py --intra 2): the 12-head, d = 128 workloads (plain and with
imbalanced heads) with 49,920 retrieved keys and the chunk's own 6,240 tokens
in 48-token key blocks
beside the 96-token history tiles (WorldAttention paper, section 3.3,
inter- and intra-chunk sparse granularity).  Checked against the float64
oracle: the active K/V bit-exact and the key-block means, the projections
over the joined sequence, every selection row, and the whole output tensors
(linear branch, sparse branch, fused output)."""
from __future__ import annotations

from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import hsa_oracle as orc
from synth import CONFIGS

from gpu_harness import (Run, assert_close, candidates_of, gpu_block_lists, host, key_blocks_of, untile_v)

pytestmark = pytest.mark.gpu

PROJ_TOL = (2e-4, 1e-5)


@pytest.mark.parametrize("name", ["c1_full", "c3_head_imbalance"])
def test_full_size_intra_step(name):
    cfg = replace(CONFIGS[name], name=f"{name}_intra2", intra_split=2)
    print(f"\n[full-size intra parity] Lh={cfg.history_tokens} Lq={cfg.query_tokens} B={cfg.block} "
          f"Bk={cfg.key_block} nKB={cfg.n_key_blocks} nC={cfg.n_candidates}", flush=True)
    r = Run(cfg)
    st = r.run()
    s = r.np
    H, d, B, Bk = cfg.n_heads, cfg.head_dim, cfg.block, cfg.key_block
    grp, nt = B // Bk, cfg.n_kblocks

    sel = host(st.sel_pages).astype(np.int64)
    k_act = np.concatenate([orc.gather_active(r.pk_np, sel), s["k_cur"].transpose(1, 0, 2)], axis=1)
    v_act = np.concatenate([orc.gather_active(r.pv_np, sel), s["v_cur"].transpose(1, 0, 2)], axis=1)
    k_gpu = st.k_act.float().cpu().numpy()
    v_gpu = untile_v(st.v_act.float().cpu().numpy())
    for h in range(H):
        assert np.array_equal(k_gpu[h], k_act[h]), f"k_act head {h} differs"
        assert np.array_equal(v_gpu[h], v_act[h]), f"v_act head {h} differs"
    del k_gpu, v_gpu
    assert_close("key-block means", host(st.kblk_mean), orc.block_means(k_act, Bk), cfg, tol=(1e-5, 1e-6))

    lin = dict(ktil=orc.project(s["e_k"], k_act), vtil=orc.project(s["e_v"], v_act))
    assert_close("k_proj", host(st.k_proj), lin["ktil"], cfg, tol=PROJ_TOL)
    assert_close("v_proj", host(st.v_proj).transpose(0, 2, 1), lin["vtil"], cfg, tol=PROJ_TOL)

    parts = orc.key_parts(cfg.history_tokens, B, cfg.query_tokens, Bk)
    bs = orc.block_selection_parts(s["q"], k_act, s["tau"], B, parts)
    gl, cnt, _ = gpu_block_lists(st)
    cands = [[None] * cfg.n_qblocks for _ in range(H)]
    differ = 0
    for h in range(H):
        for i in range(cfg.n_qblocks):
            got = candidates_of(gl[h][i], nt, grp)
            assert got is not None, f"incomplete history tile (h={h}, i={i})"
            cands[h][i] = got
            want = bs["sel"][h][i]
            if np.array_equal(got, want):
                assert np.array_equal(gl[h][i], key_blocks_of(want, nt, grp))
                continue
            assert bs["flags"][h, i], f"selection differs at unflagged row (h={h}, i={i})"
            assert orc.valid_block_selection(bs["mass"][h, i], got, s["tau"][h])
            differ += 1
    chunk_pairs = int(sum(np.sum(np.asarray(c) >= nt) for row in cands for c in row))
    print(f"  selected key blocks {int(cnt.sum())} of {cnt.size * cfg.n_key_blocks}; chunk blocks among the "
          f"selected candidates {chunk_pairs}; flagged rows {int(bs['flags'].sum())}, differing {differ}",
          flush=True)
    assert chunk_pairs > 0

    o_sp_ref = orc.sparse_attention_parts(s["q"], k_act, v_act, cands, B, parts)
    assert_close("o_sp", host(st.o_sp), o_sp_ref, cfg)
    o_lin_ref = orc.linear_attention(s["q"], lin["ktil"], lin["vtil"])
    assert_close("o_lin", host(st.o_lin), o_lin_ref, cfg)
    out_ref = orc.fuse(s["x"], s["w_g"], o_lin_ref, o_sp_ref)
    mx, rl2 = assert_close("fused output", host(st.out), out_ref, cfg)
    print(f"  fused output over all {cfg.query_tokens} x {H} x {d}: max-abs {mx:.2e}, rel-L2 {rl2:.2e}", flush=True)
    del r, st
    torch.cuda.empty_cache()
