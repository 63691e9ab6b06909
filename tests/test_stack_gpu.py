"""The chunk schedule of a layer stack (several layers x denoising steps).

Page scoring, gather and the linear-branch projection run once per layer,
in the first step, on that step's queries; later steps reuse them and run
the linear attention, block selection, sparse branch and fusion on their
own queries and gate inputs.  Pages of the configured share start in pinned
host memory and reach the gather through two device staging slots filled on
a side stream.  The oracle runs every (layer, step) with the first step's
page selection, and the streamed run (linear branch on a side stream) must
equal a run with every page resident and every call in order on one stream,
bit for bit.
"""
from __future__ import annotations

from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import hsa_oracle as orc
from synth import CONFIGS, layer_arrays, stack_host_pages

from gpu_harness import TOL, assert_close, candidates_of, check_block_selection, geom_of

pytestmark = pytest.mark.gpu


def _build(cfg, layers_needed_host=()):
    """Device inputs of every layer; returns (streamed, resident, arrays of the requested layers)."""
    from sparse_linear_attention_hsa_amd.stack import LayerInputs, make_layer_inputs
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(tdt).cuda()
    geom = geom_of(cfg)
    host_ids = stack_host_pages(cfg)
    streamed, resident, keep = [], [], {}
    for l in range(cfg.layers):
        a = layer_arrays(cfg, l, cfg.steps, workers=16)
        if l in layers_needed_host:
            keep[l] = a
        pk = [up(x) for x in a["pages_k"]]
        pv = [up(x) for x in a["pages_v"]]
        qs = [up(x) for x in a["q"]]
        xs = [up(x) for x in a["x"]]
        e_k, e_v, w_g = up(a["e_k"]), up(a["e_v"]), up(a["w_g"])
        kc = [up(x) for x in a["k_cur"]]
        vc = [up(x) for x in a["v_cur"]]
        tau = torch.from_numpy(a["tau"]).cuda()
        lay = make_layer_inputs(geom, pk, pv, host_ids[l], e_k, e_v, w_g, tau, qs, xs, kc, vc)
        streamed.append(lay)
        resident.append(LayerInputs(pages_k=pk, pages_v=pv, host_k={}, host_v={}, e_k=e_k, e_v=e_v, w_g=w_g,
                                    tau=tau, page_kmean=lay.page_kmean, q=lay.q, x=lay.x, k_cur=kc, v_cur=vc))
    return geom, host_ids, streamed, resident, keep


def _run(cfg, geom, host_ids, inputs, pairs, n_slots=4, concurrent=True):
    """Run one chunk; return per (layer, step) in `pairs`: out, o_lin, o_sp, counts, lists; and per layer the pages."""
    from sparse_linear_attention_hsa_amd.stack import HsaStack
    st = HsaStack(geom, cfg.n_pages, cfg.layers, max(len(h) for h in host_ids), n_slots=n_slots)
    outs = {p: torch.empty(cfg.query_tokens, cfg.n_heads, cfg.head_dim, dtype=inputs[0].q[0].dtype, device="cuda")
            for p in pairs}
    cap = {}

    def probe(l, s):
        if (l, s) in outs:
            cap[(l, s)] = (st.o_lin.clone(), st.o_sp.clone(), st.blk_count.clone(), st.blk_idx.clone())

    st.run_chunk(inputs, cfg.steps, outs, probe, concurrent=concurrent)
    torch.cuda.synchronize()
    res = {}
    for p in pairs:
        o_lin, o_sp, cnt, idx = (t.cpu().numpy() for t in cap[p])
        res[p] = dict(out=outs[p].float().cpu().numpy(), o_lin=o_lin, o_sp=o_sp, cnt=cnt, idx=idx)
    sel = [st.layers[l].sel_pages.cpu().numpy().astype(np.int64) for l in range(cfg.layers)]
    return res, sel


def _check_layer_step(cfg, a, s, gpu_sel, r):
    """Oracle for one (layer, step) with the first step's pages, over every
    row; with intra-chunk keys the step's own keys follow the pages."""
    B, H = cfg.block, cfg.n_heads
    sc = orc.score_and_select(a["q"][0], a["pages_k"], cfg.n_sel_pages)
    if not np.array_equal(gpu_sel, sc["sel"]):
        assert sc["tie"] and orc.valid_page_selection(sc["alpha"], gpu_sel, cfg.n_sel_pages)
    k_act = orc.gather_active(a["pages_k"], gpu_sel)
    v_act = orc.gather_active(a["pages_v"], gpu_sel)
    q, x = a["q"][s], a["x"][s]
    gl = [[r["idx"][h, i, :r["cnt"][h, i]].astype(np.int64) for i in range(cfg.n_qblocks)] for h in range(H)]
    if cfg.intra_split:
        lh = k_act.shape[1]
        k_act = np.concatenate([k_act, np.asarray(a["k_cur"][s], np.float64).transpose(1, 0, 2)], axis=1)
        v_act = np.concatenate([v_act, np.asarray(a["v_cur"][s], np.float64).transpose(1, 0, 2)], axis=1)
        parts = orc.key_parts(lh, B, cfg.query_tokens, cfg.key_block)
        bs = orc.block_selection_parts(q, k_act, a["tau"], B, parts)
        grp, nt = B // cfg.key_block, cfg.n_kblocks
        cands = [[candidates_of(gl[h][i], nt, grp) for i in range(cfg.n_qblocks)] for h in range(H)]
        assert all(c is not None for row in cands for c in row), "incomplete history tile"
        check_block_selection(bs, cands, a["tau"])
    else:
        bs = orc.block_selection(q, k_act, a["tau"], B)
        check_block_selection(bs, gl, a["tau"])
    ktil, vtil = orc.project(a["e_k"], k_act), orc.project(a["e_v"], v_act)
    o_lin_ref = orc.linear_attention(q, ktil, vtil)
    if cfg.intra_split:
        o_sp_ref = orc.sparse_attention_parts(q, k_act, v_act, cands, B, parts)
    else:
        o_sp_ref = orc.sparse_attention(q, k_act, v_act, gl, B)
    out_ref = orc.fuse(x, a["w_g"], o_lin_ref, o_sp_ref)
    assert_close("o_lin", r["o_lin"], o_lin_ref, cfg)
    assert_close("o_sp", r["o_sp"], o_sp_ref, cfg)
    assert_close("out", r["out"], out_ref, cfg)


@pytest.mark.parametrize("n_slots,intra", [(2, 0), (4, 0), (3, 2)], ids=["slots2", "slots4", "intra2"])
def test_stack_small_every_layer_step(n_slots, intra):
    cfg = CONFIGS["m6_stack"]
    if intra:  # the chunk's own keys in 48-token blocks, new keys every denoising step
        cfg = replace(cfg, name="m6_stack_intra2", intra_split=intra)
    print(f"\n[stack] {cfg.name}: {cfg.layers} layers x {cfg.steps} steps, {n_slots} staging slots, host pages "
          f"{[h.tolist() for h in stack_host_pages(cfg)]}", flush=True)
    geom, host_ids, streamed, resident, keep = _build(cfg, layers_needed_host=range(cfg.layers))
    pairs = [(l, s) for l in range(cfg.layers) for s in range(cfg.steps)]
    got, sel = _run(cfg, geom, host_ids, streamed, pairs, n_slots=n_slots)
    # the reference run: every page resident, every call in order on one stream
    ref, sel_r = _run(cfg, geom, host_ids, resident, pairs, concurrent=False)
    for p in pairs:
        for k in ("out", "o_lin", "o_sp", "cnt", "idx"):
            assert np.array_equal(got[p][k], ref[p][k]), f"streamed != resident at {p} ({k})"
    for l in range(cfg.layers):
        assert np.array_equal(sel[l], sel_r[l])
        for s in range(cfg.steps):
            _check_layer_step(cfg, keep[l], s, sel[l], got[(l, s)])


def test_stack_c4_four_layer_steps():
    """The first and last layer, first and last step: every row of the four."""
    cfg = CONFIGS["c4_stack"]
    last = cfg.layers - 1
    print(f"\n[stack] {cfg.name}: {cfg.layers} layers x {cfg.steps} steps, "
          f"{sum(len(h) for h in stack_host_pages(cfg))} host pages", flush=True)
    geom, host_ids, streamed, _, keep = _build(cfg, layers_needed_host=(0, last))
    pairs = [(0, 0), (0, cfg.steps - 1), (last, 0), (last, cfg.steps - 1)]
    got, sel = _run(cfg, geom, host_ids, streamed, pairs)
    for (l, s) in pairs:
        print(f"  layer {l} step {s}: pages {sel[l].tolist()} (host {host_ids[l].tolist()}), "
              f"selected pairs {int(got[(l, s)]['cnt'].sum())}", flush=True)
        _check_layer_step(cfg, keep[l], s, sel[l], got[(l, s)])
