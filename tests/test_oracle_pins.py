"""Pins of the CPU oracle to facts outside itself (hand-worked examples,
textbook special cases, brute force, invariants).  CPU only."""
import itertools
import math

import numpy as np
import pytest
import torch

from oracle import hsa_oracle as orc
from synth import C0, C1, M1, M2, M3, M4, M5, Workload


def sdpa(q, k, v):
    """Textbook softmax attention from torch (float64, CPU): q [n][d], k/v [m][d]."""
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))[None]
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v))[0].numpy()


# ------------------------------------------------------------------ O1 order
def test_token_order_hand_values(golden):
    g = golden("hw6_token_order.json")
    for (f, y, x), want in g["cases"]:
        assert orc.tile_major_index(f, y, x, g["frame_h"], g["frame_w"], tuple(g["tile"])) == want


@pytest.mark.parametrize("frames,fh,fw,tile", [(4, 30, 52, (4, 6, 4)), (8, 30, 52, (4, 6, 4)),
                                               (2, 6, 8, (1, 2, 8)), (4, 12, 8, (2, 6, 8))])
def test_token_order_bijection_and_cubes(frames, fh, fw, tile):
    perm = orc.raster_to_tile_major(frames, fh, fw, tile)
    assert np.array_equal(np.sort(perm), np.arange(len(perm)))
    b = tile[0] * tile[1] * tile[2]
    # every contiguous group of b tile-major tokens is one spatio-temporal cube
    inv = np.argsort(perm)
    f, rem = np.divmod(inv, fh * fw)
    y, x = np.divmod(rem, fw)
    for g in range(len(perm) // b):
        sl = slice(g * b, (g + 1) * b)
        assert len({v // tile[0] for v in f[sl]}) == 1
        assert len({v // tile[1] for v in y[sl]}) == 1
        assert len({v // tile[2] for v in x[sl]}) == 1


def test_token_order_identity_for_tiny_config():
    perm = orc.raster_to_tile_major(C0.query_frames, C0.frame_h, C0.frame_w, C0.tile)
    assert np.array_equal(perm, np.arange(len(perm)))


# ------------------------------------------------------------- S1 scoring
@pytest.mark.parametrize("name", ["hw1_page_topk.json", "hw2_head_average.json"])
def test_page_scores_hand_examples(golden, name):
    g = golden(name)
    q = np.array(g["q"], dtype=np.float64)
    pages = [np.array(p, dtype=np.float64) for p in g["pages_k"]]
    for case in g["cases"]:
        r = orc.score_and_select(q, pages, case["k"])
        np.testing.assert_allclose(r["alpha"], g["alpha"], rtol=0, atol=1e-15)
        assert r["sel"].tolist() == case["sel"]
        assert r["tie"] == case["tie"]
        assert orc.valid_page_selection(r["alpha"], case["sel"], case["k"])
        for alt in case["also_valid"]:
            assert orc.valid_page_selection(r["alpha"], alt, case["k"])
    # a wrong pick is not valid
    assert not orc.valid_page_selection(np.array(g["alpha"]), [0], 1)


def test_page_score_invariances():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((40, 3, 16))
    pages = [rng.standard_normal((24, 3, 16)) + rng.standard_normal(16) for _ in range(7)]
    base = orc.score_and_select(q, pages, 3)
    assert orc.score_and_select(2.5 * q, pages, 3)["sel"].tolist() == base["sel"].tolist()
    shuffled = [p[rng.permutation(len(p))] for p in pages]
    np.testing.assert_allclose(orc.score_and_select(q, shuffled, 3)["alpha"], base["alpha"], rtol=1e-12, atol=1e-14)
    # a brute-force check of the top-k definition
    a = base["alpha"]
    best = max(itertools.combinations(range(7), 3), key=lambda s: (sum(a[list(s)]), [-i for i in s]))
    assert sorted(best) == base["sel"].tolist()


# ------------------------------------------------ stage 1, chunk page budget
def test_prompt_retrieval_hand_example(golden):
    g = golden("hw7_prompt_retrieval.json")
    e_cur, e_past = np.array(g["e_cur"], float), np.array(g["e_past"], float)
    for case in g["cases"]:
        r = orc.prompt_retrieval(e_cur, e_past, case["k"])
        np.testing.assert_allclose(r["sims"], g["sims"], rtol=0, atol=1e-15)
        assert r["sel"].tolist() == case["sel"]
        assert not r["tie"]


def test_prompt_retrieval_invariances():
    rng = np.random.default_rng(17)
    e_cur = rng.standard_normal(24)
    e_past = rng.standard_normal((9, 24))
    base = orc.prompt_retrieval(e_cur, e_past, 3)
    # positive scaling of any embedding, and one permutation of the
    # embedding axis applied to all, leave every similarity unchanged
    scaled = orc.prompt_retrieval(3.0 * e_cur, e_past * rng.uniform(0.1, 5.0, size=(9, 1)), 3)
    np.testing.assert_allclose(scaled["sims"], base["sims"], rtol=1e-12, atol=1e-14)
    perm = rng.permutation(24)
    np.testing.assert_allclose(orc.prompt_retrieval(e_cur[perm], e_past[:, perm], 3)["sims"], base["sims"],
                               rtol=1e-12, atol=1e-14)
    # bounds, and the best chunk is the one with the largest similarity
    assert np.all(np.abs(base["sims"]) <= 1.0 + 1e-12)
    assert orc.prompt_retrieval(e_cur, e_past, 1)["sel"].tolist() == [int(np.argmax(base["sims"]))]
    # a past embedding equal to the current one (up to scale) is the top-1 chunk
    e_past[4] = 0.3 * e_cur
    r = orc.prompt_retrieval(e_cur, e_past, 1)
    assert r["sel"].tolist() == [4] and abs(r["sims"][4] - 1.0) < 1e-12


def test_ranking_readings_equal_values_nan_and_zero_embeddings():
    """Readings where the pages say nothing: equal values go to the lower id,
    a NaN ranks as -inf (so with -inf the lower id wins), a zero prompt
    embedding has similarity 0 with every chunk.  Values worked by hand."""
    nan, inf = float("nan"), float("inf")
    assert orc.top_k_lower_index(np.array([0.2, 0.2, 0.2]), 2)[1].tolist() == [0, 1]
    assert orc.top_k_lower_index(np.array([0.3, nan, 0.5, nan, 0.1]), 3)[1].tolist() == [0, 2, 4]
    assert orc.top_k_lower_index(np.array([0.3, nan, 0.5, nan, 0.1]), 4)[1].tolist() == [0, 1, 2, 4]
    assert orc.top_k_lower_index(np.array([nan, -inf, 0.2]), 2)[1].tolist() == [0, 2]
    assert orc.top_k_lower_index(np.array([-inf, nan, 0.2]), 2)[1].tolist() == [0, 2]
    sel, tie = orc.select_pages(np.array([0.1, 0.4, 0.4, 0.2]), 2)
    assert sel.tolist() == [1, 2] and not tie
    sel, tie = orc.select_pages(np.array([0.1, 0.4, 0.2, 0.2]), 2)
    assert sel.tolist() == [1, 2] and tie
    # uniform mass over 12 blocks: 7/12 < 0.6 <= 8/12, the eight lowest ids
    sel, flag = orc.select_blocks(np.full(12, 1.0 / 12.0), 0.6)
    assert sel.tolist() == list(range(8)) and flag
    # a NaN embedding ranks last; a zero one has similarity 0; a zero prompt ties every chunk at 0
    e_past = np.array([[nan, 1.0, 0.0], [0.0, 0.0, 0.0], [-1.0, 0.0, 0.0], [1.0, 1.0, 0.0]])
    r = orc.prompt_retrieval(np.array([1.0, 0.0, 0.0]), e_past, 3)
    assert np.isnan(r["sims"][0]) and r["sims"][1] == 0.0 and r["sims"][2] == -1.0
    assert abs(r["sims"][3] - 1.0 / np.sqrt(2.0)) < 1e-15 and r["sel"].tolist() == [1, 2, 3]
    r = orc.prompt_retrieval(np.zeros(3), e_past, 2)
    assert r["sims"].tolist() == [0.0] * 4 and r["sel"].tolist() == [0, 1] and r["tie"]


def test_chunk_pages_hand_examples(golden):
    g = golden("hw8_chunk_pages.json")
    for case in g["cases"]:
        sel, tie = orc.select_pages_in_chunks(np.array(case["alpha"]), case["page_chunk"], case["chunks"],
                                              case["k_p"])
        assert sel.tolist() == case["sel"], case
        assert tie == case["tie"], case


def test_chunk_pages_special_cases():
    rng = np.random.default_rng(23)
    q = rng.standard_normal((30, 2, 8))
    pages = [rng.standard_normal((12, 2, 8)) + rng.standard_normal(8) for _ in range(12)]
    # one chunk holding every page: plain top-K_p scoring
    whole = orc.score_chunk_pages(q, pages, [0] * 12, [0], 4)
    plain = orc.score_and_select(q, pages, 4)
    assert whole["sel"].tolist() == plain["sel"].tolist()
    np.testing.assert_allclose(whole["alpha"], plain["alpha"], rtol=1e-12, atol=1e-14)
    # one page per chunk (Top-K_p chunks): every chosen chunk's argmax page
    page_chunk = [j // 3 for j in range(12)]
    r = orc.score_chunk_pages(q, pages, page_chunk, [0, 2, 3], 3)
    want = sorted(3 * c + int(np.argmax(plain["alpha"][3 * c:3 * c + 3])) for c in (0, 2, 3))
    assert r["sel"].tolist() == want
    # pages outside the chosen chunks are never scored or chosen
    assert np.all(np.isneginf(r["alpha"][3:6]))
    np.testing.assert_allclose(r["alpha"][:3], plain["alpha"][:3], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("cfg", [M1, M2, M3, M4, M5])
def test_planted_pages_are_retrieved(cfg):
    w = Workload(cfg)
    pk = [w.page_k(j) for j in range(cfg.n_pages)]
    r = orc.score_and_select(w.q(), pk, cfg.n_sel_pages)
    assert r["sel"].tolist() == w.plant.target_pages.tolist()
    assert not r["tie"]


# --------------------------------------------------------------- S2 gather
def test_gather_is_an_exact_relayout():
    rng = np.random.default_rng(1)
    pages = [rng.standard_normal((10, 2, 4)).astype(np.float32) for _ in range(5)]
    sel = [1, 3, 4]
    act = orc.gather_active(pages, sel)
    assert act.shape == (2, 30, 4)
    back = act.transpose(1, 0, 2).reshape(3, 10, 2, 4)
    for s, j in enumerate(sel):
        assert np.array_equal(back[s], pages[j])


# ---------------------------------------------------------------- S3 linear
def test_linear_branch_with_identity_projection_is_dense_attention():
    rng = np.random.default_rng(2)
    H, L, Lq, d = 2, 48, 20, 16
    q = rng.standard_normal((Lq, H, d))
    k = rng.standard_normal((H, L, d))
    v = rng.standard_normal((H, L, d))
    eye = np.eye(L)
    out = orc.linear_branch(q, k, v, eye, eye)["o_lin"]
    for h in range(H):
        np.testing.assert_allclose(out[:, h, :], sdpa(q[:, h, :], k[h], v[h]), rtol=1e-10, atol=1e-12)
    # a permutation projection reorders keys and values together: same attention
    p = np.eye(L)[rng.permutation(L)]
    np.testing.assert_allclose(orc.linear_branch(q, k, v, p, p)["o_lin"], out, rtol=1e-10, atol=1e-12)


def test_linear_branch_rank_one_is_query_independent():
    rng = np.random.default_rng(3)
    H, L, Lq, d = 2, 30, 9, 8
    q = rng.standard_normal((Lq, H, d))
    k = rng.standard_normal((H, L, d))
    v = rng.standard_normal((H, L, d))
    e_k = rng.standard_normal((1, L))
    e_v = rng.standard_normal((1, L))
    out = orc.linear_branch(q, k, v, e_k, e_v)["o_lin"]
    for h in range(H):
        want = e_v[0] @ v[h]
        np.testing.assert_allclose(out[:, h, :], np.broadcast_to(want, (Lq, d)), rtol=1e-12, atol=1e-12)


# -------------------------------------------------------------- S4 selection
def test_tau_selection_hand_example(golden):
    g = golden("hw3_tau_selection.json")
    kb = np.log(np.array(g["k_is_ln_of"], dtype=np.float64))[:, None]
    m = orc.pooled_mass(np.array(g["q"]), kb)
    np.testing.assert_allclose(m, g["mass"], rtol=0, atol=1e-15)
    for case in g["cases"]:
        sel, tie = orc.select_blocks(m, case["tau"])
        assert sel.tolist() == case["sel"], case
        assert tie == case["tie"], case
        assert orc.valid_block_selection(m, case["sel"], case["tau"])
        for alt in case["also_valid"]:
            assert orc.valid_block_selection(m, alt, case["tau"])
    assert not orc.valid_block_selection(m, [0, 2], 0.7)          # not mass-ordered
    assert not orc.valid_block_selection(m, [0, 1, 2], 0.7)       # not minimal


def test_block_selection_brute_force_minimal_sets():
    rng = np.random.default_rng(4)
    for trial in range(40):
        s = rng.normal(0, rng.uniform(0.2, 3.0), size=12)
        m = orc.softmax_rows(s[None])[0]
        tau = float(rng.uniform(0.05, 0.99))
        sel, _ = orc.select_blocks(m, tau)
        best = None
        for r in range(1, 13):
            for sub in itertools.combinations(range(12), r):
                if m[list(sub)].sum() >= tau:
                    best = r
                    break
            if best:
                break
        assert len(sel) == best
        # among minimum-size sets the greedy prefix carries the largest mass
        top = max(m[list(sub)].sum() for sub in itertools.combinations(range(12), best))
        assert abs(m[sel].sum() - top) < 1e-12


def test_block_selection_limits():
    rng = np.random.default_rng(6)
    m = orc.softmax_rows(rng.standard_normal((1, 20)))[0]
    assert len(orc.select_blocks(m, 1.0)[0]) == 20
    assert orc.select_blocks(m, 1e-9)[0].tolist() == [int(np.argmax(m))]
    # uniform mass: n = ceil(tau * nKB)
    u = np.full(20, 1 / 20)
    assert len(orc.select_blocks(u, 0.33)[0]) == math.ceil(0.33 * 20)


def test_block_means_and_pooled_selection_on_planted_rows():
    # a query block aligned with exactly one key block selects it alone at small tau
    H, B, d = 1, 4, 8
    k = np.zeros((H, 5 * B, d))
    k[0, 2 * B:3 * B, 0] = 10.0
    q = np.zeros((B, H, d))
    q[:, 0, 0] = 10.0
    r = orc.block_selection(q, k, [0.5], B)
    np.testing.assert_allclose(r["kbar"][0, 2, 0], 10.0)
    assert r["sel"][0][0].tolist() == [2]


# ---------------------------------------------------------------- S5 sparse
def test_sparse_all_blocks_is_dense_attention():
    rng = np.random.default_rng(7)
    H, B, nkb, nqb, d = 2, 8, 6, 3, 16
    q = rng.standard_normal((nqb * B, H, d))
    k = rng.standard_normal((H, nkb * B, d))
    v = rng.standard_normal((H, nkb * B, d))
    sel = [[np.arange(nkb)] * nqb for _ in range(H)]
    out = orc.sparse_attention(q, k, v, sel, B)
    for h in range(H):
        np.testing.assert_allclose(out[:, h, :], sdpa(q[:, h, :], k[h], v[h]), rtol=1e-10, atol=1e-12)


def test_sparse_single_block_and_order_invariance():
    rng = np.random.default_rng(8)
    H, B, nkb, d = 1, 8, 5, 16
    q = rng.standard_normal((B, H, d))
    k = rng.standard_normal((H, nkb * B, d))
    v = rng.standard_normal((H, nkb * B, d))
    one = orc.sparse_attention(q, k, v, [[np.array([3])]], B)
    np.testing.assert_allclose(one[:, 0, :], sdpa(q[:, 0, :], k[0, 24:32], v[0, 24:32]), rtol=1e-10, atol=1e-12)
    a = orc.sparse_attention(q, k, v, [[np.array([0, 2, 4])]], B)
    b = orc.sparse_attention(q, k, v, [[np.array([4, 0, 2])]], B)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


# ------------------------------------------------------ intra-chunk keys
def test_intra_blocks_hand_example(golden):
    g = golden("hw9_intra_blocks.json")
    k = np.array(g["keys_hist"] + g["keys_chunk"], dtype=np.float64).reshape(1, -1, 1)
    v = np.array(g["vals_hist"] + g["vals_chunk"], dtype=np.float64).reshape(1, -1, 1)
    q = np.array(g["q"], dtype=np.float64).reshape(-1, 1, 1)
    parts = orc.key_parts(len(g["keys_hist"]), g["b_hist"], len(g["keys_chunk"]), g["b_intra"])
    assert parts == [(0, 2), (2, 2), (4, 1), (5, 1)]
    for case in g["cases"]:
        bs = orc.block_selection_parts(q, k, [case["tau"]], g["b_hist"], parts)
        np.testing.assert_allclose(bs["mass"][0, 0], g["mass"], atol=1e-9)
        assert bs["sel"][0][0].tolist() == case["sel"]
        out = orc.sparse_attention_parts(q, k, v, bs["sel"], g["b_hist"], parts)
        np.testing.assert_allclose(out[:, 0, 0], [case["out"]] * 2, rtol=1e-12)


def test_intra_parts_at_the_history_size_reduce_to_uniform_blocks():
    # b_intra == B: the candidates are the uniform B-token blocks of the joined
    # sequence, so selection and attention are the uniform-block ones
    rng = np.random.default_rng(21)
    H, B, d, lh, lq = 2, 8, 16, 40, 16
    q = rng.standard_normal((lq, H, d))
    k = rng.standard_normal((H, lh + lq, d))
    v = rng.standard_normal((H, lh + lq, d))
    tau = [0.7, 0.9]
    parts = orc.key_parts(lh, B, lq, B)
    a = orc.block_selection_parts(q, k, tau, B, parts)
    b = orc.block_selection(q, k, tau, B)
    np.testing.assert_allclose(a["mass"], b["mass"], rtol=1e-12, atol=1e-15)
    for h in range(H):
        for i in range(lq // B):
            assert a["sel"][h][i].tolist() == b["sel"][h][i].tolist()
    np.testing.assert_allclose(orc.sparse_attention_parts(q, k, v, a["sel"], B, parts),
                               orc.sparse_attention(q, k, v, b["sel"], B), rtol=1e-12, atol=1e-14)


def test_intra_parts_all_selected_is_dense_attention_and_means_nest():
    rng = np.random.default_rng(22)
    H, B, bi, d, lh, lq = 2, 8, 4, 16, 24, 16
    q = rng.standard_normal((lq, H, d))
    k = rng.standard_normal((H, lh + lq, d))
    v = rng.standard_normal((H, lh + lq, d))
    parts = orc.key_parts(lh, B, lq, bi)
    assert len(parts) == lh // B + lq // bi
    bs = orc.block_selection_parts(q, k, [1.0, 1.0], B, parts)
    assert all(len(s) == len(parts) for r in bs["sel"] for s in r)
    out = orc.sparse_attention_parts(q, k, v, bs["sel"], B, parts)
    for h in range(H):
        np.testing.assert_allclose(out[:, h, :], sdpa(q[:, h, :], k[h], v[h]), rtol=1e-10, atol=1e-12)
    # a history tile's mean is the mean of its two b_intra halves; a chunk
    # block's mean is the plain mean of its own tokens
    fine = orc.block_means(k, bi)
    pm = orc.part_means(k, parts)
    np.testing.assert_allclose(pm[:, :lh // B], 0.5 * (fine[:, 0:lh // bi:2] + fine[:, 1:lh // bi:2]), rtol=1e-12)
    np.testing.assert_allclose(pm[:, lh // B:], fine[:, lh // bi:], rtol=1e-12)


def test_intra_step_tau_one_is_dense_over_history_and_chunk():
    rng = np.random.default_rng(23)
    H, d, Lp, B, bi, lq, r = 2, 8, 16, 8, 4, 8, 4
    pages_k = [rng.standard_normal((Lp, H, d)) for _ in range(3)]
    pages_v = [rng.standard_normal((Lp, H, d)) for _ in range(3)]
    q = rng.standard_normal((lq, H, d))
    kc = rng.standard_normal((lq, H, d))
    vc = rng.standard_normal((lq, H, d))
    L = 2 * Lp + lq
    e_k = rng.standard_normal((r, L))
    e_v = rng.standard_normal((r, L))
    x = rng.standard_normal((lq, H * d))
    w_g = rng.standard_normal((2 * H, H * d)) * 0.1
    res = orc.hsa_step(q, pages_k, pages_v, e_k, e_v, w_g, x, [1.0, 1.0], 2, B, k_cur=kc, v_cur=vc, b_intra=bi)
    sp = res["sel_pages"]
    for h in range(H):
        keys = np.concatenate([pages_k[sp[0]][:, h], pages_k[sp[1]][:, h], kc[:, h]])
        vals = np.concatenate([pages_v[sp[0]][:, h], pages_v[sp[1]][:, h], vc[:, h]])
        np.testing.assert_allclose(res["o_sp"][:, h], sdpa(q[:, h], keys, vals), rtol=1e-10, atol=1e-12)
        # the linear branch projects the joined sequence
        np.testing.assert_allclose(res["lin"]["o_lin"][:, h], sdpa(q[:, h], e_k @ keys, e_v @ vals),
                                   rtol=1e-10, atol=1e-12)


# ------------------------------------------------------------------ S6 fuse
def test_gate_hand_example(golden):
    g = golden("hw4_gate.json")
    w = np.log(np.array(g["w_g_is_ln_of"], dtype=np.float64))
    gl, gs = orc.gates(np.array(g["x"]), w, 1)
    assert abs(gl[0, 0] - g["g_lin"]) < 1e-15 and abs(gs[0, 0] - g["g_sp"]) < 1e-15
    out = orc.fuse(np.array(g["x"]), w, np.array(g["o_lin"]), np.array(g["o_sp"]))
    np.testing.assert_allclose(out, g["out"], rtol=0, atol=1e-14)


def test_gate_limits():
    rng = np.random.default_rng(9)
    Lq, H, d = 5, 3, 4
    ol = rng.standard_normal((Lq, H, d))
    osp = rng.standard_normal((Lq, H, d))
    one, zero = np.ones((Lq, H)), np.zeros((Lq, H))
    np.testing.assert_array_equal(orc.fuse_with(zero, one, ol, osp), osp)
    np.testing.assert_array_equal(orc.fuse_with(one, zero, ol, osp), ol)
    x = rng.standard_normal((Lq, H * d))
    np.testing.assert_allclose(orc.fuse(x, np.zeros((2 * H, H * d)), ol, osp), 0.5 * (ol + osp), atol=1e-15)


# ---------------------------------------------------------------- whole step
def test_tiny_step_tau_one_is_dense_and_gates_reduce():
    w = Workload(C0)
    s = w.small_inputs()
    pk, pv = w.pages()
    r = orc.hsa_step(s["q"], pk, pv, s["e_k"], s["e_v"], s["w_g"], s["x"],
                     np.ones(C0.n_heads), C0.n_sel_pages, C0.block)
    for h in range(C0.n_heads):
        np.testing.assert_allclose(r["o_sp"][:, h, :], sdpa(s["q"][:, h, :], r["k_act"][h], r["v_act"][h]),
                                   rtol=1e-10, atol=1e-12)
    assert r["sel_pages"].tolist() == w.plant.target_pages.tolist()


def test_generator_shapes_and_determinism():
    w1, w2 = Workload(M2), Workload(M2)
    np.testing.assert_array_equal(w1.page_k(3), w2.page_k(3))
    np.testing.assert_array_equal(w1.q(), w2.q())
    assert w1.e_k().shape == (M2.rank, M2.active_tokens)
    assert w1.w_g().shape == (2 * M2.n_heads, M2.model_dim)


def test_imbalance_generator_plants_few_blocks_in_peaked_heads():
    cfg = M5
    w = Workload(cfg)
    s = w.small_inputs()
    pk, pv = w.pages()
    r = orc.hsa_step(s["q"], pk, pv, s["e_k"], s["e_v"], s["w_g"], s["x"], s["tau"], cfg.n_sel_pages, cfg.block)
    c = r["blocks"]["counts"]
    assert np.all(c[cfg.uniform_heads:] == cfg.hot_per_row)
    assert np.all(c[:cfg.uniform_heads] > cfg.n_kblocks // 2)
    for h in range(cfg.uniform_heads, cfg.n_heads):
        for i in range(cfg.n_qblocks):
            assert r["block_sel"][h][i].tolist() == sorted(w.plant.hot[h, i].tolist())


@pytest.mark.slow
def test_full_shape_planted_pages_are_retrieved():
    w = Workload(C1)
    q = w.q()
    qbar = orc.mean_over_tokens(q)
    kbars = np.stack([orc.mean_over_tokens(w.page_k(j)) for j in range(C1.n_pages)])
    a = orc.page_scores(qbar, kbars)
    sel, tie = orc.select_pages(a, C1.n_sel_pages)
    assert sel.tolist() == w.plant.target_pages.tolist() and not tie
