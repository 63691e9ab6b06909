"""hsa_sparse_attn on block lists a caller writes (not hsa_block_select's):
ids outside [0, nKB) are skipped, a count is clamped to [0, nKB], and a row
with no valid block gets zeros, also in rows the plan splits into segments
(WorldAttention paper, section 3.3 "Sparse branch": attention over exactly
the tokens of the listed blocks).  Against the float64 oracle on the valid
ids of every row."""
import numpy as np
import pytest
import torch

from oracle import hsa_oracle as orc
from sparse_linear_attention_hsa_amd import ops
from synth import M1, M3

from gpu_harness import Run, assert_close, host, untile_v

pytestmark = pytest.mark.gpu


def _lists(cfg, rng):
    """Per (head, query block): the list handed to the kernel, and its valid ids."""
    H, nqb, nkb = cfg.n_heads, cfg.n_qblocks, cfg.n_key_blocks
    given, valid = [], []
    for h in range(H):
        for i in range(nqb):
            kind = (h * nqb + i) % 6
            if kind == 0:  # no block
                ids = []
            elif kind == 1:  # every id invalid (70 of them: a row the plan splits, every segment masked)
                ids = [(-1 - j) if j % 2 else nkb + j for j in range(70)]
            elif kind == 2:  # one valid id between invalid ones
                ids = [-1, int(rng.integers(nkb)), 10 ** 6]
            elif kind == 3:  # every block, listed under a count above nKB (clamped)
                ids = list(range(nkb))
            else:  # a long random set (split rows) with invalid ids mixed in
                ids = sorted(rng.choice(nkb, size=min(nkb, 40 + 13 * kind), replace=False).tolist())
                for pos in (3, 17, 29):
                    ids.insert(min(pos, len(ids)), -1 if pos % 2 else nkb + pos)
            ids = ids[:nkb]  # a row of blk_idx holds nKB entries
            given.append(ids)
            valid.append(np.array([j for j in ids if 0 <= j < nkb], dtype=np.int64))
    return given, valid


@pytest.mark.parametrize("cfg", [M1, M3], ids=lambda c: c.name)
def test_caller_block_lists(cfg):
    rng = np.random.default_rng(77)
    r = Run(cfg)
    st = r.run()  # the gathered active buffer
    H, nqb, nkb = cfg.n_heads, cfg.n_qblocks, cfg.n_key_blocks
    given, valid = _lists(cfg, rng)
    cnt = np.zeros((H, nqb), dtype=np.int32)
    idx = np.full((H, nqb, nkb), -1, dtype=np.int32)
    for row, ids in enumerate(given):
        h, i = divmod(row, nqb)
        idx[h, i, :len(ids)] = ids
        cnt[h, i] = nkb + 5 if row % 6 == 3 else len(ids)  # (the first count is clamped to nKB)
    print(f"\n[sparse inputs] {cfg.name}: {H * nqb} rows, longest valid list "
          f"{max(len(v) for v in valid)} of {nkb} blocks", flush=True)
    o_sp = torch.full_like(st.o_sp, float("nan"))
    ops.hsa_sparse_attn(st.geom, r.q, st.k_act, st.v_act, torch.from_numpy(cnt).cuda(), torch.from_numpy(idx).cuda(),
                        o_sp, st.ws)
    torch.cuda.synchronize()
    got = host(o_sp)
    q = r.np["q"].astype(np.float64)
    k, v = host(st.k_act), untile_v(host(st.v_act))
    B = cfg.block
    want = np.zeros_like(got)
    for row, ids in enumerate(valid):
        h, i = divmod(row, nqb)
        if len(ids):
            want[i * B:(i + 1) * B, h] = orc.sparse_row(q[i * B:(i + 1) * B, h], k[h], v[h], ids, B)
    empty = [row for row, ids in enumerate(valid) if len(ids) == 0]
    for row in empty:
        h, i = divmod(row, nqb)
        assert np.all(got[i * B:(i + 1) * B, h] == 0.0), f"row {row} has no valid block: zeros"
    assert_close("o_sp", got, want, cfg)


@pytest.mark.parametrize("cfg", [M1, M3], ids=lambda c: c.name)
def test_caller_page_selection_is_clamped(cfg):
    """A page selection a caller writes, with ids below 0 and past the bank:
    the gather (host and device page tables) and, over laid-out pages, the
    block-means gather clamp them to the first and last page, as documented."""
    from sparse_linear_attention_hsa_amd.ops import DeviceTable
    r = Run(cfg)
    st = r.step
    n, kp = cfg.n_pages, cfg.n_sel_pages
    raw = [-7, n + 3] + list(range(1, kp - 1))
    clamped = np.clip(np.array(raw[:kp]), 0, n - 1)
    sel = torch.tensor(raw[:kp], dtype=torch.int32, device="cuda")
    print(f"\n[page selection] {cfg.name}: {raw[:kp]} -> pages {clamped.tolist()}", flush=True)
    want_k = orc.gather_active(r.pk_np, clamped)
    want_v = orc.gather_active(r.pv_np, clamped)
    for tables in ((r.pk, r.pv), (DeviceTable(r.pk), DeviceTable(r.pv))):
        st.k_act.zero_()
        st.v_act.zero_()
        if isinstance(tables[0], DeviceTable):
            ops.hsa_gather_active(st.geom, tables[0], tables[1], sel, None, None, st.k_act, st.v_act, st.kblk_mean)
        else:
            ops.hsa_gather_pages(st.geom, tables[0], tables[1], sel, st.k_act, st.v_act, st.kblk_mean)
        torch.cuda.synchronize()
        assert np.array_equal(host(st.k_act), want_k)
        assert np.array_equal(untile_v(host(st.v_act)), want_v)
    # over laid-out pages: the block means of the same (clamped) pages
    kblk_gathered = st.kblk_mean.clone()
    prepared = st.prepare_pages(r.pk, r.pv)
    st.kblk_mean.zero_()
    ops.hsa_gather_block_means(st.geom, prepared[2], sel, st.kblk_mean)
    torch.cuda.synchronize()
    assert torch.equal(st.kblk_mean, kblk_gathered)
