"""The C-ABI library on the host: it loads, exports every declared symbol, and
its host-side validation rejects bad arguments before launching anything.
No kernel is launched here (no GPU needed)."""
import ctypes
import glob
import os
import re

import pytest

from sparse_linear_attention_hsa_amd import _lib
from sparse_linear_attention_hsa_amd._lib import Geom

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(hsa_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def c1_geom(**kw):
    g = dict(n_heads=12, head_dim=128, frame_h=30, frame_w=52, frames_per_page=8, query_frames=4,
             tile_t=4, tile_h=6, tile_w=4, n_sel_pages=4, rank=256, dtype=_lib.HSA_BF16)
    g.update(kw)
    return Geom(**g)


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(_lib.SIGNATURES), names
    for n in names:
        assert hasattr(lib, n)
    assert lib.hsa_abi_version() == 3


def test_geometry_validation(lib):
    ok = c1_geom()
    assert lib.hsa_geom_check(ctypes.byref(ok)) == 0
    assert lib.hsa_geom_check(None) == 1
    bad = {
        "dtype": (dict(dtype=7), 3),
        "head_dim": (dict(head_dim=96), 4),
        "rank": (dict(rank=0), 4),
        "rank_big": (dict(rank=512), 4),
        "tile_not_dividing": (dict(tile_h=8), 2),         # 8 does not divide 30
        "tile_t": (dict(tile_t=3), 2),
        "block_not_16": (dict(tile_t=1, tile_h=6, tile_w=4), 2),   # B = 24
        "block_too_big": (dict(tile_t=4, tile_h=6, tile_w=13, frame_w=52), 2),  # B = 312
        "zero_frames": (dict(query_frames=0), 2),
        "zero_pages": (dict(n_sel_pages=0), 4),
        "too_many_heads": (dict(n_heads=33), 4),
    }
    for name, (kw, rc) in bad.items():
        g = c1_geom(**kw)
        assert lib.hsa_geom_check(ctypes.byref(g)) == rc, name
        assert lib.hsa_workspace_bytes(ctypes.byref(g), 16) == 0, name


def test_intra_chunk_geometry(lib):
    # B = 96: splits 1, 2 and 3 give 96-, 48- and 32-token key blocks
    for sp in (1, 2, 3):
        g = c1_geom(intra_split=sp)
        assert lib.hsa_geom_check(ctypes.byref(g)) == 0, sp
        assert lib.hsa_workspace_bytes(ctypes.byref(g), 16) > lib.hsa_workspace_bytes(ctypes.byref(c1_geom()), 16)
    bad = {
        "negative": (dict(intra_split=-1), 4),
        "above_max": (dict(intra_split=_lib.HSA_MAX_INTRA_SPLIT + 1), 4),
        "key_block_not_16": (dict(intra_split=4), 2),                # 96 / 4 = 24
        "not_dividing": (dict(tile_t=4, tile_h=2, tile_w=4, intra_split=3), 2),  # 32 / 3
        "too_many_key_blocks": (dict(intra_split=3, n_sel_pages=5), 2),          # (62400 + 6240) / 32 > 2048
    }
    for name, (kw, rc) in bad.items():
        g = c1_geom(**kw)
        assert lib.hsa_geom_check(ctypes.byref(g)) == rc, name
        assert lib.hsa_workspace_bytes(ctypes.byref(g), 16) == 0, name
    fake = ctypes.c_void_p(0x1000)
    pages = (ctypes.c_void_p * 16)(*([0x1000] * 16))
    intra, plain = c1_geom(intra_split=2), c1_geom()
    ga = lib.hsa_gather_active
    # the chunk's keys and values: required with intra keys, refused without
    assert ga(ctypes.byref(intra), pages, pages, 16, fake, None, fake, fake, fake, None, None) == 1
    assert ga(ctypes.byref(intra), pages, pages, 16, fake, fake, None, fake, fake, None, None) == 1
    assert ga(ctypes.byref(plain), pages, pages, 16, fake, fake, fake, fake, fake, None, None) == 4
    assert ga(ctypes.byref(intra), pages, pages, 200, fake, fake, fake, fake, fake, None, None) == 4
    # the plain gather does not take a geometry with intra keys
    assert lib.hsa_gather_pages(ctypes.byref(intra), pages, pages, 16, fake, fake, fake, None, None) == 4


def test_paged_entry_points_reject_bad_arguments(lib):
    g, intra = c1_geom(), c1_geom(intra_split=2)
    fake = ctypes.c_void_p(0x1000)
    pages = (ctypes.c_void_p * 16)(*([0x1000] * 16))
    null_pages = (ctypes.c_void_p * 16)()
    big = 1 << 40
    # page layout: NULL buffers
    assert lib.hsa_page_prepare(ctypes.byref(g), None, fake, fake, fake, None, None) == 1
    assert lib.hsa_page_prepare(ctypes.byref(g), fake, fake, fake, None, None, None) == 1
    assert lib.hsa_page_prepare(ctypes.byref(intra), None, fake, fake, fake, None, None) == 1
    # the chunk's page-format buffers: only with intra-chunk keys, ceil(Lq / Lp) of them
    assert lib.hsa_chunk_page_count(ctypes.byref(g)) == 0
    assert lib.hsa_chunk_page_count(ctypes.byref(intra)) == 1  # Lq = Lp / 2
    assert lib.hsa_chunk_page_count(ctypes.byref(c1_geom(intra_split=2, frames_per_page=4, query_frames=12))) == 3
    assert lib.hsa_chunk_page_count(None) == 0
    outs = (ctypes.c_void_p * 1)(0x1000)
    null_outs = (ctypes.c_void_p * 1)()
    cp = lib.hsa_chunk_prepare
    assert cp(ctypes.byref(g), fake, fake, outs, outs, None, None) == 4
    assert cp(ctypes.byref(intra), None, fake, outs, outs, None, None) == 1
    assert cp(ctypes.byref(intra), fake, fake, null_outs, outs, None, None) == 1
    assert cp(ctypes.byref(intra), fake, fake, outs, None, None, None) == 1
    # block means of the selected pages: NULL entries, page counts
    gm = lib.hsa_gather_block_means
    assert gm(ctypes.byref(g), null_pages, 16, fake, fake, None) == 1
    assert gm(ctypes.byref(g), pages, 16, None, fake, None) == 1
    assert gm(ctypes.byref(g), pages, 3, fake, fake, None) == 4
    assert gm(ctypes.byref(g), pages, 200, fake, fake, None) == 4
    assert gm(ctypes.byref(intra), null_pages, 16, fake, fake, None) == 1
    # the same three over device tables: NULL tables, bank limits
    big_bank = _lib.HSA_MAX_BANK_PAGES
    assert lib.hsa_gather_block_means_devtab(ctypes.byref(g), None, 16, fake, fake, None) == 1
    assert lib.hsa_gather_block_means_devtab(ctypes.byref(g), fake, big_bank + 1, fake, fake, None) == 4
    assert lib.hsa_gather_block_means_devtab(ctypes.byref(g), fake, 3, fake, fake, None) == 4
    lpd = lib.hsa_linear_branch_paged_devtab
    assert lpd(ctypes.byref(g), fake, None, fake, 16, fake, fake, fake, fake, fake, fake, 0, fake, big, None) == 1
    assert lpd(ctypes.byref(g), fake, fake, fake, big_bank + 1, fake, fake, fake, fake, fake, fake, 0, fake, big,
               None) == 4
    assert lpd(ctypes.byref(g), fake, fake, fake, 300, fake, fake, fake, fake, fake, fake, 0, fake, 16, None) == 5
    spd = lib.hsa_sparse_attn_paged_devtab
    assert spd(ctypes.byref(g), fake, fake, None, 16, fake, fake, fake, fake, fake, big, None, None, None) == 1
    assert spd(ctypes.byref(g), fake, fake, fake, big_bank + 1, fake, fake, fake, fake, fake, big, None, None,
               None) == 4
    assert spd(ctypes.byref(g), fake, fake, fake, 300, fake, fake, fake, fake, fake, 16, None, None, None) == 5
    # linear branch over pages: NULL pages (unless the projection is reused), counts, flags, workspace
    lp = lib.hsa_linear_branch_paged
    assert lp(ctypes.byref(g), fake, null_pages, pages, 16, fake, fake, fake, fake, fake, fake, 0, fake, big, None) == 1
    assert lp(ctypes.byref(g), fake, pages, pages, 16, None, fake, fake, fake, fake, fake, 0, fake, big, None) == 1
    assert lp(ctypes.byref(g), fake, pages, pages, 3, fake, fake, fake, fake, fake, fake, 0, fake, big, None) == 4
    assert lp(ctypes.byref(g), fake, pages, pages, 16, fake, fake, fake, fake, fake, fake, 3, fake, big, None) == 4
    assert lp(ctypes.byref(g), fake, pages, pages, 16, fake, fake, fake, fake, fake, fake, 0, fake, 16, None) == 5
    # with intra-chunk keys the paged calls get as far as the workspace check;
    # the history / chunk projection modes need them
    assert lp(ctypes.byref(intra), fake, pages, pages, 16, fake, fake, fake, fake, fake, fake, 0, fake, 16, None) == 5
    assert lp(ctypes.byref(g), fake, pages, pages, 16, fake, fake, fake, fake, fake, fake,
              _lib.HSA_LIN_HISTORY_PROJ, fake, big, None) == 4
    # sparse branch over pages
    sp = lib.hsa_sparse_attn_paged
    assert sp(ctypes.byref(g), fake, pages, null_pages, 16, fake, fake, fake, fake, fake, big, None, None, None) == 1
    assert sp(ctypes.byref(g), fake, pages, pages, 16, None, fake, fake, fake, fake, big, None, None, None) == 1
    assert sp(ctypes.byref(g), fake, pages, pages, 2, fake, fake, fake, fake, fake, big, None, None, None) == 4
    assert sp(ctypes.byref(g), fake, pages, pages, 16, fake, fake, fake, fake, fake, 16, None, None, None) == 5
    assert sp(ctypes.byref(intra), fake, pages, pages, 16, fake, fake, fake, fake, fake, 16, None, None, None) == 5


def test_workspace_sizes(lib):
    g = c1_geom()
    a = lib.hsa_workspace_bytes(ctypes.byref(g), 16)
    b = lib.hsa_workspace_bytes(ctypes.byref(g), 120)
    assert 0 < a <= b
    assert lib.hsa_workspace_bytes(ctypes.byref(g), _lib.HSA_MAX_BANK_PAGES + 1) == 0
    # the linear branch's own workspace: smaller than the full one, enough for
    # the linear branch (its check passes with exactly this size, fails below)
    lin = lib.hsa_linear_workspace_bytes(ctypes.byref(g))
    assert 0 < lin < a
    assert lib.hsa_linear_workspace_bytes(ctypes.byref(c1_geom(dtype=9))) == 0
    fake = ctypes.c_void_p(0x1000)
    assert lib.hsa_linear_branch(ctypes.byref(g), fake, fake, fake, fake, fake, fake, fake, fake, 8, fake,
                                 lin - 1, None) == 4  # bad flags still reported first
    assert lib.hsa_linear_branch(ctypes.byref(g), fake, fake, fake, fake, fake, fake, fake, fake, 0, fake,
                                 lin - 1, None) == 5


def test_entry_points_reject_bad_arguments_before_launch(lib):
    g = c1_geom()
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first
    pages = (ctypes.c_void_p * 16)(*([0x1000] * 16))
    null_pages = (ctypes.c_void_p * 16)()
    ws_small = ctypes.c_size_t(16)
    # score: NULL q, NULL page without cache, bad page counts, short workspace
    assert lib.hsa_score_pages(ctypes.byref(g), None, pages, None, 16, fake, fake, fake, 1 << 40, None) == 1
    assert lib.hsa_score_pages(ctypes.byref(g), fake, null_pages, None, 16, fake, fake, fake, 1 << 40, None) == 1
    assert lib.hsa_score_pages(ctypes.byref(g), fake, pages, None, 3, fake, fake, fake, 1 << 40, None) == 4
    assert lib.hsa_score_pages(ctypes.byref(g), fake, pages, None, 0, fake, fake, fake, 1 << 40, None) == 4
    assert lib.hsa_score_pages(ctypes.byref(g), fake, pages, None, 16, fake, fake, fake, ws_small, None) == 5
    assert lib.hsa_score_pages(ctypes.byref(g), fake, pages, None, 16, fake, fake, None, 1 << 40, None) == 5
    # chunk-restricted scoring: NULL chunk arrays, k_chunks out of range or
    # not dividing K_p (4 here), then the page checks of plain scoring
    sc = lib.hsa_score_chunk_pages
    assert sc(ctypes.byref(g), fake, pages, None, 16, None, fake, 1, fake, fake, fake, 1 << 40, None) == 1
    assert sc(ctypes.byref(g), fake, pages, None, 16, fake, None, 1, fake, fake, fake, 1 << 40, None) == 1
    for k in (0, 3, 5, -1):
        assert sc(ctypes.byref(g), fake, pages, None, 16, fake, fake, k, fake, fake, fake, 1 << 40, None) == 4, k
    assert sc(ctypes.byref(g), fake, null_pages, None, 16, fake, fake, 2, fake, fake, fake, 1 << 40, None) == 1
    assert sc(ctypes.byref(g), fake, pages, None, 16, fake, fake, 2, fake, fake, fake, ws_small, None) == 5
    # prompt-level retrieval: NULL arrays, sizes, k above the chunk count
    rc = lib.hsa_retrieve_chunks
    assert rc(None, fake, 8, 16, 1, fake, fake, None) == 1
    assert rc(fake, fake, 8, 16, 1, None, fake, None) == 1
    assert rc(fake, fake, 0, 16, 1, fake, fake, None) == 4
    assert rc(fake, fake, _lib.HSA_MAX_CHUNKS + 1, 16, 1, fake, fake, None) == 4
    assert rc(fake, fake, 8, 0, 1, fake, fake, None) == 4
    assert rc(fake, fake, 8, 16, 9, fake, fake, None) == 4
    assert rc(fake, fake, 8, 16, 0, fake, fake, None) == 4
    # gather: NULL page entry, NULL outputs
    assert lib.hsa_gather_pages(ctypes.byref(g), null_pages, pages, 16, fake, fake, fake, None, None) == 1
    assert lib.hsa_gather_pages(ctypes.byref(g), pages, pages, 16, fake, None, fake, None, None) == 1
    assert lib.hsa_gather_pages(ctypes.byref(g), pages, pages, 200, fake, fake, fake, None, None) == 4
    # linear: bad flags, missing projections, short workspace
    assert lib.hsa_linear_branch(ctypes.byref(g), fake, fake, fake, fake, fake, fake, fake, fake, 3, fake, 1 << 40, None) == 4
    assert lib.hsa_linear_branch(ctypes.byref(g), fake, fake, fake, fake, fake, fake, fake, fake, 8, fake, 1 << 40, None) == 4
    assert lib.hsa_linear_branch(ctypes.byref(g), fake, fake, fake, None, fake, fake, fake, fake, 0, fake, 1 << 40, None) == 1
    assert lib.hsa_linear_branch(ctypes.byref(g), fake, fake, fake, fake, fake, fake, fake, fake, 0, fake, ws_small, None) == 5
    # select: neither k_act nor block means
    assert lib.hsa_block_select(ctypes.byref(g), fake, None, None, fake, fake, fake, None, fake, 1 << 40, None) == 1
    assert lib.hsa_block_select(ctypes.byref(g), fake, fake, None, fake, fake, fake, None, fake, ws_small, None) == 5
    # sparse
    assert lib.hsa_sparse_attn(ctypes.byref(g), fake, fake, None, fake, fake, fake, fake, 1 << 40, None) == 1
    assert lib.hsa_sparse_attn(ctypes.byref(g), fake, fake, fake, fake, fake, fake, fake, ws_small, None) == 5
    # fuse: x without weights, neither x nor override
    assert lib.hsa_fuse(ctypes.byref(g), fake, None, None, fake, fake, fake, None) == 1
    assert lib.hsa_fuse(ctypes.byref(g), None, None, None, fake, fake, fake, None) == 1
    # geometry errors win before anything else
    bad = c1_geom(dtype=9)
    assert lib.hsa_fuse(ctypes.byref(bad), fake, fake, None, fake, fake, fake, None) == 3
    # the matrix-core probe: NULL output, workgroup and round counts out of range
    assert lib.hsa_probe_mfma_bf16(256, 10, None, None, None, None) == 1
    assert lib.hsa_probe_mfma_bf16(0, 10, fake, None, None, None) == 4
    assert lib.hsa_probe_mfma_bf16(70000, 10, fake, None, None, None) == 4
    assert lib.hsa_probe_mfma_bf16(256, 0, fake, None, None, None) == 4
    # the copy probe: NULL pointers, sizes or alignments it does not take
    assert lib.hsa_probe_hbm_copy(None, fake, 1 << 20, None, None, None) == 1
    assert lib.hsa_probe_hbm_copy(fake, fake, 0, None, None, None) == 4
    assert lib.hsa_probe_hbm_copy(fake, fake, 100, None, None, None) == 4
    assert lib.hsa_probe_hbm_copy(ctypes.c_void_p(0x1004), fake, 1 << 20, None, None, None) == 4


def test_status_strings(lib):
    for rc, name in _lib.RC_NAMES.items():
        assert lib.hsa_rc_string(rc).decode().startswith(name)


def test_noalloc_select_rejects_before_launching(lib):
    """The workspace-free block selection checks its arguments and the size
    of its fixed scratch on the host, before touching the device."""
    big = c1_geom(n_heads=24, n_sel_pages=8)    # selection scratch about 20 MB
    assert lib.hsa_geom_check(ctypes.byref(big)) == 0
    p = ctypes.c_void_p(256)                    # never dereferenced: the call returns first
    assert lib.hsa_block_select_noalloc(ctypes.byref(big), p, p, p, p, p, p, None, None) == 5
    assert lib.hsa_block_select_noalloc(ctypes.byref(c1_geom()), None, p, p, p, p, p, None, None) == 1
    assert lib.hsa_block_select_noalloc(ctypes.byref(c1_geom()), p, None, None, p, p, p, None, None) == 1
    assert lib.hsa_block_select_noalloc(ctypes.byref(c1_geom(dtype=7)), p, p, p, p, p, p, None, None) == 3
    assert _lib.HSA_NOALLOC_SCRATCH_BYTES == 16 << 20


def test_bank_limits(lib):
    """Host page tables stop at HSA_MAX_PAGES, device page tables at
    HSA_MAX_BANK_PAGES; the workspace is sized up to the latter.  Every
    rejection happens on the host, before anything is launched."""
    g = c1_geom()
    gp = ctypes.byref(g)
    assert lib.hsa_workspace_bytes(gp, _lib.HSA_MAX_BANK_PAGES) >= lib.hsa_workspace_bytes(gp, 256) >= \
        lib.hsa_workspace_bytes(gp, 16) > 0
    assert lib.hsa_workspace_bytes(gp, _lib.HSA_MAX_BANK_PAGES + 1) == 0
    p = ctypes.c_void_p(256)  # never dereferenced: each call returns before launching
    ws_big = lib.hsa_workspace_bytes(gp, _lib.HSA_MAX_BANK_PAGES)
    n_host = _lib.HSA_MAX_PAGES + 1
    host_tab = (ctypes.c_void_p * n_host)(*([256] * n_host))
    assert lib.hsa_score_pages(gp, p, host_tab, p, n_host, p, p, p, ws_big, None) == 4
    assert lib.hsa_gather_active(gp, host_tab, host_tab, n_host, p, None, None, p, p, None, None) == 4
    for n, rc in ((_lib.HSA_MAX_BANK_PAGES + 1, 4), (0, 4), (3, 4)):  # 3 < K_p = 4
        assert lib.hsa_score_pages_devtab(gp, p, p, p, n, p, p, p, ws_big, None) == rc, n
        assert lib.hsa_gather_active_devtab(gp, p, p, n, p, None, None, p, p, None, None) == rc, n
        assert lib.hsa_score_chunk_pages_devtab(gp, p, p, p, n, p, p, 1, p, p, p, ws_big, None) == rc, n
    assert lib.hsa_score_pages_devtab(gp, p, None, p, 256, p, p, p, ws_big, None) == 1
    assert lib.hsa_gather_active_devtab(gp, None, p, 256, p, None, None, p, p, None, None) == 1
    assert lib.hsa_score_chunk_pages_devtab(gp, p, p, p, 256, None, p, 1, p, p, p, ws_big, None) == 1
    small = lib.hsa_workspace_bytes(gp, 256) - 1
    assert lib.hsa_score_pages_devtab(gp, p, p, p, 256, p, p, p, small, None) == 5


def test_history_and_chunk_modes_need_intra_chunk_keys(lib):
    """The history/chunk split of the linear branch and the chunk-only gather
    exist only with intra-chunk keys; one linear mode at a time."""
    p = ctypes.c_void_p(256)
    plain, intra = c1_geom(), c1_geom(intra_split=2)
    ws = lib.hsa_workspace_bytes(ctypes.byref(intra), 16)
    for flags in (_lib.HSA_LIN_HISTORY_PROJ, _lib.HSA_LIN_CHUNK_PROJ):
        assert lib.hsa_linear_branch(ctypes.byref(plain), p, p, p, p, p, p, p, p, flags, p, ws, None) == 4
    for flags in (_lib.HSA_LIN_HISTORY_PROJ | _lib.HSA_LIN_CHUNK_PROJ, _lib.HSA_LIN_REUSE_PROJ | _lib.HSA_LIN_CHUNK_PROJ,
                  _lib.HSA_LIN_PROJ_ONLY | _lib.HSA_LIN_HISTORY_PROJ, 16):
        assert lib.hsa_linear_branch(ctypes.byref(intra), p, p, p, p, p, p, p, p, flags, p, ws, None) == 4, flags
    # the history projection needs no queries or output; the chunk mode needs both
    assert lib.hsa_linear_branch(ctypes.byref(intra), p, None, p, p, p, p, p, p, _lib.HSA_LIN_HISTORY_PROJ, p, ws,
                                 None) == 1
    assert lib.hsa_linear_branch(ctypes.byref(intra), None, p, p, p, p, p, p, p, _lib.HSA_LIN_CHUNK_PROJ, p, ws,
                                 None) == 1
    assert lib.hsa_linear_branch(ctypes.byref(intra), p, p, p, p, p, p, p, p, _lib.HSA_LIN_CHUNK_PROJ, p,
                                 lib.hsa_linear_workspace_bytes(ctypes.byref(intra)) - 1, None) == 5
    assert lib.hsa_gather_chunk(ctypes.byref(plain), p, p, p, p, None, None) == 4
    assert lib.hsa_gather_chunk(ctypes.byref(intra), None, p, p, p, None, None) == 1
