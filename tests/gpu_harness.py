"""Shared helpers of the GPU tests: upload seeded inputs, run the HIP path,
re-layout its outputs for comparison, and compare with the oracle.

Test infrastructure: it may use the oracle, and the oracle never sees a
value produced by the HIP path except a selection that the oracle has first
checked to be valid (a near-tie, where several answers are correct)."""
from __future__ import annotations

import numpy as np
import torch

from oracle import hsa_oracle as orc
from sparse_linear_attention_hsa_amd.ops import make_geom
from sparse_linear_attention_hsa_amd.step import HsaStep
from synth import Config, Workload

# Output tolerances: max-abs and relative L2 against the float64 oracle.
# bf16 workloads: the required bound (max-abs 2e-2, relative L2 1e-2).  f32 workloads: derived from float32
# arithmetic (operand rounding 2^-24, accumulation over <= 10^4 terms).
TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-4, 1e-5)}


def geom_of(cfg: Config):
    return make_geom(cfg.n_heads, cfg.head_dim, cfg.frame_h, cfg.frame_w, cfg.frames_per_page,
                     cfg.query_frames, cfg.tile, cfg.n_sel_pages, cfg.rank, cfg.dtype, cfg.intra_split)


def torch_dtype(cfg: Config):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def dev(a: np.ndarray, cfg: Config, device="cuda") -> torch.Tensor:
    """Exact upload of float32 arrays whose values are representable in the config dtype."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch_dtype(cfg)).to(device)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64) if t.is_floating_point() else t.cpu().numpy()


def untile_v(v_act: np.ndarray) -> np.ndarray:
    """[H][L/16][d][16] granule layout -> [H][L][d]."""
    H, G, d, _ = v_act.shape
    return v_act.transpose(0, 1, 3, 2).reshape(H, G * 16, d)


def max_abs_rel_l2(got: np.ndarray, want: np.ndarray):
    diff = np.asarray(got, np.float64) - np.asarray(want, np.float64)
    mx = float(np.max(np.abs(diff))) if diff.size else 0.0
    den = float(np.linalg.norm(want))
    rl2 = float(np.linalg.norm(diff) / den) if den > 0 else float(np.linalg.norm(diff))
    return mx, rl2


def assert_close(name: str, got, want, cfg: Config, tol=None):
    ma, rl = tol if tol is not None else TOL[cfg.dtype]
    mx, rl2 = max_abs_rel_l2(got, want)
    assert mx <= ma and rl2 <= rl, f"{name}: max-abs {mx:.3e} (<= {ma}), rel-L2 {rl2:.3e} (<= {rl})"
    return mx, rl2


class Run:
    """Inputs of one workload on the GPU plus the HIP step over them."""

    def __init__(self, cfg: Config, layer: int = 0, step_idx: int = 0, tau=None):
        self.cfg = cfg
        self.w = Workload(cfg, layer)
        s = self.w.small_inputs(step_idx)
        self.np = s
        if tau is not None:
            self.np["tau"] = np.asarray(tau, dtype=np.float32)
        self.pk_np, self.pv_np = self.w.pages()
        self.q = dev(s["q"], cfg)
        self.x = dev(s["x"], cfg)
        self.e_k = dev(s["e_k"], cfg)
        self.e_v = dev(s["e_v"], cfg)
        self.w_g = dev(s["w_g"], cfg)
        self.tau = torch.from_numpy(self.np["tau"]).cuda()
        self.pk = [dev(p, cfg) for p in self.pk_np]
        self.pv = [dev(p, cfg) for p in self.pv_np]
        self.k_cur = dev(s["k_cur"], cfg) if cfg.intra_split else None
        self.v_cur = dev(s["v_cur"], cfg) if cfg.intra_split else None
        self.geom = geom_of(cfg)
        self.step = HsaStep(self.geom, cfg.n_pages)

    def run(self, concurrent: bool = True, indexed: bool = False):
        self.step.run(self.q, self.pk, self.pv, self.e_k, self.e_v, self.w_g, self.x, self.tau,
                      concurrent=concurrent, indexed=indexed, k_cur=self.k_cur, v_cur=self.v_cur)
        torch.cuda.synchronize()
        return self.step

    def oracle(self, sel_pages=None, block_sel=None):
        s = self.np
        intra = {}
        if self.cfg.intra_split:
            intra = dict(k_cur=s["k_cur"], v_cur=s["v_cur"], b_intra=self.cfg.key_block)
        return orc.hsa_step(s["q"], self.pk_np, self.pv_np, s["e_k"], s["e_v"], s["w_g"], s["x"], s["tau"],
                            self.cfg.n_sel_pages, self.cfg.block, sel_pages=sel_pages, block_sel=block_sel,
                            **intra)


def gpu_block_lists(step: HsaStep):
    cnt = step.blk_count.cpu().numpy()
    idx = step.blk_idx.cpu().numpy()
    H, nqb = cnt.shape
    return [[idx[h, i, :cnt[h, i]].astype(np.int64) for i in range(nqb)] for h in range(H)], cnt, idx


def check_block_selection(ref_blocks, gpu_lists, tau):
    """Exact match on unflagged rows; validity on rows the oracle flagged as near-ties.
    Returns the number of flagged rows where the GPU picked another valid set."""
    H = len(gpu_lists)
    differ = 0
    for h in range(H):
        for i in range(len(gpu_lists[h])):
            want = ref_blocks["sel"][h][i]
            got = gpu_lists[h][i]
            if np.array_equal(got, want):
                continue
            assert ref_blocks["flags"][h, i], f"block selection differs at unflagged row (h={h}, i={i})"
            assert orc.valid_block_selection(ref_blocks["mass"][h, i], got, tau[h]), f"invalid selection at tie (h={h}, i={i})"
            differ += 1
    return differ


def key_blocks_of(cands, n_tiles: int, grp: int) -> np.ndarray:
    """Candidate ids (history tiles j < n_tiles, then the chunk's blocks) ->
    the key-block ids the library lists: tile j is key blocks grp*j ..
    grp*j+grp-1, chunk candidate j is key block grp*n_tiles + j - n_tiles."""
    out = []
    for j in cands:
        j = int(j)
        out.extend(range(grp * j, grp * j + grp) if j < n_tiles else [grp * n_tiles + j - n_tiles])
    return np.asarray(out, dtype=np.int64)


def candidates_of(blocks, n_tiles: int, grp: int):
    """Inverse of key_blocks_of; None unless every history tile is complete."""
    blocks = [int(b) for b in blocks]
    cands, i = [], 0
    while i < len(blocks):
        b = blocks[i]
        if b < grp * n_tiles:
            j = b // grp
            if b != grp * j or blocks[i:i + grp] != list(range(grp * j, grp * j + grp)):
                return None
            cands.append(j)
            i += grp
        else:
            cands.append(n_tiles + b - grp * n_tiles)
            i += 1
    return np.asarray(cands, dtype=np.int64)
