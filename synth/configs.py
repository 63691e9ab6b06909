"""Shapes of the HSA decode-step workloads.

Only geometry lives here (how many heads, tokens, blocks ...); no step of the
attention method is computed in this module.

Token order: every token buffer (queries, page keys/values, gate input) is
already in tile-major order: the flattened sequence is cut into contiguous
groups of B = tile_t*tile_h*tile_w tokens, one group per (C_t, C_h, C_w) cube
of the latent volume (WorldAttention paper, appendix A.1.3, block-sparse
attention: every contiguous group of B tokens is one cube).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Tuple


@dataclass(frozen=True)
class Config:
    name: str
    n_heads: int
    head_dim: int
    frame_h: int
    frame_w: int
    frames_per_page: int
    query_frames: int
    tile: Tuple[int, int, int]
    n_pages: int
    n_sel_pages: int
    rank: int
    dtype: str                      # "f32" or "bf16": element type of every tensor input
    structure: str = "rank8"        # "plain" | "rank8" | "imbalance"
    tau: Tuple[float, ...] = ()     # fixed per-head thresholds; empty -> drawn U[tau_lo, tau_hi]
    tau_range: Tuple[float, float] = (0.80, 0.98)
    struct_scale: float = 3.0       # s of the rank-8 spatial structure
    mu_norm: float = 2.0            # norm of the planted per-page key mean
    q_shift: float = 0.5            # query shift along the planted direction
    hot_scale: float = 4.0          # imbalance config: scale of the planted hot blocks
    hot_per_row: int = 3            # imbalance config: hot key blocks per query block
    uniform_heads: int = 4          # imbalance config: heads with iid keys
    layers: int = 1
    steps: int = 1
    host_page_frac: float = 0.0     # stack config: share of selected pages that live in host memory
    intra_split: int = 0            # 0, or the chunk's own keys join the history in B/s-token blocks
    seed: int = 1000

    # ---- derived geometry -------------------------------------------------
    @property
    def tokens_per_frame(self) -> int:
        return self.frame_h * self.frame_w

    @property
    def page_tokens(self) -> int:        # Lp
        return self.frames_per_page * self.tokens_per_frame

    @property
    def query_tokens(self) -> int:       # Lq
        return self.query_frames * self.tokens_per_frame

    @property
    def block(self) -> int:              # B
        t, h, w = self.tile
        return t * h * w

    @property
    def history_tokens(self) -> int:     # Lh: keys of the retrieved pages
        return self.n_sel_pages * self.page_tokens

    @property
    def active_tokens(self) -> int:      # L: history, then the chunk's own tokens with intra_split
        return self.history_tokens + (self.query_tokens if self.intra_split else 0)

    @property
    def n_kblocks(self) -> int:          # B-token history tiles
        return self.history_tokens // self.block

    @property
    def key_block(self) -> int:          # Bk: tokens per key block
        return self.block // self.intra_split if self.intra_split else self.block

    @property
    def n_key_blocks(self) -> int:       # nKB: key blocks of the active buffer
        return self.active_tokens // self.key_block

    @property
    def n_candidates(self) -> int:       # nC: selection candidates
        return self.n_kblocks + (self.query_tokens // self.key_block if self.intra_split else 0)

    @property
    def n_qblocks(self) -> int:          # nQB
        return self.query_tokens // self.block

    @property
    def model_dim(self) -> int:          # D = H*d
        return self.n_heads * self.head_dim

    @property
    def blocks_per_page(self) -> int:
        return self.page_tokens // self.block

    def check(self) -> None:
        t, h, w = self.tile
        assert self.frame_h % h == 0 and self.frame_w % w == 0, "tile must divide the frame"
        assert self.frames_per_page % t == 0 and self.query_frames % t == 0, "tile_t must divide page/chunk frames"
        assert self.block % 16 == 0, "block must be a multiple of 16 tokens"
        assert 1 <= self.n_sel_pages <= self.n_pages
        assert self.dtype in ("f32", "bf16")
        if self.intra_split:
            assert self.block % self.intra_split == 0 and self.key_block % 16 == 0, "B/s must be a multiple of 16"


def _c1(**kw) -> Config:
    base = dict(name="c1_full", n_heads=12, head_dim=128, frame_h=30, frame_w=52,
                frames_per_page=8, query_frames=4, tile=(4, 6, 4), n_pages=16,
                n_sel_pages=4, rank=256, dtype="bf16", structure="rank8", seed=1001)
    base.update(kw)
    return Config(**base)


# The five workloads of the scope table, by index.
C0 = Config(name="c0_tiny", n_heads=2, head_dim=64, frame_h=6, frame_w=8,
            frames_per_page=2, query_frames=1, tile=(1, 2, 8), n_pages=6,
            n_sel_pages=2, rank=16, dtype="f32", structure="plain",
            tau=(0.7, 0.9), seed=1000)
C1 = _c1()
C2 = _c1(name="c2_long_history", n_pages=120, tau=(0.95,) * 6 + (0.99,) * 6, seed=1002)
C3 = _c1(name="c3_head_imbalance", structure="imbalance", tau=(0.9,) * 12, seed=1003)
C4 = _c1(name="c4_stack", layers=30, steps=4, host_page_frac=0.3, seed=1004)

# Small parity workloads: several tiles per kernel, ragged tails, fast on the CPU oracle.
M1 = Config(name="m1_bf16_d128", n_heads=3, head_dim=128, frame_h=12, frame_w=8,
            frames_per_page=4, query_frames=2, tile=(2, 6, 8), n_pages=6,
            n_sel_pages=3, rank=64, dtype="bf16", structure="rank8",
            tau=(0.6, 0.85, 1.0), struct_scale=2.0, seed=2001)
M2 = Config(name="m2_bf16_d64_ragged", n_heads=2, head_dim=64, frame_h=6, frame_w=8,
            frames_per_page=3, query_frames=2, tile=(1, 6, 8), n_pages=7,
            n_sel_pages=3, rank=32, dtype="bf16", structure="rank8",
            tau=(0.75, 0.95), struct_scale=2.0, seed=2002)
M3 = Config(name="m3_bf16_long_rows", n_heads=2, head_dim=128, frame_h=24, frame_w=16,
            frames_per_page=4, query_frames=2, tile=(2, 6, 8), n_pages=10,
            n_sel_pages=8, rank=128, dtype="bf16", structure="rank8",
            tau=(0.97, 1.0), struct_scale=2.0, seed=2003)
M4 = Config(name="m4_f32_d128", n_heads=2, head_dim=128, frame_h=6, frame_w=8,
            frames_per_page=2, query_frames=2, tile=(1, 6, 8), n_pages=5,
            n_sel_pages=3, rank=24, dtype="f32", structure="rank8",
            tau=(0.8, 0.97), struct_scale=2.0, seed=2004)
M5 = Config(name="m5_bf16_imbalance", n_heads=4, head_dim=128, frame_h=12, frame_w=8,
            frames_per_page=4, query_frames=4, tile=(2, 6, 8), n_pages=8,
            n_sel_pages=4, rank=32, dtype="bf16", structure="imbalance",
            tau=(0.9,) * 4, uniform_heads=1, hot_per_row=2, seed=2005)

# Small layer stack: the chunk schedule (projection reuse, host-resident pages
# streamed through two staging slots) at parity-test size.
M6 = replace(M1, name="m6_stack", layers=4, steps=2, host_page_frac=0.5, seed=2006)
CONFIGS = {c.name: c for c in (C0, C1, C2, C3, C4, M1, M2, M3, M4, M5, M6)}
BY_INDEX = (C0, C1, C2, C3, C4)

for _c in CONFIGS.values():
    _c.check()


def with_(cfg: Config, **kw) -> Config:
    return replace(cfg, **kw)
