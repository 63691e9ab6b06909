"""Block selection without a workspace (the library's own device scratch)
against block selection with a caller workspace, through the C ABI: two
calls in a row on one GPU, the second on a smaller input, each bit for bit
equal to the workspace call, and the second also against the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import hsa_oracle as orc
from sparse_linear_attention_hsa_amd import ops
from synth import C3, M1

from gpu_harness import Run, check_block_selection, gpu_block_lists, host

pytestmark = pytest.mark.gpu


def _both(r: Run, use_kblk_mean: bool):
    """(workspace call, scratch call) outputs on the step's own inputs."""
    st = r.step
    kbm = st.kblk_mean if use_kblk_mean else None
    out = []
    for noalloc in (False, True):
        cnt = torch.full_like(st.blk_count, -7)
        idx = torch.full_like(st.blk_idx, -7)
        mass = torch.full_like(st.blk_mass, float("nan"))
        if noalloc:
            ops.hsa_block_select_noalloc(st.geom, r.q, st.k_act, kbm, r.tau, cnt, idx, mass)
        else:
            ops.hsa_block_select(st.geom, r.q, st.k_act, kbm, r.tau, cnt, idx, mass, st.ws)
        torch.cuda.synchronize()
        out.append((cnt, idx, mass))
    return out


def test_noalloc_block_select_matches_workspace_call_twice():
    print("\n[no-alloc] call 1: c3_head_imbalance full size", flush=True)
    big = Run(C3)
    big.run()
    (c0, i0, m0), (c1, i1, m1) = _both(big, use_kblk_mean=True)
    assert torch.equal(c0, c1) and torch.equal(i0, i1) and torch.equal(m0, m1)
    assert torch.equal(c1, big.step.blk_count) and torch.equal(i1, big.step.blk_idx)
    del big
    torch.cuda.empty_cache()

    print("[no-alloc] call 2: m1 (smaller), candidate means pooled from the active keys", flush=True)
    small = Run(M1)
    small.run()
    (c0, i0, m0), (c1, i1, m1) = _both(small, use_kblk_mean=False)
    assert torch.equal(c0, c1) and torch.equal(i0, i1) and torch.equal(m0, m1)
    # and against the oracle
    st = small.step
    st.blk_count.copy_(c1)
    st.blk_idx.copy_(i1)
    lists, _, _ = gpu_block_lists(st)
    ref = small.oracle(sel_pages=host(st.sel_pages).astype(np.int64))
    check_block_selection(ref["blocks"], lists, small.np["tau"])
    np.testing.assert_allclose(host(m1), ref["blocks"]["mass"], rtol=0, atol=1e-5)
