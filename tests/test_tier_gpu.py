"""Page tiers on the GPU: after every request of a random trace the device
slots hold exactly the requested pages (copied from pinned host slots or from
the backup store through the staging buffer), and a gather through the
tiers' page tables equals a gather from resident pages."""
import numpy as np
import pytest
import torch

from synth import M1, Workload

from gpu_harness import geom_of

pytestmark = pytest.mark.gpu


def test_page_tiers_hold_the_requested_pages():
    from sparse_linear_attention_hsa_amd.step import HsaStep
    from sparse_linear_attention_hsa_amd.tiers import PageTiers
    cfg = M1
    print(f"\n[tiers] {cfg.name}: {cfg.n_pages} pages, 2 device slots, 2 host slots", flush=True)
    w = Workload(cfg)
    pk_np, pv_np = w.pages()
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    tiers = PageTiers(pk_np, pv_np, l1_slots=cfg.n_sel_pages, l2_slots=2, dtype=dt, l2_pages=[cfg.n_pages - 1])
    rng = np.random.default_rng(3)
    main = torch.cuda.current_stream()
    for _ in range(25):
        pages = [int(p) for p in rng.choice(cfg.n_pages, size=int(rng.integers(1, cfg.n_sel_pages + 1)),
                                            replace=False)]
        slots = tiers.request(pages)
        main.wait_event(tiers.ready)
        torch.cuda.synchronize()
        for p, s in zip(pages, slots):
            assert torch.equal(tiers.l1_k[s].cpu(), tiers.l3_k[p]) and torch.equal(tiers.l1_v[s].cpu(), tiers.l3_v[p])
    st = tiers.policy.stats()
    assert st["from_l2"] > 0 and st["from_l3"] > 0 and st["l1_to_l2"] > 0 and st["l1_hits"] > 0, st
    # gather through the tiers' tables == gather from resident pages
    sel = sorted(int(p) for p in rng.choice(cfg.n_pages, size=cfg.n_sel_pages, replace=False))
    tiers.request(sel)
    main.wait_event(tiers.ready)
    geom = geom_of(cfg)
    a, b = HsaStep(geom, cfg.n_pages), HsaStep(geom, cfg.n_pages)
    for s in (a, b):
        s.sel_pages.copy_(torch.tensor(sel, dtype=torch.int32))
    pk_t, pv_t = tiers.tables()
    a.gather(pk_t, pv_t)
    b.gather([x.cuda() for x in tiers.l3_k], [x.cuda() for x in tiers.l3_v])
    torch.cuda.synchronize()
    assert torch.equal(a.k_act, b.k_act) and torch.equal(a.v_act, b.v_act) and torch.equal(a.kblk_mean, b.kblk_mean)
