"""The page-tier placement policy (library `hsa_tier_*`, host code only): a
hand-worked trace, the L2-less and seeded cases, a data-flow replay of random
traces, and argument checks.  WorldAttention paper, section 3.2 (GPU, CPU and
NVMe tiers; unselected pages sink to the lower tier, least recently used
first; NVMe keeps a full backup)."""
import ctypes

import numpy as np
import pytest

from sparse_linear_attention_hsa_amd import _lib
from sparse_linear_attention_hsa_amd.tiers import L1_TO_L2, L2_TO_L1, L3_TO_L1, TierPolicy


@pytest.fixture(scope="module", autouse=True)
def lib():
    return _lib.lib()


def test_hand_trace():
    """Two device slots, two host slots, five pages.  Worked by hand:
    1. [0,1]: both from L3 into slots 0, 1.
    2. [2]: page 0 is least recent; it sinks to L2 slot 0, page 2 comes from L3 into slot 0.
    3. [0,2]: page 1 (slot 1) is the only unpinned page; it sinks to L2 slot 1; page 0
       comes back from L2 slot 0 into slot 1; page 2 is a hit.
    4. [3]: page 0 (used before page 2 in step 3) is evicted; L2 still holds it, so no
       copy down; page 3 from L3 into slot 1.
    5. [1]: page 2 is evicted and sinks; L2's least recent page other than page 1 (which
       is about to be loaded from it) is page 0, in slot 0; page 1 from L2 slot 1."""
    t = TierPolicy(5, 2, 2)
    want = [
        ([0, 1], [0, 1], [(L3_TO_L1, 0, -1, 0), (L3_TO_L1, 1, -1, 1)]),
        ([2], [0], [(L1_TO_L2, 0, 0, 0), (L3_TO_L1, 2, -1, 0)]),
        ([0, 2], [1, 0], [(L1_TO_L2, 1, 1, 1), (L2_TO_L1, 0, 0, 1)]),
        ([3], [1], [(L3_TO_L1, 3, -1, 1)]),
        ([1], [0], [(L1_TO_L2, 2, 0, 0), (L2_TO_L1, 1, 1, 0)]),
    ]
    for pages, slots, moves in want:
        got_slots, got_moves = t.request(pages)
        assert got_slots == slots, pages
        assert got_moves == moves, pages
    assert [t.locate(j) for j in range(5)] == [(-1, -1), (0, 1), (-1, 0), (1, -1), (-1, -1)]
    assert t.stats() == dict(requested=7, l1_hits=1, from_l2=2, from_l3=4, l1_evictions=4, l1_to_l2=3)


def test_sinking_page_never_displaces_a_page_of_the_request():
    """Six pages, two device slots, two host slots; L1 holds {0, 1}, L2 holds
    {3, 2} (slots 0, 1).  Worked by hand for the request [2, 3]:
    - page 2 misses L1; the victim is page 0 (least recent, not requested).
      Both L2 slots hold pages of this request, so page 0 does not sink (L3
      keeps it); page 2 comes from L2 slot 1 into device slot 0.
    - page 3 misses L1; the victim is page 1, which does not sink either; page 3
      comes from L2 slot 0 into device slot 1.
    Both pages come from L2 and nothing is fetched from L3."""
    t = TierPolicy(6, 2, 2)
    assert t.seed([0, 1], 1) == [0, 1]
    assert t.seed([3, 2], 2) == [0, 1]
    slots, moves = t.request([2, 3])
    assert slots == [0, 1]
    assert moves == [(L2_TO_L1, 2, 1, 0), (L2_TO_L1, 3, 0, 1)]
    st = t.stats()
    assert st["from_l2"] == 2 and st["from_l3"] == 0 and st["l1_to_l2"] == 0 and st["l1_evictions"] == 2
    assert [t.locate(j) for j in range(6)] == [(-1, -1), (-1, -1), (0, 1), (1, 0), (-1, -1), (-1, -1)]
    # a later request with room in L2 lets a victim sink again: page 4 evicts
    # page 2 (least recent), whose L2 copy is still there, so no copy down
    slots, moves = t.request([4])
    assert slots == [0] and moves == [(L3_TO_L1, 4, -1, 0)]


def test_without_l2_pages_come_back_from_l3():
    t = TierPolicy(4, 2, 0)
    t.request([0, 1])
    _, moves = t.request([2])          # evicts page 0, nowhere to sink
    assert moves == [(L3_TO_L1, 2, -1, 0)]
    _, moves = t.request([0])          # evicts page 1 (least recent), page 0 from L3 again
    assert moves == [(L3_TO_L1, 0, -1, 1)]
    assert t.stats()["from_l3"] == 4 and t.stats()["l1_to_l2"] == 0


def test_seeded_l2_serves_the_first_request():
    t = TierPolicy(6, 2, 3)
    assert t.seed([4, 1], 2) == [0, 1]
    slots, moves = t.request([1, 5])
    assert slots == [0, 1]
    assert moves == [(L2_TO_L1, 1, 1, 0), (L3_TO_L1, 5, -1, 1)]
    # seeding a page twice, or beyond the free slots, is refused
    with pytest.raises(_lib.HsaError):
        t.seed([4], 2)
    with pytest.raises(_lib.HsaError):
        t.seed([0, 2, 3], 2)


@pytest.mark.parametrize("l1,l2", [(1, 0), (3, 2), (4, 8), (6, 3)])
def test_random_traces_replay(l1, l2):
    """Replaying the planned copies on a model of the slots' contents puts
    every requested page in its returned slot, keeps the policy's view
    (locate) equal to the contents, and never drops the only copy of a page
    (L3 holds all)."""
    rng = np.random.default_rng(100 * l1 + l2)
    P = 12
    t = TierPolicy(P, l1, l2)
    dev = [None] * l1
    host = [None] * l2
    for _ in range(200):
        n = int(rng.integers(1, l1 + 1))
        pages = [int(p) for p in rng.choice(P, size=n, replace=False)]
        slots, moves = t.request(pages)
        for kind, page, src, dst in moves:
            if kind == L1_TO_L2:
                assert dev[src] == page
                host[dst] = page
            elif kind == L2_TO_L1:
                assert host[src] == page
                dev[dst] = page
            else:
                assert src == -1
                dev[dst] = page
        assert [dev[s] for s in slots] == pages
        for j in range(P):
            s1, s2 = t.locate(j)
            assert (s1 >= 0) == (j in dev) and (s1 < 0 or dev[s1] == j)
            assert (s2 >= 0) == (j in host) and (s2 < 0 or host[s2] == j)
    st = t.stats()
    assert st["requested"] == st["l1_hits"] + st["from_l2"] + st["from_l3"]


def test_rejects_bad_requests_and_leaves_state_alone(lib):
    t = TierPolicy(5, 2, 1)
    t.request([0])
    before = t.stats()
    for pages in ([0, 0], [5], [-1], [0, 1, 2]):
        with pytest.raises(_lib.HsaError):
            t.request(pages)
    assert t.stats() == before and t.locate(0) == (0, -1)
    arr = (ctypes.c_int32 * 2)(1, 2)
    out = (ctypes.c_int32 * 2)()
    n = ctypes.c_int32()
    assert lib.hsa_tier_request(t._t, arr, 2, out, None, 4, ctypes.byref(n)) == 1      # NULL moves
    assert lib.hsa_tier_request(t._t, arr, 2, out, out, 3, ctypes.byref(n)) == 4       # max_moves < 2n
    assert lib.hsa_tier_create(0, 1, 0) is None and lib.hsa_tier_create(3, 0, 0) is None
    assert lib.hsa_tier_create(3, 1, -1) is None
