"""Page tiers of the KV bank: L1 device slots, L2 pinned host slots, L3 the
full backup.

WorldAttention paper, section 3.2 (the hierarchical KV bank: GPU memory, CPU
memory and NVMe with a full backup; pages not selected sink to the lower
tier, least recently used first) and the structured summary's weaknesses
discussion (prefetch the next chunk's pages from pinned memory).

The placement policy is the library's (`hsa_tier_*`, native C++): it decides
where every page goes and which copies a request needs.  `PageTiers` owns the
buffers and runs those copies on a copy stream.  L3 here is pageable host
memory standing in for the NVMe backup (a page comes back through a pinned
staging buffer, as it would from a file).
"""
from __future__ import annotations

import ctypes
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

from ._lib import check, lib

L2_TO_L1, L3_TO_L1, L1_TO_L2 = 0, 1, 2


class _Move(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("page", ctypes.c_int32), ("src_slot", ctypes.c_int32),
                ("dst_slot", ctypes.c_int32)]


class TierPolicy:
    """The library's placement policy for n_pages pages, l1 device slots and
    l2 pinned host slots (argument marshalling only)."""

    def __init__(self, n_pages: int, l1_slots: int, l2_slots: int):
        self._t = lib().hsa_tier_create(n_pages, l1_slots, l2_slots)
        if not self._t:
            raise ValueError("bad tier sizes")
        self.n_pages, self.l1_slots, self.l2_slots = n_pages, l1_slots, l2_slots

    def close(self):
        if self._t:
            lib().hsa_tier_destroy(self._t)
            self._t = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def seed(self, pages: Sequence[int], tier: int) -> List[int]:
        n = len(pages)
        arr = (ctypes.c_int32 * max(1, n))(*pages)
        out = (ctypes.c_int32 * max(1, n))()
        check("hsa_tier_seed", lib().hsa_tier_seed(self._t, arr, n, tier, out))
        return list(out)[:n]

    def request(self, pages: Sequence[int]) -> Tuple[List[int], List[Tuple[int, int, int, int]]]:
        n = len(pages)
        arr = (ctypes.c_int32 * max(1, n))(*pages)
        slots = (ctypes.c_int32 * max(1, n))()
        moves = (_Move * max(1, 2 * n))()
        n_moves = ctypes.c_int32(0)
        check("hsa_tier_request", lib().hsa_tier_request(self._t, arr, n, slots, moves, 2 * n,
                                                         ctypes.byref(n_moves)))
        return list(slots)[:n], [(m.kind, m.page, m.src_slot, m.dst_slot) for m in moves[:n_moves.value]]

    def locate(self, page: int) -> Tuple[int, int]:
        a, b = ctypes.c_int32(), ctypes.c_int32()
        check("hsa_tier_locate", lib().hsa_tier_locate(self._t, page, ctypes.byref(a), ctypes.byref(b)))
        return a.value, b.value

    def stats(self) -> dict:
        out = (ctypes.c_int64 * 6)()
        check("hsa_tier_stats", lib().hsa_tier_stats(self._t, out))
        keys = ("requested", "l1_hits", "from_l2", "from_l3", "l1_evictions", "l1_to_l2")
        return dict(zip(keys, list(out)))


class PageTiers:
    """K and V pages [Lp][H][d] of a bank in three tiers.  `request(pages)`
    makes the pages resident in device slots, enqueuing the copies on the copy
    stream after `after` (an event, e.g. the gather that last read the slots);
    `tables()` gives the page tables a gather reads; `ready` is recorded after
    the last copy."""

    def __init__(self, pages_k: Sequence[np.ndarray], pages_v: Sequence[np.ndarray], l1_slots: int,
                 l2_slots: int, dtype=torch.bfloat16, device: str = "cuda", l2_pages: Sequence[int] = ()):
        self.n_pages = len(pages_k)
        shape = tuple(pages_k[0].shape)
        dev = torch.device(device)
        # L3: the full backup (pageable host memory)
        self.l3_k = [torch.from_numpy(np.ascontiguousarray(p, dtype=np.float32)).to(dtype) for p in pages_k]
        self.l3_v = [torch.from_numpy(np.ascontiguousarray(p, dtype=np.float32)).to(dtype) for p in pages_v]
        self.l2_k = [torch.empty(shape, dtype=dtype, pin_memory=True) for _ in range(l2_slots)]
        self.l2_v = [torch.empty(shape, dtype=dtype, pin_memory=True) for _ in range(l2_slots)]
        self.l1_k = [torch.empty(shape, dtype=dtype, device=dev) for _ in range(l1_slots)]
        self.l1_v = [torch.empty(shape, dtype=dtype, device=dev) for _ in range(l1_slots)]
        self.stage_k = torch.empty(shape, dtype=dtype, pin_memory=True)
        self.stage_v = torch.empty(shape, dtype=dtype, pin_memory=True)
        self.policy = TierPolicy(self.n_pages, l1_slots, l2_slots)
        for j, s in zip(l2_pages, self.policy.seed(list(l2_pages), 2)):
            self.l2_k[s].copy_(self.l3_k[j])
            self.l2_v[s].copy_(self.l3_v[j])
        self.stream = torch.cuda.Stream(device=dev)  # default priority
        self.ready: Optional[torch.cuda.Event] = None
        self.bytes_moved = 0

    def request(self, pages: Sequence[int], after: Optional[torch.cuda.Event] = None) -> List[int]:
        slots, moves = self.policy.request([int(p) for p in pages])
        with torch.cuda.stream(self.stream):
            if after is not None:
                self.stream.wait_event(after)
            for kind, page, src, dst in moves:
                if kind == L1_TO_L2:
                    self.l2_k[dst].copy_(self.l1_k[src], non_blocking=True)
                    self.l2_v[dst].copy_(self.l1_v[src], non_blocking=True)
                elif kind == L2_TO_L1:
                    self.l1_k[dst].copy_(self.l2_k[src], non_blocking=True)
                    self.l1_v[dst].copy_(self.l2_v[src], non_blocking=True)
                else:  # from the backup through the pinned staging buffer
                    self.stream.synchronize()  # the staging buffer's last copy is done
                    self.stage_k.copy_(self.l3_k[page])
                    self.stage_v.copy_(self.l3_v[page])
                    self.l1_k[dst].copy_(self.stage_k, non_blocking=True)
                    self.l1_v[dst].copy_(self.stage_v, non_blocking=True)
                self.bytes_moved += 2 * self.l1_k[0].numel() * self.l1_k[0].element_size()
            self.ready = torch.cuda.Event()
            self.ready.record(self.stream)
        return slots

    def tables(self) -> Tuple[List[torch.Tensor], List[torch.Tensor]]:
        """Page tables over the bank: a resident page's device slot, any slot
        for the others (a gather reads only the selected pages, which the
        caller has requested)."""
        pk, pv = [], []
        for j in range(self.n_pages):
            s, _ = self.policy.locate(j)
            s = max(s, 0)
            pk.append(self.l1_k[s])
            pv.append(self.l1_v[s])
        return pk, pv
