/* Page tiers of the KV bank -- host-side policy.
 *
 * WorldAttention paper, section 3.2 (the hierarchical KV bank): history pages
 * live in tiers, L1 GPU memory, L2 CPU DRAM and L3 NVMe, which keeps a full
 * backup so that any page can be restored; pages that are not selected sink
 * to the lower tier, least recently used first.  Structured summary, method
 * step (4), and its weaknesses discussion (prefetch the next chunk's pages
 * from pinned memory).
 *
 * This policy decides where every page is and which copies a request needs;
 * it moves no data.  The caller owns the L1 slots (device buffers), the L2
 * slots (pinned host buffers) and the L3 store, and runs the returned moves
 * in order (for example on one copy stream).  Pages are immutable once
 * written, so a page leaving L2 needs no copy (L3 holds it) and a page
 * leaving L1 is copied down only if L2 does not hold it.
 *
 * All pointers are host pointers; no call touches a GPU.  Not thread-safe:
 * one policy object per thread, or a lock around it.
 */
#ifndef HSA_TIER_H
#define HSA_TIER_H

#include <stdint.h>

#include "hsa_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct hsa_tier hsa_tier;  /* opaque */

typedef enum {
  HSA_MOVE_L2_TO_L1 = 0,  /* pinned host slot -> device slot */
  HSA_MOVE_L3_TO_L1 = 1,  /* backup store -> device slot */
  HSA_MOVE_L1_TO_L2 = 2   /* device slot -> pinned host slot (a page sinking) */
} hsa_tier_move_kind;

typedef struct {
  int32_t kind;      /* hsa_tier_move_kind */
  int32_t page;      /* page id */
  int32_t src_slot;  /* slot in the source tier (-1 for L3) */
  int32_t dst_slot;  /* slot in the destination tier */
} hsa_tier_move;

/* A policy for n_pages pages (ids 0..n_pages-1), all in L3 at first, with
 * l1_slots device slots and l2_slots pinned host slots (0 for no L2).
 * Returns NULL if n_pages < 1, l1_slots < 1, l2_slots < 0 or out of memory;
 * free with hsa_tier_destroy. */
hsa_tier* hsa_tier_create(int32_t n_pages, int32_t l1_slots, int32_t l2_slots);
void hsa_tier_destroy(hsa_tier* t);

/* Declare that pages[0..n) already sit in `tier` (1 = L1, 2 = L2), filling
 * free slots in order; slot_out[i] receives page i's slot.  For setting up a
 * bank whose data the caller has already placed.  HSA_ERR_BAD_PARAM if a page
 * is out of range, repeated or already in that tier, or the tier is full. */
hsa_rc hsa_tier_seed(hsa_tier* t, const int32_t* pages, int32_t n, int32_t tier, int32_t* slot_out);

/* Make pages[0..n) resident in L1 (distinct ids, n <= l1_slots), used now in
 * this order.  l1_slot[i] receives page i's device slot; moves[0..*n_moves)
 * receives the copies to run, in order, before those slots are read: for a
 * miss, the least recently used L1 page outside the request is evicted
 * (copied to L2 first if L2 lacks it, taking L2's least recently used slot
 * that holds no page of the request; with no such slot it is not copied and
 * L3 keeps it) and the page is loaded from L2 if there, else from L3.  At
 * most 2n moves;
 * max_moves must be >= 2n.  On error nothing changes: HSA_ERR_NULL_ARG,
 * HSA_ERR_BAD_PARAM (ids, n, max_moves). */
hsa_rc hsa_tier_request(hsa_tier* t, const int32_t* pages, int32_t n, int32_t* l1_slot, hsa_tier_move* moves,
                        int32_t max_moves, int32_t* n_moves);

/* Where a page is: its L1 and L2 slots, -1 where absent (L3 always holds it). */
hsa_rc hsa_tier_locate(const hsa_tier* t, int32_t page, int32_t* l1_slot, int32_t* l2_slot);

/* Counters since creation: out[0] pages requested, out[1] L1 hits, out[2]
 * loads from L2, out[3] loads from L3, out[4] L1 evictions, out[5] copies
 * L1 -> L2. */
hsa_rc hsa_tier_stats(const hsa_tier* t, int64_t* out);

#ifdef __cplusplus
}
#endif

#endif /* HSA_TIER_H */
