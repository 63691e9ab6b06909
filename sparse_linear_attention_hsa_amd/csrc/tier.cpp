// Page tiers of the KV bank: the host-side placement policy (see hsa_tier.h).
// WorldAttention paper, section 3.2 (L1 GPU memory, L2 CPU DRAM, L3 NVMe with
// a full backup; unselected pages sink to the lower tier, least recently used
// first).  Plain C++; no GPU call.
#include <cstdint>
#include <new>
#include <vector>

#include "hsa_tier.h"

struct hsa_tier {
  int32_t n_pages = 0;
  std::vector<int32_t> l1_of, l2_of;      // page -> slot or -1
  std::vector<int32_t> l1_page, l2_page;  // slot -> page or -1
  std::vector<int64_t> l1_used, l2_used;  // slot -> last use (larger is later)
  int64_t clock = 0;
  int64_t stats[6] = {0, 0, 0, 0, 0, 0};
};

namespace {

// A free slot, else the least recently used one whose page is not pinned;
// -1 if there is none.
int32_t pick_slot(const std::vector<int32_t>& page_of_slot, const std::vector<int64_t>& used,
                  const std::vector<char>* pinned) {
  int32_t best = -1;
  for (int32_t s = 0; s < (int32_t)page_of_slot.size(); ++s) {
    const int32_t p = page_of_slot[s];
    if (p < 0) return s;
    if (pinned && (*pinned)[p]) continue;
    if (best < 0 || used[s] < used[best]) best = s;
  }
  return best;
}

bool valid_pages(const hsa_tier* t, const int32_t* pages, int32_t n, std::vector<char>& seen) {
  seen.assign(t->n_pages, 0);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t p = pages[i];
    if (p < 0 || p >= t->n_pages || seen[p]) return false;
    seen[p] = 1;
  }
  return true;
}

}  // namespace

extern "C" {

hsa_tier* hsa_tier_create(int32_t n_pages, int32_t l1_slots, int32_t l2_slots) {
  if (n_pages < 1 || l1_slots < 1 || l2_slots < 0) return nullptr;
  hsa_tier* t = new (std::nothrow) hsa_tier;
  if (!t) return nullptr;
  try {
    t->n_pages = n_pages;
    t->l1_of.assign(n_pages, -1);
    t->l2_of.assign(n_pages, -1);
    t->l1_page.assign(l1_slots, -1);
    t->l2_page.assign(l2_slots, -1);
    t->l1_used.assign(l1_slots, 0);
    t->l2_used.assign(l2_slots, 0);
  } catch (...) {
    delete t;
    return nullptr;
  }
  return t;
}

void hsa_tier_destroy(hsa_tier* t) { delete t; }

hsa_rc hsa_tier_seed(hsa_tier* t, const int32_t* pages, int32_t n, int32_t tier, int32_t* slot_out) {
  if (!t || (n > 0 && (!pages || !slot_out))) return HSA_ERR_NULL_ARG;
  if (n < 0 || (tier != 1 && tier != 2)) return HSA_ERR_BAD_PARAM;
  std::vector<char> seen;
  if (!valid_pages(t, pages, n, seen)) return HSA_ERR_BAD_PARAM;
  std::vector<int32_t>& of = tier == 1 ? t->l1_of : t->l2_of;
  std::vector<int32_t>& page_of = tier == 1 ? t->l1_page : t->l2_page;
  std::vector<int64_t>& used = tier == 1 ? t->l1_used : t->l2_used;
  int32_t free_slots = 0;
  for (int32_t p : page_of) free_slots += p < 0;
  for (int32_t i = 0; i < n; ++i)
    if (of[pages[i]] >= 0) return HSA_ERR_BAD_PARAM;
  if (n > free_slots) return HSA_ERR_BAD_PARAM;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t s = pick_slot(page_of, used, nullptr);  // a free one (checked above)
    page_of[s] = pages[i];
    of[pages[i]] = s;
    used[s] = ++t->clock;
    slot_out[i] = s;
  }
  return HSA_OK;
}

hsa_rc hsa_tier_request(hsa_tier* t, const int32_t* pages, int32_t n, int32_t* l1_slot, hsa_tier_move* moves,
                        int32_t max_moves, int32_t* n_moves) {
  if (!t || !n_moves || (n > 0 && (!pages || !l1_slot || !moves))) return HSA_ERR_NULL_ARG;
  if (n < 0 || n > (int32_t)t->l1_page.size() || max_moves < 2 * n) return HSA_ERR_BAD_PARAM;
  std::vector<char> pinned;
  if (!valid_pages(t, pages, n, pinned)) return HSA_ERR_BAD_PARAM;
  int32_t m = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t p = pages[i];
    ++t->stats[0];
    int32_t s = t->l1_of[p];
    if (s >= 0) {
      ++t->stats[1];
    } else {
      // a slot: free, or the least recently used page outside this request
      // (one exists: n <= l1_slots and the request's pages are distinct)
      s = pick_slot(t->l1_page, t->l1_used, &pinned);
      const int32_t victim = t->l1_page[s];
      if (victim >= 0) {
        ++t->stats[4];
        // the page sinks to L2, where the least recently used page outside
        // this request leaves (L3 still holds it); if every L2 slot holds a
        // page of this request, the victim does not sink (L3 keeps it)
        const int32_t s2 = t->l2_of[victim] < 0 ? pick_slot(t->l2_page, t->l2_used, &pinned) : -1;
        if (s2 >= 0) {
          const int32_t gone = t->l2_page[s2];
          if (gone >= 0) t->l2_of[gone] = -1;
          t->l2_page[s2] = victim;
          t->l2_of[victim] = s2;
          t->l2_used[s2] = ++t->clock;
          moves[m++] = hsa_tier_move{HSA_MOVE_L1_TO_L2, victim, s, s2};
          ++t->stats[5];
        }
        t->l1_of[victim] = -1;
      }
      const int32_t s2 = t->l2_of[p];
      if (s2 >= 0) {
        moves[m++] = hsa_tier_move{HSA_MOVE_L2_TO_L1, p, s2, s};
        t->l2_used[s2] = ++t->clock;
        ++t->stats[2];
      } else {
        moves[m++] = hsa_tier_move{HSA_MOVE_L3_TO_L1, p, -1, s};
        ++t->stats[3];
      }
      t->l1_page[s] = p;
      t->l1_of[p] = s;
    }
    t->l1_used[s] = ++t->clock;
    l1_slot[i] = s;
  }
  *n_moves = m;
  return HSA_OK;
}

hsa_rc hsa_tier_locate(const hsa_tier* t, int32_t page, int32_t* l1_slot, int32_t* l2_slot) {
  if (!t || !l1_slot || !l2_slot) return HSA_ERR_NULL_ARG;
  if (page < 0 || page >= t->n_pages) return HSA_ERR_BAD_PARAM;
  *l1_slot = t->l1_of[page];
  *l2_slot = t->l2_of[page];
  return HSA_OK;
}

hsa_rc hsa_tier_stats(const hsa_tier* t, int64_t* out) {
  if (!t || !out) return HSA_ERR_NULL_ARG;
  for (int k = 0; k < 6; ++k) out[k] = t->stats[k];
  return HSA_OK;
}

}  // extern "C"
