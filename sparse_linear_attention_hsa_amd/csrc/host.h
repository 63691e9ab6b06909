// Host-side geometry, validation and workspace layout of the HSA library.
// Plain C++ (no HIP), so the validation logic can be exercised without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "hsa_attn.h"

namespace hsa {

// Sizes derived from an hsa_geom.
struct Dims {
  int H, d, D, Lp, Lq, B, Kp, L, nKB, nQB, r;
  int split;  // intra_split: 0, or the chunk's own keys follow the history in B/split-token blocks
  int Bk;     // tokens per key block (B, or B / split)
  int Lh;     // keys of the retrieved pages (L = Lh, or Lh + Lq with intra-chunk keys)
  int nKBh;   // B-token history tiles, Lh / B
  int nC;     // selection candidates: nKB, or nKBh + Lq / Bk
  int bf16;  // 1 if dtype == HSA_BF16
  int esize; // bytes per element
  int rows;  // H * nQB selection rows
};

hsa_rc derive(const hsa_geom* g, Dims* out);

// Page-format buffers that hold the chunk's own keys when pages are read in
// place with intra-chunk keys: ceil(Lq / Lp) (0 without intra-chunk keys).
inline int chunk_pages(const Dims& s) { return s.split ? (s.Lq + s.Lp - 1) / s.Lp : 0; }

// Page scoring work split: units of `chunk_rows` tokens.
struct ScorePlan {
  int page_chunks;   // chunks per page
  int page_rows;     // tokens per page chunk (last one ragged)
  int q_chunks;      // chunks of the query buffer
  int q_rows;
  int units;         // n_pages * page_chunks + q_chunks
};
// few_pages: only a few of the n_pages will be read (scoring restricted to
// retrieved chunks), so every page is cut finer to keep the chip busy.
ScorePlan score_plan(const Dims& s, int n_pages, bool few_pages = false);

// Linear-branch projection split over the sequence axis.
struct ProjPlan {
  int splits;        // S: slices of the sequence axis per (head, K|V)
  int steps;         // contraction steps of the whole sequence
  int rtiles;        // ceil(r / 16)
  int rpad;          // r padded to four contraction steps (one round of the attention ring)
};
// n_tok: tokens the projection contracts (all L by default)
ProjPlan proj_plan(const Dims& s, int n_tok = -1);

// Linear-branch attention split: units of 32 queries of one head; a
// workgroup takes a run of units_per_wg of them.
struct AttendPlan {
  int units;         // ceil(Lq / 32) per head
  int units_per_wg;
  int wg_per_head;
};
AttendPlan attend_plan(const Dims& s);

// Sparse-branch segmentation of the selected-block rows.
// (head, key range) buckets the sparse plan kernel orders its work items by
// (counters in LDS)
constexpr int kPlanMaxBuckets = 2048;
// Segments per row the sparse plan handles (its per-row tables and the merge's
// LDS are sized for this many).
constexpr int kPlanMaxSegs = 64;

struct SparsePlan {
  int granules_per_block;  // Bk / 16
  int seg_granules;        // target granules per work item
  int max_segs;            // per row
  int max_items;           // rows * max_segs
  int grid;                // launch size (multiple of 8)
  int bucket_shift;        // items are ordered by (head, middle key block >> bucket_shift)
  int heads_per_phase;     // heads whose items all XCDs run before moving on to the next ones
};
// The sparse plan's metadata: {items, partial slots, first item of each head
// (H + 1 entries, the last = items), ..., per-XCD item indices in use (the
// last entry)}.
constexpr int kPlanMetaInts = 2 + 32 + 1 + 1;
SparsePlan sparse_plan(const Dims& s);

// Byte offsets inside the caller's workspace; each call uses the regions it
// needs, all starting at offset 0 of the same buffer.
struct WsLayout {
  // score
  size_t score_partial, score_qbar, score_kbar, score_end;
  // linear
  size_t lin_partial, lin_khi, lin_klo, lin_vt, lin_vlo, lin_ksum, lin_vsum, lin_end;
  // select
  size_t sel_qbar, sel_kbar, sel_logit, sel_end;
  // sparse
  size_t sp_items, sp_rowinfo, sp_meta, sp_part_o, sp_part_ml, sp_end;
  size_t total;
};
WsLayout ws_layout(const Dims& s, int n_pages);

}  // namespace hsa
