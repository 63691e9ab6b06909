// Host-side geometry validation, work plans and workspace layout.
#include "host.h"

#include <algorithm>

namespace hsa {

namespace {
inline int cdiv(int a, int b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
}  // namespace

hsa_rc derive(const hsa_geom* g, Dims* o) {
  if (!g) return HSA_ERR_NULL_ARG;
  if (g->dtype != HSA_F32 && g->dtype != HSA_BF16) return HSA_ERR_BAD_DTYPE;
  if (g->head_dim != 64 && g->head_dim != 128) return HSA_ERR_BAD_PARAM;
  if (g->n_heads < 1 || g->n_heads > 32) return HSA_ERR_BAD_PARAM;
  if (g->n_sel_pages < 1 || g->rank < 1 || g->rank > 256) return HSA_ERR_BAD_PARAM;
  if (g->frame_h < 1 || g->frame_w < 1 || g->frames_per_page < 1 || g->query_frames < 1 ||
      g->tile_t < 1 || g->tile_h < 1 || g->tile_w < 1)
    return HSA_ERR_BAD_SHAPE;
  if (g->frame_h % g->tile_h || g->frame_w % g->tile_w || g->frames_per_page % g->tile_t ||
      g->query_frames % g->tile_t)
    return HSA_ERR_BAD_SHAPE;
  const long long B = 1LL * g->tile_t * g->tile_h * g->tile_w;
  if (B % 16 || B > 192) return HSA_ERR_BAD_SHAPE;
  const int split = g->intra_split;
  if (split < 0 || split > HSA_MAX_INTRA_SPLIT) return HSA_ERR_BAD_PARAM;
  const long long Bk = split ? B / split : B;
  if (split && (B % split || Bk % 16)) return HSA_ERR_BAD_SHAPE;
  const long long tpf = 1LL * g->frame_h * g->frame_w;
  const long long Lp = tpf * g->frames_per_page, Lq = tpf * g->query_frames;
  const long long Lh = Lp * g->n_sel_pages;
  const long long L = Lh + (split ? Lq : 0);
  const long long D = 1LL * g->n_heads * g->head_dim;
  // every buffer index must fit comfortably in 32-bit element offsets per head
  if (Lp > (1LL << 24) || Lq > (1LL << 24) || L > (1LL << 24) || L * D > (1LL << 31) ||
      Lq * D > (1LL << 31) || Lp * D > (1LL << 31))
    return HSA_ERR_BAD_SHAPE;
  if (L / Bk > HSA_MAX_KBLOCKS) return HSA_ERR_BAD_SHAPE;
  if (1LL * g->n_heads * (Lq / B) > HSA_MAX_ROWS) return HSA_ERR_BAD_SHAPE;
  Dims s;
  s.H = g->n_heads; s.d = g->head_dim; s.D = (int)D;
  s.Lp = (int)Lp; s.Lq = (int)Lq; s.B = (int)B; s.Kp = g->n_sel_pages; s.L = (int)L;
  s.nKB = (int)(L / Bk); s.nQB = (int)(Lq / B); s.r = g->rank;
  s.split = split; s.Bk = (int)Bk; s.Lh = (int)Lh; s.nKBh = (int)(Lh / B);
  s.nC = split ? s.nKBh + (int)(Lq / Bk) : s.nKB;
  s.bf16 = g->dtype == HSA_BF16; s.esize = s.bf16 ? 2 : 4;
  s.rows = s.H * s.nQB;
  if (o) *o = s;
  return HSA_OK;
}

ScorePlan score_plan(const Dims& s, int n_pages, bool few_pages) {
  ScorePlan p;
  const int target = 640;
  // chunk-restricted scoring reads few pages: each is split into up to 64
  // chunks, fewer in large banks so the partials stay small
  const int few = std::max(1, std::min(64, 8192 / std::max(1, n_pages)));
  int pc = std::max(1, std::min(cdiv(s.Lp, 16), few_pages ? few : cdiv(target, std::max(1, n_pages))));
  p.page_rows = cdiv(s.Lp, pc);
  p.page_chunks = cdiv(s.Lp, p.page_rows);
  int qc = std::max(1, std::min(cdiv(s.Lq, 16), 128));
  p.q_rows = cdiv(s.Lq, qc);
  p.q_chunks = cdiv(s.Lq, p.q_rows);
  p.units = n_pages * p.page_chunks + p.q_chunks;
  return p;
}

ProjPlan proj_plan(const Dims& s, int n_tok) {
  ProjPlan p;
  const int K = s.bf16 ? 32 : 16;
  p.steps = std::max(1, cdiv(n_tok < 0 ? s.L : n_tok, K));  // stages of one contraction step
  // At most one workgroup (8 waves, two heads, 128 KB of LDS) fits on a CU,
  // so the items must not exceed the CUs: one item more would run in a
  // second round and double the kernel's time.  They take at most 224 of the
  // 256 CUs: the projection runs beside block selection and the start of
  // the sparse branch, which need CUs of their own (with all 256 the step
  // was 2-3% slower on the long-row workloads, and no faster otherwise).
  p.splits = std::max(1, std::min(p.steps, 224 / (2 * ((s.H + 1) / 2))));
  p.rtiles = cdiv(s.r, 16);
  // the linear attention streams the rank axis in chunks of K ranks through
  // a ring of four LDS slots, whole rounds of the ring per pass
  p.rpad = cdiv(s.r, 4 * K) * 4 * K;
  return p;
}

AttendPlan attend_plan(const Dims& s) {
  AttendPlan p;
  p.units = cdiv(s.Lq, 32);
  // one round of workgroups over the 256 CUs (a workgroup holds a head's
  // projected keys in LDS, so one fits per CU at the largest rank)
  const int per_head = std::max(1, std::min(p.units, 256 / std::max(1, s.H)));
  p.units_per_wg = cdiv(p.units, per_head);
  p.wg_per_head = cdiv(p.units, p.units_per_wg);
  return p;
}

SparsePlan sparse_plan(const Dims& s) {
  SparsePlan p;
  p.granules_per_block = s.Bk / 16;
  // segments of about 24 query-tile-sized blocks' worth of granules (even, so
  // two-granule steps never straddle segments), and short enough that one
  // spans at most 64 key blocks: the kernel keeps a segment's block ids one
  // per lane.  Shorter segments cover shorter key ranges, so the items an XCD
  // runs together share more of its L2 (at 49,920 keys, simulated hits 49%
  // at 32 blocks, 58% at 24), at the price of more split-row partials.
  const int seg_blocks = 24;
  int sg = seg_blocks * (s.B / 16);
  // no row may need more than kPlanMaxSegs segments
  sg = std::max(sg, cdiv(s.nKB * p.granules_per_block, kPlanMaxSegs));
  if (sg & 1) sg += 1;
  while ((sg - 1) / p.granules_per_block + 2 > 64) sg -= 2;
  p.seg_granules = sg;
  p.max_segs = cdiv(s.nKB * p.granules_per_block, sg);
  p.max_items = s.rows * p.max_segs;
  // Phases of heads: all XCDs run the items of heads_per_phase heads, each
  // XCD one contiguous range of them, before any starts on the next heads, so
  // the K/V that the misses of the XCDs' L2s fetch at one time (those heads'
  // active keys and values) stays within about 128 MB of the 256 MB
  // last-level cache.
  const double head_kv_bytes = 2.0 * s.L * s.d * s.esize;
  p.heads_per_phase = std::max(1, std::min(s.H, (int)(128.0 * (1 << 20) / head_kv_bytes)));
  const int phases = cdiv(s.H, p.heads_per_phase);
  // every phase rounds its items up to whole multiples of 8 (one per XCD)
  p.grid = (cdiv(p.max_items, 8) + phases) * 8;
  // key ranges of 8 blocks or more, and at most kPlanMaxBuckets (head, range) buckets
  p.bucket_shift = 3;
  while (s.H * cdiv(s.nKB, 1 << p.bucket_shift) > kPlanMaxBuckets) ++p.bucket_shift;
  return p;
}

WsLayout ws_layout(const Dims& s, int n_pages) {
  WsLayout w;
  const size_t hd = (size_t)s.H * s.d;
  // score
  const ScorePlan sp = score_plan(s, n_pages), spf = score_plan(s, n_pages, true);
  w.score_partial = 0;
  w.score_qbar = align256(w.score_partial + (size_t)std::max(sp.units, spf.units) * hd * 4);
  w.score_kbar = align256(w.score_qbar + hd * 4);
  w.score_end = align256(w.score_kbar + (size_t)n_pages * hd * 4);
  // linear
  ProjPlan pp = proj_plan(s);
  w.lin_partial = 0;
  const size_t kbytes = (size_t)s.H * pp.rpad * s.d * s.esize;  // one [H][rpad][d] operand
  w.lin_khi = align256((size_t)pp.splits * 2 * s.H * pp.rtiles * 16 * s.d * 4);
  w.lin_klo = align256(w.lin_khi + kbytes);
  w.lin_vt = align256(w.lin_klo + kbytes);
  w.lin_vlo = align256(w.lin_vt + kbytes);
  // float32 K~ and V~^T summed from the history and the chunk (HSA_LIN_CHUNK_PROJ)
  w.lin_ksum = align256(w.lin_vlo + kbytes);
  w.lin_vsum = align256(w.lin_ksum + (size_t)s.H * s.r * s.d * 4);
  w.lin_end = align256(w.lin_vsum + (size_t)s.H * s.r * s.d * 4);
  // select
  w.sel_qbar = 0;
  w.sel_kbar = align256((size_t)s.H * s.nQB * s.d * 4);
  w.sel_logit = align256(w.sel_kbar + (size_t)s.H * s.nKB * s.d * 4);
  w.sel_end = align256(w.sel_logit + (size_t)s.rows * s.nKB * 4);
  // sparse
  SparsePlan qp = sparse_plan(s);
  w.sp_items = 0;
  w.sp_rowinfo = align256((size_t)qp.max_items * 16);
  w.sp_meta = align256(w.sp_rowinfo + (size_t)s.rows * 8);
  w.sp_part_o = align256(w.sp_meta + (size_t)kPlanMetaInts * 4);
  w.sp_part_ml = align256(w.sp_part_o + (size_t)qp.max_items * s.B * s.d * 4);
  w.sp_end = align256(w.sp_part_ml + (size_t)qp.max_items * s.B * 2 * 4);
  w.total = std::max(std::max(w.score_end, w.lin_end), std::max(w.sel_end, w.sp_end));
  return w;
}

}  // namespace hsa

extern "C" {

size_t hsa_workspace_bytes(const hsa_geom* geom, int32_t n_pages) {
  hsa::Dims s;
  if (hsa::derive(geom, &s) != HSA_OK) return 0;
  if (n_pages < 1) n_pages = 1;
  if (n_pages > HSA_MAX_BANK_PAGES) return 0;
  return hsa::ws_layout(s, n_pages).total;
}

size_t hsa_linear_workspace_bytes(const hsa_geom* geom) {
  hsa::Dims s;
  if (hsa::derive(geom, &s) != HSA_OK) return 0;
  return hsa::ws_layout(s, 1).lin_end;
}

hsa_rc hsa_geom_check(const hsa_geom* geom) { return hsa::derive(geom, nullptr); }

const char* hsa_rc_string(hsa_rc rc) {
  switch (rc) {
    case HSA_OK: return "HSA_OK";
    case HSA_ERR_NULL_ARG: return "HSA_ERR_NULL_ARG: a required pointer is NULL";
    case HSA_ERR_BAD_SHAPE: return "HSA_ERR_BAD_SHAPE: inconsistent geometry";
    case HSA_ERR_BAD_DTYPE: return "HSA_ERR_BAD_DTYPE: dtype must be HSA_F32 or HSA_BF16";
    case HSA_ERR_BAD_PARAM: return "HSA_ERR_BAD_PARAM: parameter out of range";
    case HSA_ERR_WORKSPACE: return "HSA_ERR_WORKSPACE: workspace missing or too small";
    case HSA_ERR_HIP: return "HSA_ERR_HIP: a HIP launch failed";
  }
  return "unknown hsa_rc";
}

int32_t hsa_abi_version(void) { return HSA_ATTN_ABI_VERSION; }

}  // extern "C"
