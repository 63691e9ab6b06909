/*
 * hsa_attn.h -- C ABI of the Hybrid Sparse Attention (HSA) decode step over
 * a paged KV cache, for AMD Instinct MI355X (gfx950).
 *
 * The method is WorldAttention's (paper "WorldAttention: An Efficient
 * Attention Architecture for Interactive Video World Models"): page-level
 * retrieval of history KV pages by mean-query / mean-key score, a contiguous
 * active KV buffer, a low-rank linear branch, a head-adaptive block-sparse
 * branch, and a sigmoid-gated fusion of the two branches.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor argument is a DEVICE pointer owned by the caller, except
 *    the page pointer tables (`page_k`, `page_v`), which are HOST arrays of
 *    device pointers.  The library never allocates or frees memory; scratch
 *    memory is the caller's workspace (size from hsa_workspace_bytes).
 *    Calls are re-entrant on different streams as long as they do not share
 *    a workspace.  The one exception, hsa_block_select_noalloc, keeps its
 *    scratch in a fixed device array of the library (see there).
 *  - Every call only enqueues work on `stream` (a hipStream_t; NULL is the
 *    default stream) and returns; results are valid once the stream has
 *    reached that point.  No call synchronises with the host, so a sequence
 *    of calls can be captured into a HIP graph.
 *  - All arguments are validated on the host before anything is launched;
 *    on any error nothing is launched and nothing is written, and the error
 *    code says why.  HSA_ERR_HIP reports a failed launch (hipGetLastError);
 *    faults inside a kernel surface at the caller's next synchronisation.
 *  - Element type: Q, page K/V, the active KV, X, E_K, E_V, W_g and the
 *    fused output all have the element type
 *    geom->dtype (HSA_F32 or HSA_BF16).  Scores, means, masses, thresholds,
 *    the projected K/V, the two branch outputs and gate overrides are float32.  Every reduction
 *    and every selection decision is computed in float32 (never rounded to
 *    bfloat16); the matrix products of the bf16 path take bf16 operands with
 *    float32 accumulation.
 *  - Token order: every token buffer is in tile-major order -- the sequence
 *    is cut into contiguous groups of B = tile_t*tile_h*tile_w tokens, one
 *    per (C_t, C_h, C_w) cube of the latent volume (paper, appendix A.1.3).
 *    The library itself needs no raster knowledge.
 *  - Sizes used below: H = n_heads, d = head_dim (64 or 128), D = H*d,
 *    Lp = frames_per_page*frame_h*frame_w (tokens per page),
 *    Lq = query_frames*frame_h*frame_w (query tokens of the chunk),
 *    B = tile_t*tile_h*tile_w, r = rank, P = n_pages,
 *    Lh = n_sel_pages*Lp (keys of the retrieved pages),
 *    s = intra_split, L = Lh (s = 0) or Lh + Lq (s > 0) active keys,
 *    Bk = B (s = 0) or B/s (s > 0) tokens per key block, nKB = L/Bk key
 *    blocks, nQB = Lq/B query blocks, nKBh = Lh/B,
 *    nC = nKB (s = 0) or nKBh + Lq/Bk (s > 0) selection candidates.
 *  - Intra-chunk keys (intra_split = s > 0; paper section 3.3, "Inter- and
 *    intra-chunk sparse granularity": the retrieved history is partitioned
 *    coarsely, the current chunk's own tokens finely, both through the same
 *    block-sparse interface).  The chunk's Lq tokens follow the Lh history
 *    keys in the active buffer.  Key blocks are Bk = B/s tokens: a B-token
 *    history tile is s consecutive key blocks, selected together as one
 *    candidate; each Bk-token block of the chunk is a candidate of its own.
 *    Bk-token blocks of the chunk are consecutive slices of its B-token tiles,
 *    so the caller orders the tokens inside a tile so that each slice is a
 *    sub-cube (e.g. a (4,6,4) tile as two (4,3,4) halves).
 */
#ifndef HSA_ATTN_H
#define HSA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HSA_ATTN_ABI_VERSION 3
#define HSA_MAX_PAGES 128      /* pages per call with HOST page tables (they travel as launch arguments) */
#define HSA_MAX_BANK_PAGES 8192 /* pages per call with DEVICE page tables (the *_devtab calls) */
#define HSA_MAX_KBLOCKS 2048   /* nKB limit of the block selection (one sort per row in LDS) */
#define HSA_MAX_INTRA_SPLIT 4  /* largest intra_split */
#define HSA_MAX_ROWS 4096      /* H * nQB limit (selection rows; the sparse branch plans them in LDS) */
#define HSA_MAX_CHUNKS 4096    /* previous chunks in prompt-level retrieval (ranked in LDS) */
#define HSA_MAX_EMBED 65536    /* prompt embedding width */

typedef enum {
  HSA_OK = 0,
  HSA_ERR_NULL_ARG = 1,    /* a required pointer is NULL                                */
  HSA_ERR_BAD_SHAPE = 2,   /* geometry inconsistent (a tile does not divide, sizes <= 0) */
  HSA_ERR_BAD_DTYPE = 3,   /* dtype not HSA_F32 / HSA_BF16                              */
  HSA_ERR_BAD_PARAM = 4,   /* n_pages, K_p, head_dim, rank or flags out of range        */
  HSA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than hsa_workspace_bytes         */
  HSA_ERR_HIP = 6          /* a HIP launch failed                                        */
} hsa_rc;

typedef enum { HSA_F32 = 0, HSA_BF16 = 1 } hsa_dtype;

typedef struct {
  int32_t n_heads, head_dim;             /* H, d (d in {64, 128})                        */
  int32_t frame_h, frame_w;              /* latent frame size; tokens/frame = frame_h*frame_w */
  int32_t frames_per_page, query_frames; /* frames in one KV page, frames in the query chunk */
  int32_t tile_t, tile_h, tile_w;        /* block cube (C_t, C_h, C_w); must divide the above;
                                            B = product, a multiple of 16, at most 192    */
  int32_t n_sel_pages, rank;             /* K_p (pages retrieved), r (linear-branch rank) */
  int32_t dtype;                         /* hsa_dtype                                     */
  int32_t intra_split;                   /* s: 0 = keys of the retrieved pages only;
                                            1..HSA_MAX_INTRA_SPLIT = the chunk's own tokens
                                            follow them in key blocks of B/s tokens
                                            (B/s a multiple of 16)                         */
} hsa_geom;

typedef struct ihipStream_t* hsa_stream;  /* a hipStream_t */
typedef struct ihipEvent_t* hsa_event;    /* a hipEvent_t  */

/* Linear-branch flags. */
#define HSA_LIN_REUSE_PROJ 1  /* skip the projection: k_proj / v_proj are inputs        */
#define HSA_LIN_PROJ_ONLY 2   /* only the projection: o_lin (and q) are not touched     */
#define HSA_LIN_HISTORY_PROJ 4 /* intra_split > 0: only the projection of the history keys
                                  [0, Lh) into k_proj / v_proj; o_lin (and q) untouched  */
#define HSA_LIN_CHUNK_PROJ 8   /* intra_split > 0: k_proj / v_proj hold the history's
                                  projection (in, unchanged); the chunk's keys [Lh, L) are
                                  projected, added to it, and the attention runs on the sum */

/* ---------------------------------------------------------------------------
 * S1 -- page-level retrieval.  Paper section 3.2, "Stage 2: page-level
 * retrieval" (score equation): alpha_j = Qbar . Kbar_j / sqrt(d), Qbar the
 * mean query of the chunk, Kbar_j the mean key of page j; the top-K_p pages
 * are retrieved.  Reading for several heads: the per-head dot products are
 * averaged, alpha_j = (1/H) sum_h Qbar_h . Kbar_{j,h} / sqrt(d).  Ties go to
 * the lower page id.
 *
 *  q           [Lq][H][d] dtype.
 *  page_k      HOST array of n_pages device pointers, page j's keys [Lp][H][d]
 *              dtype.  An entry may be NULL only if page_kmean is given: that
 *              page's mean is then read from page_kmean[j] (a page that is not
 *              resident in device memory is scored from its cached mean).
 *  page_kmean  [P][H][d] float32 or NULL.  For every non-NULL page the mean
 *              key is written here (a reusable page index); for NULL pages it
 *              is read.
 *  n_pages     1 <= P <= HSA_MAX_PAGES, K_p <= P.
 *  scores      [P] float32 out: alpha_j.  A score that comes out NaN (NaN or
 *              Inf in q or a page) is reported and ranked as -inf, so the
 *              order stays total and exactly K_p pages are retrieved.
 *  sel_pages   [K_p] int32 out: the retrieved page ids, ascending.
 *  ws          workspace of ws_bytes >= hsa_workspace_bytes(geom, n_pages).
 * Larger banks (up to HSA_MAX_BANK_PAGES pages) take a device page table:
 * hsa_score_pages_devtab below.
 * ------------------------------------------------------------------------- */
hsa_rc hsa_score_pages(const hsa_geom* geom, const void* q, const void* const* page_k,
                       float* page_kmean, int32_t n_pages, float* scores, int32_t* sel_pages,
                       void* ws, size_t ws_bytes, hsa_stream stream);

/* ---------------------------------------------------------------------------
 * Stage 1 -- prompt-level retrieval.  Paper section 3.2, "Stage 1:
 * prompt-level retrieval" (the cosine similarity between the current prompt
 * embedding and the previous chunks' prompt embeddings picks the top-1 chunk)
 * and section 4.5, ablation of prompt-level candidate chunks (Top-2, Top-4);
 * structured summary, method step (2).
 *
 *  prompt         [E] float32 device: the current chunk's prompt embedding.
 *  chunk_prompts  [C][E] float32 device: the previous chunks' embeddings.
 *  n_chunks       1 <= C <= HSA_MAX_CHUNKS.
 *  emb_dim        1 <= E <= HSA_MAX_EMBED.
 *  k_chunks       1 <= k <= C.
 *  sims           [C] float32 out: cosine similarities, fp32 sums; 0 where
 *                 either embedding is all zeros; -inf (ranked last) where
 *                 the similarity comes out NaN (NaN or Inf inputs).
 *  sel_chunks     [k] int32 out: the k most similar chunks (ties to the
 *                 lower id), ascending.
 * Errors: HSA_ERR_NULL_ARG, HSA_ERR_BAD_PARAM (sizes), HSA_ERR_HIP.
 * ------------------------------------------------------------------------- */
hsa_rc hsa_retrieve_chunks(const float* prompt, const float* chunk_prompts, int32_t n_chunks, int32_t emb_dim,
                           int32_t k_chunks, float* sims, int32_t* sel_chunks, hsa_stream stream);

/* ---------------------------------------------------------------------------
 * S1 over the retrieved chunks.  Paper section 3.2, "Stage 2: page-level
 * retrieval" (the pages of the chunks retrieved in stage 1 are scored) and
 * section 4.5 (under the same K_p-page budget, Top-2 takes two pages from each
 * chunk and Top-4 one page from each).
 *
 *  Arguments as hsa_score_pages, plus:
 *  page_chunk  [P] int32 device: the chunk of every page, in
 *              [0, HSA_MAX_CHUNKS).
 *  sel_chunks  [k_chunks] int32 device: distinct chosen chunk ids (the output
 *              of hsa_retrieve_chunks).
 *  k_chunks    1 <= k <= K_p and K_p % k == 0.
 *  Pages outside the chosen chunks are not read (their page_k entry may be
 *  NULL, with page_kmean given, as for any NULL entry) and score -inf.  The
 *  K_p pages are, in this order: the best K_p / k pages of each chosen chunk
 *  (higher score, ties to the lower id); if a chosen chunk has fewer pages,
 *  the best remaining pages of the chosen chunks; then the lowest other ids.
 *  sel_pages is ascending.
 * Errors: as hsa_score_pages; HSA_ERR_NULL_ARG for a NULL page_chunk or
 * sel_chunks, HSA_ERR_BAD_PARAM for k_chunks.
 * ------------------------------------------------------------------------- */
hsa_rc hsa_score_chunk_pages(const hsa_geom* geom, const void* q, const void* const* page_k, float* page_kmean,
                             int32_t n_pages, const int32_t* page_chunk, const int32_t* sel_chunks,
                             int32_t k_chunks, float* scores, int32_t* sel_pages, void* ws, size_t ws_bytes,
                             hsa_stream stream);

/* ---------------------------------------------------------------------------
 * S2 -- active KV construction.  Paper section 3.2, "Active KV construction";
 * structured summary, method step (4): the retrieved pages are concatenated
 * (ascending page id) into one contiguous buffer in device memory.
 *
 *  page_k, page_v  HOST arrays of n_pages non-NULL device pointers, each page
 *                  [Lp][H][d] dtype (token-major, as the model writes them).
 *  sel_pages       [K_p] int32 device, ascending ids in [0, n_pages) (the
 *                  output of hsa_score_pages).  Out-of-range ids are clamped.
 *  k_act           [H][L][d] dtype out: active keys, head-major.
 *  v_act           [H][L/16][d][16] dtype out: active values, head-major, in
 *                  16-token granules stored d-major (the transposed layout the
 *                  PV and projection products read).  Element (h, t, c) is at
 *                  ((h*(L/16) + t/16)*d + c)*16 + t%16.
 *  kblk_mean       [H][nKB][d] float32 out or NULL: mean key of every
 *                  Bk-token key block of the active buffer (input of
 *                  hsa_block_select).
 *  Requires intra_split = 0 (HSA_ERR_BAD_PARAM otherwise): a geometry with
 *  intra-chunk keys uses hsa_gather_active.
 * ------------------------------------------------------------------------- */
hsa_rc hsa_gather_pages(const hsa_geom* geom, const void* const* page_k, const void* const* page_v,
                        int32_t n_pages, const int32_t* sel_pages, void* k_act, void* v_act,
                        float* kblk_mean, hsa_stream stream);

/* S2 with the current chunk's own keys.  Paper section 3.3, "Inter- and
 * intra-chunk sparse granularity" (the current chunk's tokens join the
 * retrieved history in the block-sparse attention).  As hsa_gather_pages,
 * and the chunk's own keys and values follow the Lh history keys:
 *
 *  k_cur, v_cur  [Lq][H][d] dtype device (token-major, as q): the chunk's
 *                keys and values.  Required (non-NULL) iff intra_split > 0;
 *                with intra_split = 0 both must be NULL and the call is
 *                hsa_gather_pages.
 *  k_act, v_act  as hsa_gather_pages over L = Lh + Lq keys.
 *  kblk_mean     [H][nKB][d] float32 out or NULL: the mean of every
 *                Bk-token key block (history and chunk alike).
 * Errors: as hsa_gather_pages; HSA_ERR_NULL_ARG for a missing k_cur/v_cur,
 * HSA_ERR_BAD_PARAM for k_cur/v_cur given with intra_split = 0.
 * ------------------------------------------------------------------------- */
hsa_rc hsa_gather_active(const hsa_geom* geom, const void* const* page_k, const void* const* page_v,
                         int32_t n_pages, const int32_t* sel_pages, const void* k_cur, const void* v_cur,
                         void* k_act, void* v_act, float* kblk_mean, hsa_stream stream);

/* The chunk's part of the active buffer alone: writes tokens [Lh, L) of k_act
 * and v_act and the chunk's key-block means (key blocks nKBh*B/Bk .. nKB-1 of
 * kblk_mean) from k_cur / v_cur, leaving the history part as it is (section
 * 3.3: the chunk's own keys change with every denoising step, the retrieved
 * history does not).  Arguments as hsa_gather_active; requires
 * intra_split > 0 (HSA_ERR_BAD_PARAM otherwise).
 * ------------------------------------------------------------------------- */
hsa_rc hsa_gather_chunk(const hsa_geom* geom, const void* k_cur, const void* v_cur, void* k_act, void* v_act,
                        float* kblk_mean, hsa_stream stream);

/* ---------------------------------------------------------------------------
 * Page banks larger than HSA_MAX_PAGES: S1 and S2 with the page pointer
 * tables in DEVICE memory.  Paper section 3.2 (the full history stays
 * available and restorable, the page index is built from the keys); the
 * calls are those above with the same results, for 1 <= n_pages <=
 * HSA_MAX_BANK_PAGES.
 *
 *  page_k_table, page_v_table  DEVICE arrays of n_pages device pointers
 *              (pointer j is page j, as the host tables above).  The host
 *              does not read them, so their entries are not validated:
 *              - scoring: a NULL entry is scored from page_kmean[j]; with
 *                page_kmean NULL as well the page has no mean and scores
 *                -inf (it is chosen only when fewer than K_p pages have a
 *                score, lowest id first);
 *              - gather: a NULL entry among the selected pages contributes
 *                zeros to the active buffer.
 *  ws          workspace of ws_bytes >= hsa_workspace_bytes(geom, n_pages),
 *              which grows with n_pages (per-page partial sums and means).
 * Ranking: all n_pages scores are sorted on one workgroup (a bitonic sort of
 * 64-bit keys in LDS), so the selection is the same total order as the host
 * table calls: higher score, then lower id; NaN as -inf.
 * Errors: as the host-table calls, with HSA_MAX_BANK_PAGES for the page
 * count.
 * ------------------------------------------------------------------------- */
hsa_rc hsa_score_pages_devtab(const hsa_geom* geom, const void* q, const void* const* page_k_table,
                              float* page_kmean, int32_t n_pages, float* scores, int32_t* sel_pages,
                              void* ws, size_t ws_bytes, hsa_stream stream);
hsa_rc hsa_score_chunk_pages_devtab(const hsa_geom* geom, const void* q, const void* const* page_k_table,
                                    float* page_kmean, int32_t n_pages, const int32_t* page_chunk,
                                    const int32_t* sel_chunks, int32_t k_chunks, float* scores,
                                    int32_t* sel_pages, void* ws, size_t ws_bytes, hsa_stream stream);
hsa_rc hsa_gather_active_devtab(const hsa_geom* geom, const void* const* page_k_table,
                                const void* const* page_v_table, int32_t n_pages, const int32_t* sel_pages,
                                const void* k_cur, const void* v_cur, void* k_act, void* v_act,
                                float* kblk_mean, hsa_stream stream);

/* ---------------------------------------------------------------------------
 * S3 -- linear branch.  Paper section 3.3, "Linear branch" (output equation);
 * structured summary, prerequisite "linear attention": the sequence axis of
 * K and V is projected to rank r (Linformer), Ktil_h = E_K K_h, Vtil_h = E_V V_h,
 * and O_lin_h = softmax(Q_h Ktil_h^T / sqrt(d)) Vtil_h.  One E_K and one E_V
 * per layer, shared by all heads.
 *
 *  q            [Lq][H][d] dtype.
 *  k_act/v_act  as written by hsa_gather_pages.
 *  e_k, e_v     [r][L] dtype (the weight layout of a sequence-axis Linear).
 *  k_proj       [H][r][d] float32: out, or in with HSA_LIN_REUSE_PROJ.
 *  v_proj       [H][d][r] float32 (Vtil transposed): out, or in with REUSE.
 *               The projections stay in float32: with peaked heads |Q| is
 *               large and a bf16 copy of Ktil would move the logits by more
 *               than the output tolerance; the bf16 product splits Ktil into
 *               a bf16 high and low part instead.
 *  o_lin        [Lq][H][d] float32 out (untouched with HSA_LIN_PROJ_ONLY and
 *               HSA_LIN_HISTORY_PROJ).
 *  flags        0, HSA_LIN_REUSE_PROJ, HSA_LIN_PROJ_ONLY, HSA_LIN_HISTORY_PROJ or
 *               HSA_LIN_CHUNK_PROJ (one at a time).  The last two split the
 *               projection of a geometry with intra-chunk keys (section 3.3,
 *               "Inter- and intra-chunk sparse granularity") into the history's
 *               part, reused across denoising steps, and the chunk's part,
 *               whose keys change every step: Ktil = E_K[:, :Lh] K_hist +
 *               E_K[:, Lh:] K_chunk (and the same for V).  With
 *               HSA_LIN_CHUNK_PROJ the sum stays in the workspace.  Both
 *               return HSA_ERR_BAD_PARAM when intra_split = 0.
 *  With HSA_LIN_REUSE_PROJ, k_act, v_act, e_k and e_v may be NULL.
 *  ws           workspace of ws_bytes >= hsa_workspace_bytes(geom, 1), with
 *               every flag (the projection keeps its per-slice partial sums
 *               there, the attention its element-type copies of Ktil/Vtil).
 * ------------------------------------------------------------------------- */
hsa_rc hsa_linear_branch(const hsa_geom* geom, const void* q, const void* k_act, const void* v_act,
                         const void* e_k, const void* e_v, void* k_proj, void* v_proj, float* o_lin,
                         int32_t flags, void* ws, size_t ws_bytes, hsa_stream stream);

/* ---------------------------------------------------------------------------
 * S4 -- head-adaptive block selection.  Paper section 3.3, "Head-level
 * sparsity adaptation" (per head, the smallest set of blocks whose cumulative
 * attention mass passes tau_h) and appendix A.1.2 (a cheap coarse estimate of
 * where the mass lies); structured summary, method step (5) (block pooling).
 * Readings: blocks are mean-pooled; for query block i of head h the mass of
 * key block j is m_j = softmax_j(qbar_i . kbar_j / sqrt(d)); blocks are taken
 * in order of decreasing m (ties: lower j first) until the running sum is
 * >= tau_h; tau_h >= 1 keeps every block; at least one block is kept.
 *
 *  q          [Lq][H][d] dtype.
 *  With intra-chunk keys (intra_split = s > 0) the candidates j are the nC
 *  blocks of the two granularities: j < nKBh is the B-token history tile j
 *  (key blocks s*j .. s*j+s-1), j >= nKBh the chunk's Bk-token key block
 *  s*nKBh + (j - nKBh); each is pooled by the mean over its own tokens, and
 *  one softmax runs over all nC of them.  The output lists key blocks: a
 *  selected history tile contributes its s key blocks.
 *
 *  k_act      [H][L][d] dtype; may be NULL when kblk_mean is given.
 *  kblk_mean  [H][nKB][d] float32 or NULL (computed from k_act when NULL);
 *             the mean of a history tile is the mean of its s key-block means.
 *  tau        [H] float32, each > 0.
 *  blk_count  [H][nQB] int32 out: number of selected key blocks.
 *  blk_idx    [H][nQB][nKB] int32 out: selected key-block ids, ascending;
 *             entries past the count are -1.
 *  blk_mass   [H][nQB][nC] float32 out or NULL: the pooled masses m of the
 *             candidates.
 *  Requires nKB <= HSA_MAX_KBLOCKS.
 *  Precision: pooled means are float32; each pooled logit is accumulated in
 *  float64 (products of float32 values are exact there) and rounded to
 *  float32 once, so the selection does not depend on a summation order.
 * ------------------------------------------------------------------------- */
hsa_rc hsa_block_select(const hsa_geom* geom, const void* q, const void* k_act, const float* kblk_mean,
                        const float* tau, int32_t* blk_count, int32_t* blk_idx, float* blk_mass,
                        void* ws, size_t ws_bytes, hsa_stream stream);

/* ---------------------------------------------------------------------------
 * hsa_block_select without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc).  Same arguments, kernels and results as
 * hsa_block_select, bit for bit; the scratch (pooled query means, candidate
 * means, pooled logits) lives in a device array of HSA_NOALLOC_SCRATCH_BYTES
 * inside the library, which each GPU it runs on holds until the process
 * ends.  The call allocates nothing (no hipMalloc, no hipFree, no allocating
 * library routine); its first call on a device looks up that device's copy
 * of the array (hipGetSymbolAddress).
 *
 *  Size limit: a geometry whose selection scratch (the block-selection part
 *  of hsa_workspace_bytes: H*nQB*d + H*nKB*d + H*nQB*nKB floats, each part
 *  rounded up to 256 bytes) exceeds HSA_NOALLOC_SCRATCH_BYTES is rejected
 *  with HSA_ERR_WORKSPACE before anything is launched.  That covers 12 heads
 *  of d = 128 with 49,920 retrieved keys in 96-token blocks and 6,240
 *  queries, also with the chunk's own keys in 48-token blocks.
 *  Concurrency: every call on one GPU shares that GPU's array, so calls that
 *  overlap on one GPU (different streams, or different host threads without
 *  ordering) race and give undefined results; calls ordered on one stream
 *  are safe.  Nothing in the array needs to start at zero: each call writes
 *  every scratch element it reads.
 * ------------------------------------------------------------------------- */
#define HSA_NOALLOC_SCRATCH_BYTES (16u << 20)
hsa_rc hsa_block_select_noalloc(const hsa_geom* geom, const void* q, const void* k_act, const float* kblk_mean,
                                const float* tau, int32_t* blk_count, int32_t* blk_idx, float* blk_mass,
                                hsa_stream stream);

/* ---------------------------------------------------------------------------
 * S5 -- block-sparse attention.  Paper section 3.3, "Sparse branch" and
 * appendix A.1.3: attention at token resolution, computed only between a
 * query block and its selected key blocks: for query block i of head h,
 * O = softmax(Q_i K_S^T / sqrt(d)) V_S over exactly the tokens S of the
 * selected blocks.
 *
 *  q, k_act, v_act        as above.
 *  Key block j is the Bk tokens j*Bk .. j*Bk+Bk-1 of the active buffer.
 *  blk_count, blk_idx     as written by hsa_block_select.  Entries outside
 *                         [0, nKB) are skipped; a count is clamped to [0, nKB];
 *                         a row with no valid block gets zeros.
 *  o_sp                   [Lq][H][d] float32 out.
 * ------------------------------------------------------------------------- */
hsa_rc hsa_sparse_attn(const hsa_geom* geom, const void* q, const void* k_act, const void* v_act,
                       const int32_t* blk_count, const int32_t* blk_idx, float* o_sp,
                       void* ws, size_t ws_bytes, hsa_stream stream);

/* The same call, additionally recording ev_begin / ev_end on `stream`
 * immediately before and after the attention kernel itself (between the
 * small work-planning kernel that precedes it and the merge of split rows
 * that follows), so a caller can time the dominant kernel alone.  Either
 * event may be NULL (not recorded); both are caller-created hipEvent_t.
 * Errors as hsa_sparse_attn, plus HSA_ERR_HIP if recording fails. */
hsa_rc hsa_sparse_attn_timed(const hsa_geom* geom, const void* q, const void* k_act, const void* v_act,
                             const int32_t* blk_count, const int32_t* blk_idx, float* o_sp,
                             void* ws, size_t ws_bytes, hsa_stream stream,
                             hsa_event ev_begin, hsa_event ev_end);

/* ---------------------------------------------------------------------------
 * S6 -- gated fusion.  Paper section 3.3, "Gated fusion of two branches";
 * structured summary, method step (6): G = X W, sigmoid gates, and
 * O = O_lin * G_lin + O_sp * G_sp per head and token.  Reading: W has 2H
 * output columns (no bias); column h gates the linear branch of head h and
 * column H+h its sparse branch.
 *
 *  x              [Lq][D] dtype, or NULL to use gate_override.
 *  w_g            [2H][D] dtype (row c produces gate column c); unused when x is NULL.
 *  gate_override  [Lq][2H] float32 gate VALUES (after the sigmoid), used iff x == NULL.
 *  o_lin, o_sp    [Lq][H][d] float32.
 *  out            [Lq][H][d] dtype out.
 * ------------------------------------------------------------------------- */
hsa_rc hsa_fuse(const hsa_geom* geom, const void* x, const void* w_g, const float* gate_override,
                const float* o_lin, const float* o_sp, void* out, hsa_stream stream);

/* ---------------------------------------------------------------------------
 * Pages read in place (no active-buffer copy).  Paper section 3.2 (the
 * retrieved pages are what the attention reads; the page index is built from
 * the keys when pages are written) and the copy into the active buffer that
 * the pages' own profile names as the largest cost of the step.  A page is
 * laid out once, when it is written, in the layouts the kernels read: K as
 * [H][Lp][d] and V as [H][Lp/16][d][16] (the active buffer's layouts over
 * one page), with the mean of every key block [H][Lp/Bk][d] float32 (Bk = B,
 * or B / intra_split).  A step then scores from the page index
 * (hsa_score_pages with NULL page pointers and page_kmean), takes the
 * selected pages' block means (hsa_gather_block_means, for hsa_block_select
 * with k_act = NULL), and runs the linear and sparse branches straight from
 * the laid-out pages: active key t is token t % Lp of page sel_pages[t / Lp],
 * so every result is the one the active-buffer path computes.
 *
 * Intra-chunk keys (intra_split > 0; paper section 3.3, "Inter- and
 * intra-chunk sparse granularity"): the chunk's own keys and values are laid
 * out each step into hsa_chunk_page_count() page-format buffers
 * (hsa_chunk_prepare), which the caller adds to its page table.  sel_pages
 * then holds K_p + hsa_chunk_page_count() entries: the K_p selected pages
 * (as hsa_score_pages writes them) followed by the table indices of the
 * chunk's buffers in order, so the same rule reaches the chunk's key
 * t - Lh at token (t - Lh) % Lp of its buffer (t - Lh) / Lp.
 * ------------------------------------------------------------------------- */

/* Lay out one page: k_page, v_page [Lp][H][d] dtype (as the model writes
 * them) -> k_out [H][Lp][d], v_out [H][Lp/16][d][16] dtype, blk_mean
 * [H][Lp/Bk][d] float32 (or NULL).  The output buffers are the caller's and
 * must not overlap the inputs.  Errors: HSA_ERR_NULL_ARG, geometry errors. */
hsa_rc hsa_page_prepare(const hsa_geom* geom, const void* k_page, const void* v_page, void* k_out, void* v_out,
                        float* blk_mean, hsa_stream stream);

/* Page-format buffers that hold the chunk's own keys with intra-chunk keys:
 * ceil(Lq / Lp); 0 if the geometry is invalid or has intra_split = 0. */
int32_t hsa_chunk_page_count(const hsa_geom* geom);

/* Lay out the chunk's own keys and values for the paged calls (intra_split >
 * 0): k_cur, v_cur [Lq][H][d] dtype -> buffer j = 0 .. n-1 (n =
 * hsa_chunk_page_count) holds the chunk's tokens j*Lp .. min((j+1)*Lp, Lq)-1
 * in the page layout (k_out[j] [H][Lp][d], v_out[j] [H][Lp/16][d][16]
 * dtype, blk_mean[j] [H][Lp/Bk][d] float32); entries past the chunk's last
 * token are left as they are and never read.  k_out, v_out, blk_mean are HOST
 * arrays of n device pointers (blk_mean itself may be NULL).  Errors:
 * HSA_ERR_BAD_PARAM (intra_split = 0), HSA_ERR_NULL_ARG, geometry errors. */
hsa_rc hsa_chunk_prepare(const hsa_geom* geom, const void* k_cur, const void* v_cur, void* const* k_out,
                         void* const* v_out, float* const* blk_mean, hsa_stream stream);

/* kblk_mean [H][nKB][d] float32 out: the block means of the selected pages
 * (and with intra-chunk keys the chunk's), from page_blk_mean, a HOST array
 * of n_pages device pointers, each a page's blk_mean from hsa_page_prepare
 * or hsa_chunk_prepare.  sel_pages int32 device: [K_p] as hsa_gather_pages,
 * or [K_p + hsa_chunk_page_count] with intra-chunk keys (see above);
 * out-of-range ids are clamped.  Errors: HSA_ERR_NULL_ARG (any entry NULL),
 * HSA_ERR_BAD_PARAM (n_pages). */
hsa_rc hsa_gather_block_means(const hsa_geom* geom, const float* const* page_blk_mean, int32_t n_pages,
                              const int32_t* sel_pages, float* kblk_mean, hsa_stream stream);

/* hsa_linear_branch over laid-out pages: page_k, page_v are HOST arrays of
 * n_pages device pointers, each a page's k_out / v_out from hsa_page_prepare
 * (or, with intra-chunk keys, a chunk buffer from hsa_chunk_prepare);
 * sel_pages as above.  Other arguments, flags, workspace and errors as
 * hsa_linear_branch; with HSA_LIN_REUSE_PROJ the pages may be NULL.
 * HSA_ERR_BAD_SHAPE if a page holds fewer than 32 tokens. */
hsa_rc hsa_linear_branch_paged(const hsa_geom* geom, const void* q, const void* const* page_k,
                               const void* const* page_v, int32_t n_pages, const int32_t* sel_pages,
                               const void* e_k, const void* e_v, void* k_proj, void* v_proj, float* o_lin,
                               int32_t flags, void* ws, size_t ws_bytes, hsa_stream stream);

/* hsa_sparse_attn_timed over laid-out pages (page_k, page_v, n_pages,
 * sel_pages as hsa_linear_branch_paged); the events may be NULL.  Errors as
 * hsa_sparse_attn, plus HSA_ERR_BAD_PARAM for n_pages (a valid geometry keeps
 * one head of one page within the 32-bit offsets the kernel uses). */
hsa_rc hsa_sparse_attn_paged(const hsa_geom* geom, const void* q, const void* const* page_k,
                             const void* const* page_v, int32_t n_pages, const int32_t* sel_pages,
                             const int32_t* blk_count, const int32_t* blk_idx, float* o_sp, void* ws,
                             size_t ws_bytes, hsa_stream stream, hsa_event ev_begin, hsa_event ev_end);

/* The three paged calls above with their page tables in DEVICE memory, for
 * banks beyond HSA_MAX_PAGES: page_k_table, page_v_table (and
 * page_blk_mean_table) are device arrays of n_pages (<= HSA_MAX_BANK_PAGES)
 * device pointers, read by the kernels; a NULL entry is a page without a
 * laid-out buffer, which reads as zeros (as the gather of such a page writes
 * zeros into the active buffer).  Other arguments, results and errors as the
 * host-table calls, except that no entry is checked on the host. */
hsa_rc hsa_gather_block_means_devtab(const hsa_geom* geom, const float* const* page_blk_mean_table, int32_t n_pages,
                                     const int32_t* sel_pages, float* kblk_mean, hsa_stream stream);
hsa_rc hsa_linear_branch_paged_devtab(const hsa_geom* geom, const void* q, const void* const* page_k_table,
                                      const void* const* page_v_table, int32_t n_pages, const int32_t* sel_pages,
                                      const void* e_k, const void* e_v, void* k_proj, void* v_proj, float* o_lin,
                                      int32_t flags, void* ws, size_t ws_bytes, hsa_stream stream);
hsa_rc hsa_sparse_attn_paged_devtab(const hsa_geom* geom, const void* q, const void* const* page_k_table,
                                    const void* const* page_v_table, int32_t n_pages, const int32_t* sel_pages,
                                    const int32_t* blk_count, const int32_t* blk_idx, float* o_sp, void* ws,
                                    size_t ws_bytes, hsa_stream stream, hsa_event ev_begin, hsa_event ev_end);

/* Bytes of workspace every call above needs for this geometry and a bank of
 * n_pages pages (0 if the geometry is invalid or n_pages exceeds
 * HSA_MAX_BANK_PAGES).  One workspace serves all calls on one stream. */
size_t hsa_workspace_bytes(const hsa_geom* geom, int32_t n_pages);

/* Bytes of workspace hsa_linear_branch alone needs (0 if the geometry is
 * invalid): a second, smaller workspace lets the linear branch run on its own
 * stream beside block selection and the sparse branch, which use the first
 * one (the two branches meet only in hsa_fuse). */
size_t hsa_linear_workspace_bytes(const hsa_geom* geom);

/* Host-only validation of a geometry (HSA_OK or the reason it is invalid). */
hsa_rc hsa_geom_check(const hsa_geom* geom);

/* Static text of a return code. */
const char* hsa_rc_string(hsa_rc rc);

/* HSA_ATTN_ABI_VERSION of the built library. */
int32_t hsa_abi_version(void);

/* ---------------------------------------------------------------------------
 * Measurement helper, not part of the decode step: the bf16 matrix-core rate
 * this GPU sustains (the denominator of the "% of measured peak" figures the
 * benchmark reports beside the published peak).
 *
 *  n_workgroups  1 .. 65536 workgroups of 8 waves (one per CU at a time).
 *  iters         1 .. 2^20 rounds; each wave runs 32 independent
 *                16x16x32 bf16 products per round (16*16*32*2 flops each).
 *  out           device float32 buffer of n_workgroups * 512 values (written).
 *  ev_begin/end  hipEvent_t recorded around the launch, or NULL.
 * Flops of one call: n_workgroups * 8 * iters * 32 * 16384.
 * ------------------------------------------------------------------------- */
hsa_rc hsa_probe_mfma_bf16(int32_t n_workgroups, int32_t iters, float* out, hsa_stream stream,
                           hsa_event ev_begin, hsa_event ev_end);

/* Measurement helper, not part of the decode step: an HBM stream copy of
 * `bytes` (a multiple of 16, both pointers 16-byte aligned, buffers not
 * overlapping) from src to dst, 16 bytes per lane with non-temporal loads
 * and stores.  It moves 2 * bytes; the benchmark reports its rate as the
 * measured stream-copy peak. */
hsa_rc hsa_probe_hbm_copy(const void* src, void* dst, size_t bytes, hsa_stream stream, hsa_event ev_begin,
                          hsa_event ev_end);

#ifdef __cplusplus
}
#endif

#endif /* HSA_ATTN_H */
